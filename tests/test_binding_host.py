"""Host-side helpers of the binding that lay batches out for the C ABI
(CPU only: the buffers are built on the host device)."""

from __future__ import annotations

import numpy as np

from prompt_lookup_gram_amd import binding as B


def test_strided_batch_fields():
    # min_len is the shortest history: the strided call trusts it as a lower
    # bound on every length (a bound of 0 would only switch the read-ahead
    # off, so a wrong value here changes speed, not results)
    hs = [np.arange(n, dtype=np.int32) for n in (900, 17, 300, 64)]
    sb = B.StridedBatch(hs, device="cpu")
    assert sb.batch == 4
    assert sb.min_len == 17
    assert sb.max_len == 900
    assert sb.stride >= 900 and sb.stride % 64 == 0
    assert sb.buf.shape == (4, sb.stride)
    assert sb.lengths.tolist() == [900, 17, 300, 64]
    for b, h in enumerate(hs):
        assert np.array_equal(sb.buf[b, :len(h)].numpy(), h)
        assert not sb.buf[b, len(h):].numpy().any()


def test_strided_batch_equal_lengths_pin_min_len():
    # rows of one length fill their stride when it is a multiple of the
    # alignment: min_len then equals the stride (the pinned-length case)
    hs = [np.full(4096, b, dtype=np.int32) for b in range(3)]
    sb = B.StridedBatch(hs, device="cpu")
    assert sb.min_len == sb.max_len == sb.stride == 4096


def test_strided_batch_degenerate():
    sb = B.StridedBatch([], device="cpu")
    assert sb.batch == 0 and sb.min_len == 0 and sb.max_len == 1
    sb = B.StridedBatch([np.zeros(0, np.int32), np.zeros(0, np.int32)], device="cpu")
    assert sb.min_len == 0 and sb.max_len == 1 and sb.stride == 64
    sb = B.StridedBatch([np.arange(5, dtype=np.int32)], device="cpu", stride=8)
    assert sb.stride == 8 and sb.min_len == 5
