"""The C-ABI library builds, loads and exports every symbol include/pld.h
declares, and rejects bad arguments on the host before touching the GPU
(these tests make no compute call and need no GPU)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from prompt_lookup_gram_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pld.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pld_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_symbols() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_library_is_gfx950_hip_code():
    data = open(B.LIB_PATH, "rb").read()
    assert b"gfx950" in data
    assert b"pld_scan" in data


def test_strerror_strings():
    assert B.pld_strerror(B.PLD_OK) == "success"
    assert B.pld_strerror(B.PLD_EINVAL) == "invalid argument"
    assert B.pld_strerror(B.PLD_ECAPACITY) == "history capacity exceeded"
    assert B.pld_strerror(99) == "unknown status"


def _raw(fn, *args):
    return getattr(B.load(), fn)(*args)


def test_null_context_rejected():
    assert _raw("pld_draft_batch", None, None, None, 0, 4, 12, 16, None, None,
                None, None) == B.PLD_EINVAL
    assert "ctx is null" in B.pld_last_error()
    assert _raw("pld_append", None, None, 0, None, 0, None) == B.PLD_EINVAL
    assert _raw("pld_configure", None, 4096, 1) == B.PLD_EINVAL
    assert _raw("pld_sync", None, None) == B.PLD_EINVAL
    assert _raw("pld_store_reset", None, None) == B.PLD_EINVAL
    assert _raw("pld_destroy", None) == B.PLD_OK


@pytest.mark.parametrize("max_batch,max_len,msg", [(0, 10, "max_batch"),
                                                   (-3, 10, "max_batch"),
                                                   (4, 0, "max_len"),
                                                   (4, -1, "max_len")])
def test_create_rejects_bad_sizes_before_any_hip_call(max_batch, max_len, msg):
    ctx = ctypes.c_void_p()
    assert _raw("pld_create", ctypes.byref(ctx), max_batch, max_len, 0, None) == B.PLD_EINVAL
    assert msg in B.pld_last_error()
    assert ctx.value is None


def test_create_rejects_null_out():
    assert _raw("pld_create", None, 4, 10, 0, None) == B.PLD_EINVAL


@pytest.mark.parametrize("max_len", [2**31, 2**31 + 5, 2**40])
def test_create_rejects_max_len_past_the_key_field(max_len):
    """max_len is int64 in the ABI; a position must fit the low 32 bits of
    the packed key, so 2^31 and above are refused before any HIP call."""
    ctx = ctypes.c_void_p()
    for fn, extra in (("pld_create", (0,)), ("pld_create_indexed", (4, 12)),
                      ("pld_create_ngram", (4,))):
        assert _raw(fn, ctypes.byref(ctx), 4, max_len, *extra, None) == B.PLD_EINVAL
        assert "max_len" in B.pld_last_error()
        assert ctx.value is None


# The boundary's calls and argument types as the scope table of the hot path
# names them (pld_create with an int64 max_len and a stream; pld_histories for
# the store's device views; the draft call over row pointers and lengths).
SCOPE_PROTOTYPES = {
    "pld_create": "pld_status pld_create(pld_ctx **out, int32_t max_batch, int64_t max_len, "
                  "int32_t own_store, hipStream_t stream);",
    "pld_destroy": "pld_status pld_destroy(pld_ctx *ctx);",
    "pld_append": "pld_status pld_append(pld_ctx *ctx, const int32_t *tokens, "
                  "int64_t tokens_stride, const int32_t *counts, int32_t batch, "
                  "hipStream_t stream);",
    "pld_histories": "pld_status pld_histories(pld_ctx *ctx, const int32_t *const **histories, "
                     "const int32_t **lengths);",
    "pld_draft_batch": "pld_status pld_draft_batch(pld_ctx *ctx, const int32_t *const *histories, "
                       "const int32_t *lengths, int32_t batch, int32_t n_min, int32_t n_max, "
                       "int32_t k_max, int32_t *out_draft, int32_t *out_len, "
                       "int32_t *out_match, hipStream_t stream);",
    "pld_draft_batch_pos": "pld_status pld_draft_batch_pos(pld_ctx *ctx, "
                           "const int32_t *const *histories, const int32_t *lengths, "
                           "int32_t batch, int32_t n_min, int32_t n_max, int32_t k_max, "
                           "int32_t *out_draft, int32_t *out_len, int32_t *out_match, "
                           "int32_t *out_pos, hipStream_t stream);",
    "pld_sync": "pld_status pld_sync(pld_ctx *ctx, hipStream_t stream);",
    "pld_strerror": "const char *pld_strerror(pld_status status);",
}


def _prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"([a-z_ *]+?\b(pld_[a-z_]+)\s*\([^;]*\);)", text):
        out[m.group(2)] = " ".join(m.group(1).split()).replace("( ", "(")
    return out


@pytest.mark.parametrize("name", sorted(SCOPE_PROTOTYPES))
def test_header_matches_scope_prototype(name):
    assert _prototypes()[name] == SCOPE_PROTOTYPES[name]


def test_scan_tile_query_rejects_bad_arguments():
    t = ctypes.c_int32()
    assert _raw("pld_scan_tile", None, 1, ctypes.byref(t)) == B.PLD_EINVAL
    assert "null" in B.pld_last_error()


def test_python_wrapper_raises_with_detail():
    with pytest.raises(B.PldError) as e:
        B.pld_create(0, 5)
    assert e.value.status == B.PLD_EINVAL and "max_batch" in str(e.value)


def test_fuse_params_default_is_the_page_setting():
    """HyperQwen lookup-drafting page, steps 2 and 3: 7-token drafter head,
    15 draft positions, 8 / 6 with 2 agreeing / 4, two near-full steps, hold
    3; near-full slack 1 is the reading taken where the page gives no number."""
    p = B.pld_fuse_params_default()
    assert [getattr(p, f) for f, _ in p._fields_] == [7, 15, 8, 6, 2, 4, 2, 3, 1]
    assert _raw("pld_fuse_params_default", None) == B.PLD_EINVAL


def test_fuse_null_context_or_params_rejected():
    p = B.pld_fuse_params_default()
    args = (None, 16, None, None, None, None, None, 0, None, None, None, None)
    assert _raw("pld_fuse", None, ctypes.byref(p), *args) == B.PLD_EINVAL
    assert "ctx is null" in B.pld_last_error()


def test_create_indexed_rejects_bad_lengths_before_any_hip_call():
    ctx = ctypes.c_void_p()
    for lo, hi in [(0, 4), (5, 4), (1, 65)]:
        assert _raw("pld_create_indexed", ctypes.byref(ctx), 4, 100, lo, hi,
                    None) == B.PLD_EINVAL
        assert "n_min" in B.pld_last_error()
    assert _raw("pld_draft_store", None, 1, 4, 12, 16, None, None, None, None,
                None) == B.PLD_EINVAL


def test_control_params_default():
    """Strata prompt-lookup page, sections 1 and 5: MTP drafts 3 tokens, the
    lookup must be 5% better; the rest are the readings stated in pld.h."""
    p = B.pld_control_params_default()
    assert (p.alpha, p.beta, p.margin, p.prior_accept, p.prior_time, p.mtp_tokens) == \
        (0.1, 0.1, 1.05, 0.5, 1.0, 3)
    assert list(p.bucket_edge) == [6, 8, 12]


def test_ngram_params_default():
    """llama.cpp page, its context cache: n-grams of sizes 1 to 4; the
    4-gram seen at least once with its top successor at half or more,
    used for every length."""
    p = B.pld_ngram_params_default()
    assert (p.n_min, p.n_max) == (1, 4)
    assert list(p.min_count) == [1, 1, 1, 1] and list(p.min_percent) == [50, 50, 50, 50]


def test_create_ngram_rejects_bad_lengths_before_any_hip_call():
    ctx = ctypes.c_void_p()
    for n_max in (0, 5, -1):
        assert _raw("pld_create_ngram", ctypes.byref(ctx), 4, 100, n_max, None) == B.PLD_EINVAL
        assert "n_max" in B.pld_last_error()
    p = B.pld_ngram_params_default()
    assert _raw("pld_draft_ngram", None, ctypes.byref(p), 1, 16, None, None, None,
                None) == B.PLD_EINVAL
    assert "ctx is null" in B.pld_last_error()


def test_noalloc_rejects_sizes_before_any_hip_call():
    """The no-allocation entry point refuses a batch above its static
    reduction state's size and a max_len past the key's position field,
    on the host, before touching the GPU."""
    i = ctypes.c_int32
    for batch, max_len, msg in ((B.PLD_NOALLOC_MAX_BATCH + 1, 100, "batch"),
                                (4, 2**31, "max_len"), (4, 0, "max_len"), (-1, 100, "batch")):
        st = _raw("pld_draft_batch_noalloc", None, None, i(batch), ctypes.c_int64(max_len),
                  i(4), i(12), i(16), None, None, None, None, None, None)
        assert st == B.PLD_EINVAL
        assert msg in B.pld_last_error()
    assert _raw("pld_draft_batch_noalloc", None, None, 0, 100, 4, 12, 16, None, None, None,
                None, None, None) == B.PLD_OK
