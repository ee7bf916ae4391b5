"""ctypes binding for libpld (include/pld.h), with the same entry-point names.

Argument marshalling only: every step of the drafting path runs in the HIP
kernels of ``libpld.so``. Tensors must be int32, contiguous and on the GPU;
raw device pointers (Python ints) are accepted too. The stream defaults to
PyTorch's current stream. If ``libpld.so`` cannot be loaded the calls raise:
there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpld.so")

PLD_OK = 0
PLD_EINVAL = 1
PLD_ENOMEM = 2
PLD_EHIP = 3
PLD_ECAPACITY = 4
PLD_N_MAX_LIMIT = 64
PLD_FUSE_STATE_WORDS = 4
PLD_FUSE_MAX_POSITIONS = 64

# every symbol include/pld.h declares
EXPORTS = ("pld_create", "pld_create_indexed", "pld_destroy", "pld_configure", "pld_append",
           "pld_histories", "pld_store_reset", "pld_scan_tile", "pld_draft_batch",
           "pld_draft_batch_pos", "pld_draft_batch_noalloc", "pld_draft_batch_strided",
           "pld_index_fingerprint_bits",
           "pld_draft_store", "pld_append_draft_store",
           "pld_fuse_params_default",
           "pld_fuse", "pld_draft_fuse_batch", "pld_control_params_default", "pld_control",
           "pld_ngram_params_default", "pld_create_ngram", "pld_draft_ngram",
           "pld_append_draft_ngram", "pld_draft_control_batch",
           "pld_sync", "pld_strerror",
           "pld_last_error")

_lib = None


class PldFuseParams(ctypes.Structure):
    """pld_fuse_params (include/pld.h): fusion and long-block scheduling
    parameters; pld_fuse_params_default() gives the HyperQwen page's values."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "head", "positions_long", "replace_min", "agree_min", "agree_tokens",
        "tail_min", "entry_steps", "sticky", "near_full_slack")]


class PldControlParams(ctypes.Structure):
    """pld_control_params (include/pld.h); pld_control_params_default() gives
    the defaults (the Strata page's margin 1.05 and 3 MTP tokens)."""
    _fields_ = [("alpha", ctypes.c_double), ("beta", ctypes.c_double),
                ("margin", ctypes.c_double), ("prior_accept", ctypes.c_double),
                ("prior_time", ctypes.c_double), ("mtp_tokens", ctypes.c_int32),
                ("bucket_edge", ctypes.c_int32 * 3)]


PLD_CONTROL_STATE_WORDS = 11
PLD_SOURCE_PLAIN, PLD_SOURCE_MTP, PLD_SOURCE_LOOKUP = 0, 1, 2

PLD_NGRAM_MAX_N = 4


class PldNgramParams(ctypes.Structure):
    """pld_ngram_params (include/pld.h); pld_ngram_params_default() gives the
    llama.cpp page's context-cache thresholds for every length."""
    _fields_ = [("n_min", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("min_count", ctypes.c_int32 * PLD_NGRAM_MAX_N),
                ("min_percent", ctypes.c_int32 * PLD_NGRAM_MAX_N)]


class PldError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn}: {pld_strerror(status)} ({status}): {detail}")


def load(path: str = LIB_PATH):
    """Load libpld.so (building it in-tree first if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "pld_create": [ctypes.POINTER(vp), i32, i64, i32, vp],
        "pld_create_indexed": [ctypes.POINTER(vp), i32, i64, i32, i32, vp],
        "pld_destroy": [vp],
        "pld_configure": [vp, i32, i32],
        "pld_append": [vp, vp, i64, vp, i32, vp],
        "pld_histories": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp)],
        "pld_store_reset": [vp, vp],
        "pld_draft_batch": [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp],
        "pld_draft_batch_pos": [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp],
        "pld_draft_batch_noalloc": [vp, vp, i32, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp],
        "pld_draft_batch_strided": [vp, vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp,
                                    vp, vp],
        "pld_index_fingerprint_bits": [vp, i32],
        "pld_append_draft_store": [vp, vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp],
        "pld_draft_store": [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp],
        "pld_fuse_params_default": [ctypes.POINTER(PldFuseParams)],
        "pld_fuse": [vp, ctypes.POINTER(PldFuseParams), vp, i32, vp, vp, vp, vp, vp, i32,
                     vp, vp, vp, vp],
        "pld_draft_fuse_batch": [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp,
                                 ctypes.POINTER(PldFuseParams), vp, vp, vp, vp, vp, vp, vp],
        "pld_control_params_default": [ctypes.POINTER(PldControlParams)],
        "pld_control": [vp, ctypes.POINTER(PldControlParams), vp, vp, vp, vp, vp, i32, vp, vp,
                        vp],
        "pld_ngram_params_default": [ctypes.POINTER(PldNgramParams)],
        "pld_create_ngram": [ctypes.POINTER(vp), i32, i64, i32, vp],
        "pld_scan_tile": [vp, i32, ctypes.POINTER(i32)],
        "pld_draft_ngram": [vp, ctypes.POINTER(PldNgramParams), i32, i32, vp, vp, vp, vp],
        "pld_append_draft_ngram": [vp, vp, i64, vp, i32, ctypes.POINTER(PldNgramParams), i32,
                                   vp, vp, vp, vp],
        "pld_draft_control_batch": [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp,
                                    ctypes.POINTER(PldControlParams), vp, vp, vp, vp, vp, vp],
        "pld_sync": [vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.pld_strerror.argtypes = [ctypes.c_int]
    lib.pld_strerror.restype = ctypes.c_char_p
    lib.pld_last_error.argtypes = []
    lib.pld_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_ptr(x, name: str, dtype=None) -> int:
    """Device pointer of a GPU tensor (checked), or a raw pointer int."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or a device pointer")
    if x.device.type != "cuda":
        raise ValueError(f"{name}: tensor must be on the GPU (got {x.device})")
    if not x.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name}: dtype must be {dtype} (got {x.dtype})")
    return x.data_ptr()


def _check(fn: str, status: int):
    if status != PLD_OK:
        raise PldError(fn, status, pld_last_error())


def _i32():
    import torch
    return torch.int32


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------


def pld_strerror(status: int) -> str:
    return load().pld_strerror(int(status)).decode()


def pld_last_error() -> str:
    return load().pld_last_error().decode()


def _create_stream(stream) -> int:
    """The stream a pld_create* call clears the context on: the null stream
    unless one is given (the call waits for it either way)."""
    return 0 if stream is None else _stream(stream)


def pld_create(max_batch: int, max_len: int, own_store: bool = False, stream=None) -> int:
    ctx = ctypes.c_void_p()
    _check("pld_create", load().pld_create(ctypes.byref(ctx), int(max_batch),
                                           int(max_len), int(bool(own_store)),
                                           _create_stream(stream)))
    return ctx.value


def pld_create_indexed(max_batch: int, max_len: int, n_min: int, n_max: int,
                       stream=None) -> int:
    """A context with a history store and an n-gram index over it."""
    ctx = ctypes.c_void_p()
    _check("pld_create_indexed", load().pld_create_indexed(
        ctypes.byref(ctx), int(max_batch), int(max_len), int(n_min), int(n_max),
        _create_stream(stream)))
    return ctx.value


def pld_create_ngram(max_batch: int, max_len: int, n_max: int = PLD_NGRAM_MAX_N,
                     stream=None) -> int:
    """A context with a history store and a successor-count cache over it."""
    ctx = ctypes.c_void_p()
    _check("pld_create_ngram", load().pld_create_ngram(
        ctypes.byref(ctx), int(max_batch), int(max_len), int(n_max), _create_stream(stream)))
    return ctx.value


def pld_scan_tile(ctx: int, batch: int) -> int:
    """Candidate positions per scan workgroup that a draft call of `batch`
    requests on this context uses."""
    t = ctypes.c_int32()
    _check("pld_scan_tile", load().pld_scan_tile(ctx, int(batch), ctypes.byref(t)))
    return t.value


def pld_destroy(ctx: int) -> None:
    _check("pld_destroy", load().pld_destroy(ctx))


def pld_configure(ctx: int, tile_tokens: int = 0, fused_gather: int = -1) -> None:
    _check("pld_configure", load().pld_configure(ctx, int(tile_tokens),
                                                 int(fused_gather)))


def pld_append(ctx: int, tokens, tokens_stride: int, counts, batch: int,
               stream=None) -> None:
    i32 = _i32()
    _check("pld_append", load().pld_append(
        ctx, _dev_ptr(tokens, "tokens", i32), int(tokens_stride),
        _dev_ptr(counts, "counts", i32), int(batch), _stream(stream)))


def pld_histories(ctx: int):
    """(histories, lengths) device pointers of the context's store."""
    h, n = ctypes.c_void_p(), ctypes.c_void_p()
    _check("pld_histories", load().pld_histories(ctx, ctypes.byref(h),
                                                     ctypes.byref(n)))
    return h.value, n.value


def pld_store_reset(ctx: int, stream=None) -> None:
    _check("pld_store_reset", load().pld_store_reset(ctx, _stream(stream)))


def pld_draft_batch(ctx: int, histories, lengths, batch: int, n_min: int,
                    n_max: int, k_max: int, out_draft, out_len, out_match,
                    stream=None) -> None:
    import torch
    i32 = _i32()
    _check("pld_draft_batch", load().pld_draft_batch(
        ctx, _dev_ptr(histories, "histories", torch.int64),
        _dev_ptr(lengths, "lengths", i32), int(batch), int(n_min), int(n_max),
        int(k_max), _dev_ptr(out_draft, "out_draft", i32),
        _dev_ptr(out_len, "out_len", i32), _dev_ptr(out_match, "out_match", i32),
        _stream(stream)))


def pld_draft_batch_pos(ctx: int, histories, lengths, batch: int, n_min: int,
                        n_max: int, k_max: int, out_draft, out_len, out_match,
                        out_pos, stream=None) -> None:
    import torch
    i32 = _i32()
    _check("pld_draft_batch_pos", load().pld_draft_batch_pos(
        ctx, _dev_ptr(histories, "histories", torch.int64),
        _dev_ptr(lengths, "lengths", i32), int(batch), int(n_min), int(n_max),
        int(k_max), _dev_ptr(out_draft, "out_draft", i32),
        _dev_ptr(out_len, "out_len", i32), _dev_ptr(out_match, "out_match", i32),
        _dev_ptr(out_pos, "out_pos", i32), _stream(stream)))


PLD_NOALLOC_MAX_BATCH = 4096


def pld_draft_batch_noalloc(histories, lengths, batch: int, max_len: int, n_min: int,
                            n_max: int, k_max: int, out_draft, out_len, out_match, out_pos,
                            out_err=None, stream=None) -> None:
    """pld_draft_batch_pos without a context (nothing allocated); `out_err`
    is a device uint32 tensor (or None) that error bits are OR-ed into."""
    import torch
    i32 = _i32()
    _check("pld_draft_batch_noalloc", load().pld_draft_batch_noalloc(
        _dev_ptr(histories, "histories", torch.int64), _dev_ptr(lengths, "lengths", i32),
        int(batch), int(max_len), int(n_min), int(n_max), int(k_max),
        _dev_ptr(out_draft, "out_draft", i32), _dev_ptr(out_len, "out_len", i32),
        _dev_ptr(out_match, "out_match", i32), _dev_ptr(out_pos, "out_pos", i32),
        _dev_ptr(out_err, "out_err"), _stream(stream)))


def pld_draft_batch_strided(ctx: int, base, stride: int, lengths, min_len: int,
                            batch: int, n_min: int, n_max: int, k_max: int, out_draft,
                            out_len, out_match, out_pos=None, stream=None) -> None:
    """Rows at a fixed stride: row b is base + b * stride tokens. `base` is a
    device int32 tensor (its first element is row 0's first token) or a
    pointer."""
    i32 = _i32()
    _check("pld_draft_batch_strided", load().pld_draft_batch_strided(
        ctx, _dev_ptr(base, "base", i32), int(stride), _dev_ptr(lengths, "lengths", i32),
        int(min_len), int(batch), int(n_min), int(n_max), int(k_max),
        _dev_ptr(out_draft, "out_draft", i32), _dev_ptr(out_len, "out_len", i32),
        _dev_ptr(out_match, "out_match", i32), _dev_ptr(out_pos, "out_pos", i32),
        _stream(stream)))


def pld_append_draft_store(ctx: int, tokens, tokens_stride: int, counts, batch: int,
                           n_min: int, n_max: int, k_max: int, out_draft, out_len, out_match,
                           out_pos=None, stream=None) -> None:
    """pld_append, then draft the store's first `batch` rows (include/pld.h)."""
    i32 = _i32()
    _check("pld_append_draft_store", load().pld_append_draft_store(
        ctx, _dev_ptr(tokens, "tokens", i32), int(tokens_stride),
        _dev_ptr(counts, "counts", i32), int(batch), int(n_min), int(n_max), int(k_max),
        _dev_ptr(out_draft, "out_draft", i32), _dev_ptr(out_len, "out_len", i32),
        _dev_ptr(out_match, "out_match", i32), _dev_ptr(out_pos, "out_pos", i32),
        _stream(stream)))


def pld_index_fingerprint_bits(ctx: int, bits: int) -> None:
    _check("pld_index_fingerprint_bits", load().pld_index_fingerprint_bits(ctx, int(bits)))


def pld_draft_store(ctx: int, batch: int, n_min: int, n_max: int, k_max: int, out_draft,
                    out_len, out_match, out_pos=None, stream=None) -> None:
    """Draft the store's first `batch` rows from the n-gram index."""
    i32 = _i32()
    _check("pld_draft_store", load().pld_draft_store(
        ctx, int(batch), int(n_min), int(n_max), int(k_max),
        _dev_ptr(out_draft, "out_draft", i32), _dev_ptr(out_len, "out_len", i32),
        _dev_ptr(out_match, "out_match", i32), _dev_ptr(out_pos, "out_pos", i32),
        _stream(stream)))


def pld_fuse_params_default() -> PldFuseParams:
    p = PldFuseParams()
    _check("pld_fuse_params_default", load().pld_fuse_params_default(ctypes.byref(p)))
    return p


def pld_fuse(ctx: int, params: PldFuseParams, lookup, lookup_k: int, lookup_len,
             lookup_match, drafter, accepted, state, batch: int, out_block, out_positions,
             out_src=None, stream=None) -> None:
    """One fusion step (include/pld.h). `state` is an int32 [batch, 4] device
    tensor carried across steps (zeros before the first); `out_src`, if
    given, is an int64 [batch] device tensor receiving the 64-bit masks."""
    import torch
    i32 = _i32()
    _check("pld_fuse", load().pld_fuse(
        ctx, ctypes.byref(params), _dev_ptr(lookup, "lookup", i32), int(lookup_k),
        _dev_ptr(lookup_len, "lookup_len", i32), _dev_ptr(lookup_match, "lookup_match", i32),
        _dev_ptr(drafter, "drafter", i32), _dev_ptr(accepted, "accepted", i32),
        _dev_ptr(state, "state", i32), int(batch), _dev_ptr(out_block, "out_block", i32),
        _dev_ptr(out_positions, "out_positions", i32),
        _dev_ptr(out_src, "out_src", torch.int64), _stream(stream)))


def pld_draft_fuse_batch(ctx: int, histories, lengths, batch: int, n_min: int, n_max: int,
                         k_max: int, out_draft, out_len, out_match, params: PldFuseParams,
                         drafter, accepted, state, out_block, out_positions, out_src=None,
                         stream=None) -> None:
    """pld_draft_batch and pld_fuse in one launch (include/pld.h)."""
    import torch
    i32 = _i32()
    _check("pld_draft_fuse_batch", load().pld_draft_fuse_batch(
        ctx, _dev_ptr(histories, "histories"), _dev_ptr(lengths, "lengths", i32), int(batch),
        int(n_min), int(n_max), int(k_max), _dev_ptr(out_draft, "out_draft", i32),
        _dev_ptr(out_len, "out_len", i32), _dev_ptr(out_match, "out_match", i32),
        ctypes.byref(params), _dev_ptr(drafter, "drafter", i32),
        _dev_ptr(accepted, "accepted", i32), _dev_ptr(state, "state", i32),
        _dev_ptr(out_block, "out_block", i32), _dev_ptr(out_positions, "out_positions", i32),
        _dev_ptr(out_src, "out_src", torch.int64), _stream(stream)))


def pld_control_params_default() -> PldControlParams:
    p = PldControlParams()
    _check("pld_control_params_default", load().pld_control_params_default(ctypes.byref(p)))
    return p


def pld_control(ctx: int, params: PldControlParams, accepted, round_time, lookup_len,
                lookup_match, state, batch: int, out_source, out_rates=None,
                stream=None) -> None:
    """One controller step (include/pld.h). `round_time`, `state` and
    `out_rates` are float64 device tensors."""
    import torch
    i32, f64 = _i32(), torch.float64
    _check("pld_control", load().pld_control(
        ctx, ctypes.byref(params), _dev_ptr(accepted, "accepted", i32),
        _dev_ptr(round_time, "round_time", f64), _dev_ptr(lookup_len, "lookup_len", i32),
        _dev_ptr(lookup_match, "lookup_match", i32), _dev_ptr(state, "state", f64), int(batch),
        _dev_ptr(out_source, "out_source", i32), _dev_ptr(out_rates, "out_rates", f64),
        _stream(stream)))


def pld_draft_control_batch(ctx: int, histories, lengths, batch: int, n_min: int, n_max: int,
                            k_max: int, out_draft, out_len, out_match, params: PldControlParams,
                            accepted, round_time, state, out_source, out_rates=None,
                            stream=None) -> None:
    """pld_draft_batch and pld_control in one launch (include/pld.h)."""
    import torch
    i32, f64 = _i32(), torch.float64
    _check("pld_draft_control_batch", load().pld_draft_control_batch(
        ctx, _dev_ptr(histories, "histories", torch.int64), _dev_ptr(lengths, "lengths", i32),
        int(batch), int(n_min), int(n_max), int(k_max), _dev_ptr(out_draft, "out_draft", i32),
        _dev_ptr(out_len, "out_len", i32), _dev_ptr(out_match, "out_match", i32),
        ctypes.byref(params), _dev_ptr(accepted, "accepted", i32),
        _dev_ptr(round_time, "round_time", f64), _dev_ptr(state, "state", f64),
        _dev_ptr(out_source, "out_source", i32), _dev_ptr(out_rates, "out_rates", f64),
        _stream(stream)))


def pld_ngram_params_default() -> PldNgramParams:
    p = PldNgramParams()
    _check("pld_ngram_params_default", load().pld_ngram_params_default(ctypes.byref(p)))
    return p


def pld_draft_ngram(ctx: int, params: PldNgramParams, batch: int, k_max: int, out_draft,
                    out_len, out_levels=None, stream=None) -> None:
    """Draft the store's first `batch` rows from the successor-count cache
    (include/pld.h)."""
    i32 = _i32()
    _check("pld_draft_ngram", load().pld_draft_ngram(
        ctx, ctypes.byref(params), int(batch), int(k_max), _dev_ptr(out_draft, "out_draft", i32),
        _dev_ptr(out_len, "out_len", i32), _dev_ptr(out_levels, "out_levels", i32),
        _stream(stream)))


def pld_append_draft_ngram(ctx: int, tokens, tokens_stride: int, counts, batch: int,
                           params: PldNgramParams, k_max: int, out_draft, out_len,
                           out_levels=None, stream=None) -> None:
    """pld_append, then pld_draft_ngram of the store's first `batch` rows, in
    one launch for 0 < tokens_stride <= 1024 (include/pld.h)."""
    i32 = _i32()
    _check("pld_append_draft_ngram", load().pld_append_draft_ngram(
        ctx, _dev_ptr(tokens, "tokens", i32), int(tokens_stride), _dev_ptr(counts, "counts", i32),
        int(batch), ctypes.byref(params), int(k_max), _dev_ptr(out_draft, "out_draft", i32),
        _dev_ptr(out_len, "out_len", i32), _dev_ptr(out_levels, "out_levels", i32),
        _stream(stream)))


def pld_sync(ctx: int, stream=None) -> int:
    """Wait for the stream; return (and clear) the sticky device status."""
    return int(load().pld_sync(ctx, _stream(stream)))


# ---------------------------------------------------------------------------
# device-memory plumbing for callers holding numpy histories
# ---------------------------------------------------------------------------


class DeviceBatch:
    """Histories packed into one device buffer, with a row-pointer table and
    a lengths vector, ready for pld_draft_batch.

    Row b starts at a multiple of `align` tokens plus `offsets[b]` tokens
    (offsets let tests place rows at every 4-byte alignment).
    """

    def __init__(self, histories, device="cuda", align: int = 64,
                 offsets=None, max_len: int | None = None):
        import torch
        self.batch = len(histories)
        lens = np.array([len(h) for h in histories], dtype=np.int64)
        offs = np.zeros(self.batch, np.int64) if offsets is None else np.asarray(offsets, np.int64)
        starts = np.zeros(self.batch, dtype=np.int64)
        pos = 0
        for b in range(self.batch):
            pos = -(-pos // align) * align + int(offs[b])
            starts[b] = pos
            pos += int(lens[b])
        total = -(-pos // align) * align + align
        flat = np.zeros(total, dtype=np.int32)
        for b, h in enumerate(histories):
            flat[starts[b]:starts[b] + lens[b]] = h
        self.flat = torch.from_numpy(flat).to(device)
        base = self.flat.data_ptr()
        self.rows = torch.from_numpy((base + 4 * starts).astype(np.int64)).to(device)
        self.lengths = torch.from_numpy(lens.astype(np.int32)).to(device)
        self.starts = starts
        self.max_len = int(max_len if max_len is not None else max(1, lens.max(initial=1)))

    def replicate(self):
        """A second copy at another address (same layout)."""
        other = object.__new__(DeviceBatch)
        other.batch = self.batch
        other.flat = self.flat.clone()
        other.rows = (self.rows - self.flat.data_ptr() + other.flat.data_ptr()).clone()
        other.lengths = self.lengths
        other.starts = self.starts
        other.max_len = self.max_len
        return other


class StridedBatch:
    """Histories in one padded [batch, stride] device buffer (stride rounded
    up to a multiple of `align` tokens), with a lengths vector."""

    def __init__(self, histories, device="cuda", align: int = 64, stride=None):
        import torch
        self.batch = len(histories)
        lens = np.array([len(h) for h in histories], dtype=np.int64)
        need = int(lens.max(initial=0))
        self.stride = int(stride) if stride is not None else max(align, -(-need // align) * align)
        buf = np.zeros((max(1, self.batch), self.stride), dtype=np.int32)
        for b, h in enumerate(histories):
            buf[b, :len(h)] = h
        self.buf = torch.from_numpy(buf).to(device)
        self.lengths = torch.from_numpy(lens.astype(np.int32)).to(device)
        # the shortest history (0 for an empty batch): every row's length is at least this
        self.min_len = int(lens.min()) if lens.size else 0
        self.max_len = max(1, need)


def alloc_outputs(batch: int, k_max: int, device="cuda"):
    import torch
    return (torch.empty((batch, k_max), dtype=torch.int32, device=device),
            torch.empty(batch, dtype=torch.int32, device=device),
            torch.empty(batch, dtype=torch.int32, device=device),
            torch.empty(batch, dtype=torch.int32, device=device))
