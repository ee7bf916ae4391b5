"""CPU oracle for batched prompt-lookup drafting (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product library
(``prompt_lookup_gram_amd``) never imports it.

The arithmetic lives in ``pld_oracle.c`` (lookup drafting: HyperQwen
lookup-drafting page, step 1 of the three-step principle) and
``fuse_oracle.c`` (draft fusion and long-block scheduling: steps 2 and 3 of
the same page), ``control_oracle.c`` (the online cost/benefit controller:
Strata prompt-lookup page, section 5) and ``ngram_oracle.c`` (successor-count
n-gram drafting: llama.cpp page, its context cache), plain single-threaded C compiled with
gcc at -O2 without vector intrinsics; this wrapper only marshals numpy
arrays. The rules are stated at the top of each file.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "pld_oracle.c"), os.path.join(_HERE, "fuse_oracle.c"),
         os.path.join(_HERE, "control_oracle.c"), os.path.join(_HERE, "ngram_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "libpld_oracle.so")
_lib = None


def compile_lib(out_path: str, sources=None, strict: bool = True) -> str:
    """Compile the oracle sources (default: this package's) into a shared
    library at out_path with gcc; strict turns warnings into errors."""
    # -ffp-contract=off: the controller's double arithmetic rounds each
    # operation on its own, as its file states
    warn = ["-Wall", "-Wextra", "-Werror"] if strict else []
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", *warn, "-fPIC", "-shared",
                    "-o", out_path, *(sources or _SRCS)], check=True)
    return out_path


def sources(replace=None) -> list:
    """This package's C sources, with {file name: other path} swapped in (a
    test's planted-mistake copy of one file)."""
    replace = replace or {}
    return [replace.get(os.path.basename(s), s) for s in _SRCS]


def build(force: bool = True) -> str:
    """Compile the oracle sources into libpld_oracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        compile_lib(tmp)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load(path: str | None = None):
    """Load (building first if nothing is built) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.pld_oracle_draft_one.restype = ctypes.c_int
    lib.pld_oracle_draft_one.argtypes = [i32p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, i32p,
                                         i32p, i32p, i64p]
    lib.pld_oracle_draft_batch.restype = ctypes.c_int
    lib.pld_oracle_draft_batch.argtypes = [ctypes.POINTER(i32p), i64p,
                                           ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, i32p,
                                           i32p, i32p, i64p]
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.fuse_oracle_batch.restype = ctypes.c_int
    lib.fuse_oracle_batch.argtypes = [ctypes.POINTER(FuseParams), ctypes.c_int32, i32p,
                                      ctypes.c_int32, i32p, i32p, i32p, i32p, i32p, i32p,
                                      i32p, u64p]
    lib.control_oracle_batch.restype = ctypes.c_int
    lib.control_oracle_batch.argtypes = [ctypes.POINTER(ControlParams), ctypes.c_int32, i32p,
                                         ctypes.POINTER(ctypes.c_double), i32p, i32p,
                                         ctypes.POINTER(ctypes.c_double), i32p,
                                         ctypes.POINTER(ctypes.c_double)]
    lib.ngram_oracle_draft_batch.restype = ctypes.c_int
    lib.ngram_oracle_draft_batch.argtypes = [ctypes.POINTER(NgramParams),
                                             ctypes.POINTER(i32p), i64p, ctypes.c_int32,
                                             ctypes.c_int32, i32p, i32p, i32p]
    return lib


class OracleError(RuntimeError):
    pass


class FuseParams(ctypes.Structure):
    """Fusion and scheduling parameters, defaults as the HyperQwen
    lookup-drafting page gives them (steps 2 and 3): a 7-token drafter head,
    15 draft positions in a long block, replace at a match of 8, or of 6 when
    the first 2 tokens agree, fill the tail at 4, two near-full steps to
    enter, 3 sticky steps. near_full_slack 1 is a reading (the page does not
    quantify "near-full")."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "head", "positions_long", "replace_min", "agree_min", "agree_tokens",
        "tail_min", "entry_steps", "sticky", "near_full_slack")]

    def __init__(self, head=7, positions_long=15, replace_min=8, agree_min=6,
                 agree_tokens=2, tail_min=4, entry_steps=2, sticky=3, near_full_slack=1):
        super().__init__(head, positions_long, replace_min, agree_min, agree_tokens,
                         tail_min, entry_steps, sticky, near_full_slack)


#: words of per-request fusion state (long flag, hold, near-full run, previous
#: block positions); all zero before a request's first step
FUSE_STATE_WORDS = 4


class ControlParams(ctypes.Structure):
    """Controller parameters (Strata prompt-lookup page, section 5): lookup
    must beat the MTP draft by 5% (margin 1.05); the MTP layer drafts 3
    tokens (section 1). alpha, beta, the priors and the bucket edges are
    readings (the page gives no numbers)."""
    _fields_ = [("alpha", ctypes.c_double), ("beta", ctypes.c_double),
                ("margin", ctypes.c_double), ("prior_accept", ctypes.c_double),
                ("prior_time", ctypes.c_double), ("mtp_tokens", ctypes.c_int32),
                ("edge", ctypes.c_int32 * 3)]

    def __init__(self, alpha=0.1, beta=0.1, margin=1.05, prior_accept=0.5, prior_time=1.0,
                 mtp_tokens=3, edge=(6, 8, 12)):
        super().__init__(alpha, beta, margin, prior_accept, prior_time, mtp_tokens,
                         (ctypes.c_int32 * 3)(*edge))


#: doubles of per-request controller state; all zero before the first step
CONTROL_STATE_WORDS = 11
SRC_PLAIN, SRC_MTP, SRC_LOOKUP = 0, 1, 2

#: longest context of the successor-count drafter (llama.cpp page: sizes 1 to 4)
NGRAM_MAX_N = 4


class NgramParams(ctypes.Structure):
    """Successor-count drafting parameters (llama.cpp page, its context
    cache): contexts of 1 to 4 tokens, longest tried first; per length n
    (index n - 1) the context must have been followed at least min_count
    times and its most frequent successor must hold at least min_percent of
    those. The page gives 1 and 50 for the 4-gram; every length uses them by
    default (a reading)."""
    _fields_ = [("n_min", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("min_count", ctypes.c_int32 * NGRAM_MAX_N),
                ("min_percent", ctypes.c_int32 * NGRAM_MAX_N)]

    def __init__(self, n_min=1, n_max=4, min_count=(1, 1, 1, 1), min_percent=(50, 50, 50, 50)):
        super().__init__(n_min, n_max, (ctypes.c_int32 * NGRAM_MAX_N)(*min_count),
                         (ctypes.c_int32 * NGRAM_MAX_N)(*min_percent))


def draft(histories, n_min: int, n_max: int, k_max: int, lib=None):
    """Draft every request of a batch.

    histories: sequence of 1-D int32 arrays.
    Returns (draft [B, k_max] int32, draft_len [B] int32, match_len [B] int32,
    start [B] int64 (-1 when no match)).
    """
    lib = load() if lib is None else lib
    hs = [np.ascontiguousarray(h, dtype=np.int32) for h in histories]
    batch = len(hs)
    i32p = ctypes.POINTER(ctypes.c_int32)
    ptrs = (i32p * max(batch, 1))()
    for b, h in enumerate(hs):
        ptrs[b] = h.ctypes.data_as(i32p)
    lengths = np.array([h.size for h in hs], dtype=np.int64)
    out_draft = np.empty((batch, k_max), dtype=np.int32)
    out_len = np.empty(batch, dtype=np.int32)
    out_match = np.empty(batch, dtype=np.int32)
    out_pos = np.empty(batch, dtype=np.int64)
    rc = lib.pld_oracle_draft_batch(
        ptrs, lengths.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), batch,
        n_min, n_max, k_max, out_draft.ctypes.data_as(i32p),
        out_len.ctypes.data_as(i32p), out_match.ctypes.data_as(i32p),
        out_pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    if rc != 0:
        raise OracleError(f"oracle rejected arguments (rc={rc})")
    return out_draft, out_len, out_match, out_pos


def append(histories, tokens: np.ndarray, counts: np.ndarray):
    """Streaming append: request b gains tokens[b, :counts[b]]. Returns the new
    list of histories (the inputs are not modified)."""
    return [np.concatenate([h, np.asarray(tokens[b, :int(counts[b])], dtype=np.int32)])
            for b, h in enumerate(histories)]


def fuse(params: FuseParams, lookup, lookup_len, lookup_match, drafter, accepted,
         state, lib=None):
    """One fusion step for a batch (HyperQwen page, steps 2 and 3).

    lookup [B, K] int32 lookup draft rows with lengths lookup_len [B] and
    match lengths lookup_match [B]; drafter [B, head] int32; accepted [B]
    int32 (previous step's accepted draft tokens); state [B, 4] int32.
    Returns (block [B, positions_long], positions [B], src [B] uint64 bit
    masks, new state [B, 4]); the inputs are not modified.
    """
    lib = load() if lib is None else lib
    lookup = np.ascontiguousarray(lookup, dtype=np.int32)
    batch, k = lookup.shape
    drafter = np.ascontiguousarray(drafter, dtype=np.int32).reshape(batch, params.head)
    lookup_len = np.ascontiguousarray(lookup_len, dtype=np.int32)
    lookup_match = np.ascontiguousarray(lookup_match, dtype=np.int32)
    accepted = np.ascontiguousarray(accepted, dtype=np.int32)
    st = np.array(state, dtype=np.int32).reshape(batch, FUSE_STATE_WORDS).copy()
    block = np.empty((batch, params.positions_long), dtype=np.int32)
    positions = np.empty(batch, dtype=np.int32)
    src = np.empty(batch, dtype=np.uint64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    p = lambda a: a.ctypes.data_as(i32p)  # noqa: E731
    rc = lib.fuse_oracle_batch(ctypes.byref(params), batch, p(lookup), k, p(lookup_len),
                               p(lookup_match), p(drafter), p(accepted), p(st), p(block),
                               p(positions), src.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
    if rc != 0:
        raise OracleError(f"fusion oracle rejected arguments (rc={rc})")
    return block, positions, src, st


def control(params: ControlParams, accepted, round_time, lookup_len, lookup_match, state,
            lib=None):
    """One controller step for a batch (Strata prompt-lookup page, section
    5). accepted [B] int32 and round_time [B] float64: the previous round's
    outcome (ignored at a request's first step); lookup_len, lookup_match
    [B] int32: this round's lookup draft; state [B, 11] float64. Returns
    (source [B] int32, rates [B, 3] float64, new state); inputs unchanged."""
    lib = load() if lib is None else lib
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    batch = acc.size
    rt = np.ascontiguousarray(round_time, dtype=np.float64)
    ll = np.ascontiguousarray(lookup_len, dtype=np.int32)
    lm = np.ascontiguousarray(lookup_match, dtype=np.int32)
    st = np.array(state, dtype=np.float64).reshape(batch, CONTROL_STATE_WORDS).copy()
    src = np.empty(batch, np.int32)
    rates = np.empty((batch, 3), np.float64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    rc = lib.control_oracle_batch(ctypes.byref(params), batch, acc.ctypes.data_as(i32p),
                                  rt.ctypes.data_as(f64p), ll.ctypes.data_as(i32p),
                                  lm.ctypes.data_as(i32p), st.ctypes.data_as(f64p),
                                  src.ctypes.data_as(i32p), rates.ctypes.data_as(f64p))
    if rc != 0:
        raise OracleError(f"controller oracle rejected arguments (rc={rc})")
    return src, rates, st


def ngram_draft(params: NgramParams, histories, k_max: int, lib=None):
    """Successor-count drafts for a batch (llama.cpp page, its context
    cache). histories: sequence of 1-D int32 arrays. Returns (draft [B, k_max]
    int32 padded with -1, draft_len [B] int32, levels [B, k_max] int32: the
    context length behind each draft token, 0 past draft_len)."""
    lib = load() if lib is None else lib
    hs = [np.ascontiguousarray(h, dtype=np.int32) for h in histories]
    batch = len(hs)
    i32p = ctypes.POINTER(ctypes.c_int32)
    ptrs = (i32p * max(batch, 1))()
    for b, h in enumerate(hs):
        ptrs[b] = h.ctypes.data_as(i32p)
    lengths = np.array([h.size for h in hs], dtype=np.int64)
    out_draft = np.empty((batch, k_max), dtype=np.int32)
    out_len = np.empty(batch, dtype=np.int32)
    levels = np.empty((batch, k_max), dtype=np.int32)
    rc = lib.ngram_oracle_draft_batch(ctypes.byref(params), ptrs,
                                      lengths.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                      batch, k_max, out_draft.ctypes.data_as(i32p),
                                      out_len.ctypes.data_as(i32p), levels.ctypes.data_as(i32p))
    if rc != 0:
        raise OracleError(f"n-gram oracle rejected arguments (rc={rc})")
    return out_draft, out_len, levels
