"""CPU oracle for batched prompt-lookup drafting (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product library
(``prompt_lookup_gram_amd``) never imports it.

The arithmetic lives in ``pld_oracle.c`` (plain, single-threaded C, compiled
with gcc at -O2 without vector intrinsics); this wrapper only marshals numpy
arrays. The rule it implements is stated at the top of that file (HyperQwen
lookup-drafting page, step 1 of the three-step principle).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pld_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpld_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile pld_oracle.c into libpld_oracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
                        "-fPIC", "-shared", "-o", tmp, _SRC], check=True)
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
    return lib


class OracleError(RuntimeError):
    pass


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
