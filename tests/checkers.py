"""Independent checkers that pin the oracle (and, through it, the HIP path).

None of these shares code with ``oracle/`` or with the HIP library. Each one
states the drafting rule a different way from the oracle's descending search:

* ``brute_force_set``: the answer written as the lexicographic maximum, by
  (length, start), of the set of all admissible earlier occurrences of a
  suffix, enumerated exhaustively (vectorised over many equal-length
  histories).
* ``z_function`` / ``by_z_function``: Gusfield's Z-algorithm (a textbook
  string routine) on the reversed history gives, for every end position e,
  the longest common suffix of h[..e] and h; the answer is the (length, e)
  maximum over the ones that reach n_min.
* ``certificate_errors``: given a claimed answer, checks in linear time that
  it is an occurrence of the suffix, that no more recent occurrence of that
  length exists, that no longer suffix occurs at all, and that the draft is
  the continuation.

The rule (HyperQwen lookup-drafting page, step 1 of the three-step principle):
longest suffix of n_min..n_max tokens with an earlier occurrence (overlap
allowed, the occurrence must be followed by a token), most recent occurrence,
draft = the following tokens, at most k_max of them, -1 padding.
"""

from __future__ import annotations

import itertools

import numpy as np
from numpy.lib.stride_tricks import sliding_window_view


# ---------------------------------------------------------------------------
# exhaustive set definition
# ---------------------------------------------------------------------------


def all_histories(alphabet: int, length: int) -> np.ndarray:
    """Every history of the given length over {0..alphabet-1}, as rows."""
    if length == 0:
        return np.zeros((1, 0), dtype=np.int32)
    rows = list(itertools.product(range(alphabet), repeat=length))
    return np.array(rows, dtype=np.int32)


def brute_force_set(H: np.ndarray, n_min: int, n_max: int, k_max: int):
    """H: [N, L] histories of one common length L.

    S = {(m, j): n_min <= m <= n_max, 0 <= j, j + m <= L - 1,
         H[j:j+m] == H[L-m:L]}; answer = lexicographic max of S.
    Returns (draft [N, k_max], draft_len [N], match [N], start [N]).
    """
    N, L = H.shape
    best_m = np.zeros(N, dtype=np.int64)
    best_j = np.full(N, -1, dtype=np.int64)
    for m in range(n_min, n_max + 1):
        for j in range(0, L):
            if j + m > L - 1:
                continue
            hit = np.all(H[:, j:j + m] == H[:, L - m:L], axis=1)
            better = hit & ((m > best_m) | ((m == best_m) & (j > best_j)))
            best_m = np.where(better, m, best_m)
            best_j = np.where(better, j, best_j)
    found = best_j >= 0
    d = np.where(found, np.minimum(k_max, L - (best_j + best_m)), 0)
    draft = np.full((N, k_max), -1, dtype=np.int32)
    for t in range(k_max):
        take = t < d
        if take.any():
            src = (best_j + best_m + t)[take]
            draft[take, t] = H[np.nonzero(take)[0], src]
    best_m = np.where(found, best_m, 0)
    return draft, d.astype(np.int32), best_m.astype(np.int32), best_j


# ---------------------------------------------------------------------------
# Z-function cross-check
# ---------------------------------------------------------------------------


def z_function(s) -> np.ndarray:
    """Gusfield's Z-array: z[i] = length of the longest common prefix of s and
    s[i:], with z[0] = len(s)."""
    s = list(s)
    n = len(s)
    z = [0] * n
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    z[0] = n
    left = right = 0
    for i in range(1, n):
        if i < right:
            z[i] = min(right - i, z[i - left])
        while i + z[i] < n and s[z[i]] == s[i + z[i]]:
            z[i] += 1
        if i + z[i] > right:
            left, right = i, i + z[i]
    return np.array(z, dtype=np.int64)


def by_z_function(h: np.ndarray, n_min: int, n_max: int, k_max: int):
    """Answer for one history via the Z-array of the reversed history.

    For an end position e (0 <= e <= L-2), z_rev[L-1-e] is the number of
    tokens h[..e] and h[..L-1] agree on reading backwards; it never exceeds
    e + 1, so the occurrence start e - l + 1 is >= 0.
    """
    h = np.asarray(h, dtype=np.int64)
    L = h.size
    draft = np.full(k_max, -1, dtype=np.int32)
    if L < 2:
        return draft, 0, 0, -1
    zr = z_function(h[::-1].tolist())
    e = np.arange(0, L - 1)
    ell = np.minimum(zr[L - 1 - e], n_max)
    ok = ell >= n_min
    if not ok.any():
        return draft, 0, 0, -1
    m = int(ell[ok].max())
    e_best = int(e[ok & (ell == m)].max())
    j = e_best - m + 1
    d = min(k_max, L - 1 - e_best)
    draft[:d] = h[e_best + 1:e_best + 1 + d]
    return draft, d, m, j


# ---------------------------------------------------------------------------
# linear-time certificate checker
# ---------------------------------------------------------------------------


def _occurs(h: np.ndarray, pat: np.ndarray, last_start: int, first_start: int = 0):
    """Starts s in [first_start, last_start] with h[s:s+len(pat)] == pat."""
    m = pat.size
    if last_start < first_start or m == 0:
        return np.zeros(0, dtype=np.int64)
    w = sliding_window_view(h, m)[first_start:last_start + 1]
    return np.nonzero(np.all(w == pat, axis=1))[0] + first_start


def certificate_errors(h, n_min, n_max, k_max, draft, d, m, j) -> list:
    """List of violated conditions (empty when the claimed answer is right)."""
    h = np.asarray(h, dtype=np.int64)
    draft = np.asarray(draft, dtype=np.int64)
    L = h.size
    d, m, j = int(d), int(m), int(j)
    errs = []
    m_top = min(n_max, L - 1)
    if draft.size != k_max:
        errs.append("draft row width")
    if m == 0:
        if d != 0 or j != -1:
            errs.append("no-match must have d=0, j=-1")
        if np.any(draft != -1):
            errs.append("no-match row must be all -1")
        if m_top >= n_min:
            suf = h[L - n_min:]
            if _occurs(h, suf, L - n_min - 1).size:
                errs.append("an n_min-suffix occurrence exists but none reported")
        return errs
    if not (n_min <= m <= m_top):
        errs.append(f"match length {m} outside [{n_min}, {m_top}]")
        return errs
    if not (0 <= j and j + m <= L - 1):
        errs.append(f"start {j} not admissible")
        return errs
    if not np.array_equal(h[j:j + m], h[L - m:]):
        errs.append("reported occurrence does not match the suffix")
    later = _occurs(h, h[L - m:], L - m - 1, j + 1)
    if later.size:
        errs.append(f"more recent occurrence at {int(later[-1])}")
    if m < m_top:
        if _occurs(h, h[L - m - 1:], L - m - 2).size:
            errs.append("a longer suffix occurs")
    want_d = min(k_max, L - (j + m))
    if d != want_d:
        errs.append(f"draft length {d} != {want_d}")
    dd = min(d, want_d)
    if not np.array_equal(draft[:dd], h[j + m:j + m + dd]):
        errs.append("draft is not the continuation")
    if np.any(draft[d:] != -1):
        errs.append("padding is not -1")
    return errs
