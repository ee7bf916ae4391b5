"""Seeded synthetic token histories for batched prompt-lookup drafting.

This module is the one piece shared by the HIP library's tests/bench and the
CPU oracle's tests. It holds no drafting arithmetic at all: it only draws
random token streams and plants structure in them (verbatim copies, periodic
runs, substitutions). Nothing here searches for matches.

Token statistics stand in for the workloads the pages measure on, which are
not available here:

* natural-text token frequencies: bounded Zipf, P(rank k) ~ k^-s over a
  151,936-id vocabulary with s = 1.1 (token id = rank - 1);
* "the answer repeats the prompt" (HyperQwen lookup-drafting page, opening
  table: verbatim repeat of a 25k-token document) and code-editing copies
  (Strata prompt-lookup page, section 4): a tail that copies an earlier span
  of the same history, with a small rate of random substitutions;
* list items, indentation and code fences (HyperQwen page, step 1, where the
  overlap rule is motivated): runs with a short period.

Every request draws from ``numpy.random.default_rng([config_id, request_id])``
(PCG64), so a request's tokens do not depend on the batch it sits in.
"""

from __future__ import annotations

import dataclasses
from functools import lru_cache

import numpy as np

ZIPF_S = 1.1
ZIPF_VOCAB = 151_936
UNIFORM_VOCAB_C1 = 32_000


@dataclasses.dataclass
class Workload:
    """A batch of histories plus the drafting parameters it is run with."""

    name: str
    histories: list  # list of 1-D int32 numpy arrays, one per request
    n_min: int
    n_max: int
    k_max: int
    description: str = ""

    @property
    def batch(self) -> int:
        return len(self.histories)

    @property
    def lengths(self) -> np.ndarray:
        return np.array([len(h) for h in self.histories], dtype=np.int64)

    @property
    def total_tokens(self) -> int:
        return int(sum(len(h) for h in self.histories))

    @property
    def max_len(self) -> int:
        return int(max((len(h) for h in self.histories), default=0))


# ---------------------------------------------------------------------------
# primitive draws
# ---------------------------------------------------------------------------


@lru_cache(maxsize=4)
def zipf_cdf(s: float = ZIPF_S, vocab: int = ZIPF_VOCAB) -> np.ndarray:
    """Cumulative distribution of the bounded Zipf law over ids 0..vocab-1."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    c /= c[-1]
    return c


def zipf_tokens(rng: np.random.Generator, n: int, s: float = ZIPF_S,
                vocab: int = ZIPF_VOCAB) -> np.ndarray:
    """n i.i.d. bounded-Zipf token ids by inverse-CDF sampling."""
    u = rng.random(n)
    ids = np.searchsorted(zipf_cdf(s, vocab), u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def substitute(rng: np.random.Generator, seg: np.ndarray, q: float,
               vocab: int) -> np.ndarray:
    """Replace each token independently with probability q by a uniform id
    from [0, vocab) that differs from the original."""
    seg = seg.copy()
    hit = rng.random(seg.size) < q
    k = int(hit.sum())
    if k:
        r = rng.integers(0, vocab - 1, size=k, dtype=np.int64)
        orig = seg[hit].astype(np.int64)
        seg[hit] = (r + (r >= orig)).astype(np.int32)
    return seg


def distinct_zipf_block(rng: np.random.Generator, p: int) -> np.ndarray:
    """p pairwise-distinct Zipf ids (redraw duplicates)."""
    out: list[int] = []
    seen: set[int] = set()
    while len(out) < p:
        for t in zipf_tokens(rng, 4 * p).tolist():
            if t not in seen:
                seen.add(t)
                out.append(t)
                if len(out) == p:
                    break
    return np.array(out, dtype=np.int32)


def periodic_run(block: np.ndarray, length: int) -> np.ndarray:
    reps = -(-length // block.size)
    return np.tile(block, reps)[:length].astype(np.int32)


def copy_tail(rng: np.random.Generator, doc: np.ndarray, tail: int, q: float,
              vocab: int) -> np.ndarray:
    """doc followed by `tail` tokens copying a uniformly placed span of doc,
    each copied token substituted with probability q."""
    s = int(rng.integers(0, doc.size - tail + 1))
    src = doc[s:s + tail]
    return np.concatenate([doc, substitute(rng, src, q, vocab)]).astype(np.int32)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------


def config1() -> Workload:
    """1 request, 4,096 uniform tokens from [0, 32000); the last 512 tokens
    copy a random earlier span that does not overlap them."""
    rng = np.random.default_rng([1, 0])
    h = rng.integers(0, UNIFORM_VOCAB_C1, 4096, dtype=np.int64).astype(np.int32)
    s = int(rng.integers(0, 3584 - 512 + 1))
    h[3584:] = h[s:s + 512]
    return Workload("c1_single_4k_uniform_copy", [h], 4, 12, 16,
                    "B=1, L=4096, uniform [0,32000), 512-token verbatim copy tail")


def _copy_heavy(cfg: int, b: int, length: int, tail: int, q: float) -> np.ndarray:
    rng = np.random.default_rng([cfg, b])
    doc = zipf_tokens(rng, length - tail)
    return copy_tail(rng, doc, tail, q, ZIPF_VOCAB)


def config2() -> Workload:
    """8 requests of 25,000 tokens: a 24,000-token Zipf document, then 1,000
    tokens copying a random document span with 1% substitutions."""
    hs = [_copy_heavy(2, b, 25_000, 1_000, 0.01) for b in range(8)]
    return Workload("c2_b8_25k_zipf_copy", hs, 4, 12, 15,
                    "B=8, L=25000, Zipf(1.1) doc + 1000-token copy tail, q=1%")


def config3() -> Workload:
    """64 ragged requests, L ~ U[8192, 65536]. Requests 0-31 are copy-heavy
    (1,000-token copy tail, q = 1%), 32-63 pure Zipf. Every request carries a
    200-token periodic run (period U[3, 20], distinct Zipf ids per block) at a
    random interior position; requests with b % 4 == 3 also end with one."""
    hs = []
    for b in range(64):
        rng = np.random.default_rng([3, b])
        length = int(rng.integers(8192, 65536 + 1))
        if b < 32:
            doc = zipf_tokens(rng, length - 1000)
            h = copy_tail(rng, doc, 1000, 0.01, ZIPF_VOCAB)
            interior_hi = length - 1000 - 200
        else:
            h = zipf_tokens(rng, length)
            interior_hi = length - 200 - 200
        p = int(rng.integers(3, 20 + 1))
        blk = distinct_zipf_block(rng, p)
        at = int(rng.integers(0, interior_hi + 1))
        h[at:at + 200] = periodic_run(blk, 200)
        if b % 4 == 3:
            p2 = int(rng.integers(3, 20 + 1))
            blk2 = distinct_zipf_block(rng, p2)
            h[length - 200:] = periodic_run(blk2, 200)
        hs.append(h.astype(np.int32))
    return Workload("c3_b64_ragged_8k_64k_mixed", hs, 4, 12, 16,
                    "B=64, L~U[8192,65536], half copy-heavy, half pure Zipf, "
                    "200-token periodic runs (period 3..20)")


def config4() -> Workload:
    """16 requests of 262,144 tokens: 258,048 Zipf tokens followed by a
    4,096-token copy of a random earlier span with 0.5% substitutions."""
    hs = [_copy_heavy(4, b, 262_144, 4_096, 0.005) for b in range(16)]
    return Workload("c4_b16_262k_zipf_copy", hs, 4, 12, 16,
                    "B=16, L=262144, Zipf(1.1) doc + 4096-token copy tail, q=0.5%")


# --- streaming decode --------------------------------------------------------

STREAM_BATCH = 64
STREAM_START_LEN = 32_768
STREAM_STEPS = 1_024
STREAM_MAX_APPEND = 16
STREAM_MAX_LEN = STREAM_START_LEN + STREAM_STEPS * STREAM_MAX_APPEND  # 49,152


def config5_start(start_len: int = STREAM_START_LEN) -> Workload:
    """64 requests at 32,768 tokens (start_len - 1,000 Zipf + 1,000-token copy
    tail, q = 1%), the state a streaming decode starts from. Other start
    lengths give the same decode on longer or shorter histories."""
    hs = [_copy_heavy(5, b, start_len, 1_000, 0.01)
          for b in range(STREAM_BATCH)]
    name = "c5_stream_b64_32k" if start_len == STREAM_START_LEN else f"c5_stream_b64_{start_len}"
    return Workload(name, hs, 4, 12, 16,
                    f"B=64 streaming decode from L={start_len}, 1024 steps of 1..16 "
                    "appended tokens")


def stream_step_draws(step: int, batch: int = STREAM_BATCH):
    """Per-step random draws of the streaming workload: how many tokens each
    request accepts (U[1, 16]) and 16 fresh Zipf tokens per request."""
    rng = np.random.default_rng([5, 1_000_000 + step])
    counts = rng.integers(1, STREAM_MAX_APPEND + 1, size=batch).astype(np.int32)
    fresh = zipf_tokens(rng, batch * STREAM_MAX_APPEND).reshape(
        batch, STREAM_MAX_APPEND)
    return counts, fresh


def compose_append(draft: np.ndarray, draft_len: np.ndarray,
                   counts: np.ndarray, fresh: np.ndarray) -> np.ndarray:
    """The tokens a request appends after a step: the previous draft's tokens
    while they last (the draft is taken as accepted where it exists), then
    fresh tokens. Row b holds counts[b] meaningful tokens; the rest of the
    16-wide row is padding (-1) and is never appended."""
    batch, width = fresh.shape
    t = np.arange(width)[None, :]
    dl = np.asarray(draft_len).reshape(batch, 1)
    d = np.full((batch, width), -1, dtype=np.int32)
    k = min(width, draft.shape[1])
    d[:, :k] = draft[:, :k]
    out = np.where(t < dl, d, fresh).astype(np.int32)
    return np.where(t < np.asarray(counts).reshape(batch, 1), out, -1).astype(np.int32)


# ---------------------------------------------------------------------------
# small structured cases (used by parity fuzzing; still no drafting logic)
# ---------------------------------------------------------------------------


def fuzz_batch(seed: int, max_batch: int = 24, max_len: int = 5000):
    """A ragged batch over a tiny alphabet (2..8 symbols) so that long and
    overlapping matches are common, plus random drafting parameters."""
    rng = np.random.default_rng([99, seed])
    batch = int(rng.integers(1, max_batch + 1))
    alpha = int(rng.integers(2, 9))
    hs = []
    for _ in range(batch):
        kind = int(rng.integers(0, 4))
        if kind == 0:
            length = int(rng.integers(0, 20))
        else:
            length = int(rng.integers(0, max_len + 1))
        h = rng.integers(0, alpha, length, dtype=np.int64).astype(np.int32)
        if kind == 3 and length > 64:
            p = int(rng.integers(1, 24))
            blk = rng.integers(0, alpha + 5, p, dtype=np.int64).astype(np.int32)
            run = int(rng.integers(1, length))
            h[length - run:] = periodic_run(blk, run)
        hs.append(h)
    n_min = int(rng.integers(1, 9))
    n_max = int(rng.integers(n_min, 65))
    k_max = int(rng.integers(1, 65))
    return Workload(f"fuzz{seed}", hs, n_min, n_max, k_max,
                    f"fuzz seed {seed}: alphabet {alpha}")


ALL_CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4}


# ---------------------------------------------------------------------------
# draft fusion inputs (random draws only; nothing here fuses or schedules)
# ---------------------------------------------------------------------------

#: field order of the fusion parameters (pld_fuse_params)
FUSE_PARAM_FIELDS = ("head", "positions_long", "replace_min", "agree_min", "agree_tokens",
                     "tail_min", "entry_steps", "sticky", "near_full_slack")


def fuse_params_draw(rng: np.random.Generator) -> dict:
    """Random fusion parameters covering small and page-sized blocks."""
    head = int(rng.integers(1, 9))
    return dict(head=head, positions_long=int(rng.integers(head, 17)),
                replace_min=int(rng.integers(1, 13)), agree_min=int(rng.integers(1, 13)),
                agree_tokens=int(rng.integers(1, head + 1)), tail_min=int(rng.integers(1, 13)),
                entry_steps=int(rng.integers(0, 4)), sticky=int(rng.integers(0, 5)),
                near_full_slack=int(rng.integers(0, 3)))


def fuse_step_draws(rng: np.random.Generator, batch: int, head: int, lookup_k: int = 16,
                    alphabet: int = 3):
    """One step of random lookup results and drafter proposals, over a small
    alphabet so that agreement, every match length and full tails all occur:
    (lookup [batch, lookup_k] with -1 past each draft, draft lengths,
    match lengths, drafter [batch, head]). The drafter may propose -1, a
    legal token that is also the lookup row's padding value."""
    m = rng.integers(0, 13, size=batch).astype(np.int32)
    d = np.where(m > 0, rng.integers(1, lookup_k + 1, size=batch), 0).astype(np.int32)
    lookup = rng.integers(0, alphabet, size=(batch, lookup_k)).astype(np.int32)
    lookup[np.arange(lookup_k)[None, :] >= d[:, None]] = -1
    drafter = rng.integers(-1, alphabet, size=(batch, head)).astype(np.int32)
    return lookup, d, m, drafter
