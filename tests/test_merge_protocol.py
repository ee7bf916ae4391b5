"""The fused gather's merge, as a protocol, checked by exhaustive
simulation (no GPU).

Each workgroup of a request holds a local maximum key m (0 without a
match). With a match it first performs an atomicMax on the request's key
word and waits for the old value; then it performs one atomic add on the
accumulator word: (increase << 24) + 1, where the increase is what its
atomicMax added to the key (m - old when m > old, else 0). The workgroup
whose add returns a count of n - 1 is the last; it takes (its add's return
>> 24) + its own increase as the final key. The claim: in every order the
hardware may perform these operations in (each workgroup's max before its
own add, everything else free), the last workgroup's key is the maximum of
all m. Keys are below 2^39 and fewer than 2^24 workgroups count in, so the
fields never overflow into each other."""

from __future__ import annotations

import itertools
import random

import pytest

COUNT_BITS = 24


def interleavings(n_ops_per_wg):
    """Every order of the workgroups' operations that keeps each
    workgroup's own operations in program order."""
    wgs = [w for w, k in enumerate(n_ops_per_wg) for _ in range(k)]
    seen = set()
    for perm in itertools.permutations(wgs):
        if perm not in seen:
            seen.add(perm)
            yield perm


def run_protocol(keys, order):
    key_word, acc_word = 0, 0
    state = [{"step": 0, "inc": 0} for _ in keys]
    last = []
    for w in order:
        st = state[w]
        m = keys[w]
        if m and st["step"] == 0:          # atomicMax, returning the old key
            old = key_word
            key_word = max(key_word, m)
            st["inc"] = m - old if m > old else 0
            st["step"] = 1
            continue
        prev = acc_word                    # the arrival add
        acc_word += (st["inc"] << COUNT_BITS) + 1
        st["step"] = 2
        if prev & ((1 << COUNT_BITS) - 1) == len(keys) - 1:
            last.append((prev >> COUNT_BITS) + st["inc"])
    return key_word, acc_word, last


def key(length, end):
    return (length << 32) | end


@pytest.mark.parametrize("keys", [
    [0, 0, 0],
    [key(4, 10), 0, 0],
    [key(4, 10), key(4, 99), key(12, 5)],
    [key(5, 1), key(5, 1), key(5, 2)],
    [key(64, 2**31 - 1), key(63, 7), 0, key(64, 2**31 - 2)],
    [key(3, 9), key(7, 3), key(7, 4), key(6, 100)],
])
def test_every_interleaving_gives_the_maximum(keys):
    ops = [2 if m else 1 for m in keys]
    n = 0
    for order in interleavings(ops):
        key_word, acc_word, last = run_protocol(keys, order)
        assert len(last) == 1, order                  # exactly one workgroup is last
        assert last[0] == max(keys), (order, last[0])
        assert key_word == max(keys)
        assert acc_word >> COUNT_BITS == max(keys)     # the increases telescope
        assert acc_word & ((1 << COUNT_BITS) - 1) == len(keys)
        n += 1
    assert n > 0


def test_random_orders_many_workgroups():
    """256 workgroups (a 65,536-token request at 256-token tiles), random
    keys up to the largest one, 200 random legal orders each."""
    rng = random.Random(5)
    for trial in range(20):
        keys = [key(rng.randint(1, 64), rng.randrange(2**31)) if rng.random() < 0.3 else 0
                for _ in range(256)]
        ops = [2 if m else 1 for m in keys]
        for _ in range(10):
            pending = [list(range(k)) for k in ops]
            order = []
            live = [w for w in range(len(keys))]
            while live:
                w = rng.choice(live)
                order.append(w)
                pending[w].pop()
                if not pending[w]:
                    live.remove(w)
            _, _, last = run_protocol(keys, order)
            assert last == [max(keys)]


def test_field_widths():
    """The largest key (length 64, end 2^31 - 1) fits the accumulator's 40
    upper bits, and the most tiles a request can have (max_len below 2^31
    at the smallest tile, 256) fit its 24 lower bits."""
    largest = key(64, 2**31 - 1)
    assert largest < 2 ** (64 - COUNT_BITS)
    assert -(-(2**31 - 1) // 256) < 2 ** COUNT_BITS
