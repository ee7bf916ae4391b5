"""The fused gather's merge, as a protocol, checked by exhaustive
simulation (no GPU).

Each wavefront of a workgroup holds a local maximum key (0 without a
match). A wavefront with a match performs an atomicMax on the request's key
word and waits for the old value; the increase it made (m - old when
m > old, else 0) goes to its workgroup through LDS. After the workgroup's
barrier one atomic add on the accumulator word counts the workgroup in:
(sum of its wavefronts' increases << 24) + 1. The workgroup whose add
returns a count of n - 1 is the last; it takes (its add's return >> 24) +
its own increase as the final key. The claim: in every order the hardware
may perform these operations in (each wavefront's max before its
workgroup's add, everything else free), the last workgroup's key is the
maximum of all keys. Keys are below 2^39 and fewer than 2^24 workgroups
count in, so the fields never overflow into each other. A workgroup of one
wavefront is the same protocol with one max before the add."""

from __future__ import annotations

import random

import pytest

COUNT_BITS = 24


def actors(wgs):
    """(kind, workgroup, wavefront) for every operation: one max per
    wavefront with a match, one add per workgroup."""
    ops = []
    for w, waves in enumerate(wgs):
        ops += [("max", w, v) for v, m in enumerate(waves) if m]
        ops.append(("add", w, None))
    return ops


def ready(op, done, wgs):
    kind, w, _ = op
    if kind == "max":
        return True
    return all(("max", w, v) in done for v, m in enumerate(wgs[w]) if m)


def interleavings(wgs):
    """Every order of the operations in which each workgroup's add follows
    its wavefronts' maxima."""
    ops = actors(wgs)

    def rec(done, order):
        if len(order) == len(ops):
            yield list(order)
            return
        for op in ops:
            if op not in done and ready(op, done, wgs):
                done.add(op)
                order.append(op)
                yield from rec(done, order)
                order.pop()
                done.remove(op)

    yield from rec(set(), [])


def run_protocol(wgs, order):
    key_word, acc_word = 0, 0
    inc = [0] * len(wgs)
    last = []
    for kind, w, v in order:
        if kind == "max":                  # a wavefront's atomicMax, returning the old key
            m = wgs[w][v]
            old = key_word
            key_word = max(key_word, m)
            inc[w] += m - old if m > old else 0
            continue
        prev = acc_word                    # the workgroup's arrival add
        acc_word += (inc[w] << COUNT_BITS) + 1
        if prev & ((1 << COUNT_BITS) - 1) == len(wgs) - 1:
            last.append((prev >> COUNT_BITS) + inc[w])
    return key_word, acc_word, last


def key(length, end):
    return (length << 32) | end


@pytest.mark.parametrize("wgs", [
    [[0], [0], [0]],
    [[key(4, 10)], [0], [0]],
    [[key(4, 10)], [key(4, 99)], [key(12, 5)]],
    [[key(5, 1)], [key(5, 1)], [key(5, 2)]],
    [[key(64, 2**31 - 1)], [key(63, 7)], [0], [key(64, 2**31 - 2)]],
    [[key(3, 9)], [key(7, 3)], [key(7, 4)], [key(6, 100)]],
    # several wavefronts with a match in one workgroup
    [[key(4, 10), key(5, 20)], [key(5, 30), 0], [0, 0]],
    [[key(6, 1), key(6, 2), key(6, 3)], [key(6, 4)]],
    [[key(9, 7), 0, key(9, 7), 0], [0, key(8, 900), 0, 0], [0, 0, 0, 0]],
])
def test_every_interleaving_gives_the_maximum(wgs):
    top = max(m for waves in wgs for m in waves)
    n = 0
    for order in interleavings(wgs):
        key_word, acc_word, last = run_protocol(wgs, order)
        assert len(last) == 1, order                  # exactly one workgroup is last
        assert last[0] == top, (order, last[0])
        assert key_word == top
        assert acc_word >> COUNT_BITS == top           # the increases telescope
        assert acc_word & ((1 << COUNT_BITS) - 1) == len(wgs)
        n += 1
    assert n > 0


def test_random_orders_many_workgroups():
    """256 workgroups of 4 wavefronts (a 1,048,576-token request at
    4,096-token tiles), random keys, 10 random legal orders each."""
    rng = random.Random(5)
    for trial in range(20):
        wgs = [[key(rng.randint(1, 64), rng.randrange(2**31)) if rng.random() < 0.1 else 0
                for _ in range(4)] for _ in range(256)]
        top = max(m for waves in wgs for m in waves)
        ops = actors(wgs)
        for _ in range(10):
            done, order = set(), []
            while len(order) < len(ops):
                op = rng.choice([o for o in ops if o not in done and ready(o, done, wgs)])
                done.add(op)
                order.append(op)
            _, _, last = run_protocol(wgs, order)
            assert last == [top]


def test_field_widths():
    """The largest key (length 64, end 2^31 - 1) fits the accumulator's 40
    upper bits, and the most tiles a request can have (max_len below 2^31
    at the smallest tile, 256) fit its 24 lower bits."""
    largest = key(64, 2**31 - 1)
    assert largest < 2 ** (64 - COUNT_BITS)
    assert -(-(2**31 - 1) // 256) < 2 ** COUNT_BITS
