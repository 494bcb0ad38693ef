import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a golden text fixture: '#' comments, 'key ints...' lines, digit rows."""
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head = line.split()
            if head[0].isalpha():
                meta[head[0]] = [int(x) for x in head[1:]]
            else:
                rows.append([int(ch) for ch in line])
    return meta, rows


def check_launch_rule(tasks, total, per_slice, G):
    """Position b of an order over `total` tasks is logical task tasks[b]
    (slice task // per_slice, heavy-first rank task % per_slice); position b
    is meant for XCD b mod 8.  Orders of >= 2048 tasks and >= 2 rounds of 8 G:
    an even number of rounds in which XCD x holds G consecutive tasks (group
    x of the round's 8 groups of the sequence, then group 7 - x in the next
    round), the rest in sequence order.  The sequence is rank-major where G
    divides per_slice (group k: ranks (k // slices) G .. + G - 1 of slice
    k % slices), else the task order.  Smaller orders: heavy first across
    slices (rank b // slices of slice b % slices)."""
    import numpy as np
    tasks = np.asarray(tasks)
    assert sorted(tasks.tolist()) == list(range(total))
    rounds = total // (8 * G)
    b = np.arange(total)
    n = total // per_slice

    def seq(t):
        t = np.asarray(t)
        if per_slice % G:
            return t
        k = t // G
        return (k % n) * per_slice + (k // n) * G + t % G

    if total >= 2048 and rounds >= 2:
        even = rounds - rounds % 2
        for r in range(even):
            seg = tasks[8 * G * r: 8 * G * (r + 1)]
            for x in range(8):
                g = x if r % 2 == 0 else 7 - x
                assert np.array_equal(seg[x::8], seq(8 * G * r + g * G + np.arange(G)))
        assert np.array_equal(tasks[8 * G * even:], seq(b[8 * G * even:]))
        return "grouped"
    n = total // per_slice
    assert np.array_equal(tasks, (b % n) * per_slice + b // n)
    return "interleaved"
