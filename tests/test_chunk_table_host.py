"""Host build of the packed-sequence chunk table (kda_table.h, the arithmetic
of chunk_table_kernel): exact table for well-formed cu_seqlens, and for
malformed ones (decreasing, negative, past T, overlapping) the guarantees the
kernels rely on to stay inside the caller's tensors and the workspace: spans
inside [0, T], non-decreasing chunk offsets capped at the workspace's chunk
capacity, at most ceil(len / 64) chunks per sequence and an order that is a
permutation.  Chunk size 64 ("Kimi K3 Technical Report", §2.1.1, chunkwise
form of eqs. (3)-(4), restarted at every packed sequence)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_20_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "chunk_table_harness.cpp")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("table") / "chunk_table")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", exe], check=True)
    return exe


def _run(exe, cu, T):
    cu = [int(x) for x in cu]
    N = len(cu) - 1
    cap = T // 64 + N                         # the workspace's chunk capacity for packed input
    out = subprocess.run([exe], input=f"{N} {T} {cap}\n" + " ".join(map(str, cu)) + "\n",
                         capture_output=True, text=True, check=True).stdout.split("\n")
    off, order, span = (np.array(ln.split(), dtype=np.int64) for ln in out[:3])
    return off, order, span.reshape(N, 2), cap


def _check_safe(off, order, span, cap, T):
    N = len(order)
    start, ln = span[:, 0], span[:, 1]
    assert (start >= 0).all() and (ln >= 0).all() and (start + ln <= T).all()
    assert off[0] == 0 and (np.diff(off) >= 0).all() and off[-1] <= cap
    assert (np.diff(off) <= (ln + 63) // 64).all()
    assert sorted(order.tolist()) == list(range(N))
    # every chunk a kernel can reach: token range inside [0, T], non-empty
    for c in range(int(off[-1])):
        s = int(np.searchsorted(off, c, side="right") - 1)
        tok0 = start[s] + (c - off[s]) * 64
        n = min(64, start[s] + ln[s] - tok0)
        assert 0 <= tok0 and n >= 1 and tok0 + n <= T


def test_well_formed_table_is_exact(harness):
    rng = np.random.default_rng(5)
    for N in (1, 3, 64, 1500, 2048, 2049, 5000):
        lens = rng.integers(0, 400, N)
        lens[: min(N, 4)] = [0, 1, 64, 65][: min(N, 4)]
        cu = np.concatenate([[0], np.cumsum(lens)])
        T = int(cu[-1])
        off, order, span, cap = _run(harness, cu, T)
        ch = (lens + 63) // 64
        assert (off == np.concatenate([[0], np.cumsum(ch)])).all()
        assert off[-1] <= cap
        assert (span[:, 0] == cu[:-1]).all() and (span[:, 1] == lens).all()
        if N <= 2048:
            assert (order == np.lexsort((np.arange(N), -lens))).all()   # longest first, ties by index
        else:
            assert (order == np.arange(N)).all()
        _check_safe(off, order, span, cap, T)


@pytest.mark.parametrize("cu,T", [
    ([0, 100, 50, 150], 150),                 # decreasing pair
    ([0, 5000, 6000], 1000),                  # past T
    ([-300, 10, 20], 20),                     # negative
    ([0, 1000, 0, 1000, 0, 1000], 1000),      # overlapping: chunk count over the capacity
    ([2**31 - 1, 0, 2**31 - 1], 64),          # extremes
    ([0, -2**31, 2**31 - 1, 5], 7),
    ([7, 7, 7], 7),                           # empty sequences at T
])
def test_malformed_offsets_stay_in_bounds(harness, cu, T):
    off, order, span, cap = _run(harness, cu, T)
    _check_safe(off, order, span, cap, T)


def test_random_malformed_offsets_stay_in_bounds(harness):
    rng = np.random.default_rng(11)
    for _ in range(40):
        N = int(rng.integers(1, 300))
        T = int(rng.integers(0, 20000))
        cu = rng.integers(-T - 10, 2 * T + 10, N + 1)
        off, order, span, cap = _run(harness, cu, T)
        _check_safe(off, order, span, cap, T)
