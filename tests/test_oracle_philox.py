"""Pins of the oracle's Philox4x32-10 and of its sampler counter layout."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.philox import philox4x32_10
from oracle import sampler

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(w, 16) for w in line.split()])
    return rows


def test_known_answer_vectors():
    for row in _kat():
        out = philox4x32_10(*[np.uint32(w) for w in row[:4]], row[4], row[5])
        assert [int(x) for x in out] == row[6:10]


@pytest.fixture(scope="module")
def rocrand_host(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("rr") / "rr")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "helpers", "rocrand_philox_host.cpp"),
                    "-o", exe], check=True, capture_output=True)
    return exe


def test_matches_rocrand_library_on_many_counters(rocrand_host):
    rng = np.random.default_rng(123)
    n = 2000
    seeds = rng.integers(0, 2**63, size=n, dtype=np.uint64)
    subs = rng.integers(0, 2**63, size=n, dtype=np.uint64)
    blocks = rng.integers(0, 2**61, size=n, dtype=np.uint64)
    lines = "\n".join("%x %x %x" % (int(s), int(u), int(b) * 4)
                      for s, u, b in zip(seeds, subs, blocks))
    out = subprocess.run([rocrand_host], input=lines, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    lib = np.array([[int(w, 16) for w in line.split()] for line in out if line.strip()],
                   dtype=np.uint64)
    mine = []
    for s, u, b in zip(seeds, subs, blocks):
        s, u, b = int(s), int(u), int(b)
        r = philox4x32_10(np.uint32(b & 0xFFFFFFFF), np.uint32(b >> 32),
                          np.uint32(u & 0xFFFFFFFF), np.uint32(u >> 32), s & 0xFFFFFFFF, s >> 32)
        mine.append([int(x) for x in r])
    assert np.array_equal(lib, np.array(mine, dtype=np.uint64))


def test_vectorised_equals_scalar():
    c = np.arange(64, dtype=np.uint32)
    r = philox4x32_10(c, c * 3, c ^ 7, np.uint32(9), 0x12345678, 0x9abcdef0)
    for i in range(64):
        s = philox4x32_10(np.uint32(i), np.uint32(i * 3), np.uint32(i ^ 7), np.uint32(9),
                          0x12345678, 0x9abcdef0)
        assert all(int(r[w][i]) == int(s[w]) for w in range(4))


def test_uniform_tokens_power_of_two_closed_form():
    # for V = 2^k, (x0 * V) >> 32 is the top k bits of x0
    pos = np.arange(256)
    for logv in (1, 9, 18):
        v = 1 << logv
        t = sampler.uniform_tokens(2, 3, 5, pos, v)
        x0 = philox4x32_10(np.zeros(256, np.uint32), pos.astype(np.uint32), np.uint32(5),
                           np.uint32((3 << 1) | 0), 2, 0)[0]
        assert np.array_equal(t, (x0 >> np.uint32(32 - logv)).astype(np.int64))


def test_uniform_tokens_range_and_chi2():
    from scipy.stats import chisquare
    v = 37
    t = np.concatenate([sampler.uniform_tokens(2, cid, s, np.arange(256), v)
                        for cid in range(4) for s in range(40)])
    assert t.min() >= 0 and t.max() < v
    assert chisquare(np.bincount(t, minlength=v)).pvalue > 1e-4


def test_distinct_streams():
    a = sampler.uniform_tokens(2, 0, 0, np.arange(256), 1 << 20)
    b = sampler.uniform_tokens(2, 1, 0, np.arange(256), 1 << 20)
    c = sampler.uniform_tokens(2, 0, 1, np.arange(256), 1 << 20)
    d = sampler.uniform_tokens(3, 0, 0, np.arange(256), 1 << 20)
    for other in (b, c, d):
        assert np.mean(a == other) < 0.01
