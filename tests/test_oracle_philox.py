"""Pins of the oracle's random-number path.

Philox4x32-10 (Salmon et al., SC'11) is not on the pages; the oracle's
implementation is checked against two independent installed source
implementations (PyTorch's at::philox_engine and rocRAND's
philox4x32_10_engine), compiled here from their headers.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _crosscheck_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("g++ or rocRAND headers not available")
    import torch.utils.cpp_extension as ce
    inc = [f"-I{p}" for p in ce.include_paths()]
    exe = str(tmp_path_factory.mktemp("pxc") / "pxc")
    subprocess.check_call([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *inc,
                           os.path.join(HERE, "philox_crosscheck.cpp"), "-o", exe])
    return exe


def test_philox_matches_two_independent_implementations(tmp_path_factory):
    exe = _crosscheck_binary(tmp_path_factory)
    rng = np.random.default_rng(123)
    n = 10000
    words = rng.integers(0, 2**32, size=(n, 6), dtype=np.uint64)
    edge = []
    for k in (0, 2**32 - 1):
        for c in (0, 1, 2**32 - 1):
            edge.append([c, c, c, c, k, k])
            edge.append([c, 0, c, 0, k, 0])
    words = np.concatenate([np.array(edge, dtype=np.uint64), words])
    inp = "\n".join(" ".join(str(int(v)) for v in row) for row in words) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    ref = np.array([[int(v) for v in line.split()] for line in out if line.strip()], dtype=np.uint64)
    assert ref.shape == (len(words), 8)
    # the two installed implementations agree with each other ...
    np.testing.assert_array_equal(ref[:, :4], ref[:, 4:])
    # ... and with the oracle
    mine = np.array([oracle.philox4x32_10(row[:4], row[4:]) for row in words], dtype=np.uint64)
    np.testing.assert_array_equal(mine, ref[:, :4])


def test_uniform_mapping_is_open_interval_and_fp32_exact():
    lo = oracle.uniform(0)
    hi = oracle.uniform(0xFFFFFFFF)
    assert lo == 2.0 ** -24
    assert hi == 1.0 - 2.0 ** -24
    rng = np.random.default_rng(5)
    for w in rng.integers(0, 2**32, size=2000, dtype=np.uint64):
        u = oracle.uniform(int(w))
        assert 0.0 < u < 1.0
        assert float(np.float32(u)) == u  # exactly representable in fp32
        # the 9 low bits do not matter; the 23 high bits pick one of 2^23 odd multiples of 2^-24
        assert u == (2 * (int(w) >> 9) + 1) / 2.0 ** 24


def test_coin_and_noise_use_distinct_counter_streams():
    seed = (3 << 32) | 17
    # coin of (b, r) is word 0 of counter (0, r, b, 0)
    out = oracle.philox4x32_10([0, 5, 9, 0], [17, 3])
    assert oracle.coin(seed, 9, 5) == oracle.uniform(int(out[0]))
    # race noise of vocab id y is word y&3 of counter (y>>2, r, b, 1)
    for y in (0, 1, 2, 3, 4, 1001, 128255):
        out = oracle.philox4x32_10([y >> 2, 5, 9, 1], [17, 3])
        assert oracle.noise_uniform(seed, 9, 5, y) == oracle.uniform(int(out[y & 3]))


def test_noise_uniforms_are_uniform():
    from scipy import stats
    u = np.array([oracle.noise_uniform(42, 3, 1, y) for y in range(20000)])
    assert stats.kstest(u, "uniform").pvalue > 1e-4


# Known-answer vectors of Philox4x32 with 10 rounds, as distributed with the
# Random123 library of Salmon et al. (its kat_vectors file): counter words
# c0..c3 and key words k0, k1 in, four output words out.
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answer_vectors(ctr, key, want):
    got = oracle.philox4x32_10(ctr, key)
    assert [int(w) for w in got] == list(want)
