"""Pins for the oracle's random streams and sketch construction (CPU only).

Each check compares the oracle with something other than itself: published
SplitMix64 outputs, distribution tests, scipy's Hadamard construction,
explicit matrices, or torch's bfloat16 conversion.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import scipy.stats
import torch

from oracle import rng, sketch


def test_splitmix64_published_sequence():
    # SplitMix64 started from state 0 (Steele, Lea & Flood; the reference
    # generator splitmix64.c): the first three outputs are these constants.
    # r(seed, stream, i) is that sequence started from key(seed, stream), so
    # evaluating the counter form at key 0 must reproduce them.
    expect = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    with np.errstate(over="ignore"):
        z = np.uint64(rng.PHI) * (np.arange(3, dtype=np.uint64) + np.uint64(1))
    got = [int(v) for v in rng.mix64(z)]
    assert got == expect
    assert [rng.mix64_int((rng.PHI * (i + 1)) & rng.MASK64) for i in range(3)] == expect


def test_uniform_open_interval_and_moments():
    r = rng.draw(5, 0, np.arange(200000))
    u = rng.uniform53(r)
    assert u.min() > 0.0 and u.max() < 1.0
    # mean 1/2, variance 1/12, within 4 standard errors
    n = u.size
    assert abs(u.mean() - 0.5) < 4 * math.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 4 * math.sqrt(1 / 180 / n)


@pytest.mark.parametrize("stream", [rng.STREAM_DENSE, rng.STREAM_G])
def test_gaussian_moments_and_ks(stream):
    x = rng.gaussian_fast(11, stream, np.arange(100000))
    n = x.size
    assert abs(x.mean()) < 4 / math.sqrt(n)
    assert abs(x.var() - 1.0) < 4 * math.sqrt(2 / n)
    assert scipy.stats.kstest(x, "norm").pvalue > 1e-3


def test_gaussian_exact_matches_vectorised():
    a = rng.gaussian_exact(3, 0, 4096)
    b = rng.gaussian_fast(3, 0, np.arange(4096))
    assert np.max(np.abs(a - b)) < 1e-12


def test_dither_sign_words_by_hand():
    # Key i's sign words, written out from the definition with Python ints:
    # W = ceil(m / 64) draws r(seed, 5, i W + w); 32-bit word v is the high
    # half of draw v // 2 for even v, the low half for odd v; bit j % 32 of
    # word j // 32 (LSB first) set means -1.
    seed = 9
    key = rng.mix64_int((seed + rng.PHI * (5 + 1)) & rng.MASK64)
    for m, keys in ((32, [0, 1, 77]), (64, [3]), (96, [5, 2**40 + 7]), (256, [0, 12345])):
        W = (m + 63) // 64
        got = rng.dither_signs(seed, keys, m)
        assert got.shape == (len(keys), m)
        for r, i in enumerate(keys):
            for j in range(m):
                v = j // 32
                h = rng.mix64_int((key + rng.PHI * (i * W + v // 2 + 1)) & rng.MASK64)
                word = (h >> 32) if v % 2 == 0 else (h & 0xFFFFFFFF)
                want = -1.0 if (word >> (j % 32)) & 1 else 1.0
                assert got[r, j] == want, (m, i, j)


def test_dither_magnitudes_are_float32_half_normals():
    a = rng.dither_magnitudes(4, 512)
    g = rng.gaussian_exact(4, rng.STREAM_DITHER, 512)
    assert np.array_equal(a, np.abs(g).astype(np.float32).astype(np.float64))
    assert np.all(a >= 0)
    assert np.max(np.abs(a - np.abs(g))) <= 2.0 ** -24 * np.max(np.abs(g))
    # half-normal over many draws: E a = sqrt(2 / pi), E a^2 = 1
    x = rng.dither_magnitudes(6, 200000, exact=False)
    n = x.size
    assert abs(x.mean() - math.sqrt(2 / math.pi)) < 4 * math.sqrt((1 - 2 / math.pi) / n)
    assert abs((x * x).mean() - 1.0) < 4 * math.sqrt(2 / n)
    assert scipy.stats.kstest(x, "halfnorm").pvalue > 1e-3


def test_dither_of_one_key_is_gaussian_over_sketches():
    # The estimator's unbiasing factor sqrt(1 + rho^2) needs, for one key,
    # m independent N(0, 1) dither values independent of the transform.
    # Over 3000 sketch seeds (magnitudes drawn with each sketch, the key's
    # signs with its index):
    m, N = 64, 3000
    xi = np.vstack([rng.dither(s, [17], m, rng.dither_magnitudes(s, m, exact=False))
                    for s in range(N)])
    v = xi.reshape(-1)
    n = v.size
    assert abs(v.mean()) < 4 / math.sqrt(n)
    assert abs(v.var() - 1.0) < 4 * math.sqrt(2 / n)
    assert scipy.stats.kstest(v, "norm").pvalue > 1e-3
    for p, mom in ((4, 3.0), (6, 15.0)):
        se = math.sqrt((math.prod(range(2 * p - 1, 0, -2)) - mom * mom) / n)
        assert abs(np.mean(v ** p) - mom) < 4 * se, p
    for t in (0.005, 0.5, 2.0):
        e = np.exp(-t * v * v)
        assert abs(e.mean() - 1 / math.sqrt(1 + 2 * t)) < 4 * e.std() / math.sqrt(n), t
    # coordinates of one key are uncorrelated (adjacent, and across the two
    # halves of one draw)
    for a, b in ((0, 1), (0, 32), (5, 40)):
        c = np.corrcoef(xi[:, a], xi[:, b])[0, 1]
        assert abs(c) < 4 / math.sqrt(N), (a, b)


def test_dither_signs_fair_and_distinct_per_key():
    s = rng.dither_signs(0, np.arange(4000), 256)
    n = s.size
    assert abs(s.mean()) < 4 / math.sqrt(n)
    # distinct keys: uncorrelated sign vectors (so uncorrelated dither)
    c = (s[:-1] * s[1:]).mean()
    assert abs(c) < 4 / math.sqrt(s[1:].size)
    assert not np.array_equal(rng.dither_signs(0, [7], 256), rng.dither_signs(0, [8], 256))
    assert np.array_equal(rng.dither_signs(0, [7], 256), rng.dither_signs(0, np.array([7]), 256))
    # one key's two 32-bit halves of a draw are uncorrelated
    c2 = (s[:, 0:32] * s[:, 32:64]).mean()
    assert abs(c2) < 4 / math.sqrt(s[:, 0:32].size)


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64])
def test_sylvester_matches_scipy_and_is_orthogonal(d):
    H = sketch.sylvester(d)
    assert np.array_equal(H, scipy.linalg.hadamard(d).astype(np.float64))
    assert np.array_equal(H @ H.T, d * np.eye(d))
    # entry formula (-1)^popcount(i & c)
    i, c = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    pc = np.vectorize(lambda v: bin(v).count("1"))(i & c)
    assert np.array_equal(H, (-1.0) ** pc)


@pytest.mark.parametrize("d", [2, 8, 64, 256])
def test_fwht_equals_matrix(d):
    x = np.random.default_rng(0).standard_normal((5, d))
    H = scipy.linalg.hadamard(d).astype(np.float64)
    assert np.allclose(sketch.fwht(x), x @ H.T, rtol=0, atol=1e-11 * d)


@pytest.mark.parametrize("d,nb", [(2, 1), (4, 2), (8, 1), (16, 3), (32, 2), (64, 2)])
def test_fqjl_chain_equals_explicit_product(d, nb):
    sk = sketch.make_fqjl(7, d, nb * d)
    # the explicit matrix built independently from scipy's Hadamard
    H = scipy.linalg.hadamard(d).astype(np.float64)
    blocks = []
    for b in range(nb):
        Pi = np.eye(d)[sk.P[b]]                     # row i picks u[P[i]]
        blocks.append(H @ np.diag(sk.G[b]) @ Pi @ H @ np.diag(sk.D[b]) / math.sqrt(d))
    E = np.vstack(blocks)
    assert np.allclose(sk.explicit(), E, rtol=0, atol=1e-12 * d)
    X = np.random.default_rng(1).standard_normal((9, d))
    assert np.allclose(sketch.fqjl_apply(sk, X), X @ E.T, rtol=0, atol=1e-12 * d * d)


def test_fqjl_components_valid():
    sk = sketch.make_fqjl(0, 128, 512)
    for b in range(4):
        assert sorted(sk.P[b].tolist()) == list(range(128))
        assert set(np.unique(sk.D[b]).tolist()) <= {-1.0, 1.0}
    assert not np.array_equal(sk.P[0], sk.P[1])
    # G rounded to float32
    assert np.array_equal(sk.G, sk.G.astype(np.float32).astype(np.float64))
    # Rademacher and permutation statistics over many blocks
    big = sketch.make_fqjl(1, 16, 16 * 400)
    frac = (big.D > 0).mean()
    assert abs(frac - 0.5) < 4 * 0.5 / math.sqrt(big.D.size)
    # each position of a uniform permutation is uniform on range(d)
    counts = np.zeros((16, 16))
    for b in range(400):
        counts[np.arange(16), big.P[b]] += 1
    chi2 = ((counts - 25.0) ** 2 / 25.0).sum()
    assert scipy.stats.chi2.sf(chi2, df=15 * 15) > 1e-4


def test_bf16_rounding_matches_torch():
    rs = np.random.default_rng(2)
    x = np.concatenate([rs.standard_normal(20000) * 10 ** rs.uniform(-3, 3, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.0078125, -2.5]]).astype(np.float32)
    ours = sketch.round_f32_to_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, theirs)


def test_dense_sketch_roundings():
    sk = sketch.make_dense(0, 128, 256)
    assert sk.S64.shape == (256, 128)
    assert np.array_equal(sk.S32, sk.S64.astype(np.float32).astype(np.float64))
    assert np.array_equal(sk.S16, torch.from_numpy(sk.S32.astype(np.float32))
                          .to(torch.bfloat16).double().numpy())
    # S[j, c] = N(j d + c): row-major counter layout
    assert sk.S64[3, 5] == rng.gaussian_exact(0, 0, 1, offset=3 * 128 + 5)[0]
    # moments of the whole matrix
    x = sk.S64.reshape(-1)
    assert abs(x.mean()) < 4 / math.sqrt(x.size)
    assert abs(x.var() - 1) < 4 * math.sqrt(2 / x.size)
