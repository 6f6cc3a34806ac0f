"""Pins for the oracle's quantizer and estimator (CPU only).

What the pages fix about the method, and how each is checked here:
  * sign quantization with LSB-first packing: hand-computed words;
  * the estimator is unbiased (QJL abstract): Monte Carlo over sketch seeds,
    mean within 3 standard errors of the exact q.k, for dense, FQJL and
    dithered sketches;
  * distortion shrinks with m: closed-form variance for dense rows, and the
    error's m^-1/2 slope;
  * FQJL's exact unbiasedness conditional on D and P (Gaussian second
    diagonal), which a plain Hadamard swap would lose;
  * invariances and special cases; brute force on tiny inputs.
"""
import math

import numpy as np
import pytest

from oracle import qjl, rng, sketch

SQ = math.sqrt(math.pi / 2)


# ---------------------------------------------------------------- packing
def test_hand_computed_sign_words():
    # d = 4, S[j] = e_(j mod 4) * (-1)^floor(j/4), k = (1, -2, 3, -4):
    # y_j = k_(j mod 4) * (-1)^floor(j/4).  In an even group of four the
    # signs are (+, -, +, -) -> bits 1,0,1,0 -> nibble 0b0101 = 0x5; in an odd
    # group they flip -> 0b1010 = 0xA.  LSB-first, nibble n holds group n, so
    # every word reads 0xA5A5A5A5.
    for m in (32, 64):
        S = np.array([np.eye(4)[j % 4] * (-1) ** (j // 4) for j in range(m)])
        sk = sketch.DenseSketch(0, 4, m, 0.0, S, S, S)
        bits, norms, margin, Y = qjl.quantize(sk, np.array([[1.0, -2.0, 3.0, -4.0]]), "f32")
        assert bits.dtype == np.uint32
        assert bits.tolist() == [[0xA5A5A5A5] * (m // 32)]
        assert norms[0] == math.sqrt(30.0)
        # margin = |y| / (||k|| sqrt d)
        assert np.allclose(margin[0, :4], np.array([1, 2, 3, 4]) / (math.sqrt(30) * 2))


def test_zero_key_gives_all_ones_zero_norm_zero_score():
    sk = sketch.make_dense(0, 16, 64)
    bits, norms, margin, _ = qjl.quantize(sk, np.zeros((1, 16)), "f32")
    assert bits.tolist() == [[0xFFFFFFFF, 0xFFFFFFFF]]
    assert norms[0] == 0.0 and np.all(np.isinf(margin))
    Sq = qjl.project(sk, np.ones((1, 16)), "f32")
    assert qjl.score(Sq, bits, norms, 64, 0.0, 1, 1, 1)[0, 0, 0] == 0.0


def test_pack_unpack_roundtrip_and_bit_order():
    B = np.random.default_rng(0).random((7, 96)) < 0.5
    W = qjl.pack_bits(B)
    assert np.array_equal(qjl.unpack_bits(W, 96), B)
    one = np.zeros((1, 64), dtype=bool)
    one[0, 33] = True
    assert qjl.pack_bits(one).tolist() == [[0, 2]]
    # little-endian bytes of two u32 words equal one u64 word, LSB-first
    B2 = np.random.default_rng(1).random((3, 64)) < 0.5
    w64 = qjl.pack_bits(B2).view(np.uint64)[:, 0]
    for r in range(3):
        assert all(((int(w64[r]) >> j) & 1) == int(B2[r, j]) for j in range(64))


# ---------------------------------------------------------------- brute force
def _brute_estimate(S, q, k, rho=0.0, xi=None):
    m, d = len(S), len(S[0])
    nk = math.sqrt(sum(v * v for v in k))
    tot = 0.0
    for j in range(m):
        y = sum(S[j][c] * k[c] for c in range(d))
        if xi is not None:
            y += rho * nk * xi[j]
        sq = sum(S[j][c] * q[c] for c in range(d))
        tot += sq if y >= 0 else -sq
    return SQ * math.sqrt(1 + rho * rho) / m * nk * tot


@pytest.mark.parametrize("variant,rho", [("dense", 0.0), ("dense", 0.5), ("fqjl", 0.0), ("fqjl", 0.3),
                                         ("dfqjl", 0.3), ("pfqjl", 0.0)])
def test_brute_force_tiny(variant, rho):
    d, m = 4, 32
    sk = sketch.make_sketch(3, d, m, variant, rho)
    S = sk.effective("f32")
    rs = np.random.default_rng(4)
    G, nq, nk = 2, 3, 5
    K = rs.standard_normal((G * nk, d))
    Q = rs.standard_normal((G * nq, d))
    bits, norms, _, _ = qjl.quantize(sk, K, "f32", key_index_base=10)
    out = qjl.score(qjl.project(sk, Q, "f32"), bits, norms, m, rho, G, nq, nk)
    xi = rng.dither(3, np.arange(10, 10 + G * nk), m, sk.dmag) if rho > 0 else None
    for g in range(G):
        for i in range(nq):
            for t in range(nk):
                ref = _brute_estimate(S.tolist(), Q[g * nq + i].tolist(), K[g * nk + t].tolist(),
                                      rho, xi[g * nk + t].tolist() if rho > 0 else None)
                assert abs(out[g, i, t] - ref) <= 1e-12 * (1 + abs(ref))


# ---------------------------------------------------------------- Monte Carlo
def _pairs(d, rs):
    k = rs.standard_normal(d)
    q = rs.standard_normal(d)
    qo = q - (q @ k) / (k @ k) * k                       # q orthogonal to k
    ko = rs.standard_normal(d)
    ko[rs.choice(d, 2, replace=False)] *= 15.0          # per-channel outliers
    s = np.abs(rs.standard_t(3, d))
    return [("random", q, k), ("q=k", k.copy(), k), ("q_perp_k", qo, k),
            ("outlier_k", q, ko), ("tscaled", q * s, k * s)]


def _mc(variant, d, m, rho, seeds, q, k):
    est = np.empty(len(seeds))
    for t, s in enumerate(seeds):
        sk = sketch.make_sketch(int(s), d, m, variant, rho, exact=False)
        est[t] = qjl.estimate_inner_product(sk, q, k, key_index=int(s))
    return est


@pytest.mark.parametrize("variant,rho", [("dense", 0.0), ("fqjl", 0.0), ("fqjl", 0.1), ("dense", 1.0),
                                         ("dfqjl", 0.1), ("dfqjl", 1.0), ("pfqjl", 0.0)])
def test_unbiased_over_seeds(variant, rho):
    d, m, N = 16, 64, 3000
    rs = np.random.default_rng(12)
    for name, q, k in _pairs(d, rs):
        est = _mc(variant, d, m, rho, range(N), q, k)
        se = est.std(ddof=1) / math.sqrt(N)
        assert abs(est.mean() - q @ k) <= 3 * se, (name, est.mean(), q @ k, se)


def test_dither_factor_is_needed():
    # rho = 1: without sqrt(1 + rho^2) the mean would be q.k / sqrt(2)
    d, m, N, rho = 16, 64, 3000, 1.0
    rs = np.random.default_rng(5)
    k = rs.standard_normal(d)
    q = k + 0.3 * rs.standard_normal(d)
    est = _mc("dense", d, m, rho, range(N), q, k)
    se = est.std(ddof=1) / math.sqrt(N)
    assert abs(est.mean() - q @ k) <= 3 * se
    assert abs(est.mean() / math.sqrt(2) - q @ k) > 10 * se


def test_dense_variance_closed_form():
    # Var = [(pi/2) ||k||^2 ||q||^2 (1 + rho^2) - (q.k)^2] / m for iid Gaussian rows
    d, m, N = 16, 32, 4000
    rs = np.random.default_rng(6)
    for rho in (0.0, 0.5):
        k = rs.standard_normal(d)
        q = 0.6 * k + rs.standard_normal(d)
        est = _mc("dense", d, m, rho, range(N), q, k)
        var = ((math.pi / 2) * (k @ k) * (q @ q) * (1 + rho * rho) - (q @ k) ** 2) / m
        assert abs(est.var(ddof=1) / var - 1) < 0.10


@pytest.mark.parametrize("variant,rho", [("dense", 0.0), ("fqjl", 0.0), ("dfqjl", 0.1),
                                         ("pfqjl", 0.0)])
def test_error_shrinks_like_inverse_sqrt_m(variant, rho):
    d, N = 16, 300
    rs = np.random.default_rng(7)
    k = rs.standard_normal(d)
    q = rs.standard_normal(d)
    ms = [32, 64, 128, 256, 512, 1024]
    rms = []
    for m in ms:
        est = _mc(variant, d, m, rho, range(1000, 1000 + N), q, k)
        rms.append(math.sqrt(np.mean((est - q @ k) ** 2)))
    assert all(a > b for a, b in zip(rms, rms[1:]))
    slope = np.polyfit(np.log(ms), np.log(rms), 1)[0]
    lo, hi = (-0.6, -0.4) if variant == "dense" else (-0.7, -0.3)
    assert lo <= slope <= hi, slope


def test_fqjl_unbiased_conditional_on_D_and_P():
    # Gaussian second diagonal: unbiased for every fixed D, P (mean over G only)
    d, m, N = 16, 32, 6000
    base = sketch.make_fqjl(0, d, m)
    rs = np.random.default_rng(8)
    k = rs.standard_normal(d)
    q = 0.5 * k + rs.standard_normal(d)
    est = np.empty(N)
    for t in range(N):
        G = rng.gaussian_fast(100 + t, rng.STREAM_G, np.arange(m)).reshape(m // d, d)
        sk = sketch.FqjlSketch(0, d, m, 0.0, base.D, base.P, sketch.round_to_f32(G))
        est[t] = qjl.estimate_inner_product(sk, q, k)
    se = est.std(ddof=1) / math.sqrt(N)
    assert abs(est.mean() - q @ k) <= 3 * se


def test_rademacher_second_diagonal_would_be_biased():
    # The contrast the FQJL page draws: with a +-1 second diagonal the
    # coordinates are not Gaussian and the same constant is biased for a
    # spiky key.  k = e_0 with D = 1, P = id: (H/sqrt d) k is flat, so every
    # coordinate is +-1 * (sum of +-1/sqrt d) ... the estimate of ||k||^2 = 1
    # with q = k then has mean sqrt(pi/2) E|sum_c eps_c h_c|/sqrt(d) != 1.
    d, m, N = 4, 32, 20000
    k = np.zeros(d)
    k[0] = 1.0
    ident = sketch.make_fqjl(0, d, m)
    ident.D[:] = 1.0
    ident.P[:] = np.arange(d)
    rs = np.random.default_rng(9)
    est_g, est_r = np.empty(N), np.empty(N)
    for t in range(N):
        g = rs.standard_normal((m // d, d))
        r = rs.choice([-1.0, 1.0], (m // d, d))
        for arr, diag in ((est_g, g), (est_r, r)):
            sk = sketch.FqjlSketch(0, d, m, 0.0, ident.D, ident.P, diag)
            arr[t] = qjl.estimate_inner_product(sk, k, k)
    se_g = est_g.std(ddof=1) / math.sqrt(N)
    se_r = est_r.std(ddof=1) / math.sqrt(N)
    assert abs(est_g.mean() - 1.0) <= 3 * se_g
    assert abs(est_r.mean() - 1.0) > 10 * se_r


def test_fqjl_coordinate_variance_is_norm_squared():
    d, m, N = 32, 64, 3000
    base = sketch.make_fqjl(2, d, m)
    rs = np.random.default_rng(10)
    k = rs.standard_normal(d) * np.abs(rs.standard_t(3, d))
    Y2 = np.zeros(m)
    for t in range(N):
        G = rng.gaussian_fast(500 + t, rng.STREAM_G, np.arange(m)).reshape(m // d, d)
        sk = sketch.FqjlSketch(2, d, m, 0.0, base.D, base.P, G)
        Y2 += qjl.project(sk, k[None, :], "f32")[0] ** 2
    Y2 /= N
    # each coordinate's E[Y^2] = ||k||^2; the sample mean of Y^2 (chi-square
    # with 1 dof times ||k||^2) has relative standard error sqrt(2/N)
    z = (Y2 / (k @ k) - 1) / math.sqrt(2 / N)
    assert np.max(np.abs(z)) < 4.5
    assert abs(z.mean()) < 4.5 / math.sqrt(m)


# ---------------------------------------------------------------- invariances
@pytest.mark.parametrize("variant", ["dense", "fqjl"])
def test_invariances(variant):
    d, m = 32, 128
    sk = sketch.make_sketch(4, d, m, variant)
    rs = np.random.default_rng(11)
    K = rs.standard_normal((6, d))
    Q = rs.standard_normal((1, d))
    b0, n0, mg0, _ = qjl.quantize(sk, K, "f32")
    Sq = qjl.project(sk, Q, "f32")
    s0 = qjl.score(Sq, b0, n0, m, 0.0, 1, 1, 6)
    b1, n1, _, _ = qjl.quantize(sk, 2.5 * K, "f32")          # k -> c k
    assert np.array_equal(b0, b1) and np.allclose(n1, 2.5 * n0)
    assert np.allclose(qjl.score(Sq, b1, n1, m, 0.0, 1, 1, 6), 2.5 * s0)
    assert np.allclose(qjl.score(3 * Sq, b0, n0, m, 0.0, 1, 1, 6), 3 * s0)   # q -> c q
    b2, n2, _, _ = qjl.quantize(sk, -K, "f32")               # k -> -k
    assert np.all(mg0 > 0)
    assert np.array_equal(b2, ~b0)
    assert np.allclose(qjl.score(Sq, b2, n2, m, 0.0, 1, 1, 6), -s0)


def test_unit_vector_special_case():
    # k = q = e_1: the estimate is sqrt(pi/2)/m * sum_j |S_j1| exactly, and
    # tends to 1 = <e_1, e_1> as m grows (E|N(0,1)| = sqrt(2/pi)).
    d, m = 8, 8192
    sk = sketch.make_dense(1, d, m, exact=False)
    e = np.zeros(d)
    e[1] = 1.0
    est = qjl.estimate_inner_product(sk, e, e)
    exact = SQ / m * np.abs(sk.S32[:, 1]).sum()
    assert abs(est - exact) < 1e-12
    sd = math.sqrt((math.pi / 2 - 1) / m)
    assert abs(est - 1.0) < 4 * sd


def test_estimator_constant():
    assert qjl.estimator_constant(256, 0.0) == math.sqrt(math.pi / 2) / 256
    assert abs(qjl.estimator_constant(128, 0.1) - math.sqrt(math.pi / 2) * math.sqrt(1.01) / 128) < 1e-18


# ---------------------------------------------------------------- D-FQJL / P-FQJL
def test_dfqjl_block_is_the_unpermuted_composition():
    # D-FQJL (the FQJL page's first construction) has no permutation: its
    # block is H diag(G) (H / sqrt d) diag(D), built here from scipy's
    # Hadamard matrix, while P-FQJL and the composition keep the permutation
    from scipy.linalg import hadamard
    d, m = 16, 64
    dk = sketch.make_sketch(5, d, m, "dfqjl", 0.2)
    pk = sketch.make_sketch(5, d, m, "pfqjl", 0.0)
    fk = sketch.make_sketch(5, d, m, "fqjl", 0.0)
    H = hadamard(d).astype(np.float64)
    for b in range(m // d):
        ref = H @ np.diag(dk.G[b]) @ (H / math.sqrt(d)) @ np.diag(dk.D[b])
        assert np.allclose(dk.explicit()[b * d:(b + 1) * d], ref, rtol=0, atol=1e-12)
        assert np.array_equal(dk.P[b], np.arange(d))
    # same D and G streams for one seed; the permutation is the only difference
    assert np.array_equal(dk.D, fk.D) and np.array_equal(dk.G, fk.G)
    assert np.array_equal(pk.P, fk.P) and not np.array_equal(pk.P, dk.P)
    assert np.array_equal(pk.explicit(), fk.explicit())
    X = np.random.default_rng(0).standard_normal((5, d))
    assert np.allclose(sketch.fqjl_apply(dk, X), X @ dk.explicit().T, rtol=0, atol=1e-10)


def test_variant_rho_rules():
    with pytest.raises(ValueError):
        sketch.make_sketch(0, 16, 32, "dfqjl", 0.0)
    with pytest.raises(ValueError):
        sketch.make_sketch(0, 16, 32, "pfqjl", 0.1)


def test_dfqjl_unbiased_conditional_on_D():
    # with P = I the Gaussian second diagonal still makes every coordinate
    # pair jointly Gaussian given D, so the dithered estimator with
    # sqrt(1 + rho^2) is unbiased over G and the dither (its magnitudes and
    # the key's signs) alone
    d, m, N, rho = 16, 32, 6000, 0.5
    base = sketch.make_sketch(0, d, m, "dfqjl", rho)
    rs = np.random.default_rng(13)
    k = rs.standard_normal(d)
    q = 0.5 * k + rs.standard_normal(d)
    est = np.empty(N)
    for t in range(N):
        G = rng.gaussian_fast(300 + t, rng.STREAM_G, np.arange(m)).reshape(m // d, d)
        # the dither magnitudes are drawn with the sketch, as G is
        sk = sketch.FqjlSketch(0, d, m, rho, base.D, base.P, sketch.round_to_f32(G), "dfqjl",
                               dmag=rng.dither_magnitudes(300 + t, m, exact=False))
        est[t] = qjl.estimate_inner_product(sk, q, k, key_index=t)
    se = est.std(ddof=1) / math.sqrt(N)
    assert abs(est.mean() - q @ k) <= 3 * se
