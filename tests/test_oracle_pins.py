"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test names what it pins.  The oracle is checked against closed forms, textbook
tables, invariants and brute force -- never against a retyping of its own formulas.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------ PRNG
def test_splitmix64_published_vector(O):
    want = [int(x, 16) for x in _golden_lines("splitmix64_seed0.txt")]
    got = [int(v) for v in O.splitmix64(0, 0, np.arange(len(want)))]
    assert got == want


def test_uniform_open_interval_and_moments(O):
    u = O.uniform01(123, 2, np.arange(200000))
    assert u.min() > 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 4 * math.sqrt(1 / 12 / len(u))
    # KS against U(0,1)
    assert stats.kstest(u, "uniform").pvalue > 1e-4


def test_gaussian_projection_is_standard_normal(O):
    S = O.gaussian_projection(256, 512, seed=7).astype(np.float64).ravel()
    n = S.size
    assert abs(S.mean()) < 4 / math.sqrt(n)
    assert abs(S.var() - 1.0) < 4 * math.sqrt(2.0 / n)
    assert stats.kstest(S, "norm").pvalue > 1e-4
    # deterministic per seed, different across seeds
    assert np.array_equal(O.gaussian_projection(8, 8, 7), O.gaussian_projection(8, 8, 7))
    assert not np.array_equal(O.gaussian_projection(8, 8, 7), O.gaussian_projection(8, 8, 8))


def test_rotation_signs_balanced(O):
    D = O.rotation_signs(100000, seed=3)
    assert set(np.unique(D)) == {-1.0, 1.0}
    assert abs(D.mean()) < 4 / math.sqrt(D.size)


# ------------------------------------------------------------------ codebook
@pytest.mark.parametrize("d", [8, 64, 128, 1536])
def test_marginal_density_normalised_and_unit_second_moment(O, d):
    # independent numerical quadrature of the density: mass 1, E[X^2] = 1/d
    f = lambda x: O.sphere_marginal_pdf(np.array([x]), d)[0]
    lim = min(1.0, 12.0 / math.sqrt(d))
    mass = integrate.quad(f, -lim, lim, limit=200, epsabs=1e-14)[0]
    m2 = integrate.quad(lambda x: x * x * f(x), -lim, lim, limit=200, epsabs=1e-16)[0]
    assert abs(mass - 1.0) < 1e-10
    assert abs(m2 * d - 1.0) < 1e-8


@pytest.mark.parametrize("d,bits", [(8, 2), (64, 2), (64, 3), (128, 2), (128, 3), (1536, 3)])
def test_lloyd_conditions_by_independent_quadrature(O, d, bits):
    cb = O.make_codebook(d, bits)
    c, t = cb.c64, cb.t64
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(c, -c[::-1], rtol=0, atol=1e-14)      # symmetry
    edges = np.concatenate(([-1.0], t, [1.0]))
    f = lambda x: O.sphere_marginal_pdf(np.array([x]), d)[0]
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        lo, hi = max(a, -14 / math.sqrt(d)), min(b, 14 / math.sqrt(d))
        mass = integrate.quad(f, lo, hi, limit=400, epsabs=1e-15, epsrel=1e-13)[0]
        mom = integrate.quad(lambda x: x * f(x), lo, hi, limit=400, epsabs=1e-17, epsrel=1e-13)[0]
        assert abs(mom / mass - c[k]) * math.sqrt(d) < 1e-10


@pytest.mark.parametrize("d", [8, 64, 128, 1536])
def test_one_bit_closed_form(O, d):
    # b = 1: c = +-E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    want = math.exp(math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d + 1) / 2))
    cb = O.make_codebook(d, 1)
    np.testing.assert_allclose(cb.c64, [-want, want], rtol=1e-11)  # lgamma cancellation at large d


def test_large_d_limit_is_max_gaussian_table(O):
    rows = _golden_lines("max1960_gaussian.txt")
    d = 1 << 22
    for row in rows:
        lv, mse = row.split("|")
        parts = lv.split()
        bits, levels = int(parts[0]), [float(x) for x in parts[1:]]
        cb = O.make_codebook(d, bits)
        pos = cb.c64[len(cb.c64) // 2:] * math.sqrt(d)
        np.testing.assert_allclose(pos, levels, atol=6e-4)
        assert abs(cb.mse() * d - float(mse)) < 2e-4


def test_codebook_matches_monte_carlo_conditional_means(O):
    # uniform unit vectors in R^64: empirical cell means of one coordinate ~ centroids
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200000, 64))
    u = (x / np.linalg.norm(x, axis=1, keepdims=True))[:, 0]
    cb = O.make_codebook(64, 2)
    cell = np.searchsorted(cb.t64, u)
    for k in range(4):
        sel = u[cell == k]
        assert abs(sel.mean() - cb.c64[k]) < 5 * sel.std() / math.sqrt(len(sel))


def test_stored_codebook_is_fp16_rounding_with_midpoint_boundaries(O):
    cb = O.make_codebook(128, 3)
    np.testing.assert_array_equal(cb.c, cb.c64.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(cb.t, 0.5 * (cb.c[:-1] + cb.c[1:]))
    # the midpoints are exact in fp32
    np.testing.assert_array_equal(cb.t.astype(np.float32).astype(np.float64), cb.t)


@pytest.mark.parametrize("d", [8, 64, 128, 1536])
def test_codebook_is_odd(O, d):
    # the marginal density of a rotated coordinate is even, so the Lloyd-Max optimum is an
    # odd function: c[K-1-k] = -c[k], t[K-2-k] = -t[k].  The oracle's fp64 iterate is odd up
    # to rounding, and the stored (fp16-rounded) codebook is odd exactly -- the form the
    # 2- and 3-bit plane identities of the decode and search rest on.
    for bits in (1, 2, 3, 4):
        cb = O.make_codebook(d, bits)
        np.testing.assert_allclose(cb.c64[::-1], -cb.c64, rtol=0, atol=2e-14)
        np.testing.assert_array_equal(cb.c[::-1], -cb.c)
        np.testing.assert_array_equal(cb.t[::-1], -cb.t)


# ------------------------------------------------------------------ rotation / RoPE
def test_hadamard_small_cases(O):
    np.testing.assert_array_equal(O.hadamard(2), [[1, 1], [1, -1]])
    np.testing.assert_array_equal(O.hadamard(4), [[1, 1, 1, 1], [1, -1, 1, -1],
                                                  [1, 1, -1, -1], [1, -1, -1, 1]])
    H = O.hadamard(64)
    np.testing.assert_array_equal(H @ H.T, 64 * np.eye(64))


@pytest.mark.parametrize("d", [64, 128, 1536])
def test_rotation_orthogonal_and_norm_preserving(O, d):
    P = O.rotation_matrix(d, seed=0)
    np.testing.assert_allclose(P.T @ P, np.eye(d), atol=1e-13)
    x = np.random.default_rng(0).standard_normal((50, d)) * 3
    y = x @ P.T
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    if d == 1536:   # block-diagonal of three 512 blocks
        assert np.all(P[:512, 512:] == 0) and np.all(P[512:1024, 1024:] == 0)


def test_rope_two_dim_is_plane_rotation(O):
    # d = 2: theta_0 = 1, so position p rotates by p radians
    x = np.array([[0.3, -1.7]])
    for p in [0, 1, 5, 131071]:
        c, s = math.cos(p), math.sin(p)
        want = np.array([0.3 * c + 1.7 * s, 0.3 * s - 1.7 * c])
        np.testing.assert_allclose(O.rope(x, [p], 10000.0)[0], want, atol=1e-12)


def test_rope_half_split_pairs(O):
    # d = 4, base 100: pair (0, 2) at angle p, pair (1, 3) at angle p / 10
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    p = 3.0
    a0, a1 = p, p / 10.0
    want = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
            1 * math.sin(a0) + 3 * math.cos(a0), 2 * math.sin(a1) + 4 * math.cos(a1)]
    np.testing.assert_allclose(O.rope(x, [p], 100.0)[0], want, atol=1e-14)


def test_rope_relative_position_and_rotation_invariance(O):
    # <R_i q, R_j k> = <q, R_{j-i} k>   and   <Pi R_i q, Pi R_j k> = <R_i q, R_j k>
    rng = np.random.default_rng(5)
    d = 128
    P = O.rotation_matrix(d, seed=11)
    for (i, j) in [(0, 7), (1000, 1000), (12345, 131071), (131071, 3)]:
        q, k = rng.standard_normal(d), rng.standard_normal(d) * 5
        a = O.rope(q[None], [i], 500000.0)[0] @ O.rope(k[None], [j], 500000.0)[0]
        b = q @ O.rope(k[None], [j - i], 500000.0)[0]
        c = (P @ O.rope(q[None], [i], 500000.0)[0]) @ (P @ O.rope(k[None], [j], 500000.0)[0])
        assert abs(a - b) <= 1e-9 * (1 + abs(a))
        assert abs(c - a) <= 1e-12 * (1 + np.linalg.norm(q) * np.linalg.norm(k))
    np.testing.assert_array_equal(O.rope(np.ones((2, 8)), [0, 0], 10000.0), np.ones((2, 8)))


# ------------------------------------------------------------------ encoder
@pytest.mark.parametrize("bits", [1, 2, 3])
def test_d8_exhaustive_codeword_search_equals_per_coordinate(O, bits):
    # nearest point of the product codebook C^8, searched over all 2^(8b) code vectors
    # (bits = 3 sampled over 4096 random code vectors plus the optimum), equals the
    # per-coordinate brute-force codes the encoder produces.
    codec = O.make_codec(8, bits, 0, 8, seed=2)
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((6, 8))
    enc = O.encode(x, codec, kind="db")
    c = codec.cb_k.c
    K = len(c)
    if bits <= 2:
        allcodes = np.array(list(itertools.product(range(K), repeat=8)))
    else:
        allcodes = np.concatenate([rng.integers(0, K, (4096, 8)), enc["codes"]])
    for r in range(x.shape[0]):
        dist = np.sum((enc["u"][r][None, :] - c[allcodes]) ** 2, axis=1)
        best = allcodes[np.argmin(dist)]
        assert np.array_equal(best, enc["codes"][r])
        assert np.min(dist) == pytest.approx(np.sum((enc["u"][r] - c[enc["codes"][r]]) ** 2))


def test_encode_mse_matches_codebook_mse(O):
    codec = O.make_codec(128, 2, 3, 128, seed=0)
    x = np.random.default_rng(9).standard_normal((4000, 128))
    for kind, cb in (("db", codec.cb_k), ("value", codec.cb_v)):
        enc = O.encode(x, codec, kind=kind)
        err = np.sum((enc["u"] - cb.c[enc["codes"]]) ** 2, axis=1)
        want = cb.mse() * 128
        assert abs(err.mean() - want) < 5 * err.std() / math.sqrt(len(err)) + 2e-4


def test_nearest_ties_go_to_larger_index(O):
    c = np.array([-1.0, 0.0, 1.0])
    got = O._nearest(np.array([-0.5, 0.5, -2.0, 0.25]), c)
    np.testing.assert_array_equal(got, [1, 2, 0, 1])


def test_zero_vector_and_fp16_saturation(O):
    codec = O.make_codec(64, 2, 3, 64, seed=1)
    x = np.zeros((1, 64))
    enc = O.encode(x, codec, kind="key", positions=[5], rope_base=10000.0)
    assert enc["n16"][0] == 0 and enc["rn16"][0] == 0
    assert np.all(enc["bits"] == 1)                      # sign(0) -> bit 1
    # code of u = 0: nearest stored centroid with ties up -> index 2 (first positive)
    assert np.all(enc["codes"] == 2)
    big = np.full((1, 64), 1e4)
    enc = O.encode(big, codec, kind="value")
    assert enc["n16"][0] == 65504.0 and enc["overflow"][0]


def test_residual_is_against_fp16_norm(O):
    codec = O.make_codec(64, 2, 0, 64, seed=4)
    x = np.random.default_rng(2).standard_normal((10, 64)) * 7
    enc = O.encode(x, codec, kind="db")
    recon = enc["n16"][:, None] * codec.cb_k.c[enc["codes"]]
    np.testing.assert_allclose(enc["r"], enc["y"] - recon, atol=1e-13)
    np.testing.assert_allclose(enc["z"], enc["r"] @ codec.S.T, atol=1e-12)


# ------------------------------------------------------------------ QJL estimator
def _qjl_estimates_over_seeds(O, n_seeds, d=64, m=64):
    """For one fixed key x and query q, the oracle's own score estimates under n_seeds codec
    seeds: through attend (scalar codes), search_scores and attend over a PolarQuant cache.
    Each seed draws a new rotation and a new S, so the residual changes from seed to seed.
    Also returns, per seed and path, the closed-form conditional variance of the QJL term,
    ||r||^2/m ((pi/2)||q||^2 - (q_rot . r_hat)^2), from the oracle's residual r."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(d)
    q = x + 0.5 * rng.standard_normal(d)   # correlated with x, so <q_rot, r> has a nonzero mean
    est = {"attend": np.empty(n_seeds), "search": np.empty(n_seeds), "polar": np.empty(n_seeds)}
    cvar = {k: np.empty(n_seeds) for k in est}
    one = lambda a: np.asarray(a).reshape((1, 1, 1) + np.asarray(a).shape[1:])
    for s in range(n_seeds):
        codec = O.make_codec(d, 2, 3, m, seed=1000 + s)
        qr = codec.Pi @ q
        ke = O.encode(x[None], codec, kind="key")
        f = {"kcodes": one(ke["codes"]), "n16": one(ke["n16"]), "rn16": one(ke["rn16"]), "bits": one(ke["bits"]),
             "vcodes": np.zeros((1, 1, 1, d), np.int64), "vn16": np.zeros((1, 1, 1))}
        _, sc = O.attend(f, q[None, None], codec, q_pos=0, rope_base=0.0, scale=0.0, kv_heads=1, length=1)
        est["attend"][s] = sc[0, 0, 0]
        de = O.encode(x[None], codec, kind="db")
        est["search"][s] = O.search_scores({"kcodes": de["codes"], "n16": de["n16"], "rn16": de["rn16"],
                                            "bits": de["bits"]}, q[None], codec)[0, 0]
        pe = O.polar_encode(x[None], codec, kind="key")
        pcodes = {lv: one(c) for lv, c in pe["pcodes"].items()}
        fp = {"kpc": pcodes, "n16": one(pe["n16"]), "rn16": one(pe["rn16"]), "bits": one(pe["bits"]),
              "vpc": pcodes, "vn16": np.zeros((1, 1, 1))}
        _, sc = O.attend(fp, q[None, None], codec, q_pos=0, rope_base=0.0, scale=0.0, kv_heads=1, length=1)
        est["polar"][s] = sc[0, 0, 0]
        for k, r in (("attend", ke["r"][0]), ("search", de["r"][0]), ("polar", pe["r"][0])):
            rh = r / np.linalg.norm(r)
            cvar[k][s] = (r @ r) / m * (math.pi / 2 * (q @ q) - (qr @ rh) ** 2)
    return x, q, est, cvar


def test_qjl_estimator_unbiased_over_seeds(O):
    # [TurboQuant] "QJL : une technique 1 bit a surcharge nulle": the sign sketch of the
    # residual, met by the full-precision projected query, gives an unbiased inner product.
    # With Pi orthogonal, <Pi q, n16 c_hat + r> = <q, x> for every seed, so the estimate's
    # error against <q, x> is the QJL term's error alone: over 10^4 seeds its mean must be
    # within 3 sigma / sqrt(N) of zero, and its variance must equal the mean of the
    # closed-form conditional variance ||r||^2/m ((pi/2)||q||^2 - (q_rot . r_hat)^2)
    # (E[sign(s.r)(s.q)] = sqrt(2/pi) q.r_hat for s ~ N(0, I)).  A wrong constant, a flipped
    # sign or a dropped QJL term biases the mean by a multiple of E<q_rot, r> > 0.
    n = 10000
    x, q, est, cvar = _qjl_estimates_over_seeds(O, n)
    truth = q @ x
    for path in ("attend", "search", "polar"):
        err = est[path] - truth
        sigma = err.std()
        assert abs(err.mean()) < 3 * sigma / math.sqrt(n), (path, err.mean(), sigma)
        assert abs(err.var() / cvar[path].mean() - 1.0) < 0.06, (path, err.var(), cvar[path].mean())


def test_qjl_estimator_beats_the_codes_alone(O):
    # the QJL term carries the residual's share of <q, x>: over seeds the estimate's mean
    # squared error is the conditional variance, while dropping the term leaves the whole
    # residual product <q_rot, r> (bias about ||r||^2 here, q being correlated with x)
    x, q, est, cvar = _qjl_estimates_over_seeds(O, 400)
    truth = q @ x
    for path in ("attend", "search", "polar"):
        mse = np.mean((est[path] - truth) ** 2)
        assert mse < 1.5 * cvar[path].mean(), (path, mse, cvar[path].mean())


def test_qjl_zero_residual_gives_exact_score(O):
    codec = O.make_codec(64, 2, 3, 64, seed=0)
    qr = np.random.default_rng(1).standard_normal(64)
    kc = np.random.default_rng(2).integers(0, 4, (3, 64))
    n16 = np.array([1.5, 2.0, 0.0])
    s = O.estimate_scores(qr, codec.S @ qr, kc, n16, np.zeros(3), np.ones((3, 64)), codec)
    np.testing.assert_allclose(s, n16 * (codec.cb_k.c[kc] @ qr), rtol=1e-14)


# ------------------------------------------------------------------ attention
def _fields_from_khat(O, codec, kcodes, n16, vcodes, vn16, bits=None):
    B, H, T, d = kcodes.shape
    return {"kcodes": kcodes, "n16": n16, "rn16": np.zeros((B, H, T)),
            "bits": np.ones((B, H, T, codec.m)) if bits is None else bits,
            "vcodes": vcodes, "vn16": vn16}


def test_attend_reduces_to_textbook_softmax_attention(O):
    # keys/values chosen on the codebook lattice with zero residual: the estimator is
    # then exact and the oracle's attention must equal softmax(q K^T scale) V computed
    # in the original (unrotated) coordinates, including RoPE on q and GQA mapping.
    d, B, Hkv, Hq, T = 64, 2, 2, 4, 37
    codec = O.make_codec(d, 2, 3, d, seed=3)
    rng = np.random.default_rng(4)
    kc = rng.integers(0, 4, (B, Hkv, T, d))
    vc = rng.integers(0, 8, (B, Hkv, T, d))
    n16 = rng.uniform(1, 20, (B, Hkv, T)).astype(np.float16).astype(np.float64)
    vn16 = rng.uniform(1, 20, (B, Hkv, T)).astype(np.float16).astype(np.float64)
    fields = _fields_from_khat(O, codec, kc, n16, vc, vn16)
    q = rng.standard_normal((B, Hq, d))
    q_pos, base = 900, 10000.0
    out, scores = O.attend(fields, q, codec, q_pos=q_pos, rope_base=base, scale=0.0,
                           kv_heads=Hkv, length=T)
    P = codec.Pi
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            K = (n16[b, g][:, None] * codec.cb_k.c[kc[b, g]]) @ P        # back to original coords
            V = (vn16[b, g][:, None] * codec.cb_v.c[vc[b, g]]) @ P
            qq = O.rope(q[b, h][None], [q_pos], base)[0]
            s = K @ qq
            w = np.exp(s / math.sqrt(d) - np.max(s / math.sqrt(d)))
            w /= w.sum()
            np.testing.assert_allclose(scores[b, h], s, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(out[b, h], w @ V, rtol=1e-11, atol=1e-11)


def test_attend_window_is_textbook_attention_over_both_sets(O):
    # packed tokens on the codebook lattice with zero residual (exact estimator) and a
    # full-precision window after them: the result must be softmax(q K^T scale) V over the
    # concatenation, with the window keys rotary-embedded at positions length + t, the
    # packed keys being the stored (already embedded) ones, and GQA mapping.
    d, B, Hkv, Hq, T, Wn = 64, 2, 2, 4, 23, 9
    codec = O.make_codec(d, 2, 3, d, seed=5)
    rng = np.random.default_rng(11)
    kc = rng.integers(0, 4, (B, Hkv, T, d))
    vc = rng.integers(0, 8, (B, Hkv, T, d))
    n16 = rng.uniform(1, 8, (B, Hkv, T)).astype(np.float16).astype(np.float64)
    vn16 = rng.uniform(1, 8, (B, Hkv, T)).astype(np.float16).astype(np.float64)
    fields = _fields_from_khat(O, codec, kc, n16, vc, vn16)
    wk = rng.standard_normal((B, Hkv, Wn + 3, d))
    wv = rng.standard_normal((B, Hkv, Wn + 3, d)) * 3
    q = rng.standard_normal((B, Hq, d))
    q_pos, base, scale = T + Wn, 10000.0, 0.2
    out, scores = O.attend_window(fields, wk, wv, q, codec, q_pos=q_pos, rope_base=base, scale=scale,
                                  kv_heads=Hkv, length=T, win_len=Wn)
    assert scores.shape == (B, Hq, T + Wn)
    P = codec.Pi
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Kp = (n16[b, g][:, None] * codec.cb_k.c[kc[b, g]]) @ P
            Vp = (vn16[b, g][:, None] * codec.cb_v.c[vc[b, g]]) @ P
            Kw = np.stack([O.rope(wk[b, g, t][None], [T + t], base)[0] for t in range(Wn)])
            Kall, Vall = np.concatenate([Kp, Kw]), np.concatenate([Vp, wv[b, g, :Wn]])
            qq = O.rope(q[b, h][None], [q_pos], base)[0]
            sc = Kall @ qq
            w = np.exp(scale * sc - np.max(scale * sc))
            w /= w.sum()
            np.testing.assert_allclose(scores[b, h], sc, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(out[b, h], w @ Vall, rtol=1e-11, atol=1e-11)
    # no window: the packed-only attention; no packed tokens: the window alone
    o0, s0 = O.attend_window(fields, wk, wv, q, codec, q_pos=q_pos, rope_base=base, scale=scale,
                             kv_heads=Hkv, length=T, win_len=0)
    o1, s1 = O.attend(fields, q, codec, q_pos=q_pos, rope_base=base, scale=scale, kv_heads=Hkv, length=T)
    np.testing.assert_allclose(o0, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s0, s1, rtol=1e-12, atol=1e-12)
    o2, _ = O.attend_window(fields, wk, wv, q, codec, q_pos=q_pos, rope_base=0.0, scale=0.0,
                            kv_heads=Hkv, length=0, win_len=1)
    np.testing.assert_allclose(o2[0, 0], wv[0, 0, 0], atol=1e-12)   # one token: its value


def _encode_fields(O, codec, K, V, base, means=None):
    """Tokens [0, T) of every unit; means = (o_K, o_V) [B, H, d] fp32 for an NSN cache."""
    B, H, T, d = K.shape
    ok = ov = None
    if means is not None:
        ok = np.repeat(means[0].reshape(B * H, 1, d), T, axis=1).reshape(-1, d)
        ov = np.repeat(means[1].reshape(B * H, 1, d), T, axis=1).reshape(-1, d)
    ke = O.encode(K.reshape(-1, d), codec, kind="key", positions=np.tile(np.arange(T), B * H), rope_base=base,
                  nsn_o=ok)
    ve = O.encode(V.reshape(-1, d), codec, kind="value", nsn_o=ov)
    f = {"kcodes": ke["codes"].reshape(B, H, T, d), "n16": ke["n16"].reshape(B, H, T),
         "rn16": ke["rn16"].reshape(B, H, T), "bits": ke["bits"].reshape(B, H, T, codec.m),
         "vcodes": ve["codes"].reshape(B, H, T, d), "vn16": ve["n16"].reshape(B, H, T)}
    if means is not None:
        f.update(ks1=ke["s1_16"].reshape(B, H, T), vs1=ve["s1_16"].reshape(B, H, T), ok=means[0], ov=means[1],
                 pok=O.nsn_rotated_mean(means[0].reshape(-1, d), codec).reshape(B, H, d),
                 pov=O.nsn_rotated_mean(means[1].reshape(-1, d), codec).reshape(B, H, d))
    return f


def _prefill_means(O, K, V, base):
    """NSN means of each unit over its tokens (keys at positions 0, 1, ...), fp32."""
    B, H, T, d = K.shape
    ok = np.stack([[O.nsn_mean(K[b, h], positions=np.arange(T), rope_base=base) for h in range(H)] for b in range(B)])
    ov = np.stack([[O.nsn_mean(V[b, h]) for h in range(H)] for b in range(B)])
    return ok.astype(np.float32), ov.astype(np.float32)


@pytest.mark.parametrize("nsn", [False, True])
def test_decode_step_flush_schedule(O, nsn):
    # A generation loop through decode_step against a closed form of its schedule: with L0
    # tokens packed up front and a window of cap, after step s (0-based) the packed part
    # holds L0 + cap * floor(s / cap) tokens and the window the other s % cap + 1, all
    # encoded at their own positions.  Checked by one-shot encoding of that prefix and
    # attend_window over the raw rest; with no flush yet, also against textbook attention.
    d, B, Hkv, Hq, L0, cap, steps = 64, 1, 2, 4, 5, 4, 11
    codec = O.make_codec(d, 2, 3, d, seed=9)
    rng = np.random.default_rng(21)
    K = rng.standard_normal((B, Hkv, L0 + steps, d))
    V = rng.standard_normal((B, Hkv, L0 + steps, d))
    base, scale = 10000.0, 0.0
    # NSN: the means come from the prefill (the append at position 0) and stay
    means = _prefill_means(O, K[:, :, :L0], V[:, :, :L0], base) if nsn else None
    st = {"fields": _encode_fields(O, codec, K[:, :, :L0], V[:, :, :L0], base, means), "length": L0,
          "win_k": np.zeros((B, Hkv, cap, d)), "win_v": np.zeros((B, Hkv, cap, d)), "win_len": 0}
    for s in range(steps):
        n = L0 + s + 1
        q = rng.standard_normal((B, Hq, d))
        out, sc = O.decode_step(st, K[:, :, n - 1], V[:, :, n - 1], q, codec, q_pos=n - 1, rope_base=base,
                                scale=scale, kv_heads=Hkv)
        P = L0 + cap * (s // cap)
        assert (st["length"], st["win_len"]) == (P, n - P)
        ref = _encode_fields(O, codec, K[:, :, :P], V[:, :, :P], base, means)
        for f in ref:
            np.testing.assert_array_equal(st["fields"][f], ref[f])
        o2, s2 = O.attend_window(ref, K[:, :, P:n], V[:, :, P:n], q, codec, q_pos=n - 1, rope_base=base,
                                 scale=scale, kv_heads=Hkv, length=P, win_len=n - P)
        np.testing.assert_allclose(out, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(sc, s2, rtol=0, atol=1e-12)
    if nsn:
        return
    # no packed tokens and a window that never fills: exact softmax attention over RoPE'd keys
    st = {"fields": _encode_fields(O, codec, K[:, :, :0], V[:, :, :0], base), "length": 0,
          "win_k": np.zeros((B, Hkv, 8, d)), "win_v": np.zeros((B, Hkv, 8, d)), "win_len": 0}
    for t in range(6):
        q = rng.standard_normal((B, Hq, d))
        out, _ = O.decode_step(st, K[:, :, t], V[:, :, t], q, codec, q_pos=t, rope_base=base, scale=0.0,
                               kv_heads=Hkv)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        kr = O.rope(K[0, g, :6], np.arange(6), base)
        qq = O.rope(q[0, h][None], [5], base)[0]
        lam = kr @ qq / np.sqrt(d)
        w = np.exp(lam - lam.max())
        np.testing.assert_allclose(out[0, h], (w / w.sum()) @ V[0, g, :6], rtol=0, atol=1e-12)


def test_attend_single_token_and_empty(O):
    d = 64
    codec = O.make_codec(d, 2, 3, d, seed=3)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, d))
    kenc = O.encode(x, codec, kind="key", positions=[0], rope_base=0.0)
    venc = O.encode(x * 2, codec, kind="value")
    fields = {"kcodes": kenc["codes"][None, None], "n16": kenc["n16"][None, None],
              "rn16": kenc["rn16"][None, None], "bits": kenc["bits"][None, None],
              "vcodes": venc["codes"][None, None], "vn16": venc["n16"][None, None]}
    q = rng.standard_normal((1, 1, d))
    out, _ = O.attend(fields, q, codec, q_pos=1, rope_base=0.0, scale=0.0, kv_heads=1, length=1)
    vhat = codec.Pi.T @ (venc["n16"][0] * codec.cb_v.c[venc["codes"][0]])
    np.testing.assert_allclose(out[0, 0], vhat, atol=1e-12)
    out0, s0 = O.attend(fields, q, codec, q_pos=1, rope_base=0.0, scale=0.0, kv_heads=1, length=0)
    assert np.all(out0 == 0) and s0.shape == (1, 1, 0)


# ------------------------------------------------------------------ packed format
def test_pack_handcrafted_bytes(O):
    # d = 8, bits_k = 2, m = 8, bits_v = 3, one unit, capacity 33 (two value tiles)
    desc = dict(batch=1, kv_heads=1, d=8, capacity=33, bits_k=2, bits_v=3, m=8)
    kc = np.array([[[[0, 1, 2, 3, 3, 2, 1, 0]]]])
    bits = np.array([[[[1, 0, 0, 0, 0, 0, 0, 1]]]])
    vc = np.array([[[[7, 0, 1, 2, 3, 4, 5, 6]]]])
    f = dict(kcodes=kc, bits=bits, n16=np.array([[[1.5]]]), rn16=np.array([[[0.25]]]),
             vcodes=vc, vn16=np.array([[[2.0]]]))
    img = O.pack_cache(desc, f, start_pos=32)
    lay = O.cache_layout(1, 1, 8, 33, 2, 3, 8)
    hdr = img[:16].view(np.uint32)
    assert list(hdr) == [0x564B5154, 1, 0, 0]
    assert list(img[16:44].view(np.int32)) == [1, 1, 8, 33, 2, 3, 8]
    rec = img[lay["kbits"] + 32 * 3: lay["kbits"] + 33 * 3]
    # plane 0 bits (code & 1): 0,1,0,1,1,0,1,0 -> 0b01011010 = 0x5A
    # plane 1 bits (code >> 1): 0,0,1,1,1,1,0,0 -> 0b00111100 = 0x3C;  signs -> 0x81
    assert list(rec) == [0x5A, 0x3C, 0x81]
    norms = img[lay["knorm"] + 32 * 4: lay["knorm"] + 33 * 4].view(np.float16)
    assert list(norms) == [1.5, 0.25]
    # token 32 is slot 0 of tile 1: coordinate j word = its 3-bit code in bits 0..2
    vt = img[lay["vcodes"] + 1 * 8 * 12: lay["vcodes"] + 2 * 8 * 12].reshape(8, 12)
    assert list(vt[:, 0]) == [7, 0, 1, 2, 3, 4, 5, 6] and np.all(vt[:, 1:] == 0)
    assert img[lay["vnorm"] + 64: lay["vnorm"] + 66].view(np.float16)[0] == 2.0
    u = O.unpack_cache(img, desc, length=33)
    assert list(u["vcodes"][0, 0, 32]) == [7, 0, 1, 2, 3, 4, 5, 6] and np.all(u["vcodes"][0, 0, :32] == 0)
    assert list(u["kcodes"][0, 0, 32]) == [0, 1, 2, 3, 3, 2, 1, 0] and list(u["bits"][0, 0, 32]) == [1, 0, 0, 0, 0, 0, 0, 1]
    # tokens in slots 2 and 10 of tile 0: bits 6..8 and 30..32 (straddling bytes 0/1, 3/4)
    desc0 = dict(desc)
    f2 = dict(f, vcodes=np.array([[[[5] * 8]]]))
    img0 = O.pack_cache(desc0, f2, start_pos=2)
    img0 = O.pack_cache(desc0, f2, start_pos=10, image=img0)
    w = img0[lay["vcodes"]: lay["vcodes"] + 12]
    # code 5 = 0b101 at bit 6 -> byte0 bit6 set, byte1 bit0 set; at bit 30 -> byte3 bit6, byte4 bit0
    assert list(w) == [0x40, 0x01, 0x00, 0x40, 0x01, 0, 0, 0, 0, 0, 0, 0]


def test_pack_unpack_roundtrip(O):
    rng = np.random.default_rng(3)
    desc = dict(batch=2, kv_heads=3, d=64, capacity=100, bits_k=2, bits_v=3, m=64)
    n = 70
    f = dict(kcodes=rng.integers(0, 4, (2, 3, n, 64)), bits=rng.integers(0, 2, (2, 3, n, 64)),
             n16=rng.uniform(0, 9, (2, 3, n)).astype(np.float16).astype(np.float64),
             rn16=rng.uniform(0, 9, (2, 3, n)).astype(np.float16).astype(np.float64),
             vcodes=rng.integers(0, 8, (2, 3, n, 64)),
             vn16=rng.uniform(0, 9, (2, 3, n)).astype(np.float16).astype(np.float64))
    img = O.pack_cache(desc, f, start_pos=5)
    u = O.unpack_cache(img, desc, length=75)
    for key in ("kcodes", "bits", "n16", "rn16", "vcodes", "vn16"):
        np.testing.assert_array_equal(u[key][:, :, 5:], f[key])
    assert u["magic"] == 0x564B5154 and u["version"] == 1


def test_memory_arithmetic(O):
    # record bytes: key = b_k d/8 + m/8 + 2 + 2, value = b_v d/8 + 2
    lay = O.cache_layout(1, 1, 128, 1024, 2, 3, 128)
    assert lay["kbytes"] + 4 == 52
    lay = O.cache_layout(1, 1, 64, 1024, 2, 3, 64)
    assert lay["kbytes"] + 4 == 28
    # ESM-2 650M fp32 K+V at 1024 tokens (33 layers, 20 heads, head dim 64): 330 MiB
    assert 2 * 33 * 1024 * 1280 * 4 == 346030080 == 330 * 2 ** 20


# ------------------------------------------------------------------ search
def test_topk_is_full_sort_with_lower_index_ties(O):
    s = np.array([[0.5, 0.9, 0.5, 0.1, 0.9, 0.2]])
    idx, val = O.topk(s, 4)
    assert list(idx[0]) == [1, 4, 0, 2]
    assert list(val[0]) == [0.9, 0.9, 0.5, 0.5]
    rng = np.random.default_rng(0)
    s = rng.standard_normal((5, 300))
    idx, val = O.topk(s, 10)
    for i in range(5):
        np.testing.assert_array_equal(val[i], np.sort(s[i])[::-1][:10])


def test_search_scores_match_attention_estimator_and_recall(O):
    d = 128
    codec = O.make_codec(d, 3, 0, d, seed=5)
    rng = np.random.default_rng(6)
    db = rng.standard_normal((3000, d))
    db /= np.linalg.norm(db, axis=1, keepdims=True)
    qs = rng.standard_normal((20, d))
    qs /= np.linalg.norm(qs, axis=1, keepdims=True)
    enc = O.encode(db, codec, kind="db")
    fields = {"kcodes": enc["codes"], "n16": enc["n16"], "rn16": enc["rn16"], "bits": enc["bits"]}
    s = O.search_scores(fields, qs, codec)
    for i in (0, 7):
        qr = codec.Pi @ qs[i]
        want = O.estimate_scores(qr, codec.S @ qr, enc["codes"], enc["n16"], enc["rn16"],
                                 enc["bits"], codec)
        np.testing.assert_allclose(s[i], want, rtol=1e-12, atol=1e-13)
    # the estimate tracks the exact inner product closely at 4 bits/coordinate
    exact = qs @ db.T
    assert np.sqrt(np.mean((s - exact) ** 2)) < 0.35 / math.sqrt(d)
    idx, _ = O.topk(s, 10)
    gt, _ = O.exact_topk(db, qs, 10)
    recall1 = np.mean([gt[i, 0] in idx[i] for i in range(20)])
    assert recall1 >= 0.8


# ------------------------------------------------------------------ NSN ([NSNQuant] 1, 4)
def test_nsn_mean_worked_cases(O):
    # two tokens along different axes: each is scaled to norm sqrt(4) = 2, o is their mean
    x = np.array([[2.0, 0, 0, 0], [0, 0, 0, 3.0]])
    np.testing.assert_allclose(O.nsn_mean(x), [1.0, 0, 0, 1.0], atol=1e-15)
    # zero tokens count as zero vectors; no tokens give zero
    np.testing.assert_allclose(O.nsn_mean(np.vstack([x, np.zeros(4)])), [2 / 3, 0, 0, 2 / 3], atol=1e-15)
    np.testing.assert_array_equal(O.nsn_mean(np.zeros((0, 4))), np.zeros(4))
    # keys are rotary-embedded first: d = 2 rotates position p by p radians, so (r, 0) at
    # positions 0 and 1 normalize to sqrt(2) (1, 0) and sqrt(2) (cos 1, sin 1)
    k = np.array([[5.0, 0.0], [0.5, 0.0]])
    want = math.sqrt(2) / 2 * np.array([1 + math.cos(1.0), math.sin(1.0)])
    np.testing.assert_allclose(O.nsn_mean(k, positions=[0, 1], rope_base=10000.0), want, atol=1e-14)


def test_nsn_encode_decomposition_and_zero_mean_case(O):
    # NSN writes v = s1 (s2 x + o); the encoder quantizes w = v - s1_16 o (rotated, with the
    # stored fp32 Pi o), so Pi^T w + s1_16 Pi^T (Pi o) gives back v, |w| = s1 s2 sqrt(d)
    # up to the fp16 rounding of s1, and with o = 0 every code equals the plain encoder's
    d = 64
    codec = O.make_codec(d, 2, 3, d, seed=2)
    rng = np.random.default_rng(6)
    v = rng.standard_normal((40, d)) * 3 + 5.0           # a strong common offset
    o = O.nsn_mean(v).astype(np.float32)
    e = O.encode(v, codec, kind="value", nsn_o=o)
    s1 = np.linalg.norm(v, axis=1) / math.sqrt(d)
    np.testing.assert_array_equal(e["s1_16"], s1.astype(np.float16).astype(np.float64))
    back = e["y"] @ codec.Pi + e["s1_16"][:, None] * (e["po"] @ codec.Pi)
    np.testing.assert_allclose(back, v, atol=1e-11)
    u = math.sqrt(d) * v / np.linalg.norm(v, axis=1, keepdims=True)
    w_page = u - o.astype(np.float64)                     # the page's shifted token
    s2 = np.linalg.norm(w_page, axis=1) / math.sqrt(d)
    np.testing.assert_allclose(e["n"], s1 * s2 * math.sqrt(d), rtol=2e-3)   # fp16 s1, fp32 o
    z = O.encode(v, codec, kind="value", nsn_o=np.zeros(d, np.float32))
    p = O.encode(v, codec, kind="value")
    np.testing.assert_array_equal(z["codes"], p["codes"])
    np.testing.assert_array_equal(z["n16"], p["n16"])


def test_nsn_lowers_error_on_offset_tokens(O):
    # the point of the shift: tokens sharing a large common direction are reconstructed
    # more accurately after NSN than by the plain codec (same bits); a sign error in the
    # shift or its reconstruction would make NSN worse, not better
    d = 128
    codec = O.make_codec(d, 2, 3, d, seed=1)
    rng = np.random.default_rng(8)
    mu = rng.standard_normal(d) * 4
    v = mu + rng.standard_normal((300, d))
    o = O.nsn_mean(v).astype(np.float32)

    def recon(e, nsn):
        r = (e["n16"][:, None] * codec.cb_v.c[e["codes"]]) @ codec.Pi
        return r + e["s1_16"][:, None] * (e["po"] @ codec.Pi) if nsn else r

    err_plain = np.mean(np.sum((recon(O.encode(v, codec, kind="value"), False) - v) ** 2, axis=1))
    err_nsn = np.mean(np.sum((recon(O.encode(v, codec, kind="value", nsn_o=o), True) - v) ** 2, axis=1))
    assert err_nsn < 0.2 * err_plain


def test_nsn_attention_is_textbook_on_the_lattice(O):
    # packed tokens whose shifted part lies on the codebook lattice (zero residual): the
    # NSN attention must equal softmax(q K^T scale) V with K = Pi^T (n c[code]) + s1 o_K and
    # V = Pi^T (n_v c[code_v]) + s1_v o_V, the means entering through the stored Pi o
    d, B, Hkv, Hq, T = 64, 1, 2, 4, 29
    codec = O.make_codec(d, 2, 3, d, seed=4)
    rng = np.random.default_rng(9)
    kc = rng.integers(0, 4, (B, Hkv, T, d))
    vc = rng.integers(0, 8, (B, Hkv, T, d))
    f16 = lambda a: np.asarray(a).astype(np.float16).astype(np.float64)
    fields = _fields_from_khat(O, codec, kc, f16(rng.uniform(1, 9, (B, Hkv, T))), vc,
                               f16(rng.uniform(1, 9, (B, Hkv, T))))
    ok = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    ov = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    fields.update(ks1=f16(rng.uniform(0.5, 3, (B, Hkv, T))), vs1=f16(rng.uniform(0.5, 3, (B, Hkv, T))),
                  ok=ok, ov=ov, pok=O.nsn_rotated_mean(ok.reshape(-1, d), codec).reshape(B, Hkv, d),
                  pov=O.nsn_rotated_mean(ov.reshape(-1, d), codec).reshape(B, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    q_pos, base, scale = 50, 10000.0, 0.3
    out, scores = O.attend(fields, q, codec, q_pos=q_pos, rope_base=base, scale=scale, kv_heads=Hkv, length=T)
    P = codec.Pi
    for h in range(Hq):
        g = h // (Hq // Hkv)
        K = (fields["n16"][0, g][:, None] * codec.cb_k.c[kc[0, g]]) @ P + fields["ks1"][0, g][:, None] * (fields["pok"][0, g] @ P)
        V = (fields["vn16"][0, g][:, None] * codec.cb_v.c[vc[0, g]]) @ P + fields["vs1"][0, g][:, None] * (fields["pov"][0, g] @ P)
        qq = O.rope(q[0, h][None], [q_pos], base)[0]
        sc = K @ qq
        w = np.exp(scale * sc - np.max(scale * sc))
        np.testing.assert_allclose(scores[0, h], sc, rtol=1e-11, atol=1e-10)
        np.testing.assert_allclose(out[0, h], (w / w.sum()) @ V, rtol=1e-11, atol=1e-10)
    # the same tokens plus an empty window through attend_window: identical
    o2, s2 = O.attend_window(fields, np.zeros((B, Hkv, 1, d)), np.zeros((B, Hkv, 1, d)), q, codec, q_pos=q_pos,
                             rope_base=base, scale=scale, kv_heads=Hkv, length=T, win_len=0)
    np.testing.assert_allclose(o2, out, atol=1e-12)
    np.testing.assert_allclose(s2, scores, atol=1e-12)


def test_nsn_pack_layout(O):
    # NSN records: key norms {n, |r|, s1, 0} (8 bytes), value norms {n, s1} (4 bytes), and
    # per unit [o_K, o_V, Pi o_K, Pi o_V] as fp32 after the value norms; nsn in the header
    desc = dict(batch=1, kv_heads=2, d=8, capacity=5, bits_k=2, bits_v=3, m=8, nsn=1)
    lay = O.cache_layout(1, 2, 8, 5, 2, 3, 8, 1)
    n = 2
    z = np.zeros((1, 2, n))
    means = {k: np.arange(16, dtype=np.float32).reshape(1, 2, 8) + 100 * i
             for i, k in enumerate(("ok", "ov", "pok", "pov"))}
    f = dict(kcodes=np.zeros((1, 2, n, 8), int), bits=np.zeros((1, 2, n, 8), int), n16=z + 1.5, rn16=z + 0.25,
             ks1=z + 3.0, vcodes=np.zeros((1, 2, n, 8), int), vn16=z + 2.0, vs1=z + 0.5, **means)
    img = O.pack_cache(desc, f, start_pos=3)
    assert list(img[16:48].view(np.int32)) == [1, 2, 8, 5, 2, 3, 8, 1]
    # unit 1, token 4: key record at knorm + (5 + 4) * 8, value record at vnorm + (5 + 4) * 4
    assert list(img[lay["knorm"] + 72:lay["knorm"] + 80].view(np.float16)) == [1.5, 0.25, 3.0, 0.0]
    assert list(img[lay["vnorm"] + 36:lay["vnorm"] + 40].view(np.float16)) == [2.0, 0.5]
    blk = img[lay["nsn"]:lay["nsn"] + 2 * 4 * 8 * 4].view(np.float32).reshape(2, 4, 8)
    assert blk[1, 2, 3] == means["pok"][0, 1, 3] and blk[0, 1, 7] == means["ov"][0, 0, 7]
    u = O.unpack_cache(img, desc, 5)
    np.testing.assert_array_equal(u["ks1"][:, :, 3:], z + 3.0)
    np.testing.assert_array_equal(u["vs1"][:, :, 3:], z + 0.5)
    for k in means:
        np.testing.assert_array_equal(u[k], means[k])


# ------------------------------------------------------------------ PolarQuant ([TurboQuant] "PolarQuant")
@pytest.mark.parametrize("m", [2, 4, 64])
def test_polar_angle_law_by_quadrature_and_sampling(O, m):
    # the angle between two independent m-dim Gaussian blocks' norms: density integrates to
    # 1, the closed-form CDF (incomplete beta) matches quadrature of the density, and a
    # sample of atan2(|b|, |a|) follows it (KS)
    f = lambda x: O.polar_angle_pdf(np.array([x]), m)[0]
    assert abs(integrate.quad(f, 0, math.pi / 2, limit=200, epsabs=1e-14)[0] - 1.0) < 1e-10
    for x in (0.3, math.pi / 4, 1.2):
        assert abs(integrate.quad(f, 0, x, limit=200, epsabs=1e-14)[0] - O.polar_angle_cdf(x, m)) < 1e-10
    rng = np.random.default_rng(m)
    a = np.linalg.norm(rng.standard_normal((40000, m)), axis=1)
    b = np.linalg.norm(rng.standard_normal((40000, m)), axis=1)
    assert stats.kstest(np.arctan2(b, a), lambda x: O.polar_angle_cdf(x, m)).pvalue > 1e-4


@pytest.mark.parametrize("level", [1, 2, 3, 7])
def test_polar_grids_are_lloyd_max(O, level):
    c, t = O.polar_level_codebook(level)
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    if level == 1:   # uniform on [0, 2 pi): equal sectors, centroids at their middles
        w = 2 * math.pi / 16
        np.testing.assert_allclose(c, (np.arange(16) + 0.5) * w, atol=1e-15)
        return
    m = 1 << (level - 1)
    np.testing.assert_allclose(c + c[::-1], math.pi / 2, atol=1e-13)   # the law is symmetric about pi/4
    f = lambda x: O.polar_angle_pdf(np.array([x]), m)[0]
    edges = np.concatenate(([0.0], t, [math.pi / 2]))
    for k in range(len(c)):
        mass = integrate.quad(f, edges[k], edges[k + 1], limit=400, epsabs=1e-15)[0]
        mom = integrate.quad(lambda x: x * f(x), edges[k], edges[k + 1], limit=400, epsabs=1e-15)[0]
        assert abs(mom / mass - c[k]) < 1e-10


def test_polar_encode_worked_example(O):
    # d = 4, y = (1, 1, 0, 2): level-1 angles pi/4 and pi/2 (sectors of pi/8: codes 2 and
    # 4), radii sqrt 2 and 2; level-2 angle atan(sqrt 2) against the m = 2 grid; norm sqrt 6
    pc = O.make_polar_codebook(4)
    codes, angles, n = O.polar_encode_angles(np.array([[1.0, 1.0, 0.0, 2.0]]), pc)
    assert list(codes[1][0]) == [2, 4]
    np.testing.assert_allclose(angles[2][0, 0], math.atan(math.sqrt(2)), atol=1e-15)
    assert codes[2][0, 0] == int(np.sum(math.atan(math.sqrt(2)) >= pc.t[2]))
    np.testing.assert_allclose(n[0], math.sqrt(6), atol=1e-15)
    # a negative-angle pair lands in [pi, 2 pi): (1, -1) is at 7 pi / 4, code 14
    c2, _, _ = O.polar_encode_angles(np.array([[1.0, -1.0, 1.0, 0.0]]), pc)
    assert list(c2[1][0]) == [14, 0]


def test_polar_decode_norm_and_grid_points(O):
    d = 64
    pc = O.make_polar_codebook(d)
    rng = np.random.default_rng(12)
    codes = {lv: rng.integers(0, 16 if lv == 1 else 4, (50, d >> lv)) for lv in range(1, pc.L + 1)}
    n = rng.uniform(0.5, 9, 50)
    y = O.polar_decode(codes, n, pc)
    # every level splits a radius by a stored (cos, sin) pair: the norm survives up to their
    # fp32 rounding
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), n, rtol=1e-6)
    # points built from the exact centroid angles encode back to the same codes
    exact = {lv: pc.c[lv][codes[lv]] for lv in codes}
    r = n[:, None]
    for lv in range(pc.L, 0, -1):
        out = np.empty((50, 2 * r.shape[1]))
        out[:, 0::2] = r * np.cos(exact[lv])
        out[:, 1::2] = r * np.sin(exact[lv])
        r = out
    back, _, nn = O.polar_encode_angles(r, pc)
    for lv in codes:
        np.testing.assert_array_equal(back[lv], codes[lv])
    np.testing.assert_allclose(O.polar_decode(back, nn, pc), r, rtol=0, atol=1e-6 * n.max())


def test_polar_reconstruction_error(O):
    # rotated Gaussian vectors at 3 - 2/d bits: the level-1 sectors alone cost
    # 2 - 2 sin(pi/16) / (pi/16) ~ 0.0128 of the squared norm; all levels together stay
    # well below the error of a swapped cos / sin or a wrong level order (order 1)
    d = 128
    codec = O.make_codec(d, 3, 3, d, seed=2)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((400, d))
    e = O.polar_encode(x, codec, kind="value")
    rel = np.mean(np.sum((e["yhat"] - e["y"]) ** 2, axis=1) / np.sum(e["y"] ** 2, axis=1))
    lvl1 = 2 - 2 * math.sin(math.pi / 16) / (math.pi / 16)
    assert lvl1 < rel < 4 * lvl1


def test_polar_pack_bit_positions(O):
    # d = 8: four level-1 nibbles (bits 0..15), two level-2 codes (16..19), one level-3 code
    # (20..21), two zero bits
    codes = {1: np.array([[1, 15, 0, 6]]), 2: np.array([[3, 1]]), 3: np.array([[2]])}
    rec = O.polar_pack_codes(codes, 8)
    assert list(rec[0]) == [0xF1, 0x60, 0x27]
    back = O.polar_unpack_codes(rec, 8)
    for lv in codes:
        np.testing.assert_array_equal(back[lv], codes[lv])


def test_polar_attention_is_textbook(O):
    # packed polar keys with zero residual and polar values: attention equals softmax over
    # K = Pi^T decode(codes, n) and V = Pi^T decode(codes_v, n_v), with RoPE on q and GQA
    d, B, Hkv, Hq, T = 64, 1, 2, 4, 21
    codec = O.make_codec(d, 3, 3, d, seed=6)
    pc = O.make_polar_codebook(d)
    rng = np.random.default_rng(14)
    mk = lambda: {lv: rng.integers(0, 16 if lv == 1 else 4, (B, Hkv, T, d >> lv)) for lv in range(1, pc.L + 1)}
    kpc, vpc = mk(), mk()
    f16 = lambda a: np.asarray(a).astype(np.float16).astype(np.float64)
    fields = {"kpc": kpc, "vpc": vpc, "n16": f16(rng.uniform(1, 9, (B, Hkv, T))), "rn16": np.zeros((B, Hkv, T)),
              "bits": np.ones((B, Hkv, T, d)), "vn16": f16(rng.uniform(1, 9, (B, Hkv, T)))}
    q = rng.standard_normal((B, Hq, d))
    out, scores = O.attend(fields, q, codec, q_pos=30, rope_base=10000.0, scale=0.25, kv_heads=Hkv, length=T)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        K = O.polar_decode({lv: c[0, g] for lv, c in kpc.items()}, fields["n16"][0, g], pc) @ codec.Pi
        V = O.polar_decode({lv: c[0, g] for lv, c in vpc.items()}, fields["vn16"][0, g], pc) @ codec.Pi
        qq = O.rope(q[0, h][None], [30], 10000.0)[0]
        sc = K @ qq
        w = np.exp(0.25 * (sc - sc.max()))
        np.testing.assert_allclose(scores[0, h], sc, rtol=1e-11, atol=1e-10)
        np.testing.assert_allclose(out[0, h], (w / w.sum()) @ V, rtol=1e-11, atol=1e-10)
