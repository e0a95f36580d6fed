"""Plain fp64 CPU oracle for the RoPE -> randomized-Hadamard -> Lloyd-Max (+ QJL) KV codec.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module: only
`tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py` may
import or call it.  It shares no code with the HIP library (no kernels, headers,
tables or constant generators); the two meet only in the seeded input generators,
which hold none of the method's arithmetic.

Every step is written in the slowest obvious form: a dense d x d rotation matrix
applied as a matvec, brute-force nearest codeword over all 2^b centroids, an
explicit m x d Gaussian matrix S, fp64 softmax.  Library primitives (numpy matmul,
scipy's regularized incomplete beta) serve as single steps.

Sources (titles of the pages; sections as they appear there):
  [TurboESM]  "TurboESM: Ultra-Efficient 3-Bit KV Cache Quantization for Protein
              Language Models ..." -- technical summary section 2.A (RoPE applied
              before the orthogonal rotation, invariance of the attention score
              under an orthogonal Pi), 2.C (Lloyd-Max look-up tables), 2.D (1-bit
              residual correction), 2.E (fused decode: dequantize, correct,
              inverse rotation, online softmax in one pass).
  [TurboQuant] news summary of the TurboQuant blog post -- "Etape 1" (random
              rotation then a standard scalar quantizer per coordinate), "Etape 2"
              and "QJL" (Johnson-Lindenstrauss projection reduced to sign bits,
              asymmetric estimator with a full-precision query), reader comment on
              Lloyd-Max boundaries/reconstruction values and per-dimension coding,
              "Performances en recherche vectorielle" (recall 1@k, top-k search).
  [NSNQuant]  "NSNQuant ..." technical summary section 2 (randomized Hadamard
              transform) -- cited for the choice of a seeded-sign Hadamard rotation;
              section 4 (implementation details, residuals: the cache is a quantized
              part plus a full-precision residual that is quantized and appended once
              full) -- attention over packed tokens and a full-precision window.

Readings where the pages are silent:
  * PRNG: SplitMix64 (Steele, Lea & Flood 2014) used as a counter-based generator;
    Gaussians by Box-Muller (cos branch) in fp64, rounded to fp32.
  * Rotation: Pi = blockdiag(H_B, ..., H_B) diag(D) / sqrt(B), H_B Sylvester, B the
    largest power of two dividing d (B = d for d = 64, 128; B = 512 for d = 1536).
  * RoPE: half-split pairs (j, j + d/2), theta_j = base^(-2j/d), angles in fp64.
  * Codebook: Lloyd-Max for the exact marginal of one coordinate of a uniform unit
    vector in R^d; the stored codebook is each centroid rounded to fp16, and codes
    are nearest stored centroid (ties to the larger index).
  * Residual r = y - fp16(n) * c[code]; QJL bits = [ (S r)_i >= 0 ]; estimator
    scale sqrt(pi/2)/m.

Parity pinned by tests/test_oracle_*.py (closed forms, textbook tables, invariants,
brute force).  Parity unpinned: the pages' model-level accuracy claims (cosine
similarity on protein families, lossless 3-bit LLM quality) -- no models or data.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import betainc, gammaln

__all__ = [
    "splitmix64", "uniform01", "rotation_signs", "gaussian_projection",
    "sphere_marginal_cdf", "sphere_marginal_pdf", "sphere_partial_mean", "lloyd_max",
    "Codebook", "make_codebook", "hadamard", "rotation_matrix", "rope",
    "fp16_sat", "Codec", "make_codec", "encode", "pack_cache", "unpack_cache",
    "cache_layout", "attend", "attend_window", "decode_step", "search_scores",
    "nsn_mean", "nsn_rotated_mean", "polar_angle_pdf", "polar_angle_cdf", "polar_level_codebook",
    "make_polar_codebook", "polar_encode_angles", "polar_decode", "polar_encode", "polar_pack_codes",
    "polar_unpack_codes", "estimate_scores_polar", "topk", "exact_topk",
]

_GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# PRNG stream ids (disjoint 2^32-long segments of one SplitMix64 sequence)
STREAM_SIGNS = 1
STREAM_GAUSS = 2


# ----------------------------------------------------------------------------------
# Counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
# number generators", OOPSLA 2014): output k of a generator seeded with s is
# mix(s + (k+1) * golden_gamma).  Stream t, index i uses k = t * 2^32 + i.
# ----------------------------------------------------------------------------------
def splitmix64(seed: int, stream: int, idx) -> np.ndarray:
    """uint64 SplitMix64 outputs for counter positions `idx` of `stream`."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        k = np.uint64(stream) * np.uint64(1 << 32) + idx + np.uint64(1)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * _GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, stream: int, idx) -> np.ndarray:
    """Open-interval uniforms in (0, 1): ((x >> 11) + 0.5) * 2^-53, fp64."""
    x = splitmix64(seed, stream, idx)
    return ((x >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def rotation_signs(d: int, seed: int) -> np.ndarray:
    """D_j = +1 if the top bit of SplitMix64(seed, signs stream, j) is 0, else -1."""
    x = splitmix64(seed, STREAM_SIGNS, np.arange(d, dtype=np.uint64))
    return np.where((x >> np.uint64(63)) == 0, 1.0, -1.0)


def gaussian_projection(m: int, d: int, seed: int) -> np.ndarray:
    """S (m x d): Box-Muller cos branch, u1 = U(2(i d + j)), u2 = U(2(i d + j) + 1),
    z = sqrt(-2 ln u1) * cos((2 pi) * u2) in fp64, rounded to fp32 (returned as fp32)."""
    n = np.arange(m * d, dtype=np.uint64)
    u1 = uniform01(seed, STREAM_GAUSS, 2 * n)
    u2 = uniform01(seed, STREAM_GAUSS, 2 * n + 1)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos((2.0 * math.pi) * u2)
    return z.astype(np.float32).reshape(m, d)


# ----------------------------------------------------------------------------------
# Lloyd-Max codebook for one coordinate of a uniform random unit vector in R^d
# ([TurboQuant] "Etape 1": after a random rotation each coordinate gets its own
# standard scalar quantizer; reader comment: Lloyd-Max boundaries and reconstruction
# values).  Density f_d(x) = C_d (1 - x^2)^((d-3)/2) on [-1, 1]; X^2 ~ Beta(1/2, (d-1)/2).
# ----------------------------------------------------------------------------------
def _log_cd(d: int) -> float:
    return gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)


def sphere_marginal_pdf(x, d: int):
    x = np.asarray(x, dtype=np.float64)
    inside = np.abs(x) < 1.0
    out = np.zeros_like(x)
    xi = x[inside]
    out[inside] = np.exp(_log_cd(d) + 0.5 * (d - 3) * np.log1p(-xi * xi))
    return out


def sphere_marginal_cdf(x, d: int):
    """F(x) = 1/2 + sign(x)/2 * I_{x^2}(1/2, (d-1)/2)."""
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return 0.5 + 0.5 * np.sign(x) * betainc(0.5, (d - 1) / 2.0, x * x)


def sphere_partial_mean(x, d: int):
    """M(x) = int_{-1}^{x} t f_d(t) dt = -C_d (1 - x^2)^((d-1)/2) / (d - 1)."""
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    one_m = np.maximum(1.0 - x * x, 0.0)
    with np.errstate(divide="ignore"):
        val = np.where(one_m > 0.0,
                       np.exp(_log_cd(d) + 0.5 * (d - 1) * np.log(np.where(one_m > 0, one_m, 1.0))),
                       0.0)
    return -val / (d - 1)


def lloyd_max(d: int, bits: int, tol: float = 1e-13, max_iter: int = 100000):
    """Lloyd iteration (Lloyd 1982; Max 1960) in fp64.

    t_k = (c_k + c_{k+1}) / 2;  c_k = E[X | t_{k-1} < X <= t_k], with t_{-1} = -1,
    t_{K-1} = +1.  Stops when max |sqrt(d) * delta c| < tol.
    Returns (centroids, boundaries, iterations), ascending."""
    K = 1 << bits
    # start from equal-mass cells of the N(0, 1/d) limit
    c = np.array([(k + 0.5) / K for k in range(K)], dtype=np.float64)
    c = (np.sqrt(2.0) * _erfinv(2.0 * c - 1.0)) / math.sqrt(d)
    c = np.clip(c, -0.999, 0.999)
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        F = sphere_marginal_cdf(edges, d)
        M = sphere_partial_mean(edges, d)
        c_new = (M[1:] - M[:-1]) / (F[1:] - F[:-1])
        delta = np.max(np.abs(c_new - c)) * math.sqrt(d)
        c = c_new
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it


def _erfinv(y):
    from scipy.special import erfinv
    return erfinv(y)


class Codebook:
    """Lloyd-Max codebook and the stored (fp16-rounded) form the codec uses."""

    def __init__(self, d: int, bits: int):
        self.d, self.bits = d, bits
        self.c64, self.t64, self.iterations = lloyd_max(d, bits)
        # stored codebook: each centroid rounded to the nearest fp16 (RNE)
        self.c = self.c64.astype(np.float16).astype(np.float64)
        # decision boundaries of the stored codebook: exact midpoints
        self.t = 0.5 * (self.c[:-1] + self.c[1:])

    def mse(self) -> float:
        """Per-coordinate MSE E[(X - Q(X))^2] of the fp64 codebook (closed form)."""
        d = self.d
        edges = np.concatenate(([-1.0], self.t64, [1.0]))
        F = sphere_marginal_cdf(edges, d)
        # with c_k the cell means: E[(X - Q(X))^2] = E[X^2] - sum_k c_k^2 P_k, E[X^2] = 1/d
        P = F[1:] - F[:-1]
        return 1.0 / d - float(np.sum(self.c64 ** 2 * P))


_CODEBOOK_CACHE: dict = {}


def make_codebook(d: int, bits: int) -> Codebook:
    key = (d, bits)
    if key not in _CODEBOOK_CACHE:
        _CODEBOOK_CACHE[key] = Codebook(d, bits)
    return _CODEBOOK_CACHE[key]


# ----------------------------------------------------------------------------------
# Rotation ([TurboESM] 2.A: orthogonal Pi with Pi^T Pi = I applied after RoPE;
# [TurboQuant] "Etape 1": random rotation; [NSNQuant] 2: randomized Hadamard).
# ----------------------------------------------------------------------------------
def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H[i][j] = (-1)^popcount(i & j)."""
    assert n > 0 and (n & (n - 1)) == 0
    i = np.arange(n)
    pc = np.zeros((n, n), dtype=np.int64)
    x = i[:, None] & i[None, :]
    while np.any(x):
        pc += x & 1
        x = x >> 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def hadamard_block(d: int) -> int:
    """Largest power of two dividing d."""
    return d & (-d)


def rotation_matrix(d: int, seed: int) -> np.ndarray:
    """Dense Pi = blockdiag(H_B) diag(D) / sqrt(B)."""
    B = hadamard_block(d)
    H = hadamard(B)
    P = np.zeros((d, d))
    for b in range(d // B):
        P[b * B:(b + 1) * B, b * B:(b + 1) * B] = H
    D = rotation_signs(d, seed)
    return P * D[None, :] / math.sqrt(B)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Half-split rotary embedding applied to rows of x at positions `pos` (fp64).

    For j < d/2: phi = pos * base^(-2j/d);
    (x_j, x_{j+d/2}) <- (x_j cos phi - x_{j+d/2} sin phi, x_j sin phi + x_{j+d/2} cos phi).
    base == 0 means no rotary embedding."""
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    d = x.shape[-1]
    h = d // 2
    j = np.arange(h, dtype=np.float64)
    theta = np.power(float(base), -2.0 * j / d)
    pos = np.asarray(pos, dtype=np.float64)
    phi = pos[..., None] * theta
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


FP16_MAX = 65504.0


def fp16_sat(x):
    """fp16 round-to-nearest-even; values that would round to inf become 65504.
    Returns (fp16-valued fp64 array, overflow mask)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
    over = ~np.isfinite(h)
    h = np.where(over, np.float16(FP16_MAX), h)
    return h.astype(np.float64), over


# ----------------------------------------------------------------------------------
# Codec: rotation, codebooks, S
# ----------------------------------------------------------------------------------
class Codec:
    def __init__(self, d: int, bits_k: int, bits_v: int, m: int, seed: int):
        self.d, self.bits_k, self.bits_v, self.m, self.seed = d, bits_k, bits_v, m, seed
        self.Pi = rotation_matrix(d, seed)
        self.D = rotation_signs(d, seed)
        self.cb_k = make_codebook(d, bits_k)
        self.cb_v = make_codebook(d, bits_v) if bits_v > 0 else None
        self.S = gaussian_projection(m, d, seed).astype(np.float64) if m > 0 else None

    @property
    def qjl_scale(self) -> float:
        return math.sqrt(math.pi / 2.0) / self.m


def make_codec(d, bits_k, bits_v, m, seed) -> Codec:
    return Codec(d, bits_k, bits_v, m, seed)


def _nearest(u: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Brute force over all centroids: argmin_k |u - c_k|, exact ties to larger k."""
    best = np.zeros(u.shape, dtype=np.int64)
    bestd = np.abs(u - c[0])
    for k in range(1, len(c)):
        dk = np.abs(u - c[k])
        take = dk <= bestd
        best = np.where(take, k, best)
        bestd = np.where(take, dk, bestd)
    return best


def encode(x, codec: Codec, *, kind: str, positions=None, rope_base: float = 0.0, nsn_o=None):
    """Encode rows of x ([N, d], any float dtype; converted exactly to fp64).

    kind = 'key' (RoPE if rope_base != 0, scalar codes with bits_k, QJL residual sketch),
           'value' (scalar codes with bits_v), 'db' (like 'key' without RoPE).
    nsn_o: NSN channel mean ([d] or [N, d], fp32 values; see nsn_mean).  Each token then
    gives s1 = ||x|| / sqrt(d) (fp16, s1_16) and is encoded as w = x - s1_16 o, the
    subtraction done in the rotated basis with Pi o rounded to fp32 (the stored form).
    Returns a dict with y (rotated, fp64), u, codes, n16, and for keys rn16, bits, z,
    plus overflow flags (and s1_16, po with nsn_o)."""
    x = np.asarray(x, dtype=np.float64)
    if kind == "key" and rope_base != 0:
        x = rope(x, positions, rope_base)
    y = x @ codec.Pi.T
    extra = {}
    if nsn_o is not None:
        po = nsn_rotated_mean(nsn_o, codec)
        s1 = np.sqrt(np.sum(y * y, axis=-1)) / math.sqrt(codec.d)
        s1_16, over_s = fp16_sat(s1)
        y = y - s1_16[..., None] * po
        extra = {"s1": s1, "s1_16": s1_16, "po": po, "over_s": over_s}
    n = np.sqrt(np.sum(y * y, axis=-1))
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[..., None] > 0, y / safe[..., None], 0.0)
    cb = codec.cb_v if kind == "value" else codec.cb_k
    codes = _nearest(u, cb.c)
    n16, over_n = fp16_sat(n)
    out = {"y": y, "u": u, "codes": codes, "n": n, "n16": n16, "overflow": over_n.copy()}
    if extra:
        out["s1"], out["s1_16"], out["po"] = extra["s1"], extra["s1_16"], extra["po"]
        out["overflow"] = out["overflow"] | extra["over_s"]
    if kind in ("key", "db"):
        r = y - n16[..., None] * cb.c[codes]
        rn = np.sqrt(np.sum(r * r, axis=-1))
        rn16, over_r = fp16_sat(rn)
        z = r @ codec.S.T if codec.m > 0 else np.zeros(r.shape[:-1] + (0,))
        out.update(r=r, rn=rn, rn16=rn16, z=z, bits=(z >= 0).astype(np.int64))
        out["overflow"] = out["overflow"] | over_r
    return out


# ----------------------------------------------------------------------------------
# PolarQuant stage 1 ([TurboQuant] news summary, "PolarQuant": adjacent coordinates are
# paired and turned into (radius, angle); the radii are paired again, recursively, down to
# one radius and d - 1 angles; the angles go on fixed grids whose boundaries are known in
# advance, with no per-vector normalization).  Readings: d = 2^L, pairs (2i, 2i + 1) at
# every level; a level-1 angle atan2(y_{2i+1}, y_{2i}) in [0, 2 pi) is uniform for a
# rotated vector and gets a 4-bit uniform grid; a level-l angle (l >= 2) is
# atan2(r_{2i+1}, r_{2i}) in [0, pi/2] with sin^2 psi ~ Beta(m/2, m/2), m = 2^(l-1), and
# gets a 2-bit Lloyd-Max grid for that density; the last radius is the norm (fp16).  That
# is 3 d - 2 bits of angles per vector.  Decoding uses each centroid's cos and sin rounded
# to fp32 (the stored form).
# ----------------------------------------------------------------------------------
POLAR_B1, POLAR_BH = 4, 2


def polar_angle_pdf(psi, m: int):
    """Density of psi = atan2(|b|, |a|) for independent m-dim standard Gaussian a, b:
    2^(2-m) sin^(m-1)(2 psi) / B(m/2, m/2) on [0, pi/2]."""
    psi = np.asarray(psi, dtype=np.float64)
    logc = (2 - m) * math.log(2.0) - (2 * gammaln(m / 2.0) - gammaln(float(m)))
    with np.errstate(divide="ignore"):
        s = np.sin(2.0 * psi)
        out = np.where((psi > 0) & (psi < math.pi / 2), np.exp(logc + (m - 1) * np.log(np.abs(s))), 0.0)
    return out


def polar_angle_cdf(psi, m: int):
    """F(psi) = I_{sin^2 psi}(m/2, m/2)."""
    psi = np.clip(np.asarray(psi, dtype=np.float64), 0.0, math.pi / 2)
    return betainc(m / 2.0, m / 2.0, np.sin(psi) ** 2)


def polar_level_codebook(level: int):
    """(centroids, boundaries) in fp64 of a level's angle grid, ascending."""
    if level == 1:
        K = 1 << POLAR_B1
        w = 2.0 * math.pi / K
        return np.array([(k + 0.5) * w for k in range(K)]), np.array([k * w for k in range(1, K)])
    from scipy import integrate
    m = 1 << (level - 1)
    K = 1 << POLAR_BH
    # start from equal-mass cells, then the Lloyd iteration with quadrature cell means
    c = np.array([math.pi / 2 * (k + 0.5) / K for k in range(K)])
    for _ in range(500):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([0.0], t, [math.pi / 2]))
        P = np.diff(polar_angle_cdf(edges, m))
        mom = np.array([integrate.quad(lambda x: x * polar_angle_pdf(x, m), edges[k], edges[k + 1],
                                       epsabs=1e-15, epsrel=1e-13, limit=200)[0] for k in range(K)])
        c_new = mom / P
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < 1e-13:
            break
    return c, 0.5 * (c[:-1] + c[1:])


class PolarCodebook:
    """Angle grids of every level for d = 2^L, with the stored fp32 cos / sin."""

    def __init__(self, d: int):
        self.d, self.L = d, int(round(math.log2(d)))
        assert 1 << self.L == d
        self.c, self.t, self.cos, self.sin = {}, {}, {}, {}
        for lv in range(1, self.L + 1):
            c, t = polar_level_codebook(lv)
            self.c[lv], self.t[lv] = c, t
            self.cos[lv] = np.cos(c).astype(np.float32).astype(np.float64)
            self.sin[lv] = np.sin(c).astype(np.float32).astype(np.float64)


_POLAR_CACHE: dict = {}


def make_polar_codebook(d: int) -> PolarCodebook:
    if d not in _POLAR_CACHE:
        _POLAR_CACHE[d] = PolarCodebook(d)
    return _POLAR_CACHE[d]


def polar_encode_angles(y, pc: PolarCodebook):
    """y [N, d] -> (codes {level: [N, d / 2^level]}, angles {level: ...}, norm [N])."""
    r = np.asarray(y, dtype=np.float64)
    codes, angles = {}, {}
    for lv in range(1, pc.L + 1):
        a, b = r[:, 0::2], r[:, 1::2]
        psi = np.arctan2(b + 0.0, a + 0.0)   # signed zeros count as +0 (a zero pair has angle 0)
        if lv == 1:
            psi = np.where(psi < 0, psi + 2 * math.pi, psi)
        angles[lv] = psi
        codes[lv] = np.sum(psi[..., None] >= pc.t[lv], axis=-1)
        r = np.sqrt(a * a + b * b)
    return codes, angles, r[:, 0]


def polar_decode(codes, n, pc: PolarCodebook):
    """Reconstruction from the angle codes and the norm n [N]: radii from the top level
    down, each split by the stored cos / sin of its angle's centroid."""
    r = np.asarray(n, dtype=np.float64)[:, None]
    for lv in range(pc.L, 0, -1):
        cd = np.asarray(codes[lv])
        out = np.empty((r.shape[0], 2 * r.shape[1]))
        out[:, 0::2] = r * pc.cos[lv][cd]
        out[:, 1::2] = r * pc.sin[lv][cd]
        r = out
    return r


def polar_encode(x, codec: "Codec", *, kind: str, positions=None, rope_base: float = 0.0):
    """PolarQuant encode of rows of x: y = Pi RoPE(x) (keys) or Pi x (values), angle codes,
    fp16 norm, and for keys the residual r = y - decode(codes, fp16(n)) with its QJL sketch
    as in encode (the estimator is unchanged)."""
    x = np.asarray(x, dtype=np.float64)
    if kind == "key" and rope_base != 0:
        x = rope(x, positions, rope_base)
    y = x @ codec.Pi.T
    pc = make_polar_codebook(codec.d)
    codes, angles, n = polar_encode_angles(y, pc)
    n16, over = fp16_sat(n)
    yhat = polar_decode(codes, n16, pc)
    out = {"y": y, "pcodes": codes, "angles": angles, "n": n, "n16": n16, "yhat": yhat, "overflow": over.copy()}
    if kind == "key":
        r = y - yhat
        rn = np.sqrt(np.sum(r * r, axis=-1))
        rn16, over_r = fp16_sat(rn)
        z = r @ codec.S.T if codec.m > 0 else np.zeros(r.shape[:-1] + (0,))
        out.update(r=r, rn=rn, rn16=rn16, z=z, bits=(z >= 0).astype(np.int64))
        out["overflow"] = out["overflow"] | over_r
    return out


def polar_pack_codes(codes, d: int) -> np.ndarray:
    """Angle codes {level: [N, d / 2^level]} -> [N, 3 d / 8] bytes: level-1 code i in bits
    [4 i, 4 i + 4), then the levels 2, 3, ... one after the other, 2 bits each, from bit 2 d;
    the last 2 bits are zero."""
    L = int(round(math.log2(d)))
    N = np.asarray(codes[1]).shape[0]
    bits = np.zeros((N, 3 * d), dtype=np.uint8)
    c1 = np.asarray(codes[1])
    for k in range(POLAR_B1):
        bits[:, k:2 * d:POLAR_B1] = (c1 >> k) & 1
    pos = 2 * d
    for lv in range(2, L + 1):
        cl = np.asarray(codes[lv])
        for j in range(cl.shape[1]):
            for k in range(POLAR_BH):
                bits[:, pos + POLAR_BH * j + k] = (cl[:, j] >> k) & 1
        pos += POLAR_BH * cl.shape[1]
    return _bits_to_bytes(bits)


def polar_unpack_codes(rec, d: int):
    """Inverse of polar_pack_codes."""
    L = int(round(math.log2(d)))
    bits = np.unpackbits(np.asarray(rec, dtype=np.uint8), axis=-1, bitorder="little").astype(np.int64)
    codes = {1: sum(bits[..., k:2 * d:POLAR_B1] << k for k in range(POLAR_B1))}
    pos = 2 * d
    for lv in range(2, L + 1):
        n = d >> lv
        codes[lv] = sum(bits[..., pos + k:pos + POLAR_BH * n:POLAR_BH] << k for k in range(POLAR_BH))
        pos += POLAR_BH * n
    return codes


def estimate_scores_polar(qr, sq, pcodes, n16, rn16, bits, codec: "Codec"):
    """score_t = <qr, decode(codes_t, n16_t)> + rn16_t sqrt(pi/2)/m <sq, 2 bits_t - 1>."""
    pc = make_polar_codebook(codec.d)
    yhat = polar_decode(pcodes, n16, pc)
    s = yhat @ qr
    if codec.m > 0:
        s = s + rn16 * codec.qjl_scale * ((2.0 * bits - 1.0) @ sq)
    return s


# ----------------------------------------------------------------------------------
# NSN pre-transform ([NSNQuant] section 1, normalize-shift-normalize, and section 4 for
# keys).  A token v becomes u = sqrt(d) v / ||v|| (s1 = ||v|| / sqrt(d)), the channel mean
# o of the u is subtracted, and the result is normalized again (s2); v = s1 (s2 x + o).
# The codec stores a norm and a direction, so quantizing w = v - s1 o = s1 s2 x gives NSN's
# x as the direction and s1 s2 sqrt(d) as the norm: the second normalization is the
# codec's own.  Keys are rotary-embedded first (the same order as the plain path).
# ----------------------------------------------------------------------------------
def nsn_mean(x, *, positions=None, rope_base: float = 0.0):
    """o = mean over the rows of x ([n, d]) of sqrt(d) x_i / ||x_i|| (keys: of RoPE(x_i)),
    in fp64; zero rows contribute zero vectors; no rows give o = 0."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if len(x) == 0:
        return np.zeros(d)
    if rope_base != 0:
        x = rope(x, positions, rope_base)
    n = np.sqrt(np.sum(x * x, axis=-1))
    u = np.zeros_like(x)
    nz = n > 0
    u[nz] = math.sqrt(d) * x[nz] / n[nz][:, None]
    return np.sum(u, axis=0) / len(x)


def nsn_rotated_mean(o, codec: Codec) -> np.ndarray:
    """Pi o for the stored fp32 mean o, rounded to fp32 (the form the cache stores)."""
    o32 = np.asarray(o, dtype=np.float32).astype(np.float64)
    return (o32 @ codec.Pi.T).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------
# Packed cache format, version 1 (written from the format description, independently
# of the library):
#   header: 256 bytes; u32 magic 0x564B5154 ("TQKV"), u32 version 1, u32 flags
#           (bit 0: a norm saturated to fp16 max), u32 0, then i32 batch, kv_heads, d,
#           capacity, bits_k, bits_v, m; zero padding.
#   Kbits:  [batch][kv_heads][capacity][kbytes], kbytes = (bits_k*d + m)/8: plane p of the
#           scalar code (bit p of code_j at plane bit j), p = 0..bits_k-1, then the m
#           QJL sign bits.  Plane bit j lives in byte j/8, bit j%8 (little-endian).
#   Knorm:  [batch][kv_heads][capacity] x {fp16 n, fp16 ||r||}.
#   Vcodes: [batch][kv_heads][ceil(capacity/32)][d][4*bits_v bytes]: for a tile of 32
#           tokens and coordinate j, a (32*bits_v)-bit little-endian integer whose bits
#           [bits_v*i, bits_v*(i+1)) hold the value code of token 32*tile + i.
#   Vnorm:  [batch][kv_heads][capacity] fp16 n.
#   NSN caches (desc nsn = 1, written after the desc in the header): Knorm records are 8
#   bytes {fp16 n, fp16 ||r||, fp16 s1, 0}, Vnorm records 4 bytes {fp16 n, fp16 s1}, and a
#   last region holds per unit [o_K, o_V, Pi o_K, Pi o_V] as fp32 [d] each.
#   PolarQuant caches (desc polar = 1, bits_k = bits_v = 3): a key record is the 3 d / 8
#   bytes of polar_pack_codes followed by the m QJL sign bits; values are token records of
#   3 d / 8 bytes [batch][kv_heads][capacity] in place of the tiles; norms as above.
#   Each region starts at a multiple of 256 bytes.
# ----------------------------------------------------------------------------------
CACHE_MAGIC = 0x564B5154
CACHE_VERSION = 1
HEADER_BYTES = 256


def _align(x, a=256):
    return (x + a - 1) // a * a


def cache_layout(batch, kv_heads, d, capacity, bits_k, bits_v, m, nsn=0, polar=0):
    kbytes = (bits_k * d + m) // 8   # polar: 3 d / 8 angle bytes + m / 8 (bits_k = 3)
    units = batch * kv_heads
    tiles = (capacity + 31) // 32
    off = {"knrec": 8 if nsn else 4, "vnrec": 4 if nsn else 2}
    cur = HEADER_BYTES
    off["kbits"] = cur
    cur = _align(cur + units * capacity * kbytes)
    off["knorm"] = cur
    cur = _align(cur + units * capacity * off["knrec"])
    if bits_v > 0:
        off["vcodes"] = cur
        cur = _align(cur + (units * capacity * 3 * d // 8 if polar else units * tiles * d * 4 * bits_v))
        off["vnorm"] = cur
        cur = _align(cur + units * capacity * off["vnrec"])
    if nsn:
        off["nsn"] = cur
        cur = _align(cur + units * 4 * d * 4)
    off["total"] = cur
    off["kbytes"] = kbytes
    off["tiles"] = tiles
    return off


def _bits_to_bytes(bitmat: np.ndarray) -> np.ndarray:
    """[..., nbits] of 0/1 -> [..., nbits/8] uint8, bit j in byte j/8 bit j%8."""
    sh = bitmat.shape
    b = bitmat.reshape(sh[:-1] + (sh[-1] // 8, 8)).astype(np.uint8)
    w = (1 << np.arange(8)).astype(np.uint8)
    return np.sum(b * w, axis=-1, dtype=np.uint64).astype(np.uint8)


def pack_cache(desc: dict, fields: dict, start_pos: int = 0, image: np.ndarray | None = None,
               flags: int = 0) -> np.ndarray:
    """Write tokens [start_pos, start_pos + n) of every (batch, kv-head) unit.

    fields: kcodes [B, H, n, d], n16 [B, H, n], rn16 [B, H, n], bits [B, H, n, m],
            and if bits_v > 0: vcodes [B, H, n, d], vn16 [B, H, n];
            NSN caches also ks1, vs1 [B, H, n] and the unit means ok, ov, pok, pov [B, H, d]."""
    B, H, d, cap = desc["batch"], desc["kv_heads"], desc["d"], desc["capacity"]
    bk, bv, m = desc["bits_k"], desc["bits_v"], desc["m"]
    nsn, polar = int(desc.get("nsn", 0)), int(desc.get("polar", 0))
    lay = cache_layout(B, H, d, cap, bk, bv, m, nsn, polar)
    if image is None:
        image = np.zeros(lay["total"], dtype=np.uint8)
    hdr = np.zeros(HEADER_BYTES // 4, dtype=np.uint32)
    hdr[0], hdr[1], hdr[2] = CACHE_MAGIC, CACHE_VERSION, flags
    hdr[4:13] = np.array([B, H, d, cap, bk, bv, m, nsn, polar], dtype=np.int64).astype(np.uint32)
    hdr[2] |= np.uint32(image[8:12].view(np.uint32)[0])
    image[:HEADER_BYTES] = hdr.view(np.uint8)
    if nsn:
        means = np.stack([np.asarray(fields[f], dtype=np.float32) for f in ("ok", "ov", "pok", "pov")], axis=2)
        image[lay["nsn"]:lay["nsn"] + B * H * 4 * d * 4] = means.reshape(-1).view(np.uint8)

    n = np.asarray(fields["n16"]).shape[2]
    if n == 0:
        return image
    assert start_pos + n <= cap
    kb = lay["kbytes"]
    if polar:
        ang = polar_pack_codes({lv: np.asarray(c).reshape(B * H * n, -1) for lv, c in fields["kpc"].items()}, d)
        sgn = _bits_to_bytes(np.asarray(fields["bits"]).reshape(B * H * n, m)) if m else np.zeros((B * H * n, 0), np.uint8)
        rec = np.concatenate([ang, sgn], axis=-1).reshape(B, H, n, kb)
    else:
        kcodes = np.asarray(fields["kcodes"])
        planes = [((kcodes >> p) & 1) for p in range(bk)]
        kbitsm = np.concatenate(planes + [np.asarray(fields["bits"])], axis=-1)  # [B,H,n,bk*d+m]
        rec = _bits_to_bytes(kbitsm)  # [B,H,n,kb]
    kreg = image[lay["kbits"]:lay["kbits"] + B * H * cap * kb].reshape(B, H, cap, kb)
    kreg[:, :, start_pos:start_pos + n, :] = rec
    kn = lay["knrec"] // 2
    norms = [np.asarray(fields["n16"]), np.asarray(fields["rn16"])]
    if nsn:
        norms += [np.asarray(fields["ks1"]), np.zeros_like(np.asarray(fields["n16"]))]
    nreg = image[lay["knorm"]:lay["knorm"] + B * H * cap * 2 * kn].view(np.float16).reshape(B, H, cap, kn)
    nreg[:, :, start_pos:start_pos + n, :] = np.stack(norms, axis=-1).astype(np.float16)
    if bv > 0 and polar:
        vb = 3 * d // 8
        vreg = image[lay["vcodes"]:lay["vcodes"] + B * H * cap * vb].reshape(B, H, cap, vb)
        ang = polar_pack_codes({lv: np.asarray(c).reshape(B * H * n, -1) for lv, c in fields["vpc"].items()}, d)
        vreg[:, :, start_pos:start_pos + n, :] = ang.reshape(B, H, n, vb)
        vnreg = image[lay["vnorm"]:lay["vnorm"] + B * H * cap * 2].view(np.float16).reshape(B, H, cap)
        vnreg[:, :, start_pos:start_pos + n] = np.asarray(fields["vn16"]).astype(np.float16)
    elif bv > 0:
        vcodes = np.asarray(fields["vcodes"]).astype(np.int64)
        tiles = lay["tiles"]
        wbytes = 4 * bv
        vreg = image[lay["vcodes"]:lay["vcodes"] + B * H * tiles * d * wbytes].reshape(B, H, tiles, d, wbytes)
        for i in range(n):
            t = start_pos + i
            tile, slot = divmod(t, 32)
            for p in range(bv):
                bit = (vcodes[:, :, i, :] >> p) & 1          # [B, H, d]
                pos = bv * slot + p
                byte, sh = divmod(pos, 8)
                cur = vreg[:, :, tile, :, byte].astype(np.int64)
                cur = (cur & ~(1 << sh)) | (bit << sh)
                vreg[:, :, tile, :, byte] = cur.astype(np.uint8)
        vn = lay["vnrec"] // 2
        vnorms = [np.asarray(fields["vn16"])] + ([np.asarray(fields["vs1"])] if nsn else [])
        vnreg = image[lay["vnorm"]:lay["vnorm"] + B * H * cap * 2 * vn].view(np.float16).reshape(B, H, cap, vn)
        vnreg[:, :, start_pos:start_pos + n, :] = np.stack(vnorms, axis=-1).astype(np.float16)
    return image


def unpack_cache(image: np.ndarray, desc: dict, length: int) -> dict:
    """Inverse of pack_cache for tokens [0, length).  Codes and bits come back as uint8."""
    B, H, d, cap = desc["batch"], desc["kv_heads"], desc["d"], desc["capacity"]
    bk, bv, m = desc["bits_k"], desc["bits_v"], desc["m"]
    nsn, polar = int(desc.get("nsn", 0)), int(desc.get("polar", 0))
    lay = cache_layout(B, H, d, cap, bk, bv, m, nsn, polar)
    image = np.asarray(image, dtype=np.uint8)
    hdr = image[:HEADER_BYTES].view(np.uint32)
    kb = lay["kbytes"]
    kreg = image[lay["kbits"]:lay["kbits"] + B * H * cap * kb].reshape(B, H, cap, kb)[:, :, :length]
    bitsall = np.unpackbits(kreg, axis=-1, bitorder="little")
    out = {"magic": int(hdr[0]), "version": int(hdr[1]), "flags": int(hdr[2]),
           "bits": bitsall[..., bk * d:bk * d + m]}
    if polar:
        pcs = polar_unpack_codes(kreg[..., :3 * d // 8].reshape(B * H * length, -1), d)
        out["kpc"] = {lv: c.reshape(B, H, length, -1) for lv, c in pcs.items()}
    else:
        kcodes = np.zeros((B, H, length, d), dtype=np.uint8)
        for p in range(bk):
            kcodes |= bitsall[..., p * d:(p + 1) * d] << np.uint8(p)
        out["kcodes"] = kcodes
    kn = lay["knrec"] // 2
    nreg = image[lay["knorm"]:lay["knorm"] + B * H * cap * 2 * kn].view(np.float16).reshape(B, H, cap, kn)
    out["n16"] = nreg[:, :, :length, 0].astype(np.float64)
    out["rn16"] = nreg[:, :, :length, 1].astype(np.float64)
    if nsn:
        out["ks1"] = nreg[:, :, :length, 2].astype(np.float64)
        means = image[lay["nsn"]:lay["nsn"] + B * H * 4 * d * 4].view(np.float32).reshape(B, H, 4, d)
        for i, f in enumerate(("ok", "ov", "pok", "pov")):
            out[f] = means[:, :, i].astype(np.float64)
    if bv > 0 and polar:
        vb = 3 * d // 8
        vreg = image[lay["vcodes"]:lay["vcodes"] + B * H * cap * vb].reshape(B, H, cap, vb)[:, :, :length]
        pcs = polar_unpack_codes(vreg.reshape(B * H * length, -1), d)
        out["vpc"] = {lv: c.reshape(B, H, length, -1) for lv, c in pcs.items()}
        vnreg = image[lay["vnorm"]:lay["vnorm"] + B * H * cap * 2].view(np.float16).reshape(B, H, cap)
        out["vn16"] = vnreg[:, :, :length].astype(np.float64)
    elif bv > 0:
        tiles = lay["tiles"]
        wbytes = 4 * bv
        vreg = image[lay["vcodes"]:lay["vcodes"] + B * H * tiles * d * wbytes].reshape(B, H, tiles, d, wbytes)
        used = (length + 31) // 32
        # token 32*tile + i, bit p of its code: bit bv*i + p of the tile's integer
        vbits = np.unpackbits(vreg[:, :, :used], axis=-1, bitorder="little")  # [B,H,used,d,32*bv]
        vbits = vbits.reshape(B, H, used, d, 32, bv)
        codes = np.zeros((B, H, used, d, 32), dtype=np.uint8)
        for p in range(bv):
            codes |= vbits[..., p] << np.uint8(p)
        out["vcodes"] = codes.transpose(0, 1, 2, 4, 3).reshape(B, H, used * 32, d)[:, :, :length]
        vn = lay["vnrec"] // 2
        vnreg = image[lay["vnorm"]:lay["vnorm"] + B * H * cap * 2 * vn].view(np.float16).reshape(B, H, cap, vn)
        out["vn16"] = vnreg[:, :, :length, 0].astype(np.float64)
        if nsn:
            out["vs1"] = vnreg[:, :, :length, 1].astype(np.float64)
    return out


# ----------------------------------------------------------------------------------
# Decode attention ([TurboESM] 2.E: dequantize, residual correction, online softmax,
# inverse rotation; [TurboQuant] QJL: full-precision query against sign bits).
# Written as plain full softmax (no online rescaling): mathematically identical.
# ----------------------------------------------------------------------------------
def estimate_scores(qr: np.ndarray, sq: np.ndarray, kcodes, n16, rn16, bits, codec: Codec):
    """score_t = n16_t <qr, c_k[code_t]> + rn16_t sqrt(pi/2)/m <sq, 2 bits_t - 1>."""
    khat = codec.cb_k.c[kcodes]                               # [T, d]
    mse = n16 * (khat @ qr)
    if codec.m > 0:
        qjl = rn16 * codec.qjl_scale * ((2.0 * bits - 1.0) @ sq)
    else:
        qjl = 0.0
    return mse + qjl


def _packed_scores(fields, b, g, length, qr, sq, codec):
    """Score estimates of the packed tokens [0, length) of unit (b, g): scalar codes or
    PolarQuant angles, plus the NSN mean term when the fields carry one."""
    if "kpc" in fields:
        s = estimate_scores_polar(qr, sq, {lv: c[b, g, :length] for lv, c in fields["kpc"].items()},
                                  fields["n16"][b, g, :length], fields["rn16"][b, g, :length],
                                  fields["bits"][b, g, :length], codec)
    else:
        s = estimate_scores(qr, sq, fields["kcodes"][b, g, :length], fields["n16"][b, g, :length],
                            fields["rn16"][b, g, :length], fields["bits"][b, g, :length], codec)
    if "ks1" in fields:   # NSN: the mean's share s1 <q, o>, in the rotated basis
        s = s + fields["ks1"][b, g, :length] * (fields["pok"][b, g] @ qr)
    return s


def _packed_values(fields, b, g, length, codec):
    """Reconstructed rotated values [length, d] of unit (b, g)."""
    if "vpc" in fields:
        return polar_decode({lv: c[b, g, :length] for lv, c in fields["vpc"].items()},
                            fields["vn16"][b, g, :length], make_polar_codebook(codec.d))
    vhat = fields["vn16"][b, g, :length, None] * codec.cb_v.c[fields["vcodes"][b, g, :length]]
    if "vs1" in fields:
        vhat = vhat + fields["vs1"][b, g, :length, None] * fields["pov"][b, g][None, :]
    return vhat


def attend(fields: dict, q, codec: Codec, *, q_pos: int, rope_base: float, scale: float,
           kv_heads: int, length: int):
    """fp64 decode attention of q [B, Hq, d] over tokens [0, length) of `fields`
    (as returned by unpack_cache or built from encode outputs).

    GQA: q-head h reads kv-head floor(h * Hkv / Hq).  Returns (out [B, Hq, d],
    scores [B, Hq, length]); scores are the unscaled estimates, the softmax uses
    scale * score.  length == 0 gives out = 0."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    scores = np.zeros((B, Hq, length))
    if scale == 0:
        scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(Hq):
            g = (h * kv_heads) // Hq
            qp = rope(q[b, h][None, :], [q_pos], rope_base)[0] if rope_base != 0 else q[b, h]
            qr = codec.Pi @ qp
            sq = codec.S @ qr if codec.m > 0 else None
            if length == 0:
                continue
            s = _packed_scores(fields, b, g, length, qr, sq, codec)
            scores[b, h] = s
            lam = scale * s
            p = np.exp(lam - np.max(lam))
            p = p / np.sum(p)
            o_rot = p @ _packed_values(fields, b, g, length, codec)
            out[b, h] = codec.Pi.T @ o_rot
    return out, scores


def attend_window(fields: dict, win_k, win_v, q, codec: Codec, *, q_pos: int, rope_base: float,
                  scale: float, kv_heads: int, length: int, win_len: int):
    """fp64 decode attention of q [B, Hq, d] over packed tokens [0, length) of `fields`
    and a full-precision window of win_len tokens at positions length, ..., length +
    win_len - 1 ([NSNQuant] section 4, residuals).  win_k, win_v: [B, Hkv, >= win_len, d]
    raw keys (before RoPE) and values.

    A window token's score is the exact <RoPE(q, q_pos), RoPE(k, pos)>, the rotation
    being orthogonal ([TurboESM] 2.A); packed tokens use the estimator.  One softmax over
    both sets; the packed part's value sum is rotated back by Pi^T, the window's values
    enter as they are.  Returns (out [B, Hq, d], scores [B, Hq, length + win_len])."""
    q = np.asarray(q, dtype=np.float64)
    wk = np.asarray(win_k, dtype=np.float64)
    wv = np.asarray(win_v, dtype=np.float64)
    B, Hq, d = q.shape
    n = length + win_len
    out = np.zeros((B, Hq, d))
    scores = np.zeros((B, Hq, n))
    if scale == 0:
        scale = 1.0 / math.sqrt(d)
    pos = length + np.arange(win_len)
    for b in range(B):
        for h in range(Hq):
            g = (h * kv_heads) // Hq
            qp = rope(q[b, h][None, :], [q_pos], rope_base)[0] if rope_base != 0 else q[b, h]
            qr = codec.Pi @ qp
            sq = codec.S @ qr if codec.m > 0 else None
            if n == 0:
                continue
            s = np.zeros(n)
            if length > 0:
                s[:length] = _packed_scores(fields, b, g, length, qr, sq, codec)
            if win_len > 0:
                kr = rope(wk[b, g, :win_len], pos, rope_base) if rope_base != 0 else wk[b, g, :win_len]
                s[length:] = kr @ qp
            scores[b, h] = s
            lam = scale * s
            p = np.exp(lam - np.max(lam))
            p = p / np.sum(p)
            o = np.zeros(d)
            if length > 0:
                o += codec.Pi.T @ (p[:length] @ _packed_values(fields, b, g, length, codec))
            if win_len > 0:
                o += p[length:] @ wv[b, g, :win_len]
            out[b, h] = o
    return out, scores


_ATTEND_FIELDS = ("kcodes", "n16", "rn16", "bits", "vcodes", "vn16")


def decode_step(state: dict, new_k, new_v, q, codec: Codec, *, q_pos: int, rope_base: float,
                scale: float, kv_heads: int):
    """One generation step over a packed part and a full-precision window ([NSNQuant]
    section 4, residuals: recent tokens stay unquantized in a residual buffer, which is
    quantized and appended to the packed part once it is full).

    state (updated in place): "fields" (packed tokens, [B, Hkv, length, ...] arrays as for
    attend), "length", "win_k", "win_v" ([B, Hkv, cap, d] raw keys and values), "win_len".
    new_k, new_v: [B, Hkv, d], the keys and values of position length + win_len.

    Reading (the pages do not fix the moment of the flush): a window holding cap tokens is
    flushed when the next token needs its room, so attention always sees between 1 and
    cap full-precision tokens; the flushed keys are rotary-embedded at their own
    positions.  Returns attend_window's (out, scores) after the append."""
    wk, wv = state["win_k"], state["win_v"]
    B, H, cap, d = wk.shape
    if state["win_len"] == cap:
        pos = state["length"] + np.arange(cap)
        old = state["fields"]
        nsn = "ok" in old   # NSN cache: the flushed tokens use the stored means
        ok = np.repeat(np.asarray(old["ok"]).reshape(B * H, 1, d), cap, axis=1).reshape(-1, d) if nsn else None
        ov = np.repeat(np.asarray(old["ov"]).reshape(B * H, 1, d), cap, axis=1).reshape(-1, d) if nsn else None
        ke = encode(wk.reshape(-1, d), codec, kind="key", positions=np.tile(pos, B * H), rope_base=rope_base,
                    nsn_o=ok)
        ve = encode(wv.reshape(-1, d), codec, kind="value", nsn_o=ov)
        new = {"kcodes": ke["codes"].reshape(B, H, cap, d), "n16": ke["n16"].reshape(B, H, cap),
               "rn16": ke["rn16"].reshape(B, H, cap), "bits": ke["bits"].reshape(B, H, cap, codec.m),
               "vcodes": ve["codes"].reshape(B, H, cap, d), "vn16": ve["n16"].reshape(B, H, cap)}
        names = _ATTEND_FIELDS
        if nsn:
            new["ks1"] = ke["s1_16"].reshape(B, H, cap)
            new["vs1"] = ve["s1_16"].reshape(B, H, cap)
            names = names + ("ks1", "vs1")
        state["fields"] = {f: np.concatenate([np.asarray(old[f])[:, :, :state["length"]], new[f]], axis=2)
                           for f in names}
        if nsn:
            state["fields"].update({f: old[f] for f in ("ok", "ov", "pok", "pov")})
        state["length"] += cap
        state["win_len"] = 0
    w = state["win_len"]
    wk[:, :, w] = np.asarray(new_k, dtype=np.float64)
    wv[:, :, w] = np.asarray(new_v, dtype=np.float64)
    state["win_len"] = w + 1
    return attend_window(state["fields"], wk, wv, q, codec, q_pos=q_pos, rope_base=rope_base, scale=scale,
                         kv_heads=kv_heads, length=state["length"], win_len=state["win_len"])


# ----------------------------------------------------------------------------------
# Inner-product search over packed vectors ([TurboQuant] vector search: top-k by the
# estimated inner product, recall 1@k).
# ----------------------------------------------------------------------------------
def search_scores(fields: dict, queries, codec: Codec):
    """Estimated <q, x> for every (query, database vector): [nq, n_db] fp64."""
    Q = np.asarray(queries, dtype=np.float64)
    qr = Q @ codec.Pi.T
    sq = qr @ codec.S.T
    khat = codec.cb_k.c[fields["kcodes"]]                         # [n, d]
    mse = (qr @ khat.T) * fields["n16"][None, :]
    qjl = (sq @ (2.0 * fields["bits"] - 1.0).T) * (fields["rn16"][None, :] * codec.qjl_scale)
    return mse + qjl


def topk(scores: np.ndarray, k: int):
    """Per row: the k largest scores in descending order, equal scores to the lower index."""
    nq, n = scores.shape
    k_eff = min(k, n)
    idx = np.zeros((nq, k), dtype=np.int64) - 1
    val = np.full((nq, k), -np.inf)
    for i in range(nq):
        order = np.lexsort((np.arange(n), -scores[i]))[:k_eff]
        idx[i, :k_eff] = order
        val[i, :k_eff] = scores[i, order]
    return idx, val


def exact_topk(db, queries, k: int):
    """Ground truth for recall: fp64 brute-force inner products on unquantized vectors."""
    s = np.asarray(queries, dtype=np.float64) @ np.asarray(db, dtype=np.float64).T
    return topk(s, k)
