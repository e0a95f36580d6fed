// Host half of libtq: argument validation, buffer layouts, the fp64 Lloyd-Max codebook,
// the seeded draws of the rotation signs and the Gaussian projection, and the codec table.
// Nothing here touches the GPU.

#include <cmath>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {

bool codec_desc_valid(const tq_codec_desc &c) {
  if (c.d < 8 || c.d > 4096 || (c.d % 8) != 0) return false;
  if (c.bits_k < 1 || c.bits_k > 4) return false;
  if (c.bits_v < 0 || c.bits_v > 4) return false;
  if (c.m < 0 || c.m > 2048 || (c.m % 32) != 0) return false;
  return true;
}

bool cache_desc_valid(const tq_cache_desc &c) {
  tq_codec_desc cd{c.d, c.bits_k, c.bits_v, c.m, 0};
  if (!codec_desc_valid(cd)) return false;
  if (c.batch < 1 || c.kv_heads < 1 || c.capacity < 0) return false;
  // units index a grid dimension (at most 65535), token positions and tile counts stay
  // in int, and every region size stays far inside size_t
  if (int64_t(c.batch) * int64_t(c.kv_heads) > kMaxUnits || c.capacity > kMaxCapacity) return false;
  if (c.nsn != 0 && c.nsn != 1) return false;
  if (c.nsn && (c.bits_v == 0 || (c.d != 64 && c.d != 128))) return false;
  if (c.polar != 0 && c.polar != 1) return false;
  // PolarQuant: 3 d - 2 bits of angles per vector, recorded as bits_k = bits_v = 3
  if (c.polar && (c.nsn || (c.d != 64 && c.d != 128) || c.bits_k != 3 || (c.bits_v != 0 && c.bits_v != 3)))
    return false;
  return true;
}

CacheLayout cache_layout(const tq_cache_desc &c) {
  CacheLayout L;
  L.kbytes = (c.bits_k * c.d + c.m) / 8;
  L.tiles = (c.capacity + kValueTile - 1) / kValueTile;
  L.vwords = c.bits_v;
  const size_t units = size_t(c.batch) * size_t(c.kv_heads);
  size_t cur = kHeaderBytes;
  L.kbits = cur;
  cur = align256(cur + units * size_t(c.capacity) * size_t(L.kbytes));
  L.knrec = c.nsn ? 8 : 4;
  L.vnrec = c.nsn ? 4 : 2;
  L.knorm = cur;
  cur = align256(cur + units * size_t(c.capacity) * size_t(L.knrec));
  if (c.bits_v > 0) {
    L.vcodes = cur;   // polar: token records of 3 d / 8 bytes instead of tiles
    cur = align256(cur + (c.polar ? units * size_t(c.capacity) * size_t(3 * c.d / 8)
                                  : units * size_t(L.tiles) * size_t(c.d) * size_t(4 * c.bits_v)));
    L.vnorm = cur;
    cur = align256(cur + units * size_t(c.capacity) * size_t(L.vnrec));
  }
  if (c.nsn) {
    L.nsn = cur;   // per unit [o_K, o_V, Pi o_K, Pi o_V], fp32 [d] each
    cur = align256(cur + units * 4 * size_t(c.d) * 4);
  }
  L.total = cur;
  return L;
}

CodecLayout codec_layout(int d, int bits_k, int bits_v, int m) {
  (void)bits_k;
  (void)bits_v;
  CodecLayout L;
  L.block = hadamard_block(d);
  size_t cur = kHeaderBytes;
  L.ck = cur; cur += kMaxCodes * 4;
  L.tk = cur; cur += kMaxCodes * 4;
  L.cv = cur; cur += kMaxCodes * 4;
  L.tv = cur; cur += kMaxCodes * 4;
  cur = align256(cur);
  L.D = cur; cur = align256(cur + size_t(d) * 4);
  L.S = cur; cur = align256(cur + size_t(m) * size_t(d) * 4);
  L.ST = cur; cur = align256(cur + size_t(m) * size_t(d) * 4);
  for (int i = 0; i < 3; ++i) {
    L.Sh[i] = cur;
    cur = align256(cur + size_t(m) * size_t(d) * 2);
  }
  L.pcs = cur;
  cur = align256(cur + size_t(kPolarLevels) * kPolarCodes * 2 * 4);
  L.pt = cur;
  cur = align256(cur + size_t(kPolarLevels) * kPolarCodes * 8);
  L.total = cur;
  return L;
}

double round_fp16(double x, uint16_t *bits_out) {
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs(x);
  uint16_t bits;
  double v;
  if (std::isnan(a)) {
    bits = sign | 0x7E00;
    v = x;
  } else if (a >= 65520.0) {  // 65504 + half an ulp (2^4): rounds to infinity
    bits = sign | 0x7C00;
    v = std::copysign(INFINITY, x);
  } else {
    int e = 0;
    std::frexp(a, &e);          // a = f 2^e, f in [0.5, 1)
    int E = e - 1;              // a in [2^E, 2^(E+1))
    if (E < -14) E = -14;       // subnormal range: quantum 2^-24
    const double q = std::ldexp(1.0, E - 10);
    const double r = std::nearbyint(a / q);  // default rounding: nearest, ties to even
    v = r * q;
    // encode the exactly representable fp16 value v
    if (v == 0.0) {
      bits = sign;
    } else {
      int e2 = 0;
      std::frexp(v, &e2);
      int E2 = e2 - 1;
      if (E2 < -14) {  // subnormal
        bits = uint16_t(sign | uint16_t(std::ldexp(v, 24)));
      } else {
        const uint32_t mant = uint32_t(std::ldexp(v, 10 - E2)) - 1024u;
        bits = uint16_t(sign | uint16_t((E2 + 15) << 10) | uint16_t(mant));
      }
    }
    v = std::copysign(v, x);
  }
  if (bits_out) *bits_out = bits;
  return v;
}

// ---------------------------------------------------------------------------------
// Lloyd-Max codebook for the sphere marginal f_d(x) = C_d (1 - x^2)^((d-3)/2).
// Cell masses: with x = sin(theta), int_a^b f dx = C_d int cos^(d-2)(theta) dtheta,
// integrated by composite Gauss-Legendre (the substitution removes the endpoint
// singularities of small d).  First moments: int_a^b x f dx = M(b) - M(a) with
// M(x) = -C_d (1 - x^2)^((d-1)/2) / (d - 1).
// ---------------------------------------------------------------------------------
namespace {

struct GaussLegendre {
  std::vector<double> x, w;  // nodes on [-1, 1]
  explicit GaussLegendre(int n) : x(n), w(n) {
    // Newton iteration on P_n from the Chebyshev initial guesses
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double pp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        pp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / pp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      pp = n * (z * p1 - p0) / (z * z - 1.0);
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * pp * pp);
    }
  }
};

const GaussLegendre &gl20() {
  static const GaussLegendre g(20);
  return g;
}

double log_cd(int d) {
  return std::lgamma(0.5 * d) - 0.5 * std::log(M_PI) - std::lgamma(0.5 * (d - 1));
}

// int_a^b f_d(x) dx, a <= b, both in [-1, 1]
double cell_mass(int d, double a, double b) {
  const double lc = log_cd(d);
  const double ta = std::asin(std::max(-1.0, std::min(1.0, a)));
  const double tb = std::asin(std::max(-1.0, std::min(1.0, b)));
  if (tb <= ta) return 0.0;
  // panels about a quarter of the density's width (1/sqrt(d)) in theta
  const double width = 0.25 / std::sqrt(double(d));
  const int panels = std::max(1, int(std::ceil((tb - ta) / width)));
  const double h = (tb - ta) / panels;
  const GaussLegendre &g = gl20();
  double sum = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double lo = ta + p * h, mid = lo + 0.5 * h;
    double ps = 0.0;
    for (size_t i = 0; i < g.x.size(); ++i) {
      const double th = mid + 0.5 * h * g.x[i];
      const double c = std::cos(th);
      if (c > 0.0) ps += g.w[i] * std::exp(lc + (d - 2) * std::log(c));
    }
    sum += 0.5 * h * ps;
  }
  return sum;
}

double partial_mean(int d, double x) {
  const double om = 1.0 - x * x;
  if (om <= 0.0) return 0.0;
  return -std::exp(log_cd(d) + 0.5 * (d - 1) * std::log(om)) / (d - 1);
}

void lloyd_max(int d, int bits, double *c, double *t) {
  const int K = 1 << bits;
  const double s = 1.0 / std::sqrt(double(d));
  // spread initial centroids over +-2.5 standard deviations (the iteration converges to
  // the unique optimum of this log-concave density from any ordered start)
  for (int k = 0; k < K; ++k) c[k] = (2.0 * k + 1.0 - K) / K * 2.5 * s;
  // cells far in the tails carry no mass: clip the integration range at 40 sigma
  const double lim = std::min(1.0, 40.0 * s);
  std::vector<double> e(K + 1), mass(K);
  // the step shrinks geometrically until rounding sets a floor; where that floor lies above
  // the tolerance (d = 4096 with 16 cells) stop once the step has not reached a new low
  // for a while
  double best = INFINITY;
  int stalled = 0;
  for (int it = 0; it < 200000; ++it) {
    e[0] = -lim;
    e[K] = lim;
    for (int k = 0; k + 1 < K; ++k) e[k + 1] = 0.5 * (c[k] + c[k + 1]);
    double delta = 0.0;
    for (int k = 0; k < K; ++k) {
      const double a = std::max(e[k], -lim), b = std::min(e[k + 1], lim);
      const double mk = cell_mass(d, a, b);
      const double mom = partial_mean(d, b) - partial_mean(d, a);
      const double cn = mom / mk;
      delta = std::max(delta, std::fabs(cn - c[k]));
      c[k] = cn;
    }
    if (delta / s < 1e-13) break;
    if (delta < best) {
      best = delta;
      stalled = 0;
    } else if (++stalled >= 200) {
      break;
    }
  }
  // the density is even, so the optimum is odd: c[K-1-k] = -c[k].  Make that exact (the
  // iterate differs from it only by rounding); the search kernel relies on it.
  for (int k = 0; k < K / 2; ++k) {
    const double v = 0.5 * (c[K - 1 - k] - c[k]);
    c[k] = -v;
    c[K - 1 - k] = v;
  }
  for (int k = 0; k + 1 < K; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
}

// SplitMix64 as a counter generator: output k of the generator seeded with `seed`.
// PolarQuant angle law of level l >= 2: psi = atan2(|b|, |a|) for independent
// m-dimensional standard Gaussian a, b (m = 2^(l-1)), density proportional to
// sin^(m-1)(2 psi) on [0, pi/2].  Cell mass and first moment by composite Gauss-Legendre.
void polar_cell(int m, double a, double b, double *mass, double *mom) {
  const GaussLegendre &g = gl20();
  constexpr int P = 64;
  double s0 = 0.0, s1 = 0.0;
  const double h = (b - a) / P;
  for (int p = 0; p < P; ++p) {
    const double lo = a + p * h, mid = lo + 0.5 * h;
    for (size_t i = 0; i < g.x.size(); ++i) {
      const double x = mid + 0.5 * h * g.x[i];
      const double s = std::sin(2.0 * x);
      const double f = s > 0.0 ? std::exp((m - 1) * std::log(s)) : 0.0;
      s0 += g.w[i] * f;
      s1 += g.w[i] * f * x;
    }
  }
  *mass = 0.5 * h * s0;
  *mom = 0.5 * h * s1;
}

inline uint64_t splitmix64(uint64_t seed, uint64_t k) {
  uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
constexpr uint64_t kStreamSigns = 1ull << 32;
constexpr uint64_t kStreamGauss = 2ull << 32;

inline double uniform_open(uint64_t x) { return (double(x >> 11) + 0.5) * 0x1.0p-53; }

}  // namespace

void polar_grid(int level, double *c, double *t) {
  if (level == 1) {
    const double w = 2.0 * M_PI / 16.0;
    for (int k = 0; k < 16; ++k) c[k] = (k + 0.5) * w;
    for (int k = 1; k < 16; ++k) t[k - 1] = k * w;
    return;
  }
  const int m = 1 << (level - 1), K = 4;
  for (int k = 0; k < K; ++k) c[k] = 0.5 * M_PI * (k + 0.5) / K;
  for (int it = 0; it < 1000; ++it) {
    double edges[K + 1];
    edges[0] = 0.0;
    edges[K] = 0.5 * M_PI;
    for (int k = 1; k < K; ++k) edges[k] = 0.5 * (c[k - 1] + c[k]);
    double delta = 0.0;
    for (int k = 0; k < K; ++k) {
      double mass, mom;
      polar_cell(m, edges[k], edges[k + 1], &mass, &mom);
      const double cn = mom / mass;
      delta = std::max(delta, std::fabs(cn - c[k]));
      c[k] = cn;
    }
    if (delta < 1e-13) break;
  }
  for (int k = 1; k < K; ++k) t[k - 1] = 0.5 * (c[k - 1] + c[k]);
}

}  // namespace tq

using namespace tq;

extern "C" {

const char *tq_version(void) { return "libtq 1.0 format 1"; }

const char *tq_status_str(int32_t s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported parameters";
    case TQ_ECAPACITY: return "beyond cache capacity";
    case TQ_ENOSPACE: return "buffer too small";
    case TQ_EDEVICE: return "device error";
  }
  return "unknown status";
}

tq_status tq_make_codebook_f64(int32_t d, int32_t bits, double *centroids, double *bounds) {
  if (!centroids || !bounds) return TQ_EINVAL;
  if (d < 8 || d > 4096 || bits < 1 || bits > 4) return TQ_EUNSUPPORTED;
  lloyd_max(d, bits, centroids, bounds);
  return TQ_OK;
}

tq_status tq_make_codebook(int32_t d, int32_t bits, float *centroids, float *bounds) {
  if (!centroids || !bounds) return TQ_EINVAL;
  if (d < 8 || d > 4096 || bits < 1 || bits > 4) return TQ_EUNSUPPORTED;
  double c[kMaxCodes], t[kMaxCodes];
  lloyd_max(d, bits, c, t);
  const int K = 1 << bits;
  double cs[kMaxCodes];
  for (int k = 0; k < K; ++k) cs[k] = round_fp16(c[k]);
  for (int k = 0; k < K; ++k) centroids[k] = float(cs[k]);
  for (int k = 0; k + 1 < K; ++k) bounds[k] = float(0.5 * (cs[k] + cs[k + 1]));  // exact
  return TQ_OK;
}

size_t tq_codec_bytes(const tq_codec_desc *desc) {
  if (!desc || !codec_desc_valid(*desc)) return 0;
  return codec_layout(desc->d, desc->bits_k, desc->bits_v, desc->m).total;
}

tq_status tq_codec_build(const tq_codec_desc *desc, void *host_out, size_t bytes) {
  if (!desc || !host_out) return TQ_EINVAL;
  if (!codec_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  const int d = desc->d, m = desc->m;
  const CodecLayout L = codec_layout(d, desc->bits_k, desc->bits_v, m);
  if (bytes < L.total) return TQ_ENOSPACE;
  uint8_t *base = static_cast<uint8_t *>(host_out);
  std::memset(base, 0, L.total);
  CodecHeader h{};
  h.magic = kCodecMagic;
  h.version = kFormatVersion;
  h.d = d;
  h.bits_k = desc->bits_k;
  h.bits_v = desc->bits_v;
  h.m = m;
  h.seed = desc->seed;
  h.block = L.block;
  h.qjl_scale = m > 0 ? float(std::sqrt(M_PI / 2.0) / m) : 0.0f;
  h.inv_sqrt_block = float(1.0 / std::sqrt(double(L.block)));
  std::memcpy(base, &h, sizeof(h));

  float *ck = reinterpret_cast<float *>(base + L.ck), *tk = reinterpret_cast<float *>(base + L.tk);
  float *cv = reinterpret_cast<float *>(base + L.cv), *tv = reinterpret_cast<float *>(base + L.tv);
  for (int k = 0; k < kMaxCodes; ++k) tk[k] = tv[k] = INFINITY;
  tq_status st = tq_make_codebook(d, desc->bits_k, ck, tk);
  if (st != TQ_OK) return st;
  if (desc->bits_v > 0) {
    st = tq_make_codebook(d, desc->bits_v, cv, tv);
    if (st != TQ_OK) return st;
  }
  float *D = reinterpret_cast<float *>(base + L.D);
  for (int j = 0; j < d; ++j)
    D[j] = (splitmix64(desc->seed, kStreamSigns + uint64_t(j)) >> 63) ? -1.0f : 1.0f;
  float *S = reinterpret_cast<float *>(base + L.S);
  float *ST = reinterpret_cast<float *>(base + L.ST);
  uint16_t *Sh[3];
  for (int i = 0; i < 3; ++i) Sh[i] = reinterpret_cast<uint16_t *>(base + L.Sh[i]);
  for (int i = 0; i < m; ++i) {
    for (int j = 0; j < d; ++j) {
      const uint64_t n = uint64_t(i) * uint64_t(d) + uint64_t(j);
      const double u1 = uniform_open(splitmix64(desc->seed, kStreamGauss + 2 * n));
      const double u2 = uniform_open(splitmix64(desc->seed, kStreamGauss + 2 * n + 1));
      const double z = std::sqrt(-2.0 * std::log(u1)) * std::cos((2.0 * M_PI) * u2);
      const float zf = float(z);
      S[size_t(i) * d + j] = zf;
      ST[size_t(j) * m + i] = zf;
      // three-part fp16 split: each part is the remainder rounded to fp16 (11 significant
      // bits); exact when |S| >= 1/2, where the last remainder is a multiple of the fp16
      // subnormal step, else within half of that step
      double rest = double(zf);
      for (int k = 0; k < 3; ++k) {
        uint16_t hb = 0;
        const double hv = round_fp16(rest, &hb);
        Sh[k][size_t(i) * d + j] = hb;
        rest -= hv;
      }
    }
  }
  // PolarQuant grids of the levels a vector of dimension d has (d a power of two): the
  // cos and sin of each centroid rounded to fp32, the boundaries in fp64
  float *pcs = reinterpret_cast<float *>(base + L.pcs);
  double *pt = reinterpret_cast<double *>(base + L.pt);
  if ((d & (d - 1)) == 0) {
    for (int lv = 1; (1 << lv) <= d && lv <= kPolarLevels; ++lv) {
      double c[kPolarCodes], t[kPolarCodes];
      polar_grid(lv, c, t);
      const int K = lv == 1 ? 16 : 4;
      for (int k = 0; k < K; ++k) {
        pcs[((lv - 1) * kPolarCodes + k) * 2] = float(std::cos(c[k]));
        pcs[((lv - 1) * kPolarCodes + k) * 2 + 1] = float(std::sin(c[k]));
      }
      for (int k = 0; k < K - 1; ++k) pt[(lv - 1) * kPolarCodes + k] = t[k];
    }
  }
  return TQ_OK;
}

tq_status tq_make_polar_grid(int32_t level, double *centroids, double *bounds) {
  if (!centroids || !bounds) return TQ_EINVAL;
  if (level < 1 || level > kPolarLevels) return TQ_EUNSUPPORTED;
  polar_grid(level, centroids, bounds);
  return TQ_OK;
}

size_t tq_cache_bytes(const tq_cache_desc *desc) {
  if (!desc || !cache_desc_valid(*desc)) return 0;
  return cache_layout(*desc).total;
}

}  // extern "C"
