// Device half of libtq: HIP kernels for gfx950 and the C entry points that launch them.
//
// Kernels (the step of the method each one carries out is named at its definition):
//   k_cache_init        header of a packed cache
//   k_quantize_kv       RoPE -> seeded-sign FWHT -> norm -> Lloyd-Max codes -> bit planes
//                       -> residual -> QJL sign bits (MFMA), 4 lanes per token, d in {64, 128}
//   k_quantize_db       the same for database vectors of large d (one wave per vector)
//   k_qprep_pack        query RoPE, rotation Pi q, S q_rot and their sums; for the MFMA
//                       decode also the int8 digit rows and score coefficients
//   k_decode_lds        split-K decode on MFMA with LDS-staged tiles: key scores (int8),
//                       online softmax, values (fp16 hi/lo against LUT-dequantized
//                       centroids), accumulated in the rotated basis
//   k_decode_lds16      the same for groups of at most 4 query heads at d = 128, key
//                       scores on the 16-row int8 MFMA form
//   k_decode_split      the same on plain fp32 arithmetic for the other bit widths
//   k_decode_merge      merge of the splits, normalisation, inverse rotation Pi^T (a
//                       one-wave-per-row form, k_decode_merge_wave, for d = 64 and 128)
//   k_search_tile       packed database scores for a query tile + per-tile top-k
//   k_search_merge      per-query top-k over the tile candidates

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "tq_internal.h"

namespace tq {
namespace {

// ------------------------------------------------------------------ small helpers
__device__ __forceinline__ float load_elem(const void *p, size_t i, int dtype) {
  if (dtype == TQ_F32) return static_cast<const float *>(p)[i];
  const uint16_t b = static_cast<const uint16_t *>(p)[i];
  if (dtype == TQ_BF16) return __uint_as_float(uint32_t(b) << 16);
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return float(h);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t b) {
  uint16_t s = uint16_t(b);
  _Float16 h;
  __builtin_memcpy(&h, &s, 2);
  return float(h);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sylvester FWHT of N values held in registers of one lane (natural order):
// y = H_N x with H[i][j] = (-1)^popcount(i & j).
template <int N, typename T>
__device__ __forceinline__ void fwht_regs(T *x) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const T a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
}

struct CodecPtrs {
  const float *ck, *tk, *cv, *tv, *D, *S, *ST;
  const _Float16 *Sh[3];   // S split into three fp16 parts, each [m][d]
  const float *pcs;      // PolarQuant: cos, sin of each angle centroid, [level - 1][16][2]
  const double *pt;      // PolarQuant: angle boundaries, [level - 1][16]
  int block;
  float qjl_scale, inv_sqrt_block;
};

CodecPtrs codec_ptrs(const void *codec_dev, int d, int bits_k, int bits_v, int m) {
  const CodecLayout L = codec_layout(d, bits_k, bits_v, m);
  const uint8_t *b = static_cast<const uint8_t *>(codec_dev);
  CodecPtrs p;
  p.ck = reinterpret_cast<const float *>(b + L.ck);
  p.tk = reinterpret_cast<const float *>(b + L.tk);
  p.cv = reinterpret_cast<const float *>(b + L.cv);
  p.tv = reinterpret_cast<const float *>(b + L.tv);
  p.D = reinterpret_cast<const float *>(b + L.D);
  p.S = reinterpret_cast<const float *>(b + L.S);
  p.ST = reinterpret_cast<const float *>(b + L.ST);
  for (int i = 0; i < 3; ++i) p.Sh[i] = reinterpret_cast<const _Float16 *>(b + L.Sh[i]);
  p.pcs = reinterpret_cast<const float *>(b + L.pcs);
  p.pt = reinterpret_cast<const double *>(b + L.pt);
  p.block = L.block;
  p.qjl_scale = m > 0 ? float(std::sqrt(M_PI / 2.0) / m) : 0.0f;
  p.inv_sqrt_block = float(1.0 / std::sqrt(double(L.block)));
  return p;
}

struct CachePtrs {
  uint8_t *kbits;
  uint32_t *knorm;
  uint32_t *vcodes;
  uint16_t *vnorm;
  uint32_t *flags;
  float *nsn;   // NSN caches: per unit [o_K, o_V, Pi o_K, Pi o_V] fp32 [d] each; else null
  int kbytes, tiles;
};

CachePtrs cache_ptrs(void *cache_dev, const tq_cache_desc &c) {
  const CacheLayout L = cache_layout(c);
  uint8_t *b = static_cast<uint8_t *>(cache_dev);
  CachePtrs p;
  p.kbits = b + L.kbits;
  p.knorm = reinterpret_cast<uint32_t *>(b + L.knorm);
  p.vcodes = c.bits_v > 0 ? reinterpret_cast<uint32_t *>(b + L.vcodes) : nullptr;
  p.vnorm = c.bits_v > 0 ? reinterpret_cast<uint16_t *>(b + L.vnorm) : nullptr;
  p.flags = reinterpret_cast<uint32_t *>(b + 8);
  p.nsn = c.nsn ? reinterpret_cast<float *>(b + L.nsn) : nullptr;
  p.kbytes = L.kbytes;
  p.tiles = L.tiles;
  return p;
}

__global__ void k_fill_zero(float *p, size_t n) {
  const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ------------------------------------------------------------------ cache header
__global__ void k_cache_init(uint32_t *hdr, tq_cache_desc c) {
  const int i = threadIdx.x;
  if (i >= 64) return;
  uint32_t v = 0;
  switch (i) {
    case 0: v = kCacheMagic; break;
    case 1: v = kFormatVersion; break;
    case 4: v = uint32_t(c.batch); break;
    case 5: v = uint32_t(c.kv_heads); break;
    case 6: v = uint32_t(c.d); break;
    case 7: v = uint32_t(c.capacity); break;
    case 8: v = uint32_t(c.bits_k); break;
    case 9: v = uint32_t(c.bits_v); break;
    case 10: v = uint32_t(c.m); break;
    case 11: v = uint32_t(c.nsn); break;
    case 12: v = uint32_t(c.polar); break;
    default: v = 0;
  }
  hdr[i] = v;
}

// ------------------------------------------------------------------ quantize
// RoPE frequencies of one append: theta_j = base^(-2j/d) and its cos and sin in fp64, for
// j < d/2 (d <= 128), computed once per call on the host and passed with the arguments.
struct RopeFreq {
  double theta[64], c[64], s[64];
};

// cos and sin of the query position's rotary angles q_pos * theta_j (fp64 on the host,
// rounded to fp32), j < d / 2; identity (1, 0) when the call has no RoPE
struct QueryRope {
  float c[64], s[64];
};

struct QuantArgs {
  CodecPtrs cp;
  CachePtrs ch;
  const void *k, *v;
  int start, n_new, capacity, bits_k, bits_v, m, units;
  float rope_base;
  double sqrt_b, inv_sqrt_b;   // sqrt(B) and 1 / sqrt(B) of the Hadamard block B (host fp64)
  RopeFreq rf;
};

typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ double load_d(const void *p, size_t i) {
  if constexpr (DT == TQ_F32) {
    return double(static_cast<const float *>(p)[i]);
  } else if constexpr (DT == TQ_BF16) {
    return double(__uint_as_float(uint32_t(static_cast<const uint16_t *>(p)[i]) << 16));
  } else {
    const uint16_t b = static_cast<const uint16_t *>(p)[i];
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return double(float(h));
  }
}

// fp64 -> fp16 bits, round to nearest even, for x >= 0: round toward zero to fp32 and
// set the sticky bit if inexact (round-to-odd), then let the fp32 -> fp16 conversion
// round to nearest even; 24 >= 11 + 2 bits makes the double rounding exact.  Values that
// would round to infinity are stored as 65504 and reported through *over.
__device__ __forceinline__ uint16_t f64_to_f16_sat(double x, bool *over) {
  if (!(x < 65520.0)) {
    *over = true;
    return 0x7BFF;
  }
  const float f = __double2float_rz(x);
  uint32_t b = __float_as_uint(f);
  if (double(f) != x) b |= 1u;
  _Float16 h = (_Float16)__uint_as_float(b);
  uint16_t r;
  __builtin_memcpy(&r, &h, 2);
  return r;
}

// code = #{k : u >= t_k} over ascending boundaries t[0..K-2] (fp64 compares; the fp32
// boundaries are exact in fp64); the stored centroid of that code comes from the same
// comparisons.
__device__ __forceinline__ int bucketize64(double u, const float *t, const float *c, int K,
                                           double *chat) {
  int code = 0;
  float cv = c[0];
#pragma unroll
  for (int k = 0; k < kMaxCodes - 1; ++k) {
    if (k < K - 1 && u >= double(t[k])) {
      code = k + 1;
      cv = c[k + 1];
    }
  }
  *chat = double(cv);
  return code;
}

// Exchange of a double with lane ^ 1 (kDppXor1) or lane ^ 2 (kDppXor2) inside each group
// of 4 lanes (DPP quad permutation of both halves).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(b)), CTRL, 0xF, 0xF, true));
  const uint32_t hi = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, true));
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ double group4_sum(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  return v;
}

// Unnormalised Sylvester FWHT (H_D x) of one vector spread over the 4 lanes of a group:
// lane q holds chunk A (coordinates q*HC + e) and chunk B (D/2 + q*HC + e), e < HC.
// Coordinate bits below HC are in-lane, the next two select the lane, the top bit the
// chunk.  Cross-lane butterflies use DPP; x_new = partner + s * x with s = +1 on the lower
// lane of a pair and -1 on the upper one (exact sign, one rounding, as a + b / a - b).
template <int D>
__device__ __forceinline__ void fwht_group4(double *x, int q) {
  constexpr int HC = D / 8;
  fwht_regs<HC>(x);
  fwht_regs<HC>(x + HC);
#pragma unroll
  for (int e = 0; e < HC; ++e) {
    const double a = x[e], b = x[HC + e];
    x[e] = a + b;
    x[HC + e] = a - b;
  }
  const double s1 = (q & 1) ? -1.0 : 1.0, s2 = (q & 2) ? -1.0 : 1.0;
  // (eight coordinates at a time: two DPP results per double in flight for all of them
  // would outgrow the registers of three waves per SIMD in the append)
#pragma unroll
  for (int e = 0; e < 2 * HC; ++e) {
    x[e] = fma(s1, x[e], dpp_f64<kDppXor1>(x[e]));
    if ((e & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int e = 0; e < 2 * HC; ++e) {
    x[e] = fma(s2, x[e], dpp_f64<kDppXor2>(x[e]));
    if ((e & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
}

// The 16-byte vectors of N consecutive input elements (off * sizeof(element) a multiple of
// 16), loaded into registers now and converted by raw_to_f64 later, so that the load's
// latency overlaps other work.
template <int DT, int N>
struct RawRow {
  static constexpr int NV = DT == TQ_F32 ? N / 4 : N / 8;
  uint4 v[NV];
};

template <int DT, int N>
__device__ __forceinline__ void load_raw(const void *base, size_t off, RawRow<DT, N> &r) {
  const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const char *>(base) +
                                                   off * (DT == TQ_F32 ? 4 : 2));
#pragma unroll
  for (int i = 0; i < RawRow<DT, N>::NV; ++i) r.v[i] = p[i];
}

template <int DT, int N>
__device__ __forceinline__ void raw_to_f64(const RawRow<DT, N> &r, double *x) {
#pragma unroll
  for (int i = 0; i < RawRow<DT, N>::NV; ++i) {
    const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (DT == TQ_F32) {
        x[4 * i + k] = double(__uint_as_float(w[k]));
      } else if constexpr (DT == TQ_BF16) {
        x[8 * i + 2 * k] = double(__uint_as_float(w[k] << 16));
        x[8 * i + 2 * k + 1] = double(__uint_as_float(w[k] & 0xFFFF0000u));
      } else {
        x[8 * i + 2 * k] = double(f16_bits_to_float(w[k] & 0xFFFFu));
        x[8 * i + 2 * k + 1] = double(f16_bits_to_float(w[k] >> 16));
      }
    }
  }
}

// Sign flip of a double by a mask word that holds the sign bit (bit 31) or nothing.
__device__ __forceinline__ double xor_sign(double v, uint32_t m) {
  return __builtin_bit_cast(double, __builtin_bit_cast(uint64_t, v) ^ (uint64_t(m) << 32));
}

// Sign flips of raw input elements before their conversion: m holds one mask word per
// element for fp32 rows (bit 31) and one per element pair for 2-byte rows (bits 15 and
// 31), 16-byte aligned, in the row's order.
template <int DT, int N>
__device__ __forceinline__ void xor_raw(RawRow<DT, N> &r, const uint32_t *m) {
  const uint4 *mv = reinterpret_cast<const uint4 *>(m);
#pragma unroll
  for (int i = 0; i < RawRow<DT, N>::NV; ++i) {
    const uint4 w = mv[i];
    r.v[i].x ^= w.x;
    r.v[i].y ^= w.y;
    r.v[i].z ^= w.z;
    r.v[i].w ^= w.w;
  }
}

// Bit planes of one lane's coordinates (16-bit chunk A / B halves, bit e = coordinate
// e of the chunk) joined into the plane's dwords and stored: lane q writes the word(s)
// the 4 lanes of its group are assigned.  D = 128: word (q >> 1) of chunk A is
// A(2w) | A(2w + 1) << 16; D = 64: word 0 is A(0) | A(1) << 8 | A(2) << 16 | A(3) << 24.
template <int D>
__device__ __forceinline__ void store_plane(uint32_t hA, uint32_t hB, int q, uint32_t *dst, bool valid) {
  constexpr int HC = D / 8;
  if constexpr (D == 128) {
    const uint32_t ca = hA << (HC * (q & 1)), cb = hB << (HC * (q & 1));
    const uint32_t wa = ca | dpp_u32<kDppXor1>(ca);
    const uint32_t wb = cb | dpp_u32<kDppXor1>(cb);
    // q = 0: word 0, q = 1: word 2, q = 2: word 1, q = 3: word 3
    if (valid) dst[(q & 1) ? 2 + (q >> 1) : (q >> 1)] = (q & 1) ? wb : wa;
  } else {
    uint32_t ca = hA << (HC * q), cb = hB << (HC * q);
    ca |= dpp_u32<kDppXor1>(ca);
    ca |= dpp_u32<kDppXor2>(ca);
    cb |= dpp_u32<kDppXor1>(cb);
    cb |= dpp_u32<kDppXor2>(cb);
    if (valid && q < 2) dst[q] = q ? cb : ca;
  }
}

// ------------------------------------------------------------------ PolarQuant encode
// Code of a level-1 angle psi = atan2(b, a) in [0, 2 pi) (signed zeros taken as +0): the
// number of boundaries k pi / 8 (k = 1..15) at or below psi.  Without the angle itself:
// exact half and quarter turns bring (a, b) into [0, pi / 2) (a > 0, b >= 0, or the zero
// pair), and the three boundaries inside that quarter are the tests b >= a tan(t), with
// tan(pi / 4) = 1 exact.  A test differs from the fp64 angle comparison only for angles
// within a few ulps of a boundary.
__device__ __forceinline__ int polar_code1(double a, double b) {
  a += 0.0;
  b += 0.0;
  int c = 0;
  if (b < 0.0 || (b == 0.0 && a < 0.0)) {   // [pi, 2 pi): angle - pi
    a = -a;
    b = -b;
    c = 8;
  }
  if (a <= 0.0 && b > 0.0) {   // [pi / 2, pi): angle - pi / 2
    const double t = a;
    a = b;
    b = -t;
    c += 4;
  }
  constexpr double kTan1 = 0.41421356237309503;   // tan(pi / 8) = sqrt(2) - 1
  constexpr double kTan3 = 2.4142135623730949;    // tan(3 pi / 8) = sqrt(2) + 1
  if (b > 0.0) c += int(b >= a * kTan1) + int(b >= a) + int(b >= a * kTan3);
  return c;
}

// Code of a higher-level angle psi = atan2(r1, r0) in [0, pi/2] against the level's three
// boundaries, from the squared radii s = r^2 and the boundaries' squared tangents: psi >= t
// is s1 >= s0 tan(t)^2 for s1 > 0, and the angle of r1 = 0 is 0, below every boundary.  No
// radius needs a square root until the norm.
__device__ __forceinline__ int polar_codeh(double s0, double s1, const double *tn2) {
  return s1 > 0.0 ? int(s1 >= s0 * tn2[0]) + int(s1 >= s0 * tn2[1]) + int(s1 >= s0 * tn2[2]) : 0;
}


// The in-chunk levels of HC consecutive coordinates (a power of two): codes stored level
// by level, level 1 first (HC/2 codes), the chunk's top level last (one code at HC - 2);
// returns the chunk's radius.
template <int HC>
__device__ __forceinline__ double polar_encode_chunk(const double *x, const double *ptn, int *cc) {
  double s[HC / 2];   // squared radii
#pragma unroll
  for (int i = 0; i < HC / 2; ++i) {
    cc[i] = polar_code1(x[2 * i], x[2 * i + 1]);
    s[i] = fma(x[2 * i], x[2 * i], x[2 * i + 1] * x[2 * i + 1]);
  }
#pragma unroll
  for (int lv = 2; (1 << lv) <= HC; ++lv) {
    const int n = HC >> lv, base = HC - 2 * n;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      cc[base + i] = polar_codeh(s[2 * i], s[2 * i + 1], ptn + 4 * lv);
      s[i] = s[2 * i] + s[2 * i + 1];
    }
  }
  return s[0];
}

// Reconstruction of a chunk from its radius R and codes, top level down, each radius split
// by the stored fp32 cos and sin of its angle's centroid.
template <int HC>
__device__ __forceinline__ void polar_decode_chunk(double R, const int *cc, const float *pcs, double *y) {
  constexpr int LIN = HC == 16 ? 4 : HC == 8 ? 3 : HC == 4 ? 2 : 1;   // log2 HC
  double r[HC / 2];
  r[0] = R;
#pragma unroll
  for (int lv = 0; (1 << lv) < HC / 2; ++lv) {
    // level LIN - lv has 2^lv codes at HC - 2^(lv+1)
    const int n = 1 << lv, base = HC - 2 * n, lvl = LIN - lv;
#pragma unroll
    for (int i = n - 1; i >= 0; --i) {
      const float *cs = pcs + ((lvl - 1) * kPolarCodes + cc[base + i]) * 2;
      const double rr = r[i];
      r[2 * i] = rr * double(cs[0]);
      r[2 * i + 1] = rr * double(cs[1]);
    }
  }
#pragma unroll
  for (int i = 0; i < HC / 2; ++i) {
    const float *cs = pcs + cc[i] * 2;
    y[2 * i] = r[i] * double(cs[0]);
    y[2 * i + 1] = r[i] * double(cs[1]);
  }
}

// OR a bit field into the record words (fields never straddle a dword).
template <int NW>
__device__ __forceinline__ void put_bits(uint32_t (&w)[NW], int bit, uint32_t val) {
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if ((bit >> 5) == i) w[i] |= val << (bit & 31);
}

// PolarQuant encode of one token spread over a lane group (x as in fwht_group4, in
// H-units: lane q holds chunk A, coordinates HC q .. + HC, and chunk B, D/2 + HC q .. + HC).
// In-chunk levels in registers; the next level pairs the chunks of lanes q, q ^ 1 (codes on
// even lanes), the next those of lanes 0 and 2, the last the two halves (lane 0).  Every
// lane ends with the whole record (3 D / 32 dwords); lane 0's *nh is the norm in H-units.
// With recon, x becomes the reconstruction error x - yhat, yhat built from the fp16 norm.
template <int D>
__device__ __forceinline__ void polar_encode_group(double *x, int q, const CodecPtrs &cp, const double *ptn,
                                                   uint32_t (&w)[3 * D / 32], double *nh, bool recon, double sqrt_b,
                                                   double inv_sqrt_b, uint16_t *n16b, bool *over) {
  constexpr int HC = D / 8, L1 = (HC == 16 ? 4 : 3);   // in-chunk levels
  constexpr int LC1 = L1 + 1, LC2 = L1 + 2, LT = L1 + 3;
  static_assert(HC == 8 || HC == 16, "d = 64 or 128");
  int ccA[HC - 1], ccB[HC - 1];
  // squared radii of the chunks, then of the chunk pairs, blocks and halves
  const double RA = polar_encode_chunk<HC>(x, ptn, ccA), RB = polar_encode_chunk<HC>(x + HC, ptn, ccB);
  // chunk pairs (q, q ^ 1): the even lane's chunk is the lower one
  const double RA1 = dpp_f64<kDppXor1>(RA), RB1 = dpp_f64<kDppXor1>(RB);
  const int cA1 = polar_codeh(RA, RA1, ptn + 4 * LC1);
  const int cB1 = polar_codeh(RB, RB1, ptn + 4 * LC1);
  const double RA2 = RA + RA1, RB2 = RB + RB1;
  // block pairs (lanes 0 and 2), then the halves (lane 0)
  const double RA2p = dpp_f64<kDppXor2>(RA2), RB2p = dpp_f64<kDppXor2>(RB2);
  const int cA2 = polar_codeh(RA2, RA2p, ptn + 4 * LC2);
  const int cB2 = polar_codeh(RB2, RB2p, ptn + 4 * LC2);
  const double RA3 = RA2 + RA2p, RB3 = RB2 + RB2p;
  const int cT = polar_codeh(RA3, RB3, ptn + 4 * LT);
  *nh = sqrt(RA3 + RB3);
  bool ov = false;
  *n16b = f64_to_f16_sat(*nh * inv_sqrt_b, &ov);
  if (q == 0) *over |= ov;
  // record words: level-1 nibbles, then each level's 2-bit codes from bit 2 D
#pragma unroll
  for (int i = 0; i < 3 * D / 32; ++i) w[i] = 0u;
  auto lvl_bit = [](int lv, int j) { return 2 * D + 2 * (D / 2 - (D >> (lv - 1)) + j); };
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int *cc = c ? ccB : ccA;
    const int start = c * (D / 2) + HC * q;   // first coordinate of the chunk
    uint32_t nib = 0u;
#pragma unroll
    for (int i = 0; i < HC / 2; ++i) nib |= uint32_t(cc[i]) << (4 * i);
    put_bits(w, 2 * start, nib);   // code of pair start / 2 + i at bit 4 (start / 2 + i)
#pragma unroll
    for (int lv = 2; (1 << lv) <= HC; ++lv) {
      const int n = HC >> lv, base = HC - 2 * n;
      uint32_t f = 0u;
#pragma unroll
      for (int i = 0; i < n; ++i) f |= uint32_t(cc[base + i]) << (2 * i);
      put_bits(w, lvl_bit(lv, start >> lv), f);
    }
  }
  if ((q & 1) == 0) {
    put_bits(w, lvl_bit(LC1, (HC * q) >> LC1), uint32_t(cA1));
    put_bits(w, lvl_bit(LC1, (D / 2 + HC * q) >> LC1), uint32_t(cB1));
  }
  if (q == 0) {
    put_bits(w, lvl_bit(LC2, 0), uint32_t(cA2));
    put_bits(w, lvl_bit(LC2, 1), uint32_t(cB2));
    put_bits(w, lvl_bit(LT, 0), uint32_t(cT));
  }
#pragma unroll
  for (int i = 0; i < 3 * D / 32; ++i) {
    w[i] |= dpp_u32<kDppXor1>(w[i]);
    w[i] |= dpp_u32<kDppXor2>(w[i]);
  }
  if (!recon) return;
  // reconstruction from the fp16 norm, top down: lane 0 splits the halves and the blocks,
  // lane 2 takes its block radius from lane 0, odd lanes their chunk radius from the even
  const float *pcs = cp.pcs;
  const double nb = double(f16_bits_to_float(*n16b)) * sqrt_b;
  const float *cst = pcs + ((LT - 1) * kPolarCodes + cT) * 2;
  const double hA = nb * double(cst[0]), hB = nb * double(cst[1]);
  const float *csa = pcs + ((LC2 - 1) * kPolarCodes + cA2) * 2, *csb = pcs + ((LC2 - 1) * kPolarCodes + cB2) * 2;
  const double bA0 = hA * double(csa[0]), bA2 = hA * double(csa[1]);
  const double bB0 = hB * double(csb[0]), bB2 = hB * double(csb[1]);
  const double tA2 = dpp_f64<kDppXor2>(bA2), tB2 = dpp_f64<kDppXor2>(bB2);
  const double rA = q == 0 ? bA0 : tA2, rB = q == 0 ? bB0 : tB2;   // meaningful on lanes 0, 2
  const float *c1a = pcs + ((LC1 - 1) * kPolarCodes + cA1) * 2, *c1b = pcs + ((LC1 - 1) * kPolarCodes + cB1) * 2;
  const double oA = rA * double(c1a[0]), pA = rA * double(c1a[1]);
  const double oB = rB * double(c1b[0]), pB = rB * double(c1b[1]);
  const double qA = dpp_f64<kDppXor1>(pA), qB = dpp_f64<kDppXor1>(pB);
  const double RAh = (q & 1) ? qA : oA, RBh = (q & 1) ? qB : oB;
  double y[HC];
  polar_decode_chunk<HC>(RAh, ccA, pcs, y);
#pragma unroll
  for (int e = 0; e < HC; ++e) x[e] -= y[e];
  polar_decode_chunk<HC>(RBh, ccB, pcs, y);
#pragma unroll
  for (int e = 0; e < HC; ++e) x[HC + e] -= y[e];
}

// NSN shift ([NSNQuant] section 1) of one token spread over a lane group as in
// fwht_group4 (x in H-units, sqrt(B) times the rotated coordinates): s1 = ||y|| / sqrt(d)
// is rounded to fp16, then y -= s1 (Pi o) with the unit's stored fp32 Pi o.  The codec's
// norm and direction of what remains are NSN's second normalization.
template <int D>
__device__ __forceinline__ void nsn_shift(double *x, int q, const float *po, double sqrt_b, double inv_sqrt_b,
                                          uint16_t *s1b, bool *over) {
  constexpr int HC = D / 8, H = D / 2, C = 2 * HC;
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < C; ++e) ss = fma(x[e], x[e], ss);
  const double nu = sqrt(group4_sum(ss));   // sqrt(B) ||y||
  *s1b = f64_to_f16_sat(nu * inv_sqrt_b / sqrt(double(D)), over);
  const double s1h = double(f16_bits_to_float(*s1b)) * sqrt_b;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const int j = e < HC ? HC * q + e : H + HC * q + (e - HC);
    x[e] = fma(-s1h, double(po[j]), x[e]);
  }
}

// One workgroup (4 waves) per 64-token window aligned to value tiles; 4 lanes per token.
// Keys: RoPE (fp64 angles from two small LDS tables, the window's rows of 8 tokens and the
// offsets inside a row), the seeded signs D, the unnormalised FWHT H_B, norm, codes and
// residual in fp64, with the 1/sqrt(B) of Pi folded into the norms; the QJL projection
// z = S r runs on fp16 MFMA (v_mfma_f32_32x32x16_f16, split operands) over the window's 64
// residuals.  Values: signs, FWHT, norm and codes in fp64, then the window's codes are
// packed into value tiles.  Three workgroups per CU (at most 168 VGPRs; the PolarQuant
// encode needs more and runs two).
// KK / KV: number of key / value codes when known at compile time (0: from the
// descriptor, a slower loop).  Codes compare the unnormalised coordinate y_j with
// ||y|| * t_k, which is u_j >= t_k up to one rounding.
template <int D, int DT, int KK, int KV, bool POLAR = false>
__global__ __launch_bounds__(256, POLAR ? 2 : 3) void k_quantize_kv(QuantArgs a) {
  constexpr int H = D / 2;
  constexpr int HC = D / 8;     // coordinates per chunk
  constexpr int C = 2 * HC;     // coordinates per lane
  constexpr int W = D / 32;     // dwords per plane
  constexpr int RS = D + 8;     // padded residual row (fp16 elements)
  // RoPE tables: rows of (cos, sin) of the window's angles (p0 + 8 a) theta_j and of the
  // in-group offsets b theta_j (a, b < 8); token slot 8 a + b combines row a of the first
  // with row b of the second.  Entry j = HC q + e sits at (HC + 1) q + e of its row (rows of
  // 4 (HC + 1) entries): the 8 rows times 4 lane chunks a wave reads at once then fall on
  // distinct 16-byte bank groups, two to a group.
  constexpr int RW = 4 * (HC + 1);
  constexpr int ROPE_BYTES = 2 * 8 * RW * 16;
  constexpr int R_BYTES = 2 * 64 * RS * 2;
  constexpr int U_BYTES = ROPE_BYTES > R_BYTES ? ROPE_BYTES : R_BYTES;
  __shared__ __align__(16) unsigned char u_s[U_BYTES];   // RoPE table, later residuals
  // value codes, one byte each; rows padded by a dword so that the 16 tokens of a wave,
  // which write the same columns, land on different banks
  __shared__ __align__(16) uint8_t vcode_s[64][D + 4];
  __shared__ float cb_s[4][kMaxCodes];
  // PolarQuant: the squared tangents of each level's three angle boundaries, [4 level + k]
  __shared__ double ptan_s[POLAR ? 32 : 1];
  // the seeded signs D as sign masks: one word per coordinate (bit 31 set where D_j = -1),
  // then one word per coordinate pair (bits 15 and 31) for 2-byte value rows
  __shared__ __align__(16) uint32_t dsg_s[D + D / 2];
  double2 *ropeA_s = reinterpret_cast<double2 *>(u_s);   // [8][RW]
  double2 *ropeB_s = ropeA_s + 8 * RW;                    // [8][RW]
  _Float16 *r_s = reinterpret_cast<_Float16 *>(u_s);     // [2 parts][64][RS]

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int slot = wv * 16 + (lane >> 2), q = lane & 3;
  const int unit = blockIdx.y;
  const int first_tile = a.start / kValueTile;
  const int p0 = (first_tile + 2 * int(blockIdx.x)) * kValueTile;
  const int p = p0 + slot;
  const int end = a.start + a.n_new;
  const bool valid = p >= a.start && p < end;
  const size_t row = size_t(unit) * size_t(a.n_new) + size_t(valid ? p - a.start : 0);
  bool over = false;

  // the token's key row is requested before the RoPE tables are built, so that its latency
  // overlaps them (the value row is requested once the key codes are done: holding it
  // through the key work would cost the registers of the third wave per SIMD)
  RawRow<DT, HC> rk0, rk1, rv0, rv1;
  if (valid) {
    load_raw<DT, HC>(a.k, row * D + HC * q, rk0);
    load_raw<DT, HC>(a.k, row * D + H + HC * q, rk1);
  }

  if (tid < kMaxCodes) {
    cb_s[0][tid] = a.cp.ck[tid];
    cb_s[1][tid] = a.cp.tk[tid];
    cb_s[2][tid] = a.cp.cv[tid];
    cb_s[3][tid] = a.cp.tv[tid];
  }
  if constexpr (POLAR) {
    constexpr int L = D == 128 ? 7 : 6;
    if (tid < 32) {
      const int lv = tid >> 2, k = tid & 3;
      const double tn = lv >= 2 && lv <= L && k < 3 ? tan(a.cp.pt[(lv - 1) * kPolarCodes + k]) : 0.0;
      ptan_s[tid] = tn * tn;
    }
  }
  const bool use_rope = a.rope_base != 0.0f;
  if (use_rope && tid < 2 * H) {
    // threads j < H: row a of table A by the rotation recurrence from sincos(p0 theta_j) in
    // steps of 8 theta_j (three doublings of theta_j); threads H + j: table B from (1, 0)
    // in steps of theta_j.  Doublings, products and the recurrences involve no argument
    // reduction; the angles match the fp64 ones to about 1e-14.
    const int j = tid % H;
    const int col = (j / HC) * (HC + 1) + j % HC;
    const double cd = a.rf.c[j], sd = a.rf.s[j];
    double c, s, cs, ss;
    double2 *tab;
    if (tid < H) {
      sincos(double(p0) * a.rf.theta[j], &s, &c);
      cs = cd;
      ss = sd;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const double c2 = cs * cs - ss * ss;
        ss = 2.0 * cs * ss;
        cs = c2;
      }
      tab = ropeA_s;
    } else {
      c = 1.0;
      s = 0.0;
      cs = cd;
      ss = sd;
      tab = ropeB_s;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tab[i * RW + col] = make_double2(c, s);
      const double cn = c * cs - s * ss;
      s = s * cs + c * ss;
      c = cn;
    }
  }
  for (int i = tid; i < D + D / 2; i += 256) {
    if (i < D) {
      dsg_s[i] = a.cp.D[i] < 0.0f ? 0x80000000u : 0u;
    } else {
      const int k = 2 * (i - D);
      dsg_s[i] = (a.cp.D[k] < 0.0f ? 0x8000u : 0u) | (a.cp.D[k + 1] < 0.0f ? 0x80000000u : 0u);
    }
  }
  __syncthreads();

  const double sqrt_b = a.sqrt_b, inv_sqrt_b = a.inv_sqrt_b;
  uint32_t *rec = reinterpret_cast<uint32_t *>(a.ch.kbits + (size_t(unit) * a.capacity + (valid ? p : 0)) * a.ch.kbytes);

  // ------------------------------------------------------------ keys
  double x[C];
  float r32[C];   // the key residual rounded to fp32, for the QJL projection
  if (valid) {
    raw_to_f64<DT, HC>(rk0, x);
    raw_to_f64<DT, HC>(rk1, x + HC);
  } else {
#pragma unroll
    for (int e = 0; e < C; ++e) x[e] = 0.0;
  }
  if (use_rope) {
    const double2 *ta = ropeA_s + (slot >> 3) * RW + (HC + 1) * q;
    const double2 *tb = ropeB_s + (slot & 7) * RW + (HC + 1) * q;
#pragma unroll
    for (int e = 0; e < HC; ++e) {
      const double2 u = ta[e], w = tb[e];
      const double c = u.x * w.x - u.y * w.y, sn = u.y * w.x + u.x * w.y;
      const double x0 = x[e], x1 = x[HC + e];
      x[e] = x0 * c - x1 * sn;
      x[HC + e] = x0 * sn + x1 * c;
    }
  }
  {
    // the signs D after the rotary step (sign flips of the fp64 high words)
    const uint4 *ma = reinterpret_cast<const uint4 *>(dsg_s + HC * q);
    const uint4 *mb = reinterpret_cast<const uint4 *>(dsg_s + H + HC * q);
#pragma unroll
    for (int i = 0; i < HC / 4; ++i) {
      const uint4 wa = ma[i], wb = mb[i];
      x[4 * i] = xor_sign(x[4 * i], wa.x);
      x[4 * i + 1] = xor_sign(x[4 * i + 1], wa.y);
      x[4 * i + 2] = xor_sign(x[4 * i + 2], wa.z);
      x[4 * i + 3] = xor_sign(x[4 * i + 3], wa.w);
      x[HC + 4 * i] = xor_sign(x[HC + 4 * i], wb.x);
      x[HC + 4 * i + 1] = xor_sign(x[HC + 4 * i + 1], wb.y);
      x[HC + 4 * i + 2] = xor_sign(x[HC + 4 * i + 2], wb.z);
      x[HC + 4 * i + 3] = xor_sign(x[HC + 4 * i + 3], wb.w);
    }
  }
  fwht_group4<D>(x, q);
  uint16_t ks1b = 0;
  if (a.ch.nsn) nsn_shift<D>(x, q, a.ch.nsn + size_t(unit) * 4 * D + 2 * D, sqrt_b, inv_sqrt_b, &ks1b, &over);
  if constexpr (POLAR) {
    // PolarQuant: angle codes of the rotated key, the reconstruction error left in x
    uint32_t w[3 * D / 32];
    double nh;
    uint16_t n16b;
    polar_encode_group<D>(x, q, a.cp, ptan_s, w, &nh, true, sqrt_b, inv_sqrt_b, &n16b, &over);
#pragma unroll
    for (int i = 0; i < 3 * D / 32; ++i)
      if ((i & 3) == q && valid) rec[i] = w[i];
    double rr = 0.0;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      rr = fma(x[e], x[e], rr);
      r32[e] = float(x[e]);
    }
    const uint16_t rn16b = f64_to_f16_sat(sqrt(group4_sum(rr)) * inv_sqrt_b, &over);
    if (valid && q == 0) a.ch.knorm[size_t(unit) * a.capacity + p] = uint32_t(n16b) | (uint32_t(rn16b) << 16);
  } else {
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < C; ++e) ss = fma(x[e], x[e], ss);
    const double nu = sqrt(group4_sum(ss));           // ||H D x'|| = sqrt(B) ||y||
    const uint16_t n16b = f64_to_f16_sat(nu * inv_sqrt_b, &over);
    const double nb16 = double(f16_bits_to_float(n16b)) * sqrt_b;   // fp16(n) in H-units
    const double sc = nu > 0.0 ? nu : 1.0;
    // planes that can be non-zero: log2(KK) when the code count is fixed, else up to 4
    constexpr int NP = KK == 2 ? 1 : KK == 4 ? 2 : KK == 8 ? 3 : 4;
    uint32_t hA[4] = {0u, 0u, 0u, 0u}, hB[4] = {0u, 0u, 0u, 0u};
    double rr = 0.0;
    if constexpr (KK == 4) {
      // The stored codebook is odd (c[3 - k] = -c[k], t = {-s, 0, s} / sc).  With a = |x|
      // and d = a - s, the code's upper bit is [x >= 0] and its lower bit
      // [x >= copysign(s, x)]: the sign bits of x and of d agree.  The centroid is
      // +-outer when d >= 0, else +-inner, with the sign of x.  The sign bits come from
      // the fp64 high words and are shifted into the plane words (top coordinate first);
      // an exact tie a = s falls to the sign of d's zero, on a decision boundary.  A zero
      // coordinate can carry a negative sign only in a zero vector, fixed after the loop.
      const double s1 = sc * double(cb_s[1][2]);
      const double wo = nb16 * double(cb_s[0][3]), wi = nb16 * double(cb_s[0][2]);
      const uint64_t uo = uint64_t(__double_as_longlong(wo)), ui = uint64_t(__double_as_longlong(wi));
      const uint32_t olo = uint32_t(uo), ohi = uint32_t(uo >> 32), ilo = uint32_t(ui), ihi = uint32_t(ui >> 32);
      uint32_t sxA = 0u, sxB = 0u, sgA = 0u, sgB = 0u;   // sign bits of x; sign(x) xor sign(d)
      auto code2 = [&](int i, uint32_t &sx, uint32_t &sg) {
        double xe = x[i];
        const uint32_t xh = uint32_t(uint64_t(__double_as_longlong(xe)) >> 32);
        const uint32_t dh = uint32_t(uint64_t(__double_as_longlong(fabs(xe) - s1)) >> 32);
        sx = __builtin_amdgcn_alignbit(sx, xh, 31);        // sx << 1 | sign(x)
        sg = __builtin_amdgcn_alignbit(sg, xh ^ dh, 31);   // sg << 1 | (sign(x) != sign(d))
        const uint32_t m = uint32_t(int32_t(dh) >> 31);    // all ones: the inner centroid
        const uint32_t wl = (ilo & m) | (olo & ~m);
        const uint32_t wh = (((ihi & m) | (ohi & ~m)) & 0x7FFFFFFFu) | (xh & 0x80000000u);
        xe -= __longlong_as_double(int64_t((uint64_t(wh) << 32) | wl));
        rr = fma(xe, xe, rr);
        float rf = float(xe);
        asm volatile("" : "+v"(rf));   // convert here: the fp64 residual dies at once
        r32[i] = rf;
      };
#pragma unroll
      for (int e = HC - 1; e >= 0; --e) {
        code2(e, sxA, sgA);
        code2(HC + e, sxB, sgB);
        // in order, four coordinates at a time: interleaving the whole loop holds more
        // residuals than the registers of three waves per SIMD allow
        if ((e & 1) == 0) __builtin_amdgcn_sched_barrier(0);
      }
      constexpr uint32_t hm = HC >= 32 ? 0xFFFFFFFFu : (1u << HC) - 1u;
      // a zero vector takes code 2 (the first positive centroid) everywhere
      const uint32_t zm = nu > 0.0 ? 0u : 0xFFFFFFFFu;
      hA[0] = ~sgA & hm & ~zm;
      hB[0] = ~sgB & hm & ~zm;
      hA[1] = (~sxA | zm) & hm;
      hB[1] = (~sxB | zm) & hm;
    } else if constexpr (KK > 0) {
      double sk[KK - 1], wk[KK];
#pragma unroll
      for (int k = 0; k < KK - 1; ++k) sk[k] = sc * double(cb_s[1][k]);
#pragma unroll
      for (int k = 0; k < KK; ++k) wk[k] = nb16 * double(cb_s[0][k]);
#pragma unroll
      for (int e = 0; e < C; ++e) {
        int code = 0;
        double w = wk[0];
#pragma unroll
        for (int k = 0; k < KK - 1; ++k) {
          const bool ge = x[e] >= sk[k];
          code += ge ? 1 : 0;
          w = ge ? wk[k + 1] : w;
        }
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          const uint32_t bit = uint32_t((code >> pp) & 1) << (e % HC);
          if (e < HC) hA[pp] |= bit; else hB[pp] |= bit;
        }
        x[e] -= w;
        rr = fma(x[e], x[e], rr);
        r32[e] = float(x[e]);
      }
    } else {
      const int K = 1 << a.bits_k;
#pragma unroll
      for (int e = 0; e < C; ++e) {
        int code = 0;
        for (int k = 0; k < K - 1; ++k) code += x[e] >= sc * double(cb_s[1][k]) ? 1 : 0;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint32_t bit = uint32_t((code >> pp) & 1) << (e % HC);
          if (e < HC) hA[pp] |= bit; else hB[pp] |= bit;
        }
        x[e] -= nb16 * double(cb_s[0][code]);
        rr = fma(x[e], x[e], rr);
        r32[e] = float(x[e]);
      }
    }
    const uint16_t rn16b = f64_to_f16_sat(sqrt(group4_sum(rr)) * inv_sqrt_b, &over);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
      if (pp < a.bits_k) store_plane<D>(hA[pp], hB[pp], q, rec + pp * W, valid);
    if (valid && q == 0) {
      const uint32_t nw = uint32_t(n16b) | (uint32_t(rn16b) << 16);
      if (a.ch.nsn)
        reinterpret_cast<uint2 *>(a.ch.knorm)[size_t(unit) * a.capacity + p] = make_uint2(nw, uint32_t(ks1b));
      else
        a.ch.knorm[size_t(unit) * a.capacity + p] = nw;
    }
  }   // scalar codes
  // the value row is requested now: the key doubles are dead, and its latency overlaps the
  // barrier and the residual staging
  if (valid && a.bits_v > 0) {
    load_raw<DT, HC>(a.v, row * D + HC * q, rv0);
    load_raw<DT, HC>(a.v, row * D + H + HC * q, rv1);
  }
  __syncthreads();   // every wave is done with the RoPE table before residuals overwrite it
  {
    // residual r_H = H D x' - fp16(n) sqrt(B) c = sqrt(B) r (same signs of S r), rounded
    // to fp32, scaled by a power of two that brings the token's largest |r_j| into
    // [2^13, 2^14) (the signs of S r do not change), and split into fp16 hi + lo parts
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < C; ++e) amax = fmaxf(amax, fabsf(r32[e]));
    amax = fmaxf(amax, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(amax))));
    amax = fmaxf(amax, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(amax))));
    const float rscale = amax > 0.0f ? __builtin_ldexpf(1.0f, 14 - __builtin_amdgcn_frexp_expf(amax)) : 1.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      v8h part[2][HC / 8];
#pragma unroll
      for (int e = 0; e < HC; ++e) {
        const float rr = r32[c * HC + e] * rscale;
        const _Float16 hv = _Float16(rr);
        part[0][e / 8][e % 8] = hv;
        part[1][e / 8][e % 8] = _Float16(rr - float(hv));
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        v8h *dst = reinterpret_cast<v8h *>(r_s + (k * 64 + slot) * RS + c * H + HC * q);
#pragma unroll
        for (int i = 0; i < HC / 8; ++i) dst[i] = part[k][i];
      }
    }
  }

  // ------------------------------------------------------------ values
  if (a.bits_v > 0) {
    if (valid) {
      // the signs D on the raw elements (no rotary step on values)
      constexpr bool w32 = DT == TQ_F32;
      xor_raw<DT, HC>(rv0, w32 ? dsg_s + HC * q : dsg_s + D + HC * q / 2);
      xor_raw<DT, HC>(rv1, w32 ? dsg_s + H + HC * q : dsg_s + D + (H + HC * q) / 2);
      raw_to_f64<DT, HC>(rv0, x);
      raw_to_f64<DT, HC>(rv1, x + HC);
    } else {
#pragma unroll
      for (int e = 0; e < C; ++e) x[e] = 0.0;
    }
    fwht_group4<D>(x, q);
    uint16_t vs1b = 0;
    if (a.ch.nsn) nsn_shift<D>(x, q, a.ch.nsn + size_t(unit) * 4 * D + 3 * D, sqrt_b, inv_sqrt_b, &vs1b, &over);
    if constexpr (POLAR) {
      // PolarQuant values: token records of 3 D / 8 bytes in the value region
      uint32_t w[3 * D / 32];
      double nh;
      uint16_t n16b;
      polar_encode_group<D>(x, q, a.cp, ptan_s, w, &nh, false, sqrt_b, inv_sqrt_b, &n16b, &over);
      uint32_t *vrec = reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.ch.vcodes) +
                                                    (size_t(unit) * a.capacity + (valid ? p : 0)) * (3 * D / 8));
#pragma unroll
      for (int i = 0; i < 3 * D / 32; ++i)
        if ((i & 3) == q && valid) vrec[i] = w[i];
      if (valid && q == 0) a.ch.vnorm[size_t(unit) * a.capacity + p] = n16b;
    } else {
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < C; ++e) ss = fma(x[e], x[e], ss);
    const double nu = sqrt(group4_sum(ss));
    const uint16_t n16b = f64_to_f16_sat(nu * inv_sqrt_b, &over);
    const double sc = nu > 0.0 ? nu : 1.0;
    uint32_t cw[C / 4];
#pragma unroll
    for (int i = 0; i < C / 4; ++i) cw[i] = 0u;
    if constexpr (KV > 0) {
      // odd codebook: the code counts the boundaries at or below x; with the h - 1 positive
      // thresholds s_i = sc t_{h-1+i} it follows from |x| against them and the sign of x
      constexpr int h = KV / 2;
      double sp[h > 1 ? h - 1 : 1];
#pragma unroll
      for (int i = 1; i < h; ++i) sp[i - 1] = sc * double(cb_s[3][h - 1 + i]);
#pragma unroll
      for (int e = 0; e < C; ++e) {
        // nb = the thresholds above |x|: the code is nb for x < 0 and 2h - 1 - nb =
        // nb ^ (2h - 1) for x >= 0 (h a power of two); sign bits from the fp64 high words
        const uint32_t xh = uint32_t(uint64_t(__double_as_longlong(x[e])) >> 32);
        const double ax = fabs(x[e]);
        uint32_t nb = 0u;
#pragma unroll
        for (int i = 1; i < h; ++i) nb += ax < sp[i - 1] ? 1u : 0u;
        const uint32_t code = nb ^ ((2u * uint32_t(h) - 1u) & ~uint32_t(int32_t(xh) >> 31));
        cw[e / 4] |= code << (8 * (e % 4));
      }
      // a zero vector (whose coordinates may carry negative zeros) takes code h everywhere
      if (!(nu > 0.0)) {
#pragma unroll
        for (int i = 0; i < C / 4; ++i) cw[i] = uint32_t(h) * 0x01010101u;
      }
    } else {
      const int K = 1 << a.bits_v;
#pragma unroll
      for (int e = 0; e < C; ++e) {
        int code = 0;
        for (int k = 0; k < K - 1; ++k) code += x[e] >= sc * double(cb_s[3][k]) ? 1 : 0;
        cw[e / 4] |= uint32_t(code) << (8 * (e % 4));
      }
    }
    uint32_t *va = reinterpret_cast<uint32_t *>(&vcode_s[slot][HC * q]);
    uint32_t *vb = reinterpret_cast<uint32_t *>(&vcode_s[slot][H + HC * q]);
#pragma unroll
    for (int i = 0; i < HC / 4; ++i) {
      va[i] = cw[i];
      vb[i] = cw[HC / 4 + i];
    }
    if (valid && q == 0) {
      if (a.ch.nsn)
        reinterpret_cast<uint32_t *>(a.ch.vnorm)[size_t(unit) * a.capacity + p] = uint32_t(n16b) | (uint32_t(vs1b) << 16);
      else
        a.ch.vnorm[size_t(unit) * a.capacity + p] = n16b;
    }
    }   // scalar codes
  }
  __syncthreads();

  // ------------------------------------------------------------ QJL signs: z = S r
  // z^T[32 rows x 64 tokens] per 32-row block of S, both 32-token halves sharing the S
  // operand, on fp16 MFMA (v_mfma_f32_32x32x16_f16): S in fp16 parts hi + mid (the codec's
  // third part, lo, is not needed here), the scaled residual in two (hi, lo).  The three
  // products hi.hi, mid.hi and hi.lo leave out lo.hi and mid.lo (each at most 2^-22 of
  // the leading term) and lo.lo (2^-33), and the residual's own split costs 2^-23: z to
  // a few 2^-22 relative per term, a few 1e-7 of |r| over the d-term sum, so a sign can
  // move only for |z| that close to zero (the parity rule's band is 1e-6 |r|).
  // Step i contracts k = 16 i + 8 (lane / 32) + 0..7 on both operands.
  {
    const int mt_n = a.m / 32;
    const int half = lane >> 5;
    for (int mt = wv; mt < mt_n; mt += 4) {
      v16f acc0 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      v16f acc1 = acc0;
      const size_t srow = size_t(32 * mt + (lane & 31)) * D + 8 * half;
      const _Float16 *r0 = r_s + (lane & 31) * RS + 8 * half;
      const _Float16 *r1 = r0 + 32 * RS;
      // Every step's S slices are requested at once, so their L2 latency is paid once per
      // block of rows (fetched one step ahead, the loop waited on them at every step).  The
      // scheduling barrier keeps the loads here: hoisted into the value work their 64 VGPRs
      // spill.  (Requested before the barrier above they were slower.)
      constexpr int NS = D / 16;
      v8h sv[NS][2];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int k = 0; k < 2; ++k) sv[i][k] = *reinterpret_cast<const v8h *>(a.cp.Sh[k] + srow + 16 * i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        v8h ra[2], rb[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          ra[k] = *reinterpret_cast<const v8h *>(r0 + k * 64 * RS + 16 * i);
          rb[k] = *reinterpret_cast<const v8h *>(r1 + k * 64 * RS + 16 * i);
        }
#define TQ_SR(A, B)                                                             \
  acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sv[i][A], ra[B], acc0, 0, 0, 0); \
  acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sv[i][A], rb[B], acc1, 0, 0, 0)
        TQ_SR(0, 1);
        TQ_SR(1, 0);
        TQ_SR(0, 0);
#undef TQ_SR
      }
      // lane holds rows 8 (r / 4) + 4 (lane / 32) + r % 4 of token column lane % 32
      uint32_t b0 = 0u, b1 = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int sh = 8 * (r >> 2) + 4 * half + (r & 3);
        b0 |= uint32_t(acc0[r] >= 0.0f) << sh;
        b1 |= uint32_t(acc1[r] >= 0.0f) << sh;
      }
      b0 |= __shfl_xor(b0, 32, 64);
      b1 |= __shfl_xor(b1, 32, 64);
      const int ts = lane & 31;
      const int pt = p0 + ts + (half ? 32 : 0);
      if (pt >= a.start && pt < end) {
        uint32_t *rt = reinterpret_cast<uint32_t *>(a.ch.kbits + (size_t(unit) * a.capacity + pt) * a.ch.kbytes);
        rt[a.bits_k * W + mt] = half ? b1 : b0;
      }
    }
  }

  // ------------------------------------------------------------ value tiles
  if (!POLAR && a.bits_v > 0) {
    // one (tile, coordinate) word group per thread; tokens outside the written range
    // keep their previous bits
    const int bv = a.bits_v;
    const uint32_t mask = (1u << bv) - 1u;
    for (int wi = tid; wi < 2 * D; wi += 256) {
      const int tloc = wi / D, j = wi % D;
      const int tile = first_tile + 2 * int(blockIdx.x) + tloc;
      const int tstart = tile * kValueTile;
      if (tstart >= end || tile >= a.ch.tiles) continue;
      uint32_t *wp = a.ch.vcodes + ((size_t(unit) * a.ch.tiles + tile) * D + j) * bv;
      const bool full = tstart >= a.start && tstart + kValueTile <= end;
      if constexpr (KV > 0) {
        // whole tile with a fixed code width: every shift is a constant
        constexpr int BV = KV == 2 ? 1 : KV == 4 ? 2 : KV == 8 ? 3 : 4;
        if (full) {
          uint32_t fw[BV];
#pragma unroll
          for (int k = 0; k < BV; ++k) fw[k] = 0u;
#pragma unroll
          for (int i = 0; i < kValueTile; ++i) {
            const uint32_t code = vcode_s[tloc * kValueTile + i][j];
            const int bit = BV * i;
            fw[bit >> 5] |= code << (bit & 31);
            if ((bit & 31) + BV > 32) fw[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
          }
#pragma unroll
          for (int k = 0; k < BV; ++k) wp[k] = fw[k];
          continue;
        }
      }
      uint32_t word[4] = {0u, 0u, 0u, 0u};
      if (!full)
        for (int qq = 0; qq < bv; ++qq) word[qq] = wp[qq];
      for (int i = 0; i < kValueTile; ++i) {
        const int t = tstart + i;
        if (t < a.start || t >= end) continue;
        const uint32_t code = vcode_s[tloc * kValueTile + i][j];
        const int bit = bv * i;
        const int qq = bit >> 5, sh = bit & 31;
        word[qq] = (word[qq] & ~(mask << sh)) | (code << sh);
        if (sh + bv > 32) {
          const int s2 = 32 - sh;
          word[qq + 1] = (word[qq + 1] & ~(mask >> s2)) | (code >> s2);
        }
      }
      for (int qq = 0; qq < bv; ++qq) wp[qq] = word[qq];
    }
  }
  if (over) atomicOr(a.ch.flags, 1u);
}

// Database vectors of large d (keys only, no RoPE): one wave per vector for the fp64
// rotation, norm, codes and residual (lane l holds, in each Hadamard block b, the E
// consecutive coordinates b*B + E*l + e); the workgroup's 16 residuals then go through
// z = S r on MFMA with S streamed from L2.  Eight waves, two per SIMD, so that one wave's
// S loads are in flight while the other multiplies.  For d <= 1536 a workgroup takes 24
// vectors, whose residuals fit in LDS as fp16 hi + lo parts, and the products run on fp16
// MFMA (v_mfma_f32_32x32x16_f16: S hi.r hi + S mid.r hi + S hi.r lo, as in the append);
// at d = 2048 it takes 16 vectors with fp32 residuals on v_mfma_f32_16x16x4f32.
constexpr int kDbWaves = 8;
__host__ __device__ constexpr int db_group(int c) { return c <= 24 ? 24 : 16; }
__host__ __device__ constexpr size_t db_lds_bytes(int c) {
  return c <= 24 ? size_t(2) * db_group(c) * (64 * c + 8) * 2 : size_t(db_group(c)) * (64 * c + 4) * 4;
}

template <int C, int E, int DT>
__global__ __launch_bounds__(64 * kDbWaves) void k_quantize_db(QuantArgs a) {
  constexpr int NB = C / E;
  constexpr int B = 64 * E;
  constexpr int Dm = C * 64;
  constexpr bool F16 = C <= 24;
  constexpr int GV = db_group(C);
  constexpr int RS = Dm + 4;        // fp32 residual row
  constexpr int RS16 = Dm + 8;      // fp16 residual row
  static_assert(GV % kDbWaves == 0, "whole vectors per wave");
  extern __shared__ float r_s[];   // fp32: [GV][RS]; fp16: [2 parts][GV][RS16]
  _Float16 *r16 = reinterpret_cast<_Float16 *>(r_s);
  __shared__ float cb_s[2][kMaxCodes];
  // (the wave index is wave-uniform: what derives from it, the S rows' buffer resource
  // included, lives in scalar registers)
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.y;
  const int g0 = a.start + int(blockIdx.x) * GV;
  const int end = a.start + a.n_new;
  if (tid < kMaxCodes) {
    cb_s[0][tid] = a.cp.ck[tid];
    cb_s[1][tid] = a.cp.tk[tid];
  }
  __syncthreads();
  const double inv_sqrt_b = 1.0 / sqrt(double(B));
  const int K = 1 << a.bits_k;
  const int dbytes = Dm / 8;
  // the rows of both of this wave's vectors (and the signs D) are requested up front, so
  // that one memory latency, not one per vector, precedes the encodes; elements as fp32,
  // exact for every input type (at d >= 1536 one row ahead: more would not fit beside the
  // encode's registers)
  constexpr int NVW = GV / kDbWaves, NPRE = C >= 24 ? 1 : NVW;
  float xr[NPRE][C], dj[C];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < E; ++e) dj[b * E + e] = a.cp.D[b * B + E * lane + e];
  auto load_row = [&](int v, float *dst) {
    const int p = g0 + wv + kDbWaves * v;
    const size_t row = size_t(unit) * size_t(a.n_new) + size_t(p < end ? p - a.start : 0);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < E; ++e)
        dst[b * E + e] = p < end ? float(load_d<DT>(a.k, row * Dm + b * B + E * lane + e)) : 0.0f;
  };
#pragma unroll
  for (int v = 0; v < NPRE; ++v) load_row(v, xr[v]);
#pragma unroll
  for (int v = 0; v < NVW; ++v) {
    const int vi = wv + kDbWaves * v;
    const int p = g0 + vi;
    const bool valid = p < end;
    double x[C];
#pragma unroll
    for (int c = 0; c < C; ++c) x[c] = double(xr[v % NPRE][c]) * double(dj[c]);
    if (v + NPRE < NVW) load_row(v + NPRE, xr[v % NPRE]);   // the slot just read: the next row it serves
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      fwht_regs<E>(x + b * E);
#pragma unroll
      for (int dist = 1; dist < 64; dist <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const double o = __shfl_xor(x[b * E + e], dist, 64);
          x[b * E + e] = (lane & dist) ? (o - x[b * E + e]) : (x[b * E + e] + o);
        }
      }
    }
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      x[c] *= inv_sqrt_b;
      ss += x[c] * x[c];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const double n = sqrt(ss);
    bool over = false;
    const uint16_t n16b = f64_to_f16_sat(n, &over);
    const double n16 = double(f16_bits_to_float(n16b));
    const double inv = n > 0.0 ? 1.0 / n : 0.0;
    uint32_t planebits[4][NB];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int b = 0; b < NB; ++b) planebits[pp][b] = 0u;
    double rr = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      double chat;
      const int code = bucketize64(x[c] * inv, cb_s[1], cb_s[0], K, &chat);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) planebits[pp][c / E] |= uint32_t((code >> pp) & 1) << (c % E);
      x[c] -= n16 * chat;
      rr += x[c] * x[c];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rr += __shfl_xor(rr, o, 64);
    const uint16_t rn16b = f64_to_f16_sat(sqrt(rr), &over);
    uint8_t *rec = a.ch.kbits + (size_t(unit) * a.capacity + (valid ? p : 0)) * a.ch.kbytes;
    for (int pp = 0; pp < a.bits_k; ++pp) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t v = planebits[pp][b];
        if (E >= 8) {
#pragma unroll
          for (int by = 0; by < E / 8; ++by)
            if (valid) rec[pp * dbytes + (b * B + E * lane) / 8 + by] = uint8_t(v >> (8 * by));
        } else {
          uint32_t acc = v << ((E * lane) & 7);
#pragma unroll
          for (int o = 1; o < 8 / E; o <<= 1) acc |= __shfl_xor(acc, o, 64);
          if (valid && ((E * lane) & 7) == 0) rec[pp * dbytes + (b * B + E * lane) / 8] = uint8_t(acc);
        }
      }
    }
    if constexpr (F16) {
      // the residual rounded to fp32, scaled by a power of two that brings its largest
      // |r_j| into [2^13, 2^14) (the signs of S r do not change), split into fp16 hi + lo
      float amax = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) amax = fmaxf(amax, fabsf(float(x[c])));
      amax = wave_max(amax);
      const float rscale = amax > 0.0f ? __builtin_ldexpf(1.0f, 14 - __builtin_amdgcn_frexp_expf(amax)) : 1.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float rv = float(x[b * E + e]) * rscale;
          const _Float16 hv = _Float16(rv);
          r16[size_t(vi) * RS16 + b * B + E * lane + e] = hv;
          r16[size_t(GV + vi) * RS16 + b * B + E * lane + e] = _Float16(rv - float(hv));
        }
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) r_s[vi * RS + b * B + E * lane + e] = float(x[b * E + e]);
    }
    if (valid && lane == 0) {
      a.ch.knorm[size_t(unit) * a.capacity + p] = uint32_t(n16b) | (uint32_t(rn16b) << 16);
      if (over) atomicOr(a.ch.flags, 1u);
    }
  }
  __syncthreads();
  if constexpr (F16) {
    // z^T[32 rows x 32 columns] per 32-row tile of S, the group's GV vectors in columns
    // 0..GV-1 (the other columns read vector GV-1 again and are not stored), on
    // v_mfma_f32_32x32x16_f16: S in its fp16 parts hi + mid, the scaled residual in hi + lo,
    // and the products hi.hi, mid.hi and hi.lo (each term left out is at most 2^-22 of the
    // leading one).  Step i contracts k = 16 i + 8 (lane / 32) + 0..7 on both operands.
    // The S parts of the next kDbPf16 steps are in flight while a step is multiplied
    // (buffer loads, for the same reason as in the fp32 form below).
    constexpr int kDbPf16 = 4;
    constexpr int NS = Dm / 16;
    static_assert(NS % kDbPf16 == 0, "whole prefetch rounds");
    const int mt_n = a.m / 32;
    const int half = lane >> 5, col = lane & 31;
    const _Float16 *rh = r16 + size_t(col < GV ? col : GV - 1) * RS16 + 8 * half;
    const _Float16 *rl = rh + size_t(GV) * RS16;
    const int soff = (col * Dm + 8 * half) * 2;   // bytes: the lane's row and k half
    for (int mt = wv; mt < mt_n; mt += kDbWaves) {
      v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const __amdgpu_buffer_rsrc_t sr0 = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<_Float16 *>(a.cp.Sh[0] + size_t(32 * mt) * Dm), 0, 32 * Dm * 2, 0x00020000);
      const __amdgpu_buffer_rsrc_t sr1 = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<_Float16 *>(a.cp.Sh[1] + size_t(32 * mt) * Dm), 0, 32 * Dm * 2, 0x00020000);
      v8h sb[kDbPf16][2];
#pragma unroll
      for (int f = 0; f < kDbPf16; ++f) {
        sb[f][0] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(sr0, soff + 32 * f, 0, 0));
        sb[f][1] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(sr1, soff + 32 * f, 0, 0));
      }
      for (int i0 = 0; i0 < NS; i0 += kDbPf16) {
        v8h cur[kDbPf16][2];
#pragma unroll
        for (int f = 0; f < kDbPf16; ++f) {
          cur[f][0] = sb[f][0];
          cur[f][1] = sb[f][1];
        }
        __builtin_amdgcn_sched_barrier(0);
        if (i0 + kDbPf16 < NS) {
#pragma unroll
          for (int f = 0; f < kDbPf16; ++f) {
            const int o = soff + 32 * (i0 + kDbPf16 + f);
            sb[f][0] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(sr0, o, 0, 0));
            sb[f][1] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(sr1, o, 0, 0));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < kDbPf16; ++f) {
          const int i = i0 + f;
          const v8h ra = *reinterpret_cast<const v8h *>(rh + 16 * i);
          const v8h rb = *reinterpret_cast<const v8h *>(rl + 16 * i);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[f][0], rb, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[f][1], ra, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[f][0], ra, acc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane holds rows 8 (r / 4) + 4 (lane / 32) + r % 4 of the tile, column lane % 32
      uint32_t bits = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) bits |= uint32_t(acc[r] >= 0.0f) << (8 * (r >> 2) + 4 * half + (r & 3));
      bits |= __shfl_xor(bits, 32, 64);
      const int p = g0 + col;
      if (half == 0 && col < GV && p < end) {
        uint8_t *rec = a.ch.kbits + (size_t(unit) * a.capacity + p) * a.ch.kbytes;
        *reinterpret_cast<uint32_t *>(rec + a.bits_k * dbytes + 4 * mt) = bits;
      }
    }
  } else {
    // z^T[m x 16] = S[m x Dm] . R^T[Dm x 16], 16-row output tiles spread over the waves.
    // The contraction runs in chunks of 16 coordinates; in chunk c, MFMA i takes from lane
    // group g = lane / 16 the coordinate 16 c + 4 g + i (any order of k serves, A and B
    // using the same), so a lane reads S and R as one 16-byte vector per chunk.  The S
    // vectors of the next kDbPf chunks are in flight while a chunk is multiplied: S comes
    // from L2 / the last-level cache, and two waves per SIMD cannot hide that latency by
    // themselves.
    constexpr int kDbPf = 8;
    constexpr int NCK = Dm / 16;
    static_assert(NCK % kDbPf == 0, "whole prefetch rounds");
    const int mt_n = a.m / 16;
    for (int mt = wv; mt < mt_n; mt += kDbWaves) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      // (buffer loads: S is read-only, and from plain loads the compiler would load each
      // vector again where it is used instead of keeping the early load's result)
      const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float *>(a.cp.S + size_t(16 * mt) * Dm), 0, 16 * Dm * 4, 0x00020000);
      const int soff = ((lane & 15) * Dm + 4 * (lane >> 4)) * 4;   // bytes: the lane's row, group
      auto sload = [&](int c) {
        return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(srs, soff + 64 * c, 0, 0));
      };
      const float4 *rrow = reinterpret_cast<const float4 *>(r_s + (lane & 15) * RS) + (lane >> 4);
      v4f sb[kDbPf];
  #pragma unroll
      for (int f = 0; f < kDbPf; ++f) sb[f] = sload(f);
      for (int c0 = 0; c0 < NCK; c0 += kDbPf) {
        // this round's vectors, then the next round's requested in one block (the scheduling
        // barriers keep the compiler from sinking each load to its use)
        v4f cur[kDbPf];
  #pragma unroll
        for (int f = 0; f < kDbPf; ++f) cur[f] = sb[f];
        __builtin_amdgcn_sched_barrier(0);
        if (c0 + kDbPf < NCK) {
  #pragma unroll
          for (int f = 0; f < kDbPf; ++f) sb[f] = sload(c0 + kDbPf + f);
        }
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int f = 0; f < kDbPf; ++f) {
          const float4 rv = rrow[4 * (c0 + f)];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[f][0], rv.x, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[f][1], rv.y, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[f][2], rv.z, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[f][3], rv.w, acc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane holds outputs 16 mt + 4 (lane / 16) + r of vector lane % 16
      uint32_t bits = 0u;
  #pragma unroll
      for (int r = 0; r < 4; ++r) bits |= uint32_t(acc[r] >= 0.0f) << (4 * (lane >> 4) + r);
      bits |= __shfl_xor(bits, 16, 64);
      bits |= __shfl_xor(bits, 32, 64);
      const int p = g0 + (lane & 15);
      if (lane < 16 && p < end) {
        uint8_t *rec = a.ch.kbits + (size_t(unit) * a.capacity + p) * a.ch.kbytes;
        uint16_t *sb = reinterpret_cast<uint16_t *>(rec + a.bits_k * dbytes + 2 * mt);
        *sb = uint16_t(bits);
      }
    }
  }
}

// ------------------------------------------------------------------ decode (split-K)
struct DecodeArgs {
  CodecPtrs cp;
  const uint8_t *kbits;
  const uint32_t *knorm;
  const uint32_t *vcodes;
  const uint16_t *vnorm;
  int kbytes, tiles, capacity, bits_k, bits_v, m;
  int kv_heads, q_heads, G, length, splits, chunk;
  float scale;
  const float *qp;   // prepared queries, row stride qstride
  int qstride;
  float *part;       // [B*Hq][splits][d + 2]
  float *scores;     // optional [B][Hq][score_stride]
  int score_stride;  // length, or length + the full-precision window's tokens
};

constexpr int kDecThreads = 256;
constexpr int kMaxG = 16;

// One block per (unit, split).  Tokens of the split are processed in tiles of 256: one
// thread per token computes the G scores from the packed key (dequantized planes
// against q_rot, sign bits against S q_rot), the block keeps an online softmax, and
// threads then switch to one coordinate each to accumulate p * n_v * c_v[code].
template <int D>
__global__ __launch_bounds__(kDecThreads) void k_decode_split(DecodeArgs a) {
  const int unit = blockIdx.x;       // b * kv_heads + g
  const int split = blockIdx.y;
  const int tid = threadIdx.x;
  const int b = unit / a.kv_heads, g = unit % a.kv_heads;
  const int G = a.G;
  const int hq0 = g * G;             // first q-head of this kv-head
  extern __shared__ float sm[];
  float *qr_s = sm;                          // [G][D]
  float *sq_s = qr_s + kMaxG * D;            // [G][m]
  float *p_s = sq_s + kMaxG * a.m;           // [G][256]
  float *red = p_s + kMaxG * kDecThreads;    // [4 waves][G]
  __shared__ float ck_s[kMaxCodes], cv_s[kMaxCodes];
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int h = i / D, j = i % D;
    qr_s[h * D + j] = a.qp[size_t(b * a.q_heads + hq0 + h) * a.qstride + j];
  }
  for (int i = tid; i < G * a.m; i += kDecThreads) {
    const int h = i / a.m, j = i % a.m;
    sq_s[h * a.m + j] = a.qp[size_t(b * a.q_heads + hq0 + h) * a.qstride + D + j];
  }
  if (tid < kMaxCodes) {
    ck_s[tid] = a.cp.ck[tid];
    cv_s[tid] = a.cp.cv[tid];
  }
  __syncthreads();
  float sumsq[kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h)
    sumsq[h] = (h < G) ? a.qp[size_t(b * a.q_heads + hq0 + h) * a.qstride + D + a.m + 1] : 0.0f;

  const int t_begin = split * a.chunk;
  const int t_end = min(a.length, t_begin + a.chunk);
  float M[kMaxG], Lsum[kMaxG], acc[kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    M[h] = -INFINITY;
    Lsum[h] = 0.0f;
    acc[h] = 0.0f;
  }
  const int j_own = tid % D;            // coordinate owned in the value phase
  const int part_id = tid / D;          // token sub-range owned in the value phase
  const int parts = kDecThreads / D;
  const int kw = D / 32;
  const int bv = a.bits_v;
  const size_t ubase = size_t(unit) * a.capacity;

  for (int t0 = t_begin; t0 < t_end; t0 += kDecThreads) {
    const int t = t0 + tid;
    float lam[kMaxG];
    if (t < t_end) {
      const uint32_t *rec = reinterpret_cast<const uint32_t *>(a.kbits + (ubase + t) * a.kbytes);
      const uint32_t nr = a.knorm[ubase + t];
      const float n16 = f16_bits_to_float(nr & 0xFFFF), rn16 = f16_bits_to_float(nr >> 16);
      float dot[kMaxG], qj[kMaxG];
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) dot[h] = qj[h] = 0.0f;
      for (int w = 0; w < kw; ++w) {
        uint32_t pl[4] = {0u, 0u, 0u, 0u};
        for (int pp = 0; pp < a.bits_k; ++pp) pl[pp] = rec[pp * kw + w];
        for (int i = 0; i < 32; ++i) {
          int code = 0;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) code |= int((pl[pp] >> i) & 1u) << pp;
          const float kh = ck_s[code];
          const int j = w * 32 + i;
#pragma unroll
          for (int h = 0; h < kMaxG; ++h)
            if (h < G) dot[h] = fmaf(qr_s[h * D + j], kh, dot[h]);
        }
      }
      for (int w = 0; w < a.m / 32; ++w) {
        const uint32_t sb = rec[a.bits_k * kw + w];
        for (int i = 0; i < 32; ++i) {
          const int ii = w * 32 + i;
          if ((sb >> i) & 1u) {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h)
              if (h < G) qj[h] += sq_s[h * a.m + ii];
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
          // <sq, 2 s - 1> = 2 sum_{s=1} sq - sum sq
          const float score = n16 * dot[h] + rn16 * a.cp.qjl_scale * (2.0f * qj[h] - sumsq[h]);
          if (a.scores) a.scores[(size_t(b) * a.q_heads + hq0 + h) * a.score_stride + t] = score;
          lam[h] = a.scale * score;
        } else {
          lam[h] = -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) lam[h] = -INFINITY;
    }
    // tile maxima per head
    const int wv = tid >> 6;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        const float mx = wave_max(lam[h]);
        if ((tid & 63) == 0) red[wv * kMaxG + h] = mx;
      }
    }
    __syncthreads();
    float alpha[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float mx = red[h];
        for (int w = 1; w < kDecThreads / 64; ++w) mx = fmaxf(mx, red[w * kMaxG + h]);
        const float Mn = fmaxf(M[h], mx);
        alpha[h] = (M[h] == -INFINITY) ? 0.0f : __expf(M[h] - Mn);
        M[h] = Mn;
        const float pv = (lam[h] == -INFINITY) ? 0.0f : __expf(lam[h] - Mn);
        Lsum[h] = Lsum[h] * alpha[h] + pv;
        const float vn = (t < t_end) ? f16_bits_to_float(a.vnorm[ubase + t]) : 0.0f;
        p_s[h * kDecThreads + tid] = pv * vn;
      } else {
        alpha[h] = 1.0f;
      }
    }
    __syncthreads();
    // value phase: coordinate j_own, tokens of sub-range part_id
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) acc[h] *= alpha[h];
    const int per = kDecThreads / parts;
    const int tl0 = part_id * per;
    for (int tl = tl0; tl < tl0 + per; ++tl) {
      const int tt = t0 + tl;
      if (tt >= t_end) break;
      const int tile = tt / kValueTile, slot = tt % kValueTile;
      const uint32_t *wp = a.vcodes + ((size_t(unit) * a.tiles + tile) * D + j_own) * bv;
      const int bit = bv * slot;
      const int q = bit >> 5, s = bit & 31;
      uint32_t code = wp[q] >> s;
      if (s + bv > 32) code |= wp[q + 1] << (32 - s);
      code &= (1u << bv) - 1u;
      const float vh = cv_s[code];
#pragma unroll
      for (int h = 0; h < kMaxG; ++h)
        if (h < G) acc[h] = fmaf(p_s[h * kDecThreads + tl], vh, acc[h]);
    }
    __syncthreads();
  }
  // reduce: Lsum over all threads, acc over token sub-ranges
  const int wv = tid >> 6;
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      const float s = wave_sum(Lsum[h]);
      if ((tid & 63) == 0) red[wv * kMaxG + h] = s;
    }
  }
  __syncthreads();
  float *accs = p_s;  // reuse: [parts][G][D]
#pragma unroll
  for (int h = 0; h < kMaxG; ++h)
    if (h < G) accs[(part_id * G + h) * D + j_own] = acc[h];
  __syncthreads();
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int h = i / D, j = i % D;
    float v = 0.0f;
    for (int pp = 0; pp < parts; ++pp) v += accs[(pp * G + h) * D + j];
    float *o = a.part + ((size_t(b * a.q_heads + hq0 + h) * a.splits) + split) * (D + 2);
    o[j] = v;
    if (j == 0) {
      float L = 0.0f;
      for (int w = 0; w < kDecThreads / 64; ++w) L += red[w * kMaxG + h];
      o[D] = M[h];
      o[D + 1] = L;
    }
  }
}

// ------------------------------------------------------------------ decode (MFMA path)
// For bits_k = 2, m = d, bits_v = 3, d in {64, 128} and up to 8 q-heads per kv-head.
//
// Keys: with c[code] = c0 + (c1 - c0) b0 + (c2 - c0) b1 (symmetric 2-bit codebook),
//   score = n (c0 sum q + (c1-c0) q.b0 + (c2-c0) q.b1) + ||r|| sqrt(pi/2)/m (2 sq.s - sum sq).
// The vectors (c1-c0) q and (c2-c0) q (one shared exponent) and sq = S q are written as
// 32-bit fixed point in four signed int8 digits (rows digit * 8 + head of a 32-row A
// operand), and the packed bit planes of 32 tokens are the B operand of
// v_mfma_i32_32x32x32_i8.  A B byte is one plane bit masked in place within its nibble,
// b 2^e with e in 0..3 (no shifts per bit), and the query element it meets carries 2^-e
// in its digits, which leaves it 29 to 32 bits.  The products are exact integers, both
// planes accumulate into one sum, and the digit sums recombine in-lane.  That precision
// keeps every query element near its fp32 value even when a few outlier coordinates set
// the exponent.
// Values: p n_v is split into fp16 hi + lo rows (16 rows for 8 heads) and multiplied on
// v_mfma_f32_16x16x32_f16 with the fp16 centroids of 32 tokens, looked up 4 codes at a
// time from a 4096-entry LDS table (the stored centroids are fp16 values, so this B is
// exact).  Accumulation is fp32 in the rotated basis; the combine applies Pi^T.
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kMfmaMaxG = 8;
constexpr int kQpackCoef = 8;   // floats per head: k0..k4, padding
constexpr int kQpackVecs = 5;   // digit-row vector slots: up to 4 key-plane weight vectors, S q
constexpr int kSqVec = 4;       // slot of the S q vector
constexpr int kDigits = 4;      // int8 digits per value: 32-bit fixed point, rows digit * 8 + head

// Per unit: [kQpackVecs][32 rows][2 halves][d/32 chunks][16 bytes] of int8 digits, then
// [8 heads][kQpackCoef] floats.
__host__ __device__ constexpr size_t qpack_unit_bytes(int d) { return size_t(kQpackVecs) * 32 * 2 * (d / 32) * 16 + kMfmaMaxG * kQpackCoef * 4; }

struct MfmaArgs {
  const uint8_t *kbits;
  const uint32_t *knorm;
  const uint32_t *vcodes;
  const uint16_t *vnorm;
  const float *cv;
  const uint8_t *qpack;
  float *part;
  float *scores;
  const float *nsn;   // NSN caches: per unit [o_K, o_V, Pi o_K, Pi o_V]; else null
  int kbytes, tiles, capacity, length, chunk, splits, kv_heads, q_heads, G;
  int score_stride;   // row stride of scores: length, or length + the window's tokens
  float scale_log2, inv_scale_log2;
};

__device__ __forceinline__ uint32_t f16bits(float x) {
  _Float16 h = (_Float16)x;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// Max over each group of 32 lanes with DPP row operations: within rows of 16 (quad
// swaps, half-row mirror, row mirror), then row_bcast15 folds row 0 into row 1 and row 2
// into row 3; the group maxima end up in lanes 31 and 63.  The floats are compared as
// integers under the order-preserving map x -> x ^ ((x >> 31) & 0x7fffffff), which keeps
// the reduction free of NaN canonicalization and lets the moves fold into v_max_i32_dpp.
__device__ __forceinline__ int f2ord(float v) {
  const int x = __float_as_int(v);
  return x ^ ((x >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float ord2f(int x) { return __int_as_float(x ^ ((x >> 31) & 0x7fffffff)); }

__device__ __forceinline__ int dpp_max32_tail(int x) {
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false));
  return x;
}

__device__ __forceinline__ float sum32(float v) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Tail shared by the two query-prep kernels, run by all 256 threads once q_rot (qs) and
// sq (sqs) are complete, thread i < d having written sqs[i] itself: the fp32 row, the
// sums, the two fixed-point exponents, the score coefficients and the int8 digit rows.
// nsn: the cache's NSN means (null for a plain cache); the head's coefficient 2 is then
// <q_rot, Pi o_K>, the score of the keys' mean per unit of s1.
__device__ __forceinline__ void qprep_tail(const float *qs, const float *sqs, int d, int m,
                                           const CodecPtrs &cp, float *o, float (*red)[4], int tid,
                                           int lane, int wv, int b, int g, int h, int G,
                                           int kv_heads, int bits_k, uint8_t *qpack, const float *nsn,
                                           bool l16 = false) {
  // fp32 rows and sums; maxima for the fixed-point scaling (the two plane vectors
  // (c1 - c0) q and (c2 - c0) q share one exponent, set by the larger weight)
  // Key-plane weights of the odd codebook: c[code] = c0 + sum_p pw[p] bit_p(code).  For
  // 3-bit codes, c = a0 s0 + a1 s1 + a2 s2 + a3 s0 s1 s2 (s = 2 bit - 1; the only odd
  // multilinear terms), and s0 s1 s2 = 2 (b0 ^ b1 ^ b2) - 1, so the parity of the three
  // bits is a fourth plane: pw = 2 a.  All planes share one exponent (the largest weight).
  float pw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int np = 0;
  if (bits_k == 1) {
    np = 1;
    pw[0] = cp.ck[1] - cp.ck[0];
  } else if (bits_k == 2) {
    np = 2;
    pw[0] = cp.ck[1] - cp.ck[0];
    pw[1] = cp.ck[2] - cp.ck[0];
  } else if (bits_k == 3) {
    np = 4;
    const float c4 = cp.ck[4], c5 = cp.ck[5], c6 = cp.ck[6], c7 = cp.ck[7];
    pw[0] = 0.5f * (c7 - c6 + c5 - c4);
    pw[1] = 0.5f * (c7 + c6 - c5 - c4);
    pw[2] = 0.5f * (c7 + c6 + c5 + c4);
    pw[3] = 0.5f * (c7 - c6 - c5 + c4);
  }
  const float wmax = fmaxf(fmaxf(fabsf(pw[0]), fabsf(pw[1])), fmaxf(fabsf(pw[2]), fabsf(pw[3])));
  float s0 = 0.0f, s1 = 0.0f, m0 = 0.0f, m1 = 0.0f, sb = 0.0f;
  const float *pok = nsn ? nsn + size_t(b * kv_heads + g) * 4 * d + 2 * d : nullptr;
  for (int j = tid; j < d; j += 256) {
    o[j] = qs[j];
    s0 += qs[j];
    m0 = fmaxf(m0, fabsf(qs[j]) * wmax);
    if (pok) sb = fmaf(qs[j], pok[j], sb);
  }
  for (int i = tid; i < m; i += 256) {
    o[d + i] = sqs[i];
    s1 += sqs[i];
    m1 = fmaxf(m1, fabsf(sqs[i]));
  }
  s0 = wave_sum(s0);
  s1 = wave_sum(s1);
  m0 = wave_max(m0);
  m1 = wave_max(m1);
  sb = wave_sum(sb);
  if (lane == 0) {
    red[0][wv] = s0;
    red[1][wv] = s1;
    red[2][wv] = m0;
    red[3][wv] = m1;
    red[4][wv] = sb;
  }
  __syncthreads();
  // every thread derives the two fixed-point exponents from the wave maxima
  int sexp[2];
  for (int v = 0; v < 2; ++v) {
    const float mx = fmaxf(fmaxf(red[2 + v][0], red[2 + v][1]), fmaxf(red[2 + v][2], red[2 + v][3]));
    int e = 0;
    if (mx > 0.0f) {
      int ex;
      frexpf(mx, &ex);   // mx < 2^ex
      e = 30 - ex;   // |x| 2^e < 2^30: four signed int8 digits
    }
    sexp[v] = e;
  }
  if (tid == 0) {
    const float S0 = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const float S1 = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    o[d + m] = S0;
    o[d + m + 1] = S1;
    if (qpack) {
      float *coef = reinterpret_cast<float *>(qpack + size_t(b * kv_heads + g) * qpack_unit_bytes(d) +
                                              size_t(kQpackVecs) * 32 * 2 * (d / 32) * 16);
      // the decode kernel forms a digit sum as hi + lo 2^-16 (= sum / 65536)
      const float iq = ldexpf(1.0f, 16 - sexp[0]), is = ldexpf(1.0f, 16 - sexp[1]);
      const float c0 = cp.ck[0];
      float *k = coef + h * kQpackCoef;
      k[0] = c0 * S0;
      k[1] = iq;
      k[2] = (red[4][0] + red[4][1]) + (red[4][2] + red[4][3]);   // NSN: <q_rot, Pi o_K>
      k[3] = 2.0f * cp.qjl_scale * is;
      k[4] = cp.qjl_scale * S1;
      k[5] = k[6] = k[7] = 0.0f;
      if (h == 0)
        for (int hz = G; hz < kMfmaMaxG; ++hz)
          for (int i = 0; i < kQpackCoef; ++i) coef[hz * kQpackCoef + i] = 0.0f;
    }
  }
  if (!qpack) return;
  const int nch = d / 32;
  uint32_t *o32 = reinterpret_cast<uint32_t *>(qpack + size_t(b * kv_heads + g) * qpack_unit_bytes(d));
  // this head's rows digit * 8 + h of the np plane vectors and the S q vector (slot
  // kSqVec): [slot][digit][half][chunk][e]
  const int ndw = (np + 1) * kDigits * 2 * nch * 4;
  for (int i = tid; i < ndw; i += 256) {
    const int e = i & 3, c = (i >> 2) % nch, half = (i / (4 * nch)) & 1;
    const int digit = (i / (8 * nch)) % kDigits, vi = i / (8 * kDigits * nch);
    const bool is_sq = vi == np;
    const int v = is_sq ? kSqVec : vi;
    const float *src = is_sq ? sqs : qs;
    const float wgt = is_sq ? 1.0f : pw[vi];
    // the decode kernel keeps bit e of each nibble in place (token byte = b 2^e), so the
    // query element that meets it carries the factor 2^-e
    const int ex = sexp[is_sq ? 1 : 0] - e;
    uint32_t word = 0u;
#pragma unroll
    for (int beta = 0; beta < 4; ++beta) {
      const int j = 32 * (half * (d / 64) + (c >> 1)) + 8 * beta + 4 * (c & 1) + e;
      const int xi = int(rintf(ldexpf(src[j] * wgt, ex)));
      const int d0 = ((xi + 128) & 255) - 128;
      const int x1 = (xi - d0) >> 8;
      const int d1 = ((x1 + 128) & 255) - 128;
      const int x2 = (x1 - d1) >> 8;
      const int d2 = ((x2 + 128) & 255) - 128;
      const int d3 = (x2 - d2) >> 8;
      const int dg = digit == 0 ? d0 : (digit == 1 ? d1 : (digit == 2 ? d2 : d3));
      word |= uint32_t(dg & 255) << (8 * beta);
    }
    // l16 (d = 128, G <= 4): the A operand of the 16-row key-score MFMA, rows 4 head + digit,
    // the same 16-byte fragments at [slot][row][dword kg = 2 half + c / 2][nibble c % 2]
    const int row = digit * 8 + h;
    const int oi = l16 ? ((((v * 16 + 4 * h + digit) * 4 + 2 * half + (c >> 1)) * 2 + (c & 1)) * 4 + e)
                       : ((((v * 32 + row) * 2 + half) * nch + c) * 4 + e);
    o32[oi] = word;
  }
  if (h == 0 && l16 && G < 4) {
    // rows 4 head + digit of the absent heads G <= head < 4, 32 words each
    const int nrow = kDigits * (4 - G);
    for (int i = tid; i < kQpackVecs * nrow * 32; i += 256) {
      const int w = i & 31, ri = (i >> 5) % nrow, v = i / (32 * nrow);
      o32[(v * 16 + 4 * (G + ri / kDigits) + ri % kDigits) * 32 + w] = 0u;
    }
  }
  if (h == 0 && !l16 && G < 8) {
    // rows (digit, head) of the absent heads h >= G
    const int nrow = kDigits * (8 - G);
    for (int i = tid; i < kQpackVecs * nrow * 2 * nch * 4; i += 256) {
      const int e = i & 3, c = (i >> 2) % nch, half = (i / (4 * nch)) & 1;
      const int ri = (i / (8 * nch)) % nrow, v = i / (8 * nch * nrow);   // every slot
      const int row = (ri / (8 - G)) * 8 + G + ri % (8 - G);
      o32[(((v * 32 + row) * 2 + half) * nch + c) * 4 + e] = 0u;
    }
  }
}

// Query preparation for the MFMA path, one block per (batch, q-head) row: q_rot =
// Pi RoPE(q, q_pos) (LDS FWHT), sq = S q_rot, their sums (kept in the fp32 rows for the
// plain path as well), then the head's three int8 digit rows of the key-score A operand
// and its score coefficients.  The first head of each kv-head also clears the unused
// rows (digit 3, heads >= G) of its unit.
__global__ __launch_bounds__(256) void k_qprep_pack(const void *q, int dtype, int d, int m,
                                                    int q_pos, float rope_base, CodecPtrs cp,
                                                    float *qrows, int qstride, int q_heads,
                                                    int G, int bits_k, uint8_t *qpack, const float *nsn) {
  extern __shared__ float qs[];   // d floats (q_rot), m floats (sq), max(1024, m) partial sums
  float *sqs = qs + d;
  __shared__ float red[5][4];
  const int rowi = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = rowi / q_heads, hq = rowi % q_heads;
  const int g = hq / G, h = hq % G;
  const int kv_heads = q_heads / G;
  const size_t base = size_t(rowi) * d;
  const int hh = d / 2;
  if (rope_base != 0.0f) {
    for (int j = tid; j < hh; j += 256) {
      const double theta = pow(double(rope_base), -2.0 * double(j) / double(d));
      double s, c;
      sincos(double(q_pos) * theta, &s, &c);
      const float x0 = load_elem(q, base + j, dtype), x1 = load_elem(q, base + j + hh, dtype);
      qs[j] = (x0 * float(c) - x1 * float(s)) * cp.D[j];
      qs[j + hh] = (x0 * float(s) + x1 * float(c)) * cp.D[j + hh];
    }
  } else {
    for (int j = tid; j < d; j += 256) qs[j] = load_elem(q, base + j, dtype) * cp.D[j];
  }
  __syncthreads();
  const int B = cp.block;
  if (B == d && d >= 64 && d <= 256) {
    // one wave: d / 64 consecutive values per lane, the first stages in registers, the
    // rest across lanes, and the 1/sqrt(B) scale on the way out
    if (tid < 64) {
      float x[4];
      const int E = d / 64;
      for (int e = 0; e < E; ++e) x[e] = qs[E * tid + e];
      for (int st = 1; st < E; st <<= 1)
        for (int e = 0; e < E; ++e)
          if (!(e & st)) {
            const float u = x[e], v = x[e + st];
            x[e] = u + v;
            x[e + st] = u - v;
          }
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1)
        for (int e = 0; e < E; ++e) {
          const float pv = __shfl_xor(x[e], msk, 64);
          x[e] = (tid & msk) ? pv - x[e] : x[e] + pv;
        }
      for (int e = 0; e < E; ++e) qs[E * tid + e] = x[e] * cp.inv_sqrt_block;
    }
  } else {
    for (int st = 1; st < B; st <<= 1) {
      for (int k = tid; k < d / 2; k += 256) {
        const int blk = k / (B / 2), kk = k % (B / 2);
        const int i = blk * B + (kk / st) * 2 * st + (kk % st);
        const float x0 = qs[i], x1 = qs[i + st];
        qs[i] = x0 + x1;
        qs[i + st] = x0 - x1;
      }
      __syncthreads();
    }
    for (int j = tid; j < d; j += 256) qs[j] *= cp.inv_sqrt_block;
  }
  __syncthreads();
  // sq = S q_rot: each thread takes 4 consecutive outputs (a float4 of a row of S^T) over
  // one of `slices` slices of the inner dimension; the slices are summed through LDS
  if (m > 0) {
    const int g4 = m / 4;
    int slices = 1;                                 // largest power of two <= 256 / g4
    while (2 * slices * g4 <= 256) slices *= 2;
    const int jl = d / slices;
    float *part = sqs + m;                          // [slices][m] (shared with the final sq)
    for (int og = tid % g4 + (tid / g4 >= slices ? g4 : 0), sl = tid / g4; og < g4; og += 256) {
      const int j0 = (slices > 1 ? sl : 0) * jl, j1 = slices > 1 ? j0 + jl : d;
      float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 *st = reinterpret_cast<const float4 *>(cp.ST) + og;
#pragma unroll 8
      for (int j = j0; j < j1; ++j) {
        const float4 sv = st[size_t(j) * g4];
        const float x = qs[j];
        z.x = fmaf(sv.x, x, z.x);
        z.y = fmaf(sv.y, x, z.y);
        z.z = fmaf(sv.z, x, z.z);
        z.w = fmaf(sv.w, x, z.w);
      }
      float *o4 = part + (slices > 1 ? sl : 0) * m + 4 * og;
      o4[0] = z.x;
      o4[1] = z.y;
      o4[2] = z.z;
      o4[3] = z.w;
      if (slices > 1) break;
    }
    __syncthreads();
    for (int i = tid; i < m; i += 256) {
      float z = 0.0f;
      for (int sl = 0; sl < slices; ++sl) z += part[sl * m + i];
      sqs[i] = z;
    }
  }
  __syncthreads();
  qprep_tail(qs, sqs, d, m, cp, qrows + size_t(rowi) * qstride, red, tid, lane, wv, b, g, h, G, kv_heads, bits_k, qpack,
             nsn);
}

// Query preparation for d = m in {64, 128} with Hadamard block d (the decode MFMA path):
// the same arithmetic as k_qprep_pack in the same order, but every global load (this
// thread's slice of S^T, the query pair and its signs) is issued before the fp64 RoPE
// angle is computed, the FWHT runs in one wave's registers, and one barrier less.
template <int D>
__global__ __launch_bounds__(256) void k_qprep_fast(const void *q, int dtype, QueryRope qr,
                                                    CodecPtrs cp, float *qrows, int qstride,
                                                    int q_heads, int G, int bits_k, uint8_t *qpack,
                                                    const float *nsn, int l16) {
  constexpr int H2 = D / 2, G4 = D / 4, SL = 256 / G4, JL = D / SL, E = D / 64;
  __shared__ float qs[D], sqs[D], part[SL * D];
  __shared__ float red[5][4];
  const int rowi = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = rowi / q_heads, hq = rowi % q_heads;
  const int g = hq / G, h = hq % G;
  const int kv_heads = q_heads / G;
  const size_t base = size_t(rowi) * D;
  const int og = tid % G4, sl = tid / G4;
  float4 sv[JL];
  const float4 *st = reinterpret_cast<const float4 *>(cp.ST) + og;
#pragma unroll
  for (int jj = 0; jj < JL; ++jj) sv[jj] = st[size_t(sl * JL + jj) * G4];
  if (tid < H2) {
    const int j = tid;
    const float x0 = load_elem(q, base + j, dtype), x1 = load_elem(q, base + j + H2, dtype);
    const float d0 = cp.D[j], d1 = cp.D[j + H2];
    const float c = qr.c[j], sn = qr.s[j];
    qs[j] = (x0 * c - x1 * sn) * d0;
    qs[j + H2] = (x0 * sn + x1 * c) * d1;
  }
  __syncthreads();
  if (tid < 64) {
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = qs[E * tid + e];
#pragma unroll
    for (int s = 1; s < E; s <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (!(e & s)) {
          const float u = x[e], v = x[e + s];
          x[e] = u + v;
          x[e + s] = u - v;
        }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float pv = __shfl_xor(x[e], msk, 64);
        x[e] = (tid & msk) ? pv - x[e] : x[e] + pv;
      }
#pragma unroll
    for (int e = 0; e < E; ++e) qs[E * tid + e] = x[e] * cp.inv_sqrt_block;
  }
  __syncthreads();
  {
    float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int jj = 0; jj < JL; ++jj) {
      const float x = qs[sl * JL + jj];
      z.x = fmaf(sv[jj].x, x, z.x);
      z.y = fmaf(sv[jj].y, x, z.y);
      z.z = fmaf(sv[jj].z, x, z.z);
      z.w = fmaf(sv[jj].w, x, z.w);
    }
    float *o4 = part + sl * D + 4 * og;
    o4[0] = z.x;
    o4[1] = z.y;
    o4[2] = z.z;
    o4[3] = z.w;
  }
  __syncthreads();
  if (tid < D) {
    float z = 0.0f;
#pragma unroll
    for (int s = 0; s < SL; ++s) z += part[s * D + tid];
    sqs[tid] = z;
  }
  qprep_tail(qs, sqs, D, D, cp, qrows + size_t(rowi) * qstride, red, tid, lane, wv, b, g, h, G, kv_heads, bits_k, qpack,
             nsn, l16 != 0);
}

// LDS-staged split-K decode.  Each wave streams its tiles through a ring of kRing LDS
// slots filled by direct global->LDS loads, kRing - 1 tiles ahead of the one it computes,
// so the packed bytes in flight do not cost registers.  Per tile: int8 MFMA key scores,
// online softmax, fp16 MFMA value accumulation.  Blocks of kDecWaves waves,
// kDecBlocksPerCU of them resident per CU.
constexpr int kRing = 3;
constexpr int kDecWaves = 8;
constexpr int kDecBlocksPerCU = 1;

// Reads of a ring slot written by direct global->LDS loads are inline assembly, each
// block waiting for its own results (lgkmcnt(0)), because the compiler would otherwise
// wait for every direct-to-LDS load in flight (including the prefetches into the other
// slots) before any LDS read; the ring's own vmcnt waits order them instead.
template <int D, int KBITS, bool NSN = false>
struct LdsGeom {
  static constexpr int KB = (KBITS + 1) * D / 8;   // key record bytes (KBITS planes + m = d sign bits)
  static constexpr int KT = 32 * KB;       // key bytes per 32-token tile
  static constexpr int VT = 12 * D;        // value-code bytes per 32-token tile
  // direct-to-LDS loads land lane-contiguously for 4- and 16-byte sizes: key records whose
  // size is a multiple of 16 and all value tiles go as 16-byte chunks, other key records
  // (24 bytes at d = 64 with 2-bit codes: not 16-byte aligned in general) as dwords
  static constexpr int KCH = KB % 16 == 0 ? 16 : 4;   // key chunk bytes
  static constexpr int NK = (KT / KCH + 63) / 64; // key DMA instructions
  static constexpr int NV = (VT / 16 + 63) / 64;  // value DMA instructions
  static constexpr int NDMA = NK + NV + 2;        // + key norms + value norms
  // key norm records: 4 bytes, or 8 with NSN ({n, |r|, s1, 0}); value norm records: 2
  // bytes (read as 17 dwords from the dword at or below the tile's first), or 4 with NSN
  static constexpr int KNR = NSN ? 8 : 4;
  static constexpr int KN = KT + VT;       // offset of the 32 key norms
  static constexpr int VN = KN + 32 * KNR; // offset of the value norms
  static constexpr int SLOT = VN + (NSN ? 128 : 80);
};

template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  // s_waitcnt with vmcnt = N and expcnt / lgkmcnt left at their "no wait" maxima (gfx9
  // encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14])
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// a where mask bits are set, else b (a bitwise select: the compiler keeps it a v_bfi
// rather than turning a choice between array elements into an indexed stack access)
__device__ __forceinline__ float pick_bits(uint32_t mask, float a, float b) {
  return __uint_as_float((mask & __float_as_uint(a)) | (~mask & __float_as_uint(b)));
}

// KBITS = key code bits (1, 2 or 3).  The key score's code term is a weighted sum of
// NP 0/1 planes: the code bits, and for 3-bit codes also their parity (odd codebook).
// NSN: the cache's tokens carry fp16 s1 next to the norms; a key's score gains
// s1 <q, o_K> (the query coefficient 2) and a value's share of s1 Pi o_V is summed per head
// next to the softmax sum and added to the accumulator at the end.
template <int D, int KBITS, bool NSN, bool SCORES>
__global__ __launch_bounds__(64 * kDecWaves, kDecBlocksPerCU) void k_decode_lds(MfmaArgs a) {
  // The body is device code only (its local lambdas call device builtins); the host pass
  // needs nothing but the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using Gm = LdsGeom<D, KBITS, NSN>;
  constexpr int NCH = D / 32, NT = D / 16, NW = kDecWaves, NTH = 64 * NW, R = kRing;
  constexpr int NP = KBITS == 3 ? 4 : KBITS;
  static_assert(KBITS >= 1 && KBITS <= 3, "key planes");
  // The 32 KB LUT has the largest alignment, so it is laid out first, at address 0: a
  // lookup's address is then its masked index itself, with no base to add per lookup.
  // (Separate arrays, not one struct: the compiler then knows that the direct-to-LDS loads
  // into the ring cannot alias the LUT or the other arrays, and waits for none of them.)
  __shared__ __align__(32768) uint2 lut[4096];
  __shared__ __align__(16) uint8_t ring[R][NW][Gm::SLOT];
  __shared__ __align__(16) _Float16 pt_s[NW][16][40];
  __shared__ __align__(16) float coef_s[2][5][4];
  __shared__ float red_s[NW][3][kMfmaMaxG];
  static_assert(NW * 16 * D * 4 <= int(sizeof(ring)), "the waves' accumulators fit in the ring for the merge");

  // the wave index goes through readfirstlane so that everything derived from it (token
  // ranges, tile addresses) is known to be wave-uniform and lives in scalar registers
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / a.kv_heads, g = unit % a.kv_heads;
  const int hq0 = g * a.G;
  for (int i = tid; i < 4096; i += NTH) {
    const uint32_t h0 = f16bits(a.cv[i & 7]), h1 = f16bits(a.cv[(i >> 3) & 7]);
    const uint32_t h2 = f16bits(a.cv[(i >> 6) & 7]), h3 = f16bits(a.cv[(i >> 9) & 7]);
    lut[i] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
  }
  const uint8_t *qpk = a.qpack + size_t(unit) * qpack_unit_bytes(D);
  const float *coef = reinterpret_cast<const float *>(qpk + size_t(kQpackVecs) * 32 * 2 * NCH * 16);
  if (tid < 40) {
    // the coefficients carry the softmax scale (log2 domain): the loop forms scale * score
    const int hf = tid / 20, k = (tid / 4) % 5, r = tid % 4;
    coef_s[hf][k][r] = coef[(4 * hf + r) * kQpackCoef + k] * a.scale_log2;
  }
  const int row = lane & 31, half = lane >> 5;
  // int8 digit rows: the NP plane-weight vectors and S q
  v4i Aq[NP][NCH], As[NCH];
  {
    const v4i *src = reinterpret_cast<const v4i *>(qpk);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) Aq[pp][c] = src[((pp * 32 + row) * 2 + half) * NCH + c];
      As[c] = src[((kSqVec * 32 + row) * 2 + half) * NCH + c];
    }
  }
  __syncthreads();

  // this lane's 4 heads' score coefficients: held in registers for the whole loop, except
  // with 3-bit keys, whose two more digit-row vectors leave no registers for them (they are
  // then read from LDS each tile)
  constexpr bool kCoefRegs = KBITS < 3;
  float K0[4], K1[4], K2[4], K3[4], K4[4];
  auto load_coef = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      K0[r] = coef_s[half][0][r];
      K1[r] = coef_s[half][1][r];
      K2[r] = NSN ? coef_s[half][2][r] : 0.0f;
      K3[r] = coef_s[half][3][r];
      K4[r] = coef_s[half][4][r];
    }
  };
  if constexpr (kCoefRegs) load_coef();
  const int t_begin = split * a.chunk;
  const int t_end = min(a.length, t_begin + a.chunk);
  const size_t ubase = size_t(unit) * a.capacity;
  const int t_first = t_begin + 32 * wv;
  constexpr int TS = 32 * NW;   // tokens between a wave's consecutive tiles
  const int nk = t_end > t_first ? (t_end - t_first + TS - 1) / TS : 0;
  float M[kMfmaMaxG], Mh[4], lsum[4];   // Mh: the running maxima of this lane's 4 heads
  float so[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // NSN: sum of p s1_v per head
  const uint32_t hmask = half ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int h = 0; h < kMfmaMaxG; ++h) M[h] = h < a.G ? -INFINITY : 0.0f;   // absent heads: any finite value
#pragma unroll
  for (int r = 0; r < 4; ++r) Mh[r] = pick_bits(hmask, M[4 + r], M[r]);
#pragma unroll
  for (int r = 0; r < 4; ++r) lsum[r] = 0.0f;
  v4f acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = v4f{0.f, 0.f, 0.f, 0.f};
  const int vq = lane >> 4, vn = lane & 15;
  // A lane's 8 tokens of a coordinate are bits [24 vq, 24 vq + 24) of the coordinate's 96
  // bits.  The lane reads the dword pair holding them and funnel-shifts it so that the two
  // 12-bit LUT indices come out already scaled by the 8-byte entry size: by 24 vq - 3 bits
  // from dword vidx, or for vq = 0 by 29 bits from the pair that starts one dword earlier
  // (the 3 bits shifted in from below are masked off).
  const int vidx = vq == 0 ? -1 : (24 * vq) >> 5;
  const uint32_t vsh = vq == 0 ? 29u : uint32_t(((24 * vq) & 31) - 3);
  const uint8_t *vbase = reinterpret_cast<const uint8_t *>(a.vcodes) + size_t(unit) * a.tiles * Gm::VT;
  const uint8_t *vnbase = reinterpret_cast<const uint8_t *>(a.vnorm);

  // Tile k of this wave starts at t_first + TS k.  Every chunk a lane loads stays inside
  // the tokens [t0, t_end); tiles past the end reload the last one into a slot that is
  // never read, so every step issues the same Gm::NDMA loads.
  // Each load is a uniform base (per tile, in SGPRs) plus a 32-bit per-lane byte offset;
  // for whole tiles the offsets are fixed, so a step spends almost no VALU on addresses.
  uint32_t koff[Gm::NK];
#pragma unroll
  for (int i = 0; i < Gm::NK; ++i) koff[i] = uint32_t(Gm::KCH * (64 * i + lane));
  // the wave's first tile in each stream; tile k is a fixed stride further
  const uint8_t *kb0 = a.kbits + (ubase + t_first) * Gm::KB;
  const uint8_t *vb0 = vbase + size_t(t_first / kValueTile) * Gm::VT;
  const uint8_t *kn0 = reinterpret_cast<const uint8_t *>(a.knorm) + (ubase + t_first) * Gm::KNR;
  const uint8_t *vn0 = vnbase + (ubase + t_first) * (NSN ? 4 : 2);
  auto issue_dma = [&](int k, uint8_t *slot) {
    const int kk = k < nk ? k : nk - 1;
    const int t0 = t_first + TS * kk;
    const int nv = t_end - t0;   // valid tokens in the tile (1..32)
    const bool whole = nv >= 32;   // wave-uniform: no clamping needed
    const size_t tk0 = size_t(kk) * TS;   // the tile's first token, from the wave's first
    const uint8_t *ksrc = kb0 + tk0 * Gm::KB;
    const int last = nv * Gm::KB / Gm::KCH - 1;
    constexpr int kchunks = Gm::KT / Gm::KCH;
#pragma unroll
    for (int i = 0; i < Gm::NK; ++i) {
      if (64 * i + 64 <= kchunks || lane < kchunks - 64 * i) {
        const uint32_t o = whole ? koff[i] : uint32_t(Gm::KCH * min(64 * i + lane, last));
        __builtin_amdgcn_global_load_lds(ksrc + o, slot + 64 * Gm::KCH * i, Gm::KCH, 0, 0);
      }
    }
    const uint8_t *vsrc = vb0 + (tk0 / kValueTile) * Gm::VT;
    constexpr int vchunks = Gm::VT / 16;
#pragma unroll
    for (int i = 0; i < Gm::NV; ++i) {
      if (64 * i + 64 <= vchunks || lane < vchunks - 64 * i)
        __builtin_amdgcn_global_load_lds(vsrc + 1024 * i + uint32_t(16 * lane), slot + Gm::KT + 1024 * i, 16, 0, 0);
    }
    if constexpr (NSN) {
      // 32 key norm records of 8 bytes (64 dwords), 32 value norm records of 4 bytes
      const uint8_t *kn = kn0 + tk0 * 8;
      const uint32_t tk = uint32_t(whole ? lane >> 1 : min(lane >> 1, nv - 1));
      __builtin_amdgcn_global_load_lds(kn + 8 * tk + 4 * uint32_t(lane & 1), slot + Gm::KN, 4, 0, 0);
      if (lane < 32) {
        const uint8_t *vn4 = vn0 + tk0 * 4;
        __builtin_amdgcn_global_load_lds(vn4 + 4 * uint32_t(whole ? lane : min(lane, nv - 1)), slot + Gm::VN, 4, 0, 0);
      }
    } else {
    if (lane < 32) {
      const uint8_t *kn = kn0 + tk0 * 4;
      __builtin_amdgcn_global_load_lds(kn + uint32_t(4 * (whole ? lane : min(lane, nv - 1))), slot + Gm::KN, 4, 0, 0);
    }
    if (lane < 17) {
      // value norms: 17 dwords from the 4-byte boundary at or below token t0's norm, none
      // past the dword holding the tile's last token (the region may end right there)
      // (tiles are TS tokens = a multiple of 4 bytes of norms apart, so the dword offset of
      // token t0's norm, r, is the same for all of the wave's tiles)
      const uint8_t *v2 = vn0 + tk0 * 2;
      const uint32_t r = uint32_t(reinterpret_cast<uintptr_t>(vn0)) & 3u;
      const uint32_t span = (r + 2u * uint32_t(nv - 1)) & ~3u;
      __builtin_amdgcn_global_load_lds(v2 - r + min(uint32_t(4 * lane), span), slot + Gm::VN, 4, 0, 0);
    }
    }
  };

  auto step = [&](int k, const uint8_t *slot, uint8_t *nxt) {
    // every read of the slot refilled here was waited for inside its own read block
    issue_dma(k + R - 1, nxt);
    if constexpr (SCORES)
      __builtin_amdgcn_s_waitcnt(0);
    else
      wait_vmcnt_le<(R - 1) * Gm::NDMA>();   // this tile's loads are the oldest still counted
    const int t0 = t_first + TS * k;
    const int t = t0 + row;
    const bool valid = t < t_end;
    const uint32_t sbase = uint32_t(reinterpret_cast<uintptr_t>(slot));
    // ---- this lane's key words, its token's norms and its value-code words, read in one
    // block; the value LUT lookups follow at once so their latency overlaps the key MFMAs
    // four key words per lane: the planes of the record (D / 8 bytes each, the lane's half
    // of them) and its sign bits; with fewer than three planes the extra reads fall on the
    // next record or the value region of the slot and are not used
    uint2 kw[4];
    uint32_t nr, vnb;
    uint32_t vwr[NT][2];
    {
      const uint32_t kaddr = sbase + row * Gm::KB + half * (D / 16);
      const uint32_t naddr = sbase + Gm::KN + Gm::KNR * row;
      const uint32_t vaddr = NSN ? sbase + Gm::VN + 4 * row : sbase + Gm::VN + uint32_t(((ubase + t0) * 2) & 3) + 2 * row;
      const uint32_t caddr = sbase + Gm::KT + vn * 12 + 4 * vidx;
#if defined(__HIP_DEVICE_COMPILE__)
      // The outputs are early-clobber ("=&v"): a read's destination must not share a
      // register with an address that a later read of the block still uses.
      if constexpr (D >= 128) {
        asm volatile(
            "ds_read_b64 %0, %22\n"
            "ds_read_b64 %1, %22 offset:16\n"
            "ds_read_b64 %2, %22 offset:32\n"
            "ds_read_b64 %3, %22 offset:48\n"
            "ds_read_b32 %4, %23\n"
            "ds_read_u16 %5, %24\n"
            "ds_read_b32 %6, %25\n"
            "ds_read_b32 %7, %25 offset:4\n"
            "ds_read_b32 %8, %25 offset:192\n"
            "ds_read_b32 %9, %25 offset:196\n"
            "ds_read_b32 %10, %25 offset:384\n"
            "ds_read_b32 %11, %25 offset:388\n"
            "ds_read_b32 %12, %25 offset:576\n"
            "ds_read_b32 %13, %25 offset:580\n"
            "ds_read_b32 %14, %25 offset:768\n"
            "ds_read_b32 %15, %25 offset:772\n"
            "ds_read_b32 %16, %25 offset:960\n"
            "ds_read_b32 %17, %25 offset:964\n"
            "ds_read_b32 %18, %25 offset:1152\n"
            "ds_read_b32 %19, %25 offset:1156\n"
            "ds_read_b32 %20, %25 offset:1344\n"
            "ds_read_b32 %21, %25 offset:1348\n"
            "s_waitcnt lgkmcnt(0)\n"
            : "=&v"(kw[0]), "=&v"(kw[1]), "=&v"(kw[2]), "=&v"(kw[3]), "=&v"(nr), "=&v"(vnb),
              "=&v"(vwr[0][0]), "=&v"(vwr[0][1]), "=&v"(vwr[1][0]), "=&v"(vwr[1][1]), "=&v"(vwr[2][0]),
              "=&v"(vwr[2][1]), "=&v"(vwr[3][0]), "=&v"(vwr[3][1]), "=&v"(vwr[4][0]), "=&v"(vwr[4][1]),
              "=&v"(vwr[5][0]), "=&v"(vwr[5][1]), "=&v"(vwr[6][0]), "=&v"(vwr[6][1]), "=&v"(vwr[7][0]),
              "=&v"(vwr[7][1])
            : "v"(kaddr), "v"(naddr), "v"(vaddr), "v"(caddr)
            : "memory");
      } else {
        uint32_t x0, x1, x2, x3;
        asm volatile(
            "ds_read_b32 %0, %14\n"
            "ds_read_b32 %1, %14 offset:8\n"
            "ds_read_b32 %2, %14 offset:16\n"
            "ds_read_b32 %3, %14 offset:24\n"
            "ds_read_b32 %4, %15\n"
            "ds_read_u16 %5, %16\n"
            "ds_read_b32 %6, %17\n"
            "ds_read_b32 %7, %17 offset:4\n"
            "ds_read_b32 %8, %17 offset:192\n"
            "ds_read_b32 %9, %17 offset:196\n"
            "ds_read_b32 %10, %17 offset:384\n"
            "ds_read_b32 %11, %17 offset:388\n"
            "ds_read_b32 %12, %17 offset:576\n"
            "ds_read_b32 %13, %17 offset:580\n"
            "s_waitcnt lgkmcnt(0)\n"
            : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(nr), "=&v"(vnb),
              "=&v"(vwr[0][0]), "=&v"(vwr[0][1]), "=&v"(vwr[1][0]), "=&v"(vwr[1][1]), "=&v"(vwr[2][0]),
              "=&v"(vwr[2][1]), "=&v"(vwr[3][0]), "=&v"(vwr[3][1])
            : "v"(kaddr), "v"(naddr), "v"(vaddr), "v"(caddr)
            : "memory");
        kw[0] = make_uint2(x0, 0u);
        kw[1] = make_uint2(x1, 0u);
        kw[2] = make_uint2(x2, 0u);
        kw[3] = make_uint2(x3, 0u);
      }
#else
      (void)kaddr;
      (void)naddr;
      (void)vaddr;
      (void)caddr;
      nr = vnb = 0u;
      kw[0] = kw[1] = kw[2] = kw[3] = make_uint2(0u, 0u);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vwr[nt][0] = vwr[nt][1] = 0u;
#endif
    }
    // value B operands: 8 tokens' fp16 centroids of coordinate 16 nt + vn, two LUT lookups
    v8h Bv[NT];
    const uint8_t *lutb = reinterpret_cast<const uint8_t *>(lut);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t y = __builtin_amdgcn_alignbit(vwr[nt][1], vwr[nt][0], vsh);   // 8 x (low bits junk)
      const uint2 e0 = *reinterpret_cast<const uint2 *>(lutb + (y & 0x7FF8u));
      const uint2 e1 = *reinterpret_cast<const uint2 *>(lutb + ((y >> 12) & 0x7FF8u));
      v4i bw = {int(e0.x), int(e0.y), int(e1.x), int(e1.y)};
      __builtin_memcpy(&Bv[nt], &bw, 16);
    }
    // ---- key scores on int8 MFMA: every code plane accumulates into s01 (its digit rows
    // carry the plane weight), the sign bits into s2.  The B bytes of coordinate-chunk c
    // are bit e of the low (c even) or high (c odd) nibble of each byte of the lane's plane
    // dword for c / 2, masked in place: byte value b 2^e, the 2^-e being in the query digits.
    // Plane words: the code bits, then for 3-bit codes their parity; signs follow the codes.
    uint2 pl[NP + 1];
#pragma unroll
    for (int pp = 0; pp < KBITS; ++pp) pl[pp] = kw[pp];
    if constexpr (KBITS == 3) pl[3] = make_uint2(kw[0].x ^ kw[1].x ^ kw[2].x, kw[0].y ^ kw[1].y ^ kw[2].y);
    pl[NP] = kw[KBITS];
    v16i s01 = {}, s2 = {};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      v4i bp[NP + 1];
#pragma unroll
      for (int pp = 0; pp <= NP; ++pp) {
        const uint32_t w = (c >> 1) ? pl[pp].y : pl[pp].x;
        const uint32_t nb = (c & 1) ? w >> 4 : w;
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[pp][e] = int(nb & (0x01010101u << e));
      }
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) s01 = __builtin_amdgcn_mfma_i32_32x32x32_i8(Aq[pp][c], bp[pp], s01, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(As[c], bp[NP], s2, 0, 0, 0);
    }
    const float n16 = f16_bits_to_float(nr & 0xFFFFu), rn16 = f16_bits_to_float(nr >> 16);
    const float vnorm = f16_bits_to_float(vnb & 0xFFFFu);
    float ks1 = 0.0f, vs1 = 0.0f;
    if constexpr (NSN) {
      // the s1 halves of this token's norm records (LDS reads, waited for in the block)
      uint32_t k1b = 0u, v1b = 0u;
      asm volatile(
          "ds_read_u16 %0, %2 offset:4\n"
          "ds_read_u16 %1, %3 offset:2\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(k1b), "=&v"(v1b)
          : "v"(sbase + Gm::KN + 8 * row), "v"(sbase + Gm::VN + 4 * row)
          : "memory");
      ks1 = f16_bits_to_float(k1b);
      vs1 = f16_bits_to_float(v1b);
    }
    // lam = scale * score in the log2 domain; a token past the end gets -inf through the
    // innermost fma.  Heads h >= G (zero coefficients and digits) get lam = 0: their rows
    // are carried along and never written out.
    if constexpr (!kCoefRegs) load_coef();
    const float vbias = valid ? 0.0f : -INFINITY;
    float lam[4], rel[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // digit sums: rows 8 digit + head are accumulator registers 4 digit + r
      const float S01 = fmaf(float(s01[r] + 256 * s01[4 + r]), 0x1p-16f, float(s01[8 + r] + 256 * s01[12 + r]));
      const float S2 = fmaf(float(s2[r] + 256 * s2[4 + r]), 0x1p-16f, float(s2[8 + r] + 256 * s2[12 + r]));
      const float vb = NSN ? fmaf(ks1, K2[r], vbias) : vbias;   // NSN: + s1 <q, o_K>
      lam[r] = fmaf(n16, fmaf(K1[r], S01, K0[r]), fmaf(rn16, fmaf(K3[r], S2, -K4[r]), vb));
      rel[r] = lam[r] - Mh[r];
    }
    if constexpr (SCORES) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * half + r;
        if (valid && h < a.G) a.scores[(size_t(b) * a.q_heads + hq0 + h) * a.score_stride + t] = lam[r] * a.inv_scale_log2;
      }
    }
    // ---- online softmax (log2 domain); tile maxima and running maxima are wave-uniform.
    // The running maxima are raised (and the accumulators rescaled) only when a score
    // exceeds its head's maximum by more than 8, so p = 2^(lam - M) <= 256 between raises;
    // a token whose value norm is 255 or more allows no slack, which keeps p * n_v within
    // fp16 range (256 * 255 < 65504) for the hi/lo split below.  In the first tile the
    // maxima are -inf, so every valid token is above them.
    const float slack = vnorm < 255.0f ? 8.0f : 0.0f;
    uint64_t above = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) above |= __builtin_amdgcn_ballot_w64(rel[r] > slack);
    if (above != 0) {
      float tm[kMfmaMaxG];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = dpp_max32_tail(f2ord(lam[r]));
        tm[r] = ord2f(__builtin_amdgcn_readlane(v, 31));
        tm[4 + r] = ord2f(__builtin_amdgcn_readlane(v, 63));
      }
      float alpha[kMfmaMaxG];
#pragma unroll
      for (int h = 0; h < kMfmaMaxG; ++h) {
        const float nm = fmaxf(M[h], tm[h]);
        alpha[h] = (nm == M[h]) ? 1.0f : __builtin_amdgcn_exp2f(M[h] - nm);
        M[h] = nm;
      }
      // accumulator row 4 vq + r holds head 4 (vq & 1) + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float al = (vq & 1) ? alpha[4 + r] : alpha[r];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= al;
        lsum[r] *= half ? alpha[4 + r] : alpha[r];
        if constexpr (NSN) so[r] *= half ? alpha[4 + r] : alpha[r];
        Mh[r] = pick_bits(hmask, M[4 + r], M[r]);
        rel[r] = lam[r] - Mh[r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * half + r;
      // lam = -inf (token past the end) gives p = 0: Mh is finite after the first tile
      const float p = __builtin_amdgcn_exp2f(rel[r]);
      lsum[r] += p;
      if constexpr (NSN) so[r] = fmaf(p, vs1, so[r]);
      const float pv = p * vnorm;
      const _Float16 hi = (_Float16)pv;
      const _Float16 lo = (_Float16)(pv - float(hi));
      pt_s[wv][h][row] = hi;
      pt_s[wv][8 + h][row] = lo;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const v8h A = *reinterpret_cast<const v8h *>(&pt_s[wv][vn][8 * vq]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bv[nt], acc[nt], 0, 0, 0);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };

  if (nk > 0) {
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue_dma(k, &ring[k][wv][0]);
    for (int k = 0; k < nk; k += R) {
#pragma unroll
      for (int sl = 0; sl < R; ++sl)
        if (k + sl < nk) step(k + sl, &ring[sl][wv][0], &ring[(sl + R - 1) % R][wv][0]);
    }
    __builtin_amdgcn_s_waitcnt(0);   // drain the tail loads before the slots are reused
  }
  // ---- merge the block's waves
#pragma unroll
  for (int r = 0; r < 4; ++r) lsum[r] = sum32(lsum[r]);
  if constexpr (NSN) {
#pragma unroll
    for (int r = 0; r < 4; ++r) so[r] = sum32(so[r]);
  }
  __syncthreads();
  float *acc_s = reinterpret_cast<float *>(&ring[0][0][0]);   // [NW waves][16 rows][D]
  if (lane == 0 || lane == 32) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red_s[wv][1][4 * half + r] = lsum[r];
    if constexpr (NSN) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red_s[wv][2][4 * half + r] = so[r];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kMfmaMaxG; ++h) red_s[wv][0][h] = M[h];
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_s[(wv * 16 + 4 * vq + r) * D + 16 * nt + vn] = acc[nt][r];
  __syncthreads();
  for (int i = tid; i < a.G * D; i += NTH) {
    const int h = i / D, j = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red_s[w][0][h]);
    float v = 0.0f, L = 0.0f, SO = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red_s[w][0][h];
      if (mw == -INFINITY) continue;
      const float f = exp2f(mw - mx);
      v += (acc_s[(w * 16 + h) * D + j] + acc_s[(w * 16 + 8 + h) * D + j]) * f;
      L += red_s[w][1][h] * f;
      if constexpr (NSN) SO += red_s[w][2][h] * f;
    }
    // NSN: the values' mean, sum_t p_t s1_t Pi o_V, joins the rotated accumulator
    if constexpr (NSN) v = fmaf(SO, a.nsn[size_t(unit) * 4 * D + 3 * D + j], v);
    float *o = a.part + ((size_t(b * a.q_heads + hq0 + h) * a.splits) + split) * (D + 2);
    o[j] = v;
    if (j == 0) {
      o[D] = mx == -INFINITY ? -INFINITY : mx * 0.69314718055994531f;
      o[D + 1] = L;
    }
  }
#else
  (void)a;
#endif
}

// Maxima of x over each row of 16 lanes, left in every lane of the row (quad swaps, then
// half-row and row mirrors).
__device__ __forceinline__ int dpp_max16(int x) {
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true));
  return x;
}

// The split-K decode of k_decode_lds for groups of at most 4 query heads per kv-head
// (G <= 4) at d = 128, plain caches.  Tiles, ring, value LUT and value MFMAs are the same;
// the key scores run on v_mfma_i32_16x16x64_i8 with the 16 A rows 4 head + digit, where
// the 32x32x32 form would leave half of its 32 rows (digit x head for 8 heads) idle: half
// the matrix-core cycles per tile.  Lane l holds, for head l / 16, tokens l % 16 and
// 16 + l % 16 of the tile: its B operands are dword l / 16 of those tokens' plane and sign
// words (low nibbles for coordinates chunk 0, high nibbles for chunk 1, as the 32x32 form
// splits a dword), and its four accumulator rows are the four digits of its head, so the
// digit sums recombine in-lane as before.  The query prep writes the matching A operand
// (the same 16-byte fragments, indexed [slot][4 head + digit][dword][nibble]).
template <int KBITS, bool SCORES>
__global__ __launch_bounds__(64 * kDecWaves, kDecBlocksPerCU) void k_decode_lds16(MfmaArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int D = 128;
  using Gm = LdsGeom<D, KBITS, false>;
  constexpr int NT = D / 16, NW = kDecWaves, NTH = 64 * NW, R = kRing;
  constexpr int NP = KBITS == 3 ? 4 : KBITS;
  static_assert(KBITS >= 1 && KBITS <= 3, "key planes");
  __shared__ __align__(32768) uint2 lut[4096];
  __shared__ __align__(16) uint8_t ring[R][NW][Gm::SLOT];
  __shared__ __align__(16) _Float16 pt_s[NW][16][40];
  __shared__ float red_s[NW][2][4];
  static_assert(NW * 16 * D * 4 <= int(sizeof(ring)), "the waves' accumulators fit in the ring for the merge");

  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / a.kv_heads, kvh = unit % a.kv_heads;
  const int hq0 = kvh * a.G;
  for (int i = tid; i < 4096; i += NTH) {
    const uint32_t h0 = f16bits(a.cv[i & 7]), h1 = f16bits(a.cv[(i >> 3) & 7]);
    const uint32_t h2 = f16bits(a.cv[(i >> 6) & 7]), h3 = f16bits(a.cv[(i >> 9) & 7]);
    lut[i] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
  }
  // P rows 4..7 and 12..15 (heads 4..7) are never written: zero once
  {
    uint32_t *pz = reinterpret_cast<uint32_t *>(&pt_s[0][0][0]);
    for (int i = tid; i < NW * 16 * 40 / 2; i += NTH) pz[i] = 0u;
  }
  const int n = lane & 15, gh = lane >> 4;   // token of 16 (and its B/A lane group), head
  const uint8_t *qpk = a.qpack + size_t(unit) * qpack_unit_bytes(D);
  const float *coef = reinterpret_cast<const float *>(qpk + size_t(kQpackVecs) * 32 * 2 * (D / 32) * 16);
  // this lane's head's score coefficients with the softmax scale (log2 domain)
  const float K0 = coef[gh * kQpackCoef + 0] * a.scale_log2, K1 = coef[gh * kQpackCoef + 1] * a.scale_log2;
  const float K3 = coef[gh * kQpackCoef + 3] * a.scale_log2, K4 = coef[gh * kQpackCoef + 4] * a.scale_log2;
  // int8 digit rows: A lane (row n = 4 head + digit, K group gh), chunks 0 and 1
  v4i Aq[NP][2], As[2];
  {
    const v4i *src = reinterpret_cast<const v4i *>(qpk);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) Aq[pp][c] = src[((pp * 16 + n) * 4 + gh) * 2 + c];
      As[c] = src[((kSqVec * 16 + n) * 4 + gh) * 2 + c];
    }
  }
  __syncthreads();

  const int t_begin = split * a.chunk;
  const int t_end = min(a.length, t_begin + a.chunk);
  const size_t ubase = size_t(unit) * a.capacity;
  const int t_first = t_begin + 32 * wv;
  constexpr int TS = 32 * NW;
  const int nk = t_end > t_first ? (t_end - t_first + TS - 1) / TS : 0;
  float M[4];   // running maxima per head (wave-uniform); absent heads: any finite value
#pragma unroll
  for (int h = 0; h < 4; ++h) M[h] = h < a.G ? -INFINITY : 0.0f;
  const uint32_t gm0 = (gh & 1) ? 0xFFFFFFFFu : 0u, gm1 = (gh & 2) ? 0xFFFFFFFFu : 0u;
  auto head_of = [&](const float *v) { return pick_bits(gm1, pick_bits(gm0, v[3], v[2]), pick_bits(gm0, v[1], v[0])); };
  float Mh = head_of(M), lsum = 0.0f;
  v4f acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = v4f{0.f, 0.f, 0.f, 0.f};
  const int vq = lane >> 4, vn = lane & 15;
  const int vidx = vq == 0 ? -1 : (24 * vq) >> 5;
  const uint32_t vsh = vq == 0 ? 29u : uint32_t(((24 * vq) & 31) - 3);
  const uint8_t *vbase = reinterpret_cast<const uint8_t *>(a.vcodes) + size_t(unit) * a.tiles * Gm::VT;
  const uint8_t *vnbase = reinterpret_cast<const uint8_t *>(a.vnorm);
  uint32_t koff[Gm::NK];
#pragma unroll
  for (int i = 0; i < Gm::NK; ++i) koff[i] = uint32_t(Gm::KCH * (64 * i + lane));
  const uint8_t *kb0 = a.kbits + (ubase + t_first) * Gm::KB;
  const uint8_t *vb0 = vbase + size_t(t_first / kValueTile) * Gm::VT;
  const uint8_t *kn0 = reinterpret_cast<const uint8_t *>(a.knorm) + (ubase + t_first) * Gm::KNR;
  const uint8_t *vn0 = vnbase + (ubase + t_first) * 2;
  auto issue_dma = [&](int k, uint8_t *slot) {
    const int kk = k < nk ? k : nk - 1;
    const int t0 = t_first + TS * kk;
    const int nv = t_end - t0;
    const bool whole = nv >= 32;
    const size_t tk0 = size_t(kk) * TS;
    const uint8_t *ksrc = kb0 + tk0 * Gm::KB;
    const int last = nv * Gm::KB / Gm::KCH - 1;
    constexpr int kchunks = Gm::KT / Gm::KCH;
#pragma unroll
    for (int i = 0; i < Gm::NK; ++i) {
      if (64 * i + 64 <= kchunks || lane < kchunks - 64 * i) {
        const uint32_t o = whole ? koff[i] : uint32_t(Gm::KCH * min(64 * i + lane, last));
        __builtin_amdgcn_global_load_lds(ksrc + o, slot + 64 * Gm::KCH * i, Gm::KCH, 0, 0);
      }
    }
    const uint8_t *vsrc = vb0 + (tk0 / kValueTile) * Gm::VT;
    constexpr int vchunks = Gm::VT / 16;
#pragma unroll
    for (int i = 0; i < Gm::NV; ++i) {
      if (64 * i + 64 <= vchunks || lane < vchunks - 64 * i)
        __builtin_amdgcn_global_load_lds(vsrc + 1024 * i + uint32_t(16 * lane), slot + Gm::KT + 1024 * i, 16, 0, 0);
    }
    if (lane < 32) {
      const uint8_t *kn = kn0 + tk0 * 4;
      __builtin_amdgcn_global_load_lds(kn + uint32_t(4 * (whole ? lane : min(lane, nv - 1))), slot + Gm::KN, 4, 0, 0);
    }
    if (lane < 17) {
      const uint8_t *v2 = vn0 + tk0 * 2;
      const uint32_t r = uint32_t(reinterpret_cast<uintptr_t>(vn0)) & 3u;
      const uint32_t span = (r + 2u * uint32_t(nv - 1)) & ~3u;
      __builtin_amdgcn_global_load_lds(v2 - r + min(uint32_t(4 * lane), span), slot + Gm::VN, 4, 0, 0);
    }
  };

  auto step = [&](int k, const uint8_t *slot, uint8_t *nxt) {
    issue_dma(k + R - 1, nxt);
    if constexpr (SCORES)
      __builtin_amdgcn_s_waitcnt(0);
    else
      wait_vmcnt_le<(R - 1) * Gm::NDMA>();
    const int t0 = t_first + TS * k;
    const int ta = t0 + n, tb = ta + 16;
    const bool va = ta < t_end, vb = tb < t_end;
    const uint32_t sbase = uint32_t(reinterpret_cast<uintptr_t>(slot));
    // dword gh of the plane and sign words of tokens n and 16 + n (four words each: with
    // fewer than three planes the extra reads fall on the next record or the value region
    // of the slot and are not used), their norms and value norms, and the value-code words
    uint32_t wa[4], wb[4], nra, nrb, vna, vnb2;
    uint32_t vwr[NT][2];
    {
      const uint32_t kaddr = sbase + n * Gm::KB + 4 * gh;
      const uint32_t naddr = sbase + Gm::KN + 4 * n;
      const uint32_t vaddr = sbase + Gm::VN + uint32_t(((ubase + t0) * 2) & 3) + 2 * n;
      const uint32_t caddr = sbase + Gm::KT + vn * 12 + 4 * vidx;
      asm volatile(
          "ds_read_b32 %0, %28\n"
          "ds_read_b32 %1, %28 offset:16\n"
          "ds_read_b32 %2, %28 offset:32\n"
          "ds_read_b32 %3, %28 offset:48\n"
          "ds_read_b32 %4, %32\n"
          "ds_read_b32 %5, %32 offset:16\n"
          "ds_read_b32 %6, %32 offset:32\n"
          "ds_read_b32 %7, %32 offset:48\n"
          "ds_read_b32 %8, %29\n"
          "ds_read_b32 %9, %29 offset:64\n"
          "ds_read_u16 %10, %30\n"
          "ds_read_u16 %11, %30 offset:32\n"
          "ds_read_b32 %12, %31\n"
          "ds_read_b32 %13, %31 offset:4\n"
          "ds_read_b32 %14, %31 offset:192\n"
          "ds_read_b32 %15, %31 offset:196\n"
          "ds_read_b32 %16, %31 offset:384\n"
          "ds_read_b32 %17, %31 offset:388\n"
          "ds_read_b32 %18, %31 offset:576\n"
          "ds_read_b32 %19, %31 offset:580\n"
          "ds_read_b32 %20, %31 offset:768\n"
          "ds_read_b32 %21, %31 offset:772\n"
          "ds_read_b32 %22, %31 offset:960\n"
          "ds_read_b32 %23, %31 offset:964\n"
          "ds_read_b32 %24, %31 offset:1152\n"
          "ds_read_b32 %25, %31 offset:1156\n"
          "ds_read_b32 %26, %31 offset:1344\n"
          "ds_read_b32 %27, %31 offset:1348\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(wa[0]), "=&v"(wa[1]), "=&v"(wa[2]), "=&v"(wa[3]), "=&v"(wb[0]), "=&v"(wb[1]), "=&v"(wb[2]),
            "=&v"(wb[3]), "=&v"(nra), "=&v"(nrb), "=&v"(vna), "=&v"(vnb2), "=&v"(vwr[0][0]), "=&v"(vwr[0][1]),
            "=&v"(vwr[1][0]), "=&v"(vwr[1][1]), "=&v"(vwr[2][0]), "=&v"(vwr[2][1]), "=&v"(vwr[3][0]),
            "=&v"(vwr[3][1]), "=&v"(vwr[4][0]), "=&v"(vwr[4][1]), "=&v"(vwr[5][0]), "=&v"(vwr[5][1]),
            "=&v"(vwr[6][0]), "=&v"(vwr[6][1]), "=&v"(vwr[7][0]), "=&v"(vwr[7][1])
          : "v"(kaddr), "v"(naddr), "v"(vaddr), "v"(caddr), "v"(kaddr + 16 * Gm::KB)
          : "memory");
    }
    v8h Bv[NT];
    const uint8_t *lutb = reinterpret_cast<const uint8_t *>(lut);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t y = __builtin_amdgcn_alignbit(vwr[nt][1], vwr[nt][0], vsh);
      const uint2 e0 = *reinterpret_cast<const uint2 *>(lutb + (y & 0x7FF8u));
      const uint2 e1 = *reinterpret_cast<const uint2 *>(lutb + ((y >> 12) & 0x7FF8u));
      v4i bw = {int(e0.x), int(e0.y), int(e1.x), int(e1.y)};
      __builtin_memcpy(&Bv[nt], &bw, 16);
    }
    // ---- key scores: for each token half, chunk and plane, the B bytes are bit e of the
    // low (chunk 0) or high (chunk 1) nibbles of the lane's plane word, masked in place
    v4i s01[2] = {}, s2[2] = {};
#pragma unroll
    for (int tbk = 0; tbk < 2; ++tbk) {
      const uint32_t *w = tbk ? wb : wa;
      uint32_t pl[NP + 1];
#pragma unroll
      for (int pp = 0; pp < KBITS; ++pp) pl[pp] = w[pp];
      if constexpr (KBITS == 3) pl[3] = w[0] ^ w[1] ^ w[2];
      pl[NP] = w[KBITS];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        v4i bp[NP + 1];
#pragma unroll
        for (int pp = 0; pp <= NP; ++pp) {
          const uint32_t nb = c ? pl[pp] >> 4 : pl[pp];
#pragma unroll
          for (int e = 0; e < 4; ++e) bp[pp][e] = int(nb & (0x01010101u << e));
        }
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) s01[tbk] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aq[pp][c], bp[pp], s01[tbk], 0, 0, 0);
        s2[tbk] = __builtin_amdgcn_mfma_i32_16x16x64_i8(As[c], bp[NP], s2[tbk], 0, 0, 0);
      }
    }
    float lam[2], rel[2], vnorm[2];
#pragma unroll
    for (int tbk = 0; tbk < 2; ++tbk) {
      const uint32_t nr = tbk ? nrb : nra;
      const float n16 = f16_bits_to_float(nr & 0xFFFFu), rn16 = f16_bits_to_float(nr >> 16);
      vnorm[tbk] = f16_bits_to_float((tbk ? vnb2 : vna) & 0xFFFFu);
      // the four accumulator rows are digits 0..3 of the lane's head
      const float S01 = fmaf(float(s01[tbk][0] + 256 * s01[tbk][1]), 0x1p-16f, float(s01[tbk][2] + 256 * s01[tbk][3]));
      const float S2 = fmaf(float(s2[tbk][0] + 256 * s2[tbk][1]), 0x1p-16f, float(s2[tbk][2] + 256 * s2[tbk][3]));
      const float vbias = (tbk ? vb : va) ? 0.0f : -INFINITY;
      lam[tbk] = fmaf(n16, fmaf(K1, S01, K0), fmaf(rn16, fmaf(K3, S2, -K4), vbias));
      rel[tbk] = lam[tbk] - Mh;
    }
    if constexpr (SCORES) {
      if (gh < a.G) {
        float *srow = a.scores + (size_t(b) * a.q_heads + hq0 + gh) * a.score_stride;
        if (va) srow[ta] = lam[0] * a.inv_scale_log2;
        if (vb) srow[tb] = lam[1] * a.inv_scale_log2;
      }
    }
    // ---- online softmax (log2 domain), maxima raised only past a slack of 8 (as in
    // k_decode_lds); the tile maximum of a head is the maximum over its row of 16 lanes
    const float sla = vnorm[0] < 255.0f ? 8.0f : 0.0f, slb = vnorm[1] < 255.0f ? 8.0f : 0.0f;
    const uint64_t above = __builtin_amdgcn_ballot_w64(rel[0] > sla || rel[1] > slb);
    if (above != 0) {
      const int v = dpp_max16(max(f2ord(lam[0]), f2ord(lam[1])));
      float alpha[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float tm = ord2f(__builtin_amdgcn_readlane(v, 16 * h + 15));
        const float nm = fmaxf(M[h], tm);
        alpha[h] = (nm == M[h]) ? 1.0f : __builtin_amdgcn_exp2f(M[h] - nm);
        M[h] = nm;
      }
      // accumulator row 4 vq + r holds head r (hi for vq = 0, lo for vq = 2; the rows of
      // vq = 1 and 3 are the zero P rows of heads 4..7)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= alpha[r];
      lsum *= head_of(alpha);
      Mh = head_of(M);
      rel[0] = lam[0] - Mh;
      rel[1] = lam[1] - Mh;
    }
#pragma unroll
    for (int tbk = 0; tbk < 2; ++tbk) {
      const float p = __builtin_amdgcn_exp2f(rel[tbk]);
      lsum += p;
      const float pv = p * vnorm[tbk];
      const _Float16 hi = (_Float16)pv;
      const _Float16 lo = (_Float16)(pv - float(hi));
      pt_s[wv][gh][n + 16 * tbk] = hi;
      pt_s[wv][8 + gh][n + 16 * tbk] = lo;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const v8h A = *reinterpret_cast<const v8h *>(&pt_s[wv][vn][8 * vq]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bv[nt], acc[nt], 0, 0, 0);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };

  if (nk > 0) {
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue_dma(k, &ring[k][wv][0]);
    for (int k = 0; k < nk; k += R) {
#pragma unroll
      for (int sl = 0; sl < R; ++sl)
        if (k + sl < nk) step(k + sl, &ring[sl][wv][0], &ring[(sl + R - 1) % R][wv][0]);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  // ---- merge the block's waves: the head's sum over its row of 16 lanes
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) lsum += __shfl_xor(lsum, o, 64);
  __syncthreads();
  float *acc_s = reinterpret_cast<float *>(&ring[0][0][0]);   // [NW waves][16 rows][D]
  if (n == 0) red_s[wv][1][gh] = lsum;
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) red_s[wv][0][h] = M[h];
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_s[(wv * 16 + 4 * vq + r) * D + 16 * nt + vn] = acc[nt][r];
  __syncthreads();
  for (int i = tid; i < a.G * D; i += NTH) {
    const int h = i / D, j = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red_s[w][0][h]);
    float v = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red_s[w][0][h];
      if (mw == -INFINITY) continue;
      const float f = exp2f(mw - mx);
      v += (acc_s[(w * 16 + h) * D + j] + acc_s[(w * 16 + 8 + h) * D + j]) * f;
      L += red_s[w][1][h] * f;
    }
    float *o = a.part + ((size_t(b * a.q_heads + hq0 + h) * a.splits) + split) * (D + 2);
    o[j] = v;
    if (j == 0) {
      o[D] = mx == -INFINITY ? -INFINITY : mx * 0.69314718055994531f;
      o[D + 1] = L;
    }
  }
#else
  (void)a;
#endif
}

// Attention logits only (tq_decode_attend with out = NULL): the key-score half of
// k_decode_lds, for the same key formats and query digit rows, writing the unscaled
// estimates.  With no value stream to stage, each lane loads its own token's key words
// (its half of every plane and of the signs) and norms straight into registers two tiles
// ahead; 4 waves per block, wave w taking tiles w, w + 4, ... of the block's chunk.
template <int D, int KBITS, bool NSN>
__global__ __launch_bounds__(256) void k_logits(MfmaArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NCH = D / 32, NP = KBITS == 3 ? 4 : KBITS, KB = (KBITS + 1) * D / 8;
  __shared__ __align__(16) float coef_s[2][5][4];
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / a.kv_heads, g = unit % a.kv_heads;
  const int hq0 = g * a.G;
  const uint8_t *qpk = a.qpack + size_t(unit) * qpack_unit_bytes(D);
  const float *coef = reinterpret_cast<const float *>(qpk + size_t(kQpackVecs) * 32 * 2 * NCH * 16);
  if (tid < 40) {
    const int hf = tid / 20, k = (tid / 4) % 5, r = tid % 4;
    coef_s[hf][k][r] = coef[(4 * hf + r) * kQpackCoef + k];
  }
  const int row = lane & 31, half = lane >> 5;
  v4i Aq[NP][NCH], As[NCH];
  {
    const v4i *src = reinterpret_cast<const v4i *>(qpk);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) Aq[pp][c] = src[((pp * 32 + row) * 2 + half) * NCH + c];
      As[c] = src[((kSqVec * 32 + row) * 2 + half) * NCH + c];
    }
  }
  __syncthreads();
  const int t_begin = split * a.chunk;
  const int t_end = min(a.length, t_begin + a.chunk);
  const size_t ubase = size_t(unit) * a.capacity;
  const int t_first = t_begin + 32 * wv;
  const int nk = t_end > t_first ? (t_end - t_first + 127) / 128 : 0;
  // a lane's words of tile k (tokens past the end read the last token of the range)
  auto load = [&](int k, uint2 (&kw)[KBITS + 1], uint32_t &nr, uint32_t &ns) {
    const int tc = min(t_first + 128 * k + row, t_end - 1);
    const uint8_t *rec = a.kbits + (ubase + tc) * KB + half * (D / 16);
#pragma unroll
    for (int pp = 0; pp <= KBITS; ++pp) {
      if constexpr (D >= 128)
        kw[pp] = *reinterpret_cast<const uint2 *>(rec + pp * (D / 8));
      else
        kw[pp] = make_uint2(*reinterpret_cast<const uint32_t *>(rec + pp * (D / 8)), 0u);
    }
    if constexpr (NSN) {
      const uint2 r = reinterpret_cast<const uint2 *>(a.knorm)[ubase + tc];   // {n | |r|, s1}
      nr = r.x;
      ns = r.y;
    } else {
      nr = a.knorm[ubase + tc];
      ns = 0u;
    }
  };
  uint2 kwn[KBITS + 1], kwm[KBITS + 1];   // tiles k + 1 and k + 2 in flight
  uint32_t nrn = 0u, nrm = 0u, nsn_n = 0u, nsn_m = 0u;
  if (nk > 0) load(0, kwn, nrn, nsn_n);
  if (nk > 1) load(1, kwm, nrm, nsn_m);
  for (int k = 0; k < nk; ++k) {
    uint2 kw[KBITS + 1];
#pragma unroll
    for (int pp = 0; pp <= KBITS; ++pp) {
      kw[pp] = kwn[pp];
      kwn[pp] = kwm[pp];
    }
    const uint32_t nr = nrn, ns = nsn_n;
    nrn = nrm;
    nsn_n = nsn_m;
    if (k + 2 < nk) load(k + 2, kwm, nrm, nsn_m);
    uint2 pl[NP + 1];
#pragma unroll
    for (int pp = 0; pp < KBITS; ++pp) pl[pp] = kw[pp];
    if constexpr (KBITS == 3) pl[3] = make_uint2(kw[0].x ^ kw[1].x ^ kw[2].x, kw[0].y ^ kw[1].y ^ kw[2].y);
    pl[NP] = kw[KBITS];
    v16i s01 = {}, s2 = {};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      v4i bp[NP + 1];
#pragma unroll
      for (int pp = 0; pp <= NP; ++pp) {
        const uint32_t w = (c >> 1) ? pl[pp].y : pl[pp].x;
        const uint32_t nb = (c & 1) ? w >> 4 : w;
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[pp][e] = int(nb & (0x01010101u << e));
      }
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) s01 = __builtin_amdgcn_mfma_i32_32x32x32_i8(Aq[pp][c], bp[pp], s01, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(As[c], bp[NP], s2, 0, 0, 0);
    }
    const float n16 = f16_bits_to_float(nr & 0xFFFFu), rn16 = f16_bits_to_float(nr >> 16);
    const float ks1 = NSN ? f16_bits_to_float(ns & 0xFFFFu) : 0.0f;
    const int t = t_first + 128 * k + row;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float S01 = fmaf(float(s01[r] + 256 * s01[4 + r]), 0x1p-16f, float(s01[8 + r] + 256 * s01[12 + r]));
      const float S2 = fmaf(float(s2[r] + 256 * s2[4 + r]), 0x1p-16f, float(s2[8 + r] + 256 * s2[12 + r]));
      float sc = fmaf(n16, fmaf(coef_s[half][1][r], S01, coef_s[half][0][r]),
                      rn16 * fmaf(coef_s[half][3][r], S2, -coef_s[half][4][r]));
      if constexpr (NSN) sc = fmaf(ks1, coef_s[half][2][r], sc);   // + s1 <q, o_K>
      const int h = 4 * half + r;
      if (t < t_end && h < a.G) a.scores[(size_t(b) * a.q_heads + hq0 + h) * a.score_stride + t] = sc;
    }
  }
#else
  (void)a;
#endif
}

// ------------------------------------------------------------------ full-precision window
// The recent tokens not yet packed ([NSNQuant] section 4, residuals: a quantized part plus
// a full-precision residual that is quantized and appended once full).  One block per
// (batch, kv-head) unit scores its G q-heads against the window exactly,
// <RoPE(q, q_pos), RoPE(k, pos)> (the rotation Pi being orthogonal, the same score as in
// the rotated basis, [TurboESM] 2.A), runs the online softmax over 64-token chunks,
// accumulates the raw values, rotates the sum once by Pi and stores it as one more split
// partial (max, sum, acc) for the merge, which then weighs it against the packed splits.
struct WindowArgs {
  const void *k, *v;          // [batch][kv_heads][cap][d] of dtype: raw keys, values
  const void *nk, *nv;        // optional [batch][kv_heads][d]: token len - 1, appended here
  void *ak, *av;              // the window buffers the appended token is stored into
  const void *q;              // [batch][q_heads][d] of qdtype
  const float *Dsg;           // rotation signs
  float *part;                // [B*Hq][splits_total][d + 2]
  float *scores;              // optional [B][Hq][score_stride]
  int dtype, qdtype, len, cap, length, q_pos, kv_heads, q_heads, G;
  int splits_total, split_idx, score_stride;
  int chunks_per_block;       // 64-token chunks per block; blockIdx.y picks the block's range
  float rope_base, scale_log2, inv_sqrt_block;
};

// 16-byte vector of window elements -> fp32 (bf16, f16: 8 elements; f32: 4)
template <int ES>
__device__ __forceinline__ void unpack_vec(const uint4 &r, bool bf, float *dst) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if constexpr (ES == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(w[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (bf) {
        dst[2 * e] = __uint_as_float(w[e] << 16);
        dst[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      } else {
        const uint16_t lo = uint16_t(w[e]), hi = uint16_t(w[e] >> 16);
        _Float16 a, b;
        __builtin_memcpy(&a, &lo, 2);
        __builtin_memcpy(&b, &hi, 2);
        dst[2 * e] = float(a);
        dst[2 * e + 1] = float(b);
      }
    }
  }
}

// D: head dim; ES: element bytes of the window (2: bf16 / f16, 4: f32).  A chunk of 64
// tokens of K and V is read with 16-byte loads (the next chunk's are in flight while the
// current one is scored), converted into LDS, rotary-embedded there by a per-pair fp64
// angle recurrence, scored against the G rotary-embedded queries, and folded into the
// online softmax (one lane per token) and the value sums.
template <int D, int ES, int GM>
__global__ __launch_bounds__(256) void k_window(WindowArgs a) {
  constexpr int H2 = D / 2, CH = 64, RS = D + 1;     // padded rows: conflict-free column reads
  constexpr int VPR = D * ES / 16, EPV = 16 / ES;    // 16-byte vectors per row, elements per vector
  constexpr int NV = CH * VPR / 256;                 // vectors per thread per chunk, K and V each
  static_assert(NV * 256 == CH * VPR, "a chunk splits evenly over the block");
  constexpr int NGRP = 256 / H2, TPG = CH / NGRP;    // RoPE: token groups per pair index
  // GM: heads per unit rounded up (8 or 16); every thread runs HPT head slots without a
  // branch per head, slots past G working on zero rows
  constexpr int HS = 256 / D, HPT = GM / HS;
  static_assert(GM == 8 || GM == 16, "head slots");
  __shared__ __align__(16) float qr[GM][D];
  __shared__ float kr[CH * RS];
  __shared__ float vr[CH * RS];
  __shared__ __align__(16) float ps[GM][CH];
  __shared__ float mstat[3][GM];   // running max (log2 units), sum, this chunk's rescale
  __shared__ float qrot[2][H2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, unit = blockIdx.x;
  const int b = unit / a.kv_heads, g = unit % a.kv_heads, G = a.G, hq0 = g * G;
  const bool rope = a.rope_base != 0.0f, bf = a.dtype == TQ_BF16;
  const size_t ubase = size_t(unit) * a.cap;
  // this block's tokens: chunks [blockIdx.y * cpb, ...) of the window
  const int t_begin = blockIdx.y * a.chunks_per_block * CH;
  const int t_end = min(a.len, t_begin + a.chunks_per_block * CH);
  const char *kb = static_cast<const char *>(a.k), *vb = static_cast<const char *>(a.v);
  uint4 kreg[NV], vreg[NV];
  // chunk c0 into registers; the token this call appends (row len - 1) comes from nk, nv
  auto fetch = [&](int c0) {
    const int cn = min(CH, t_end - c0);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = tid + k * 256, t = vi / VPR, col = (vi % VPR) * EPV;
      if (t < cn) {
        const bool fresh = a.nk && c0 + t == a.len - 1;
        const size_t off = (fresh ? size_t(unit) * D + col : (ubase + c0 + t) * D + col) * ES;
        kreg[k] = *reinterpret_cast<const uint4 *>((fresh ? static_cast<const char *>(a.nk) : kb) + off);
        vreg[k] = *reinterpret_cast<const uint4 *>((fresh ? static_cast<const char *>(a.nv) : vb) + off);
      }
    }
  };
  fetch(t_begin);
  // this thread's query pairs, loaded before the fp64 angles are computed
  constexpr int QPT = GM * H2 / 256;
  static_assert(QPT * 256 == GM * H2, "query pairs split evenly over the block");
  float qx0[QPT], qx1[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * 256, h = i / H2, j = i % H2;
    qx0[k] = 0.0f;
    qx1[k] = 0.0f;
    if (i < G * H2) {
      const size_t base = (size_t(b) * a.q_heads + hq0 + h) * D;
      qx0[k] = load_elem(a.q, base + j, a.qdtype);
      qx1[k] = load_elem(a.q, base + j + H2, a.qdtype);
    }
  }
  // fp64 frequency of this thread's pair index (the keys' RoPE steps token by token)
  const int jp = tid % H2, grp = tid / H2;
  const double theta = rope ? exp2(-2.0 * double(jp) / double(D) * log2(double(a.rope_base))) : 0.0;
  // angle of token grp * TPG of this block's first chunk, stepped by theta within a chunk
  // and by (CH - TPG) theta from one chunk to the next, all in fp64
  double sd = 0.0, cd = 1.0, sj = 0.0, cj = 1.0, sg = 0.0, cg = 1.0;
  if (rope) {
    sincos(theta, &sd, &cd);
    sincos(double(CH - TPG) * theta, &sj, &cj);
    sincos(double(a.length + t_begin + grp * TPG) * theta, &sg, &cg);
  }
  if (tid < H2) {
    double sn = 0.0, c = 1.0;
    if (rope) sincos(double(a.q_pos) * theta, &sn, &c);
    qrot[0][tid] = float(c);
    qrot[1][tid] = float(sn);
  }
  if (tid < GM) {
    mstat[0][tid] = -INFINITY;
    mstat[1][tid] = 0.0f;
    mstat[2][tid] = 0.0f;
  }
  for (int i = tid; i < GM * CH; i += 256) (&ps[0][0])[i] = 0.0f;
  for (int i = G * D + tid; i < GM * D; i += 256) (&qr[0][0])[i] = 0.0f;
  __syncthreads();
  // RoPE(q) of the unit's heads, unrotated
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * 256, h = i / H2, j = i % H2;
    if (i >= G * H2) break;
    const float x0 = qx0[k], x1 = qx1[k];
    if (rope) {
      const float c = qrot[0][j], sn = qrot[1][j];
      qr[h][j] = x0 * c - x1 * sn;
      qr[h][j + H2] = x0 * sn + x1 * c;
    } else {
      qr[h][j] = x0;
      qr[h][j + H2] = x1;
    }
  }
  const int jv = tid % D, hs = tid / D;
  float acc[HPT];
#pragma unroll
  for (int k = 0; k < HPT; ++k) acc[k] = 0.0f;
  for (int c0 = t_begin; c0 < t_end; c0 += CH) {
    const int cn = min(CH, t_end - c0);
    __syncthreads();   // the previous chunk's readers are done
    // rows past the chunk's end are zero, so the loops below run over whole chunks
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = tid + k * 256, t = vi / VPR, col = (vi % VPR) * EPV;
      if (t < cn) {
        unpack_vec<ES>(kreg[k], bf, &kr[t * RS + col]);
        unpack_vec<ES>(vreg[k], bf, &vr[t * RS + col]);
        if (a.nk && c0 + t == a.len - 1) {   // store the appended token into its window row
          const size_t off = ((ubase + c0 + t) * D + col) * ES;
          *reinterpret_cast<uint4 *>(static_cast<char *>(a.ak) + off) = kreg[k];
          *reinterpret_cast<uint4 *>(static_cast<char *>(a.av) + off) = vreg[k];
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          kr[t * RS + col + e] = 0.0f;
          vr[t * RS + col + e] = 0.0f;
        }
      }
    }
    if (c0 + CH < t_end) fetch(c0 + CH);
    __syncthreads();
    if (rope) {
      // pair jp of tokens grp * TPG .. + TPG: angles stepped from one fp64 sincos, then
      // all reads, then all rotations
      const int t0 = grp * TPG;
      float cf[TPG], sf[TPG], x0[TPG], x1[TPG];
      double sn = sg, c = cg;
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        cf[i] = float(c);
        sf[i] = float(sn);
        const double cn2 = c * cd - sn * sd;
        sn = sn * cd + c * sd;
        c = cn2;
      }
      {   // the same token group of the next chunk
        const double cn2 = c * cj - sn * sj;
        sg = sn * cj + c * sj;
        cg = cn2;
      }
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        x0[i] = kr[(t0 + i) * RS + jp];
        x1[i] = kr[(t0 + i) * RS + jp + H2];
      }
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        kr[(t0 + i) * RS + jp] = x0[i] * cf[i] - x1[i] * sf[i];
        kr[(t0 + i) * RS + jp + H2] = x0[i] * sf[i] + x1[i] * cf[i];
      }
      __syncthreads();
    }
    // scores: token = lane, heads wv + 8i and wv + 8i + 4; one read of the key row serves both
    for (int h0 = wv; h0 < G; h0 += 8) {
      const int t = lane;
      const float *krow = &kr[t * RS];
      if (h0 + 4 < G) {
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll 8
        for (int j = 0; j < D; j += 4) {
          const float4 qa = *reinterpret_cast<const float4 *>(&qr[h0][j]);
          const float4 qb = *reinterpret_cast<const float4 *>(&qr[h0 + 4][j]);
          const float k0 = krow[j], k1 = krow[j + 1], k2 = krow[j + 2], k3 = krow[j + 3];
          s0 = fmaf(qa.x, k0, s0);
          s1 = fmaf(qa.y, k1, s1);
          s0 = fmaf(qa.z, k2, s0);
          s1 = fmaf(qa.w, k3, s1);
          s2 = fmaf(qb.x, k0, s2);
          s3 = fmaf(qb.y, k1, s3);
          s2 = fmaf(qb.z, k2, s2);
          s3 = fmaf(qb.w, k3, s3);
        }
        ps[h0][t] = s0 + s1;
        ps[h0 + 4][t] = s2 + s3;
      } else {
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll 8
        for (int j = 0; j < D; j += 4) {
          const float4 qa = *reinterpret_cast<const float4 *>(&qr[h0][j]);
          s0 = fmaf(qa.x, krow[j], s0);
          s1 = fmaf(qa.y, krow[j + 1], s1);
          s2 = fmaf(qa.z, krow[j + 2], s2);
          s3 = fmaf(qa.w, krow[j + 3], s3);
        }
        ps[h0][t] = (s0 + s1) + (s2 + s3);
      }
    }
    __syncthreads();
    // online softmax, one lane per token, heads h0 and h0 + 4 of a wave side by side (the
    // second is a zero row when h0 + 4 >= G); the scores go out unscaled
    for (int h0 = wv; h0 < G; h0 += 8) {
      const int h1 = h0 + 4;
      const bool two = h1 < G;
      const float s0 = ps[h0][lane], s1 = ps[h1 < GM ? h1 : h0][lane];
      if (a.scores && lane < cn) {
        float *srow = a.scores + (size_t(b) * a.q_heads + hq0) * a.score_stride + a.length + c0 + lane;
        srow[size_t(h0) * a.score_stride] = s0;
        if (two) srow[size_t(h1) * a.score_stride] = s1;
      }
      float v0 = lane < cn ? s0 * a.scale_log2 : -INFINITY;
      float v1 = lane < cn ? s1 * a.scale_log2 : -INFINITY;
      float m0 = v0, m1 = v1;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        m0 = fmaxf(m0, __shfl_xor(m0, o, 64));
        m1 = fmaxf(m1, __shfl_xor(m1, o, 64));
      }
      const float mold0 = mstat[0][h0], mnew0 = fmaxf(mold0, m0);
      const float mold1 = two ? mstat[0][h1] : -INFINITY, mnew1 = fmaxf(mold1, m1);
      const float al0 = mold0 == -INFINITY ? 0.0f : exp2f(mold0 - mnew0);
      const float al1 = mold1 == -INFINITY ? 0.0f : exp2f(mold1 - mnew1);
      const float p0 = lane < cn ? exp2f(v0 - mnew0) : 0.0f;
      const float p1 = lane < cn ? exp2f(v1 - mnew1) : 0.0f;
      float l0 = p0, l1 = p1;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        l0 += __shfl_xor(l0, o, 64);
        l1 += __shfl_xor(l1, o, 64);
      }
      ps[h0][lane] = p0;
      if (two) ps[h1][lane] = p1;
      if (lane == 0) {
        mstat[0][h0] = mnew0;
        mstat[1][h0] = mstat[1][h0] * al0 + l0;
        mstat[2][h0] = al0;
        if (two) {
          mstat[0][h1] = mnew1;
          mstat[1][h1] = mstat[1][h1] * al1 + l1;
          mstat[2][h1] = al1;
        }
      }
    }
    __syncthreads();
    // values: one read of vr per token serves all of this thread's heads
    {
      float o[HPT];
#pragma unroll
      for (int k = 0; k < HPT; ++k) o[k] = acc[k] * mstat[2][hs + k * HS];
#pragma unroll 4
      for (int t = 0; t < CH; t += 4) {
        const float v0 = vr[t * RS + jv], v1 = vr[(t + 1) * RS + jv];
        const float v2 = vr[(t + 2) * RS + jv], v3 = vr[(t + 3) * RS + jv];
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
          const float4 p = *reinterpret_cast<const float4 *>(&ps[hs + k * HS][t]);
          o[k] = fmaf(p.x, v0, o[k]);
          o[k] = fmaf(p.y, v1, o[k]);
          o[k] = fmaf(p.z, v2, o[k]);
          o[k] = fmaf(p.w, v3, o[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < HPT; ++k) acc[k] = o[k];
    }
  }
  __syncthreads();
  // Pi acc = H (D .* acc) / sqrt(B) per head (Hadamard block = d here), then the partial
  float *ys = kr;   // [GM][D]
#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    const int h = hs + k * HS;
    if (h < G) ys[h * D + jv] = acc[k] * a.Dsg[jv];
  }
  __syncthreads();
  for (int st = 1; st < D; st <<= 1) {
    for (int i = tid; i < G * H2; i += 256) {
      const int h = i / H2, kk = i % H2;
      const int j = (kk / st) * 2 * st + (kk % st);
      const float x0 = ys[h * D + j], x1 = ys[h * D + j + st];
      ys[h * D + j] = x0 + x1;
      ys[h * D + j + st] = x0 - x1;
    }
    __syncthreads();
  }
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, j = i % D;
    float *o = a.part + ((size_t(b) * a.q_heads + hq0 + h) * a.splits_total + a.split_idx + blockIdx.y) * (D + 2);
    o[j] = ys[h * D + j] * a.inv_sqrt_block;
    if (j == 0) {
      o[D] = mstat[0][h] * 0.69314718055994531f;   // natural-log units, as the packed splits
      o[D + 1] = mstat[1][h];
    }
  }
}

// Max over the 64 lanes, in every lane: DPP within rows of 16 (quad swaps, rotations by 4
// and 8), then the four row results read lane by lane.
__device__ __forceinline__ float row_dpp_f32(float x, bool mx) {
  const auto op = [mx](float u, float v) { return mx ? fmaxf(u, v) : u + v; };
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true)));
  return x;
}
__device__ __forceinline__ float lane_f32(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = row_dpp_f32(x, true);
  return fmaxf(fmaxf(lane_f32(x, 0), lane_f32(x, 16)), fmaxf(lane_f32(x, 32), lane_f32(x, 48)));
}

// ------------------------------------------------------------------ PolarQuant decode
// Split-K decode over PolarQuant records ([TurboQuant] "PolarQuant" as stage 1, QJL on
// the key residual).  Each of a block's 8 waves walks its own 32-token steps of the
// block's range with its own online-softmax state (a split inside the split); the block
// combines the 8 states at the end.  A step's records come in with 16- and 8-byte loads
// (the wave's next step in flight meanwhile) and are staged in the wave's own LDS rows.
//   keys: lane = (token, quarter of the coordinates): the lane decodes its quarter's
//         angle subtree (the two top levels give the quarter's radius), splits the
//         coordinates into fp16 hi + lo and feeds them to v_mfma_f32_16x16x32_f16 as the
//         B operand; the A rows are the heads' rotated queries as fp16 hi + lo, so the
//         four cross products of hi and lo parts all land in fp32.
//   QJL:  the sign bits against the S q digit rows on v_mfma_i32_32x32x32_i8.
//   values: lane = (subtree of d / 16 coordinates, 4 consecutive tokens): the decoded
//         coordinates, times the value norm, split into fp16 hi + lo, are already the B
//         operand of v_mfma_f32_16x16x16_f16 (k = token) without any transposition; the
//         A rows are the softmax weights as fp16 hi + lo.
// The sums stay in the rotated basis: the partials are the merge's usual input.

// a compile-time int carried by a value (selects a templated lambda body)
template <int V>
struct IntTag {
  static constexpr int value = V;
};

// f(IntTag<B>), f(IntTag<B - 1>), ..., f(IntTag<E>)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for_down(F &&f) {
  if constexpr (B >= E) {
    f(IntTag<B>{});
    static_for_down<B - 1, E>(f);
  }
}

// First bit of the 2-bit angle codes of level lv >= 2 in a PolarQuant record of d
// coordinates: the d / 2 level-1 codes (4 bits each) come first, then every level's
// nodes in order, root last.
__host__ __device__ constexpr int polar_level_bit(int d, int lv) { return 2 * d + 2 * (d / 2 - (d >> (lv - 1))); }

// Bits from C + W j on of a record held as dwords, for 0 <= j < JN: one read of a fixed
// dword when every j's W bits lie in the dword holding bit C.
template <int C, int W, int JN>
__device__ __forceinline__ uint32_t rec_bits(const uint32_t *w, int j) {
  if constexpr ((C & 31) + W * JN <= 32) {
    return w[C >> 5] >> ((C & 31) + W * j);
  } else {
    const int p = C + W * j;
    return w[p >> 5] >> (p & 31);
  }
}

// 2-bit code j (0 <= j < JN) of the level whose codes start at bit C
template <int C, int JN>
__device__ __forceinline__ uint32_t rec_code(const uint32_t *w, int j) {
  if constexpr ((C & 31) + 2 * JN <= 32) {
    return __builtin_amdgcn_ubfe(w[C >> 5], (C & 31) + 2 * j, 2);
  } else {
    const int p = C + 2 * j;
    return __builtin_amdgcn_ubfe(w[p >> 5], p & 31, 2);
  }
}

// Radius of subtree J (root at level S, 0 <= J < JN) of a record, times r0: cos or sin
// of each ancestor's angle, by the branch J takes.
template <int D, int S, int JN>
__device__ __forceinline__ float polar_path_radius(const uint32_t *w, int J, float r0, const float2 (*csh)[4]) {
  constexpr int L = D == 128 ? 7 : 6;
  // cos or sin of each ancestor's code, read as one float (the branch picks the
  // component), every level's read in flight before the first product
  float c[L - S];
  static_for_down<L, S + 1>([&](auto t) {
    constexpr int lv = decltype(t)::value, up = lv - S;
    constexpr int nodes = (JN + (1 << up) - 1) >> up;
    const uint32_t code = rec_code<polar_level_bit(D, lv), nodes>(w, J >> up);
    const uint32_t off = (code << 3) + uint32_t(((J >> (up - 1)) & 1) << 2);   // bytes into the level's table
    c[lv - S - 1] = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(&csh[lv - 2][0]) + off);
  });
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = L - S - 1; i >= 0; --i) r0 *= c[i];
  return r0;
}

// Radii of the level-1 pairs of subtree J (root at level S, radius r0): each subtree
// level splits every radius into its cos and sin parts.  r gets 2^(S-1) radii.
template <int D, int S, int JN>
__device__ __forceinline__ void polar_sub_radii(const uint32_t *w, int J, float r0, const float2 (*csh)[4],
                                                float *r) {
  r[0] = r0;
  static_for_down<S, 2>([&](auto t) {
    constexpr int lv = decltype(t)::value, n = 1 << (S - lv);
    const uint32_t f = rec_bits<polar_level_bit(D, lv), 2 * n, JN>(w, J);
    // the level's lookups are all issued before the first product waits on one
    float2 cs[n];
#pragma unroll
    for (int i = 0; i < n; ++i) cs[i] = csh[lv - 2][(f >> (2 * i)) & 3u];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = n - 1; i >= 0; --i) {
      const float rr = r[i];
      r[2 * i] = rr * cs[i].x;
      r[2 * i + 1] = rr * cs[i].y;
    }
  });
}

template <int D, int S, int JN>
__device__ __forceinline__ void polar_pair_radii(const uint32_t *w, int J, float r0, const float2 (*csh)[4],
                                                 float *r) {
  polar_sub_radii<D, S, JN>(w, J, polar_path_radius<D, S, JN>(w, J, r0, csh), csh, r);
}

// Orders a wave's LDS writes before its later reads of other lanes' data (and the reads
// before later writes): the LDS serves one wave's requests in order, so only the
// compiler's ordering is at stake.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct PolarArgs {
  const uint8_t *krec;     // [units][capacity][kb]: 3 D / 8 angle bytes, m / 8 sign bytes
  const uint32_t *knorm;   // {fp16 n, fp16 |r|}
  const uint8_t *vrec;     // [units][capacity][3 D / 8]
  const uint16_t *vnorm;
  const float *qp;         // query rows: Pi RoPE(q) [D], S q [m], sum q_rot, sum S q
  const uint8_t *qpack;    // per unit: int8 digit rows (the S q rows are used) and coefficients
  const float *pcs;        // cos, sin of the angle centroids [level - 1][16][2]
  float *part, *scores;
  int kb, capacity, length, chunk, splits, kv_heads, q_heads, G, m, qstride, score_stride;
  float scale_log2;
};

typedef __fp16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// PolarQuant decode blocks: 4 waves, 3 blocks per CU (3 waves per SIMD, up to 168
// registers each: room for the table lookups of a decode level to be in flight together)
constexpr int kPolarWaves = 4, kPolarBlocksPerCU = 3;

template <int D>
__global__ __launch_bounds__(64 * kPolarWaves, kPolarBlocksPerCU * kPolarWaves / 4) void k_decode_polar(PolarArgs a) {
  // m = D QJL rows, at most 8 heads
  constexpr int L = D == 128 ? 7 : 6, NW = kPolarWaves, NT = 64 * NW, ST = 32;
  constexpr int KW = D / 8, VW = 3 * D / 32;    // record dwords: key (angles, signs), value
  constexpr int KWP = KW + 1, VWP = VW + 1;     // odd LDS strides: one token per bank
  constexpr int NQ = D / 4, NK = D / 32;        // key quarter; f16 MFMAs per hi or lo part
  constexpr int CPL = D / 16;                   // value coordinates per lane (a subtree)
  constexpr int SK = L - 2, SV = CPL == 8 ? 3 : 2;
  constexpr int KQ = ST * KW / 4, KQL = (KQ + 63) / 64;   // 16-byte key loads per step, per lane
  constexpr int VQ = ST * VW / 2, VQL = (VQ + 63) / 64;   // 8-byte value loads
  // the decoded key coordinates (|y| <= 1) are scaled by 2^8 before the split, and each
  // head's query by a power of two that brings its largest element into [2^7, 2^8): the
  // fp16 parts stay normal and far from overflow; the dot products are scaled back
  constexpr float kYScale = 256.0f;
  __shared__ __align__(16) v8h qa[NK][64];      // key A operands in lane order
  __shared__ __align__(16) v4i qsa[NK][64];     // QJL A operands (S q digit rows) in lane order
  __shared__ float2 cs1[16];                    // level-1 centroids' (cos, sin)
  __shared__ float2 csh[L - 1][4];              // higher levels' (cos, sin): [level - 2][code]
  __shared__ float qsc[8], qiv[8];              // query scale per head and 1 / (scale 2^8)
  __shared__ float qjc[2][8];                   // 2 qjl 2^16 / 2^e and qjl sum S q per head
  __shared__ uint32_t krs[NW][ST * KWP];        // each wave's staged records
  __shared__ uint32_t vrs[NW][ST * VWP];
  __shared__ uint32_t kns[NW][ST];
  __shared__ float vns[NW][ST];
  __shared__ __align__(16) float dts[NW][ST][8];   // <q_rot, yhat> by token and head
  __shared__ __align__(16) float pts[NW][8][ST];   // softmax weights by head and token
  __shared__ float wst[2][NW][8];               // per wave: reference maximum and sum per head
  __shared__ float ys[8][D];                    // the block's value sums
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / a.kv_heads, g = unit % a.kv_heads, G = a.G, hq0 = g * G;
  const int t_begin = split * a.chunk, t_end = min(a.length, t_begin + a.chunk);
  const size_t ubase = size_t(unit) * a.capacity;
  const float *qrow = a.qp + size_t(b * a.q_heads + hq0) * a.qstride;
  if (tid < 16) cs1[tid] = make_float2(a.pcs[2 * tid], a.pcs[2 * tid + 1]);
  if (tid < 4 * (L - 1)) {
    const int lv = 2 + tid / 4, c = tid % 4;
    csh[lv - 2][c] = make_float2(a.pcs[((lv - 1) * 16 + c) * 2], a.pcs[((lv - 1) * 16 + c) * 2 + 1]);
  }
  const uint8_t *qpk = a.qpack + size_t(unit) * qpack_unit_bytes(D);
  if (tid < 8) {
    const float *coef = reinterpret_cast<const float *>(qpk + size_t(kQpackVecs) * 32 * 2 * NK * 16);
    qjc[0][tid] = coef[tid * kQpackCoef + 3];
    qjc[1][tid] = coef[tid * kQpackCoef + 4];
  }
  for (int i = tid; i < 8 * D; i += NT) (&ys[0][0])[i] = 0.0f;
  for (int h = wv; h < 8; h += NW) {
    // the scale of head h's query
    float mx = 0.0f;
    if (h < G)
      for (int j = lane; j < D; j += 64) mx = fmaxf(mx, fabsf(qrow[size_t(h) * a.qstride + j]));
    mx = wave_max_dpp(mx);
    if (lane == 0) {
      int ex = 0;
      if (mx > 0.0f) frexpf(mx, &ex);   // mx < 2^ex
      const float s = mx > 0.0f ? ldexpf(1.0f, 8 - ex) : 1.0f;
      qsc[h] = h < G ? s : 0.0f;
      qiv[h] = h < G ? 1.0f / (s * kYScale) : 0.0f;
    }
  }
  __syncthreads();
  // key A operand of MFMA k: lane (row m, group q) holds coordinates q NQ + 8 k .. + 7 of
  // row m; rows 4 i .. 4 i + 3 are head 2 i hi, lo and head 2 i + 1 hi, lo, so that the
  // lanes of result row group i hold both parts of two heads
  for (int i = tid; i < NK * 64; i += NT) {
    const int k = i / 64, l = i % 64, mrow = l & 15, qg = l >> 4;
    const int h = 2 * (mrow >> 2) + ((mrow >> 1) & 1), part = mrow & 1;
    v8h v;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = h < G ? qrow[size_t(h) * a.qstride + qg * NQ + 8 * k + j] * qsc[h] : 0.0f;
      const _Float16 hi = _Float16(q);
      v[j] = part ? _Float16(q - float(hi)) : hi;
    }
    qa[k][l] = v;
  }
  {
    const v4i *src = reinterpret_cast<const v4i *>(qpk);
    for (int i = tid; i < NK * 64; i += NT) {
      const int c = i / 64, l = i % 64;
      qsa[c][l] = src[((kSqVec * 32 + (l & 31)) * 2 + (l >> 5)) * NK + c];
    }
  }
  __syncthreads();

  const int nsteps = t_end > t_begin ? (t_end - t_begin + ST - 1) / ST : 0;
  float mref[4], lsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mref[r] = -INFINITY;
    lsum[r] = 0.0f;
  }
  v4f acc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  uint4 pk[KQL];
  uint2 pv[VQL];
  uint32_t pn = 0u;
  auto fetch = [&](int s) {
    const int t0 = t_begin + s * ST, cn = min(ST, t_end - t0);
    const int t32 = lane & 31, hf = lane >> 5;
    const size_t tb = ubase + size_t(t0);   // uniform bases, lane offsets below 2^31
    const uint4 *ks = reinterpret_cast<const uint4 *>(a.krec + tb * (KW * 4));
    const uint2 *vs = reinterpret_cast<const uint2 *>(a.vrec + tb * (VW * 4));
    const uint32_t *kn = a.knorm + tb;
    const uint16_t *vn = a.vnorm + tb;
#pragma unroll
    for (int r = 0; r < KQL; ++r) {
      const int i = lane + 64 * r;
      pk[r] = i < KQ && i / (KW / 4) < cn ? ks[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < VQL; ++r) {
      const int i = lane + 64 * r;
      pv[r] = i < VQ && i / (VW / 2) < cn ? vs[i] : make_uint2(0u, 0u);
    }
    if (hf == 0)
      pn = t32 < cn ? kn[t32] : 0u;
    else
      pn = t32 < cn ? uint32_t(vn[t32]) : 0u;
  };
  if (wv < nsteps) fetch(wv);
  for (int s = wv; s < nsteps; s += NW) {
    const int t0 = t_begin + s * ST, cn = min(ST, t_end - t0);
    // the lane index is made opaque to the compiler in each step, so that the many lane
    // dependent LDS addresses and shifts below are formed where they are used instead of
    // being held in registers across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n16 = ln & 15, grp = ln >> 4;   // MFMA column and lane group
    const int t32 = ln & 31, hf = ln >> 5;    // QJL / softmax: token and half of the heads
    // ---- stage this step's records (rows past the range are zero), then start the next
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < KQL; ++r) {
      const int i = lane + 64 * r;
      if (i < KQ) {
        uint32_t *d = &krs[wv][(i / (KW / 4)) * KWP + (i % (KW / 4)) * 4];
        d[0] = pk[r].x;
        d[1] = pk[r].y;
        d[2] = pk[r].z;
        d[3] = pk[r].w;
      }
    }
#pragma unroll
    for (int r = 0; r < VQL; ++r) {
      const int i = lane + 64 * r;
      if (i < VQ) {
        uint32_t *d = &vrs[wv][(i / (VW / 2)) * VWP + (i % (VW / 2)) * 2];
        d[0] = pv[r].x;
        d[1] = pv[r].y;
      }
    }
    if (hf == 0)
      kns[wv][t32] = pn;
    else
      vns[wv][t32] = f16_bits_to_float(pn);
    if (s + NW < nsteps) fetch(s + NW);
    wave_lds_sync();

    // ---- keys, 16 tokens at a time: lane = (token n16, quarter grp)
#pragma unroll 1
    for (int sb = 0; sb < 2; ++sb) {
      const uint32_t *w = &krs[wv][(16 * sb + n16) * KWP];
      float r[NQ / 2];
      polar_pair_radii<D, SK, 4>(w, grp, kYScale, csh, r);
      v4f kacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        // coordinates 8 k .. 8 k + 7 of the quarter: level-1 pairs 4 k .. 4 k + 3
        const uint32_t nib = w[(2 * NQ * grp + 16 * k) >> 5] >> ((16 * k) & 31);
        float2 cs4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) cs4[p] = cs1[(nib >> (4 * p)) & 15u];
        __builtin_amdgcn_sched_barrier(0);
        v4u hb, lb;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float2 cs = cs4[p];
          const float y0 = r[4 * k + p] * cs.x, y1 = r[4 * k + p] * cs.y;
          const h2v hh = __builtin_amdgcn_cvt_pkrtz(y0, y1);
          const h2v hl = __builtin_amdgcn_cvt_pkrtz(y0 - float(hh.x), y1 - float(hh.y));
          hb[p] = __builtin_bit_cast(uint32_t, hh);
          lb[p] = __builtin_bit_cast(uint32_t, hl);
        }
        const v8h A = qa[k][lane];
        kacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(v8h, hb), kacc, 0, 0, 0);
        kacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(v8h, lb), kacc, 0, 0, 0);
      }
      // lane (token n16, group grp): heads 2 grp and 2 grp + 1, hi + lo rows
      *reinterpret_cast<float2 *>(&dts[wv][16 * sb + n16][2 * grp]) =
          make_float2((kacc[0] + kacc[1]) * qiv[2 * grp], (kacc[2] + kacc[3]) * qiv[2 * grp + 1]);
    }

    // ---- QJL sums: the sign bits as int8 bytes (bit e of each nibble in place) against
    // the S q digit rows; lane = (token t32, half hf of the digit rows)
    float sc[4];
    {
      const uint32_t *sgw = &krs[wv][t32 * KWP + 3 * D / 32 + hf * (D / 64)];
      const uint2 sw = make_uint2(sgw[0], D >= 128 ? sgw[1] : 0u);
      v16i s2 = {};
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        const uint32_t w = (c >> 1) ? sw.y : sw.x;
        const uint32_t nb = (c & 1) ? w >> 4 : w;
        v4i bp;
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[e] = int(nb & (0x01010101u << e));
        s2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qsa[c][lane], bp, s2, 0, 0, 0);
      }
      const uint32_t kn = kns[wv][t32];
      const float n16f = f16_bits_to_float(kn & 0xFFFFu), rn16 = f16_bits_to_float(kn >> 16);
      const float4 dt = *reinterpret_cast<const float4 *>(&dts[wv][t32][4 * hf]);
      const float dv[4] = {dt.x, dt.y, dt.z, dt.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * hf + r;
        // digit sums: rows 8 digit + head are accumulator registers 4 digit + r
        const float S2 = fmaf(float(s2[r] + 256 * s2[4 + r]), 0x1p-16f, float(s2[8 + r] + 256 * s2[12 + r]));
        sc[r] = fmaf(n16f, dv[r], rn16 * fmaf(qjc[0][h], S2, -qjc[1][h]));
      }
    }
    const bool live = t32 < cn;
    if (a.scores && live) {
      // one head half at a time, so that every row address is uniform
      float *srow = a.scores + (size_t(b) * a.q_heads + hq0) * a.score_stride + t0;
      const size_t ss = size_t(a.score_stride);
      if (hf == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < G) srow[ss * r + t32] = sc[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 + r < G) srow[ss * (4 + r) + t32] = sc[r];
      }
    }
    // ---- online softmax with a lazy reference: the weights are 2^(v - mref), and mref
    // moves only when a logit passes it by more than 8, so the weights stay below 2^8
    float v[4];
    bool up = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = live ? sc[r] * a.scale_log2 : -INFINITY;
      up = up || v[r] > mref[r] + 8.0f;
    }
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // the maximum over each half's 32 tokens ends in lanes 31 and 63
        const int mx = dpp_max32_tail(f2ord(v[r]));
        const float m0 = ord2f(__builtin_amdgcn_readlane(mx, 31)), m1 = ord2f(__builtin_amdgcn_readlane(mx, 63));
        const float mn = fmaxf(mref[r], hf ? m1 : m0);
        al[r] = mref[r] == -INFINITY ? 0.0f : exp2f(mref[r] - mn);
        mref[r] = mn;
        lsum[r] *= al[r];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al[i]), 0));
        const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al[i]), 32));
        const float ai = (grp & 1) ? a1 : a0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) acc[j][i] *= ai;
      }
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = exp2f(v[r] - mref[r]);   // 0 past the range
      lsum[r] += p[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) pts[wv][4 * hf + r][t32] = p[r];
    wave_lds_sync();

    // ---- values, 16 tokens at a time: lane = (subtree n16, tokens 4 grp .. 4 grp + 3),
    // which is the B layout of v_mfma_f32_16x16x16_f16 (k = token); the A rows are the
    // weights as fp16 hi (rows 0..7) and lo (rows 8..15), B the coordinates as fp16 hi
    // and lo in two products, so every cross product of the parts lands in fp32.
    // acc[j] (rows = head parts, columns = subtrees) sums coordinate CPL n16 + j.
#pragma unroll 1
    for (int vb = 0; vb < ST / 16; ++vb) {
      if (16 * vb < cn) {
        const float4 p4 = *reinterpret_cast<const float4 *>(&pts[wv][n16 & 7][16 * vb + 4 * grp]);
        h2v pa0 = __builtin_amdgcn_cvt_pkrtz(p4.x, p4.y), pa1 = __builtin_amdgcn_cvt_pkrtz(p4.z, p4.w);
        if (n16 & 8) {
          pa0 = __builtin_amdgcn_cvt_pkrtz(p4.x - float(pa0.x), p4.y - float(pa0.y));
          pa1 = __builtin_amdgcn_cvt_pkrtz(p4.z - float(pa1.x), p4.w - float(pa1.y));
        }
        const v4h A = __builtin_bit_cast(v4h, make_uint2(__builtin_bit_cast(uint32_t, pa0),
                                                         __builtin_bit_cast(uint32_t, pa1)));
        // the subtree in two halves (the children of its root), so that only half of
        // the B operands are live at a time; the second half's radius is kept per token
        constexpr int HC = CPL / 2;   // coordinates per half
        float rho1[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t bh[HC][2], bl[HC][2];   // coordinate j of tokens (0, 1) and (2, 3)
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            float vc[2][HC];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int tk = 16 * vb + 4 * grp + 2 * i2 + i;
              const uint32_t *w = &vrs[wv][tk * VWP];
              float rh;
              if (hh == 0) {
                const float rho = polar_path_radius<D, SV, 16>(w, n16, vns[wv][tk], csh);
                const float2 cs = csh[SV - 2][rec_bits<polar_level_bit(D, SV), 2, 16>(w, n16) & 3u];
                rh = rho * cs.x;
                rho1[2 * i2 + i] = rho * cs.y;
              } else {
                rh = rho1[2 * i2 + i];
              }
              float r[HC / 2];
              polar_sub_radii<D, SV - 1, 32>(w, 2 * n16 + hh, rh, csh, r);
              const uint32_t nib = rec_bits<0, CPL, 32>(w, 2 * n16 + hh);
              float2 cs2[HC / 2];
#pragma unroll
              for (int e = 0; e < HC / 2; ++e) cs2[e] = cs1[(nib >> (4 * e)) & 15u];
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int e = 0; e < HC / 2; ++e) {
                vc[i][2 * e] = r[e] * cs2[e].x;
                vc[i][2 * e + 1] = r[e] * cs2[e].y;
              }
            }
#pragma unroll
            for (int j = 0; j < HC; ++j) {
              const h2v hv = __builtin_amdgcn_cvt_pkrtz(vc[0][j], vc[1][j]);
              const h2v lv = __builtin_amdgcn_cvt_pkrtz(vc[0][j] - float(hv.x), vc[1][j] - float(hv.y));
              bh[j][i2] = __builtin_bit_cast(uint32_t, hv);
              bl[j][i2] = __builtin_bit_cast(uint32_t, lv);
            }
          }
#pragma unroll
          for (int j = 0; j < HC; ++j) {
            v4f &c = acc[HC * hh + j];
            c = __builtin_amdgcn_mfma_f32_16x16x16f16(A, __builtin_bit_cast(v4h, make_uint2(bh[j][0], bh[j][1])), c,
                                                      0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x16f16(A, __builtin_bit_cast(v4h, make_uint2(bl[j][0], bl[j][1])), c,
                                                      0, 0, 0);
          }
        }
      }
    }
  }

  // ---- the block's combination of its 8 wave states: sums per head over each half's
  // lanes, the block maximum, then the waves' scaled value sums added in wave order
  const int n16 = lane & 15, grp = lane >> 4, t32 = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float ls = lsum[r];
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) ls += __shfl_xor(ls, o, 64);
    if (t32 == 0) {
      wst[0][wv][4 * hf + r] = mref[r];
      wst[1][wv][4 * hf + r] = ls;
    }
  }
  __syncthreads();
  float fac[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * (grp & 1) + i;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wst[0][w][h]);
    const float mw = wst[0][wv][h];
    fac[i] = mw == -INFINITY ? 0.0f : exp2f(mw - M);
  }
  // the lo rows (lane groups 2, 3) onto the hi rows of the same heads
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] += __shfl_xor(acc[j][i], 32, 64);
  for (int w = 0; w < NW; ++w) {
    if (wv == w && grp < 2) {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) ys[4 * grp + i][CPL * n16 + j] += acc[j][i] * fac[i];
    }
    __syncthreads();
  }
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, j = i % D;
    float *o = a.part + ((size_t(b) * a.q_heads + hq0 + h) * a.splits + split) * (D + 2);
    o[j] = ys[h][j];
    if (j == 0) {
      float M = -INFINITY;
      for (int w = 0; w < NW; ++w) M = fmaxf(M, wst[0][w][h]);
      float l = 0.0f;
      for (int w = 0; w < NW; ++w)
        if (wst[0][w][h] != -INFINITY) l += wst[1][w][h] * exp2f(wst[0][w][h] - M);
      o[D] = M == -INFINITY ? -INFINITY : M * 0.69314718055994531f;   // natural-log units
      o[D + 1] = l;
    }
  }
}

// Merge of the splits and inverse rotation: out = D .* (H o) / sqrt(B) = Pi^T o.
// One block per (batch, q-head) row; split maxima and sums go through LDS first.
__global__ __launch_bounds__(256) void k_decode_merge(const float *part, int splits, int d,
                                                      CodecPtrs cp, float *out) {
  extern __shared__ float ms[];   // [splits] weights, d outputs, then [256 / d][d] partial sums
  float *os = ms + splits;
  __shared__ float red[2][4];
  const int rowi = blockIdx.x, tid = threadIdx.x;
  const float *pr = part + size_t(rowi) * splits * (d + 2);
  float mx = -INFINITY;
  for (int s = tid; s < splits; s += 256) mx = fmaxf(mx, pr[size_t(s) * (d + 2) + d]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[0][tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float L = 0.0f;
  for (int s = tid; s < splits; s += 256) {
    const float m_s = pr[size_t(s) * (d + 2) + d];
    const float w = m_s == -INFINITY ? 0.0f : __expf(m_s - mx);
    ms[s] = w;
    L += w * pr[size_t(s) * (d + 2) + d + 1];
  }
  L = wave_sum(L);
  if ((tid & 63) == 0) red[1][tid >> 6] = L;
  __syncthreads();
  L = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float invL = L > 0.0f ? 1.0f / L : 0.0f;
  // coordinate j over the splits of one parity class per thread group, 8 loads in flight
  const int groups = 256 / d > 0 ? 256 / d : 1;
  float *acc2 = os + d;   // [groups][d]
  for (int jt = tid; jt < d * groups; jt += 256) {
    const int j = jt % d, g0 = jt / d;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int s = g0;
    for (; s + 7 * groups < splits; s += 8 * groups) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] += pr[size_t(s + u * groups) * (d + 2) + j] * ms[s + u * groups];
    }
    for (; s < splits; s += groups) v[0] += pr[size_t(s) * (d + 2) + j] * ms[s];
    acc2[g0 * d + j] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  }
  __syncthreads();
  for (int j = tid; j < d; j += 256) {
    float v = 0.0f;
    for (int g0 = 0; g0 < groups; ++g0) v += acc2[g0 * d + j];
    os[j] = v * invL;
  }
  __syncthreads();
  const int B = cp.block;
  for (int hh = 1; hh < B; hh <<= 1) {
    for (int k = tid; k < d / 2; k += 256) {
      const int blk = k / (B / 2), kk = k % (B / 2);
      const int i = blk * B + (kk / hh) * 2 * hh + (kk % hh);
      const float x0 = os[i], x1 = os[i + hh];
      os[i] = x0 + x1;
      os[i + hh] = x0 - x1;
    }
    __syncthreads();
  }
  for (int j = tid; j < d; j += 256) out[size_t(rowi) * d + j] = os[j] * cp.inv_sqrt_block * cp.D[j];
}

// The same merge for d = 64 or 128 (Hadamard block = d) with one wave per (batch, q-head)
// row and no block barriers: lane l holds coordinates E l .. E l + E - 1, the split
// weights are broadcast from the lanes that computed them, and the FWHT runs in registers
// and across lanes.
template <int D>
__global__ __launch_bounds__(256) void k_decode_merge_wave(const float *part, int splits, int rows,
                                                           CodecPtrs cp, float *out) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int rowi = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rowi >= rows) return;
  const float *pr = part + size_t(rowi) * splits * (D + 2);
  float dsc[E];   // output scale D_j / sqrt(B), loaded up front with everything else
#pragma unroll
  for (int e = 0; e < E; ++e) dsc[e] = cp.D[E * lane + e] * cp.inv_sqrt_block;
  float x[E], L = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = 0.0f;
  constexpr int SMAX = 16;
  if (splits <= SMAX) {
    // all loads issued before any arithmetic: one memory round trip
    float m_s = -INFINITY, l_s = 0.0f, xs[SMAX][E];
    if (lane < splits) {
      m_s = pr[size_t(lane) * (D + 2) + D];
      l_s = pr[size_t(lane) * (D + 2) + D + 1];
    }
#pragma unroll
    for (int u = 0; u < SMAX; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) xs[u][e] = u < splits ? pr[size_t(u) * (D + 2) + E * lane + e] : 0.0f;
    const float mx = wave_max(m_s);
    const float w = m_s == -INFINITY ? 0.0f : __expf(m_s - mx);
    L = w * l_s;
#pragma unroll
    for (int u = 0; u < SMAX; ++u) {
      const float wu = __shfl(w, u, 64);
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = fmaf(xs[u][e], wu, x[e]);
    }
  } else {
  float mx = -INFINITY;
  for (int s = lane; s < splits; s += 64) mx = fmaxf(mx, pr[size_t(s) * (D + 2) + D]);
  mx = wave_max(mx);
  for (int s0 = 0; s0 < splits; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.0f;
    if (s < splits) {
      const float m_s = pr[size_t(s) * (D + 2) + D];
      w = m_s == -INFINITY ? 0.0f : __expf(m_s - mx);
      L += w * pr[size_t(s) * (D + 2) + D + 1];
    }
    const int n = min(64, splits - s0);
    for (int u = 0; u < n; ++u) {
      const float wu = __shfl(w, u, 64);
      const float *ps = pr + size_t(s0 + u) * (D + 2) + E * lane;
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = fmaf(ps[e], wu, x[e]);
    }
  }
  }
  L = wave_sum(L);
  const float invL = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] *= invL;
#pragma unroll
  for (int st = 1; st < E; st <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (!(e & st)) {
        const float u = x[e], v = x[e + st];
        x[e] = u + v;
        x[e + st] = u - v;
      }
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float p = __shfl_xor(x[e], msk, 64);
      x[e] = (lane & msk) ? p - x[e] : x[e] + p;
    }
#pragma unroll
  for (int e = 0; e < E; ++e) out[size_t(rowi) * D + E * lane + e] = x[e] * dsc[e];
}

// ------------------------------------------------------------------ search
constexpr int kSearchQ = 8;        // queries per block
constexpr int kSearchTile = 256;   // database vectors per block (one per thread)

struct SearchArgs {
  CodecPtrs cp;
  const uint8_t *kbits;
  const uint32_t *knorm;
  int kbytes, d, m, bits_k, n_db, nq, k, ntiles;
  const float *qp;
  int qstride;
  float *cand_s;
  int *cand_i;
};

// Scores of one database tile against kSearchQ queries with the decode estimator, then
// the tile's top-k per query (descending score, ties to the lower index).
__global__ __launch_bounds__(kSearchTile) void k_search_tile(SearchArgs a) {
  extern __shared__ float sm[];
  float *qr_s = sm;                         // [Q][d]
  float *sq_s = qr_s + kSearchQ * a.d;      // [Q][m]
  float *sc_s = sq_s + kSearchQ * a.m;      // [Q][tile]
  __shared__ float ck_s[kMaxCodes];
  const int tid = threadIdx.x;
  const int qt = blockIdx.y, tile = blockIdx.x;
  const int q0 = qt * kSearchQ;
  const int nqb = min(kSearchQ, a.nq - q0);
  for (int i = tid; i < kSearchQ * a.d; i += kSearchTile) {
    const int q = i / a.d, j = i % a.d;
    qr_s[i] = q < nqb ? a.qp[size_t(q0 + q) * a.qstride + j] : 0.0f;
  }
  for (int i = tid; i < kSearchQ * a.m; i += kSearchTile) {
    const int q = i / a.m, j = i % a.m;
    sq_s[i] = q < nqb ? a.qp[size_t(q0 + q) * a.qstride + a.d + j] : 0.0f;
  }
  if (tid < kMaxCodes) ck_s[tid] = a.cp.ck[tid];
  __syncthreads();
  const int x = tile * kSearchTile + tid;
  float dot[kSearchQ], qj[kSearchQ];
#pragma unroll
  for (int q = 0; q < kSearchQ; ++q) dot[q] = qj[q] = 0.0f;
  if (x < a.n_db) {
    const uint32_t *rec = reinterpret_cast<const uint32_t *>(a.kbits + size_t(x) * a.kbytes);
    const int kw = a.d / 32;
    for (int w = 0; w < kw; ++w) {
      uint32_t pl[4] = {0u, 0u, 0u, 0u};
      for (int pp = 0; pp < a.bits_k; ++pp) pl[pp] = rec[pp * kw + w];
      for (int i = 0; i < 32; ++i) {
        int code = 0;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) code |= int((pl[pp] >> i) & 1u) << pp;
        const float kh = ck_s[code];
        const int j = w * 32 + i;
#pragma unroll
        for (int q = 0; q < kSearchQ; ++q) dot[q] = fmaf(qr_s[q * a.d + j], kh, dot[q]);
      }
    }
    for (int w = 0; w < a.m / 32; ++w) {
      const uint32_t sb = rec[a.bits_k * kw + w];
      for (int i = 0; i < 32; ++i) {
        const float sgn = ((sb >> i) & 1u) ? 1.0f : -1.0f;
        const int ii = w * 32 + i;
#pragma unroll
        for (int q = 0; q < kSearchQ; ++q) qj[q] = fmaf(sq_s[q * a.m + ii], sgn, qj[q]);
      }
    }
    const uint32_t nr = a.knorm[x];
    const float n16 = f16_bits_to_float(nr & 0xFFFF), rn16 = f16_bits_to_float(nr >> 16);
#pragma unroll
    for (int q = 0; q < kSearchQ; ++q)
      sc_s[q * kSearchTile + tid] = n16 * dot[q] + rn16 * a.cp.qjl_scale * qj[q];
  } else {
#pragma unroll
    for (int q = 0; q < kSearchQ; ++q) sc_s[q * kSearchTile + tid] = -INFINITY;
  }
  __syncthreads();
  // per-tile top-k: one wave per query, k rounds of arg-max
  const int lane = tid & 63, wv = tid >> 6;
  for (int q = wv; q < nqb; q += kSearchTile / 64) {
    float prev_s = INFINITY;
    int prev_i = -1;
    for (int r = 0; r < a.k; ++r) {
      float bs = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int e = lane; e < kSearchTile; e += 64) {
        const float s = sc_s[q * kSearchTile + e];
        const int idx = tile * kSearchTile + e;
        if (idx >= a.n_db) continue;
        const bool after = (s < prev_s) || (s == prev_s && idx > prev_i);
        const bool better = (s > bs) || (s == bs && idx < bi);
        if (after && better) {
          bs = s;
          bi = idx;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float os = __shfl_xor(bs, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (os > bs || (os == bs && oi < bi)) {
          bs = os;
          bi = oi;
        }
      }
      if (lane == 0) {
        const size_t c = (size_t(q0 + q) * a.ntiles + tile) * a.k + r;
        a.cand_s[c] = bs;
        a.cand_i[c] = (bi == 0x7FFFFFFF) ? -1 : bi;
      }
      prev_s = bs;
      prev_i = bi;
    }
  }
}

// Per-query top-k over all tile candidates.
__global__ __launch_bounds__(256) void k_search_merge(const float *cand_s, const int *cand_i,
                                                      int ntiles, int k, int *idx_out,
                                                      float *score_out) {
  const int q = blockIdx.x, tid = threadIdx.x;
  const size_t n = size_t(ntiles) * k;
  const float *cs = cand_s + size_t(q) * n;
  const int *ci = cand_i + size_t(q) * n;
  __shared__ float rs[4];
  __shared__ int ri[4];
  float prev_s = INFINITY;
  int prev_i = -1;
  for (int r = 0; r < k; ++r) {
    float bs = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (size_t e = tid; e < n; e += 256) {
      const int idx = ci[e];
      if (idx < 0) continue;
      const float s = cs[e];
      const bool after = (s < prev_s) || (s == prev_s && idx > prev_i);
      const bool better = (s > bs) || (s == bs && idx < bi);
      if (after && better) {
        bs = s;
        bi = idx;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float os = __shfl_xor(bs, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (os > bs || (os == bs && oi < bi)) {
        bs = os;
        bi = oi;
      }
    }
    if ((tid & 63) == 0) {
      rs[tid >> 6] = bs;
      ri[tid >> 6] = bi;
    }
    __syncthreads();
    bs = rs[0];
    bi = ri[0];
    for (int w = 1; w < 4; ++w)
      if (rs[w] > bs || (rs[w] == bs && ri[w] < bi)) {
        bs = rs[w];
        bi = ri[w];
      }
    __syncthreads();
    if (tid == 0) {
      idx_out[size_t(q) * k + r] = (bi == 0x7FFFFFFF) ? -1 : bi;
      score_out[size_t(q) * k + r] = (bi == 0x7FFFFFFF) ? -INFINITY : bs;
    }
    prev_s = bs;
    prev_i = bi;
  }
}

// Inner-product search on int8 MFMA for 3-bit database codes with m = d.  For a symmetric
// 8-level codebook (c[7 - k] = -c[k]) a centroid is an odd function of the three code
// bits, c = a0 s0 + a1 s1 + a2 s2 + a3 s0 s1 s2 with s = 2 b - 1 and s0 s1 s2 = 2 (b0^b1^b2) - 1,
// so <q, c[codes]> = sum_k a_k (2 q.b_k - sum q) over four 0/1 planes (the three code planes
// and their XOR).  The query rows are written as 32-bit fixed point in four int8 digits
// (A rows digit * 8 + query, 8 queries per block) and kept in LDS; each wave streams
// 32-vector database tiles, expands the plane and sign bits to 0/1 bytes (B) and runs five
// v_mfma_i32_32x32x32_i8 per 32 coordinates (four code planes, the sign bits).  The tile's
// scores update per-(wave, query) top-k lists in LDS; the block then merges its waves'
// lists into one candidate list per query.
constexpr int kSmQ = 8;        // queries per block
constexpr int kSmWaves = 8;    // waves per block (512 threads), one block per CU
constexpr int kSmTopMax = 16;  // list length per (wave, query); k <= 16 on this path

struct SearchMfmaArgs {
  const uint8_t *kbits;
  const uint32_t *knorm;
  const float *ck;
  const float *qp;   // prepared query rows: qr [d], sq [d], sum qr, sum sq
  float *cand_s;     // [nq][slices][k]
  int *cand_i;
  int kbytes, d, n_db, nq, k, slices, per, qstride;
  float qjl_scale;
};

__global__ __launch_bounds__(512, 1) void k_search_mfma(SearchMfmaArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ __align__(16) uint8_t sm_u8[];
  const int nch = a.d / 32;
  uint8_t *Aq = sm_u8;                              // [nch][64 lanes][16 B]
  uint8_t *As = sm_u8 + size_t(nch) * 1024;
  float *lst_s = reinterpret_cast<float *>(sm_u8 + size_t(nch) * 2048);   // [waves][8][kSmTopMax]
  int *lst_i = reinterpret_cast<int *>(lst_s + kSmWaves * kSmQ * kSmTopMax);
  __shared__ int exps[kSmQ][2];
  __shared__ float sums[kSmQ][2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, half = lane >> 5;
  const int q0 = blockIdx.x * kSmQ, slice = blockIdx.y;
  const int nqb = min(kSmQ, a.nq - q0);
  // ---- per-query exponents and sums (wave w takes query w)
  {
    const int qi = wv;
    float m0 = 0.0f, m1 = 0.0f;
    if (qi < nqb) {
      const float *qr = a.qp + size_t(q0 + qi) * a.qstride;
      for (int j = lane; j < a.d; j += 64) {
        m0 = fmaxf(m0, fabsf(qr[j]));
        m1 = fmaxf(m1, fabsf(qr[a.d + j]));
      }
    }
    m0 = wave_max(m0);
    m1 = wave_max(m1);
    if (lane == 0) {
      const float mx[2] = {m0, m1};
      for (int v = 0; v < 2; ++v) {
        int e = 0;
        if (mx[v] > 0.0f) {
          int ex;
          frexpf(mx[v], &ex);   // mx < 2^ex
          e = 30 - ex;          // |x| 2^e < 2^30: four signed int8 digits
        }
        exps[qi][v] = e;
        sums[qi][v] = qi < nqb ? a.qp[size_t(q0 + qi) * a.qstride + 2 * a.d + v] : 0.0f;
      }
    }
  }
  for (int i = tid; i < kSmWaves * kSmQ * kSmTopMax; i += 512) {
    lst_s[i] = -INFINITY;
    lst_i[i] = -1;
  }
  __syncthreads();
  // ---- A digits: lane (row = digit * 8 + query, half h), dword e, byte b of chunk c holds
  // coordinate 32 c + 8 b + 4 h + e
  for (int i = tid; i < 2 * nch * 256; i += 512) {
    const int e = i & 3, ln = (i >> 2) & 63, c = (i >> 8) % nch, v = i / (256 * nch);
    const int row = ln & 31, h = ln >> 5, digit = row >> 3, qi = row & 7;
    uint32_t word = 0u;
    if (qi < nqb) {
      const float *src = a.qp + size_t(q0 + qi) * a.qstride + (v ? a.d : 0);
      const int ex = exps[qi][v];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = 32 * c + 8 * b + 4 * h + e;
        const int xi = int(rintf(ldexpf(src[j], ex)));
        const int d0 = ((xi + 128) & 255) - 128;
        const int x1v = (xi - d0) >> 8;
        const int d1 = ((x1v + 128) & 255) - 128;
        const int x2 = (x1v - d1) >> 8;
        const int d2 = ((x2 + 128) & 255) - 128;
        const int d3 = (x2 - d2) >> 8;
        const int dg = digit == 0 ? d0 : (digit == 1 ? d1 : (digit == 2 ? d2 : d3));
        word |= uint32_t(dg & 255) << (8 * b);
      }
    }
    reinterpret_cast<uint32_t *>(v ? As : Aq)[i - v * 256 * nch] = word;
  }
  __syncthreads();
  // ---- per-lane constants for its queries 4 half + r
  const float c4 = a.ck[4], c5 = a.ck[5], c6 = a.ck[6], c7 = a.ck[7];
  const float al[4] = {0.25f * (c7 - c6 + c5 - c4), 0.25f * (c7 + c6 - c5 - c4),
                       0.25f * (c7 + c6 + c5 + c4), 0.25f * (c7 - c6 - c5 + c4)};
  const float alsum = (al[0] + al[1]) + (al[2] + al[3]);
  float sq_q[4], ss_q[4], cq[4], cs[4], thr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qi = 4 * half + r;
    sq_q[r] = ldexpf(2.0f, 16 - exps[qi][0]);   // 2 x (digit sum scale)
    ss_q[r] = ldexpf(2.0f, 16 - exps[qi][1]);
    cq[r] = sums[qi][0] * alsum;
    cs[r] = sums[qi][1];
    thr[r] = -INFINITY;
  }
  const int x0 = slice * a.per;
  const int x1 = min(a.n_db, x0 + a.per);
  const int ntile = x1 > x0 ? (x1 - x0 + 31) / 32 : 0;
  const int pb = a.d / 8;   // plane bytes
  const v4i *Aq4 = reinterpret_cast<const v4i *>(Aq);
  const v4i *As4 = reinterpret_cast<const v4i *>(As);
  const int sh0 = 4 * half;
  for (int t = wv; t < ntile; t += kSmWaves) {
    const int n = x0 + 32 * t + (lane & 31);
    const bool valid = n < x1;
    const uint8_t *rec = a.kbits + size_t(valid ? n : x0) * a.kbytes;
    v16i acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {}, accs = {};
    for (int g = 0; g < nch / 4; ++g) {
      const uint4 p0 = *reinterpret_cast<const uint4 *>(rec + 16 * g);
      const uint4 p1 = *reinterpret_cast<const uint4 *>(rec + pb + 16 * g);
      const uint4 p2 = *reinterpret_cast<const uint4 *>(rec + 2 * pb + 16 * g);
      const uint4 ps = *reinterpret_cast<const uint4 *>(rec + 3 * pb + 16 * g);
      const uint32_t w0s[4] = {p0.x, p0.y, p0.z, p0.w}, w1s[4] = {p1.x, p1.y, p1.z, p1.w};
      const uint32_t w2s[4] = {p2.x, p2.y, p2.z, p2.w}, wss[4] = {ps.x, ps.y, ps.z, ps.w};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int c = 4 * g + cc;
        const uint32_t w0 = w0s[cc] >> sh0, w1 = w1s[cc] >> sh0, w2 = w2s[cc] >> sh0;
        const uint32_t wsg = wss[cc] >> sh0, wx = w0 ^ w1 ^ w2;
        v4i b0, b1, b2, bx, bs;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b0[e] = int((w0 >> e) & 0x01010101u);
          b1[e] = int((w1 >> e) & 0x01010101u);
          b2[e] = int((w2 >> e) & 0x01010101u);
          bx[e] = int((wx >> e) & 0x01010101u);
          bs[e] = int((wsg >> e) & 0x01010101u);
        }
        const v4i aq = Aq4[c * 64 + lane], as = As4[c * 64 + lane];
        acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq, b0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq, b1, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq, b2, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq, bx, acc3, 0, 0, 0);
        accs = __builtin_amdgcn_mfma_i32_32x32x32_i8(as, bs, accs, 0, 0, 0);
      }
    }
    // scores of vector n for queries 4 half + r (accumulator registers 4 digit + r)
    const uint32_t nr = valid ? a.knorm[n] : 0u;
    const float n16 = f16_bits_to_float(nr & 0xFFFFu), rn16 = f16_bits_to_float(nr >> 16);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#define TQ_DS(acc) fmaf(float(acc[r] + 256 * acc[4 + r]), 0x1p-16f, float(acc[8 + r] + 256 * acc[12 + r]))
      const float code = (al[0] * TQ_DS(acc0) + al[1] * TQ_DS(acc1) + al[2] * TQ_DS(acc2) + al[3] * TQ_DS(acc3)) *
                             sq_q[r] - cq[r];
      const float qjl = TQ_DS(accs) * ss_q[r] - cs[r];
#undef TQ_DS
      const bool live = valid && (4 * half + r) < nqb;
      sc[r] = live ? n16 * code + rn16 * a.qjl_scale * qjl : -INFINITY;
    }
    // ---- top-k lists: candidates beating their list's k-th score, lowest lane first
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bool pending = sc[r] > thr[r];
      uint64_t mask = __builtin_amdgcn_ballot_w64(pending);
      while (mask) {
        const int bl = __builtin_ctzll(mask);
        const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc[r]), bl));
        const int qi = (bl < 32 ? 0 : 4) + r;
        float *ls = lst_s + (wv * kSmQ + qi) * kSmTopMax;
        int *li = lst_i + (wv * kSmQ + qi) * kSmTopMax;
        if (lane == 0) {
          int pos = a.k - 1;
          while (pos > 0 && s > ls[pos - 1]) {
            ls[pos] = ls[pos - 1];
            li[pos] = li[pos - 1];
            --pos;
          }
          ls[pos] = s;
          li[pos] = x0 + 32 * t + (bl & 31);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const float nt = ls[a.k - 1];
        if ((bl < 32) == (half == 0)) thr[r] = nt;
        if (lane == bl) pending = false;
        pending = pending && sc[r] > thr[r];
        mask = __builtin_amdgcn_ballot_w64(pending);
      }
    }
  }
  __syncthreads();
  // ---- merge the waves' lists: wave w takes query w, k rounds of arg-max over 8 k entries
  if (wv < nqb) {
    const int qi = wv;
    const int ncand = kSmWaves * a.k;
    float cs0 = -INFINITY, cs1 = -INFINITY;
    int ci0 = 0x7FFFFFFF, ci1 = 0x7FFFFFFF;
    if (lane < ncand) {
      const int w = lane / a.k, e = lane % a.k;
      cs0 = lst_s[(w * kSmQ + qi) * kSmTopMax + e];
      ci0 = lst_i[(w * kSmQ + qi) * kSmTopMax + e];
      if (ci0 < 0) { cs0 = -INFINITY; ci0 = 0x7FFFFFFF; }
    }
    if (lane + 64 < ncand) {
      const int w = (lane + 64) / a.k, e = (lane + 64) % a.k;
      cs1 = lst_s[(w * kSmQ + qi) * kSmTopMax + e];
      ci1 = lst_i[(w * kSmQ + qi) * kSmTopMax + e];
      if (ci1 < 0) { cs1 = -INFINITY; ci1 = 0x7FFFFFFF; }
    }
    for (int r = 0; r < a.k; ++r) {
      float bs;
      int bi;
      if (cs1 > cs0 || (cs1 == cs0 && ci1 < ci0)) { bs = cs1; bi = ci1; } else { bs = cs0; bi = ci0; }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float os = __shfl_xor(bs, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (os > bs || (os == bs && oi < bi)) {
          bs = os;
          bi = oi;
        }
      }
      if (lane == 0) {
        const size_t cdx = (size_t(q0 + qi) * a.slices + slice) * a.k + r;
        a.cand_s[cdx] = bs;
        a.cand_i[cdx] = bi == 0x7FFFFFFF ? -1 : bi;
      }
      // remove the taken entry
      if (ci0 == bi && cs0 == bs) { cs0 = -INFINITY; ci0 = 0x7FFFFFFF; }
      if (ci1 == bi && cs1 == bs) { cs1 = -INFINITY; ci1 = 0x7FFFFFFF; }
    }
  }
#else
  (void)a;
#endif
}

// ------------------------------------------------------------------ NSN means
// [NSNQuant] section 1, the shift: o = mean over a unit's tokens of sqrt(d) x / ||x||,
// keys rotary-embedded first.  k_nsn_partial: grid (units, slices); a token is spread over
// LPT lanes, each holding NP rotary pairs (j, j + D/2) of it (two 4-element loads), so a
// wave takes TPW tokens at once: wave w of a block takes tokens t0 + TPW (w + 4 i) + sub,
// with the fp64 RoPE angles of its pairs stepped by 4 TPW theta per iteration.  Sums in
// fp64, combined in a fixed order (deterministic).
struct NsnArgs {
  const void *k, *v;
  double *part;   // [units][slices][2][D]
  int n, start, slices, per;
  float rope_base;
};

// Raw bits of 4 consecutive input elements starting at element `off` (one 8-byte load for
// 16-bit types, 16 bytes for fp32; off * sizeof(element) is a multiple of that size).
template <int DT>
struct Raw4 {
  using T = uint2;
};
template <>
struct Raw4<TQ_F32> {
  using T = uint4;
};
template <int DT>
__device__ __forceinline__ typename Raw4<DT>::T load_raw4(const void *base, size_t off) {
  if constexpr (DT == TQ_F32)
    return *reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + off);
  else
    return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + off);
}
template <int DT>
__device__ __forceinline__ void raw4_to_f64(const typename Raw4<DT>::T &r, double *x) {
  if constexpr (DT == TQ_F32) {
    x[0] = __uint_as_float(r.x);
    x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z);
    x[3] = __uint_as_float(r.w);
  } else if constexpr (DT == TQ_BF16) {
    x[0] = __uint_as_float(r.x << 16);
    x[1] = __uint_as_float(r.x & 0xFFFF0000u);
    x[2] = __uint_as_float(r.y << 16);
    x[3] = __uint_as_float(r.y & 0xFFFF0000u);
  } else {
    x[0] = f16_bits_to_float(r.x & 0xFFFFu);
    x[1] = f16_bits_to_float(r.x >> 16);
    x[2] = f16_bits_to_float(r.y & 0xFFFFu);
    x[3] = f16_bits_to_float(r.y >> 16);
  }
}

// Sum of a double over each aligned group of N lanes (N = 8 or 16), in every lane of the
// group (DPP: quad swaps, then the half-row mirror, then a rotation by 8 in the row).
template <int N>
__device__ __forceinline__ double group_sum_f64(double x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp_f64<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_f64<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_f64<0x141>(x);   // row_half_mirror: the other quad of the half row
  if constexpr (N == 16) x += dpp_f64<0x128>(x);   // row_ror:8: the other half row
  return x;
}

template <int D, int DT>
__global__ __launch_bounds__(256) void k_nsn_partial(NsnArgs a) {
  constexpr int H2 = D / 2, NP = 4, LPT = H2 / NP, TPW = 64 / LPT, STEP = 4 * TPW;
  constexpr int U = 4;   // iterations whose loads are issued together
  __shared__ double acc_s[4][2][D];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int jg = lane % LPT, sub = lane / LPT, j0 = NP * jg;
  const int unit = blockIdx.x, sl = blockIdx.y;
  const int t0 = sl * a.per, t1 = min(a.n, t0 + a.per);
  const bool rope = a.rope_base != 0.0f;
  const double sqd = sqrt(double(D));
  // this lane's pairs: (cos, sin) at its current token and the step rotation
  double c[NP], sn[NP], cs[NP], ss[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    c[e] = 1.0;
    sn[e] = 0.0;
    cs[e] = 1.0;
    ss[e] = 0.0;
    if (rope) {
      const double theta = pow(double(a.rope_base), -2.0 * double(j0 + e) / double(D));
      sincos(double(a.start + t0 + TPW * wv + sub) * theta, &sn[e], &c[e]);
      sincos(double(STEP) * theta, &ss[e], &cs[e]);
    }
  }
  double ak[2 * NP], av[2 * NP];
#pragma unroll
  for (int e = 0; e < 2 * NP; ++e) ak[e] = av[e] = 0.0;
  const size_t ub = size_t(unit) * a.n;
  using R4 = typename Raw4<DT>::T;
  for (int tb = t0 + TPW * wv; tb < t1; tb += U * STEP) {   // wave-uniform
    R4 rk[U][2], rv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u * STEP + sub;
      const size_t o = (ub + size_t(t < t1 ? t : t0)) * D + j0;
      rk[u][0] = load_raw4<DT>(a.k, o);
      rk[u][1] = load_raw4<DT>(a.k, o + H2);
      rv[u][0] = load_raw4<DT>(a.v, o);
      rv[u][1] = load_raw4<DT>(a.v, o + H2);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = tb + u * STEP + sub < t1;
      double x[2 * NP], y[2 * NP];
      raw4_to_f64<DT>(rk[u][0], x);
      raw4_to_f64<DT>(rk[u][1], x + NP);
      raw4_to_f64<DT>(rv[u][0], y);
      raw4_to_f64<DT>(rv[u][1], y + NP);
      if (rope) {
#pragma unroll
        for (int e = 0; e < NP; ++e) {
          const double r0 = x[e] * c[e] - x[NP + e] * sn[e], r1 = x[e] * sn[e] + x[NP + e] * c[e];
          x[e] = r0;
          x[NP + e] = r1;
          const double cn = c[e] * cs[e] - sn[e] * ss[e];
          sn[e] = sn[e] * cs[e] + c[e] * ss[e];
          c[e] = cn;
        }
      }
      double nk = 0.0, nv = 0.0;
#pragma unroll
      for (int e = 0; e < 2 * NP; ++e) {
        nk = fma(x[e], x[e], nk);
        nv = fma(y[e], y[e], nv);
      }
      nk = group_sum_f64<LPT>(nk);
      nv = group_sum_f64<LPT>(nv);
      // sqrt(d) / ||x||: hardware reciprocal square root refined by two Newton steps (each
      // squares the relative error; the mean is rounded to fp32)
      double rk_ = __builtin_amdgcn_rsq(nk), rv_ = __builtin_amdgcn_rsq(nv);
      rk_ *= fma(-0.5 * nk * rk_, rk_, 1.5);
      rv_ *= fma(-0.5 * nv * rv_, rv_, 1.5);
      rk_ *= fma(-0.5 * nk * rk_, rk_, 1.5);
      rv_ *= fma(-0.5 * nv * rv_, rv_, 1.5);
      const double fk = live && nk > 0.0 ? sqd * rk_ : 0.0, fv = live && nv > 0.0 ? sqd * rv_ : 0.0;
#pragma unroll
      for (int e = 0; e < 2 * NP; ++e) {
        ak[e] = fma(x[e], fk, ak[e]);
        av[e] = fma(y[e], fv, av[e]);
      }
    }
  }
  // the wave's token groups: lanes with the same pairs, in a fixed order
#pragma unroll
  for (int msk = LPT; msk < 64; msk <<= 1)
#pragma unroll
    for (int e = 0; e < 2 * NP; ++e) {
      ak[e] += __shfl_xor(ak[e], msk, 64);
      av[e] += __shfl_xor(av[e], msk, 64);
    }
  if (sub == 0) {
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      acc_s[wv][0][j0 + e] = ak[e];
      acc_s[wv][0][H2 + j0 + e] = ak[NP + e];
      acc_s[wv][1][j0 + e] = av[e];
      acc_s[wv][1][H2 + j0 + e] = av[NP + e];
    }
  }
  __syncthreads();
  for (int i = tid; i < 2 * D; i += 256) {
    const int kv = i / D, jj = i % D;
    a.part[((size_t(unit) * a.slices + sl) * 2 + kv) * D + jj] =
        (acc_s[0][kv][jj] + acc_s[1][kv][jj]) + (acc_s[2][kv][jj] + acc_s[3][kv][jj]);
  }
}

// o = (sum of the slices' partials) / n, stored in fp32, then Pi o = H (D .* o) / sqrt(B)
// in fp64 (LDS FWHT), stored in fp32: per unit [o_K, o_V, Pi o_K, Pi o_V].
template <int D>
__global__ __launch_bounds__(256) void k_nsn_final(const double *part, int slices, int n, const float *Dsg,
                                                   float *nsn) {
  __shared__ double y_s[2][D];
  const int tid = threadIdx.x, unit = blockIdx.x;
  float *dst = nsn + size_t(unit) * 4 * D;
  for (int i = tid; i < 2 * D; i += 256) {
    const int kv = i / D, jj = i % D;
    double acc = 0.0;
    for (int sl = 0; sl < slices; ++sl) acc += part[((size_t(unit) * slices + sl) * 2 + kv) * D + jj];
    const float o32 = float(acc / double(n));
    dst[kv * D + jj] = o32;
    y_s[kv][jj] = double(o32) * double(Dsg[jj]);
  }
  __syncthreads();
  for (int st = 1; st < D; st <<= 1) {
    for (int i = tid; i < D; i += 256) {   // D / 2 butterflies per vector, two vectors
      const int kv = i / (D / 2), kk = i % (D / 2);
      const int jj = (kk / st) * 2 * st + (kk % st);
      const double x0 = y_s[kv][jj], x1 = y_s[kv][jj + st];
      y_s[kv][jj] = x0 + x1;
      y_s[kv][jj + st] = x0 - x1;
    }
    __syncthreads();
  }
  const double isb = 1.0 / sqrt(double(D));
  for (int i = tid; i < 2 * D; i += 256) dst[2 * D + i] = float(y_s[i / D][i % D] * isb);
}

int nsn_slices(int n, int units) {
  const int want = (1024 + units - 1) / units;   // about four blocks per CU in all
  const int by_n = int((int64_t(n) + 255) / 256);
  return std::max(1, std::min(want, by_n));
}

// ------------------------------------------------------------------ host-side helpers
tq_status launch_status() {
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EDEVICE;
}

bool decode_supported(const tq_cache_desc &c) {
  return (c.d == 64 || c.d == 128) && c.bits_v > 0;
}

// The MFMA path covers the 2-bit + QJL (m = d) keys, 3-bit values configuration.
bool decode_mfma_path(const tq_cache_desc &c, int q_heads) {
  return !c.polar && (c.d == 64 || c.d == 128) && c.bits_k >= 1 && c.bits_k <= 3 && c.bits_v == 3 &&
         c.m == c.d && q_heads / c.kv_heads <= kMfmaMaxG;
}

constexpr int kMfmaChunk = 32 * kDecWaves;   // tokens per block iteration (one tile per wave)

constexpr int kDecodeBlocks = 256 * kDecBlocksPerCU;   // MI355X: 256 CUs
constexpr int kLogitsBlocks = 1024;                    // logits-only kernel: 4 blocks per CU
constexpr int kMaxWindow = 4096;                      // full-precision window capacity
constexpr int kWinMaxSplits = 8;                      // window partials per unit, at most

int default_splits(const tq_cache_desc &c, int length) {
  if (length <= 0) return 1;
  const int units = c.batch * c.kv_heads;
  const int by_len = (length + kMfmaChunk - 1) / kMfmaChunk;
  // one round of blocks: the split kernel keeps kDecBlocksPerCU blocks resident per CU
  // and MI355X has 256 CUs, so all blocks start together and none waits for a second round
  // (PolarQuant's decode kernel keeps kPolarBlocksPerCU)
  const int want = ((c.polar ? 256 * kPolarBlocksPerCU : kDecodeBlocks) + units - 1) / units;
  int s = by_len < want ? by_len : want;
  if (s < 1) s = 1;
  if (s > 4096) s = 4096;
  return s;
}

// Tokens per split: a multiple of kMfmaChunk, so that every wave of a block gets the same
// number of whole 32-token tiles.
int split_chunk(int length, int splits) {
  const int per = (length + splits - 1) / splits;
  return (per + kMfmaChunk - 1) / kMfmaChunk * kMfmaChunk;
}

size_t decode_ws(const tq_cache_desc &c, int q_heads, int splits) {
  const size_t rows = size_t(c.batch) * q_heads;
  const size_t qstride = size_t(c.d) + c.m + 2;
  const size_t units = size_t(c.batch) * c.kv_heads;
  return align256(rows * qstride * 4) + align256(units * qpack_unit_bytes(c.d)) +
         align256(rows * size_t(splits) * (c.d + 2) * 4);
}

int search_tiles(int n_db) { return (n_db + kSearchTile - 1) / kSearchTile; }

}  // namespace
}  // namespace tq

using namespace tq;

// MFMA-path kernels by head dim, key bits and NSN: the logits-only kernel or the split
// decode kernel (with or without the scores output, so that the loop carries no test of it).
template <bool LOGITS, bool NSN>
static void launch_mfma(int d, int bk, dim3 grid, dim3 blk, hipStream_t s, const MfmaArgs &ma) {
#define TQ_MFMA(DD, BK)                                                                 \
  if (d == DD && bk == BK) {                                                            \
    if constexpr (LOGITS)                                                               \
      hipLaunchKernelGGL((k_logits<DD, BK, NSN>), grid, blk, 0, s, ma);                 \
    else if (ma.scores)                                                                 \
      hipLaunchKernelGGL((k_decode_lds<DD, BK, NSN, true>), grid, blk, 0, s, ma);       \
    else                                                                                \
      hipLaunchKernelGGL((k_decode_lds<DD, BK, NSN, false>), grid, blk, 0, s, ma);      \
  }
  TQ_MFMA(64, 1)
  TQ_MFMA(64, 2)
  TQ_MFMA(64, 3)
  TQ_MFMA(128, 1)
  TQ_MFMA(128, 2)
  TQ_MFMA(128, 3)
#undef TQ_MFMA
}

static void launch_mfma16(int bk, dim3 grid, dim3 blk, hipStream_t s, const MfmaArgs &ma) {
#define TQ_MFMA16(BK)                                                                   \
  if (bk == BK) {                                                                       \
    if (ma.scores)                                                                      \
      hipLaunchKernelGGL((k_decode_lds16<BK, true>), grid, blk, 0, s, ma);              \
    else                                                                                \
      hipLaunchKernelGGL((k_decode_lds16<BK, false>), grid, blk, 0, s, ma);             \
  }
  TQ_MFMA16(1)
  TQ_MFMA16(2)
  TQ_MFMA16(3)
#undef TQ_MFMA16
}

extern "C" {

tq_status tq_cache_init(const tq_cache_desc *desc, void *cache_dev, tq_stream_t stream) {
  if (!desc || !cache_dev) return TQ_EINVAL;
  if (!cache_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  hipLaunchKernelGGL(k_cache_init, dim3(1), dim3(64), 0, hipStream_t(stream),
                     static_cast<uint32_t *>(cache_dev), *desc);
  if (desc->nsn) {
    // means start at zero: a fill kernel rather than a memset node, for graph capture
    const size_t n = size_t(desc->batch) * desc->kv_heads * 4 * desc->d;
    hipLaunchKernelGGL(k_fill_zero, dim3(unsigned((n + 255) / 256)), dim3(256), 0, hipStream_t(stream),
                       cache_ptrs(cache_dev, *desc).nsn, n);
  }
  return launch_status();
}

tq_status tq_quantize_kv_profiled(const tq_cache_desc *desc, const void *codec_dev,
                                  void *cache_dev, const void *k, const void *v,
                                  int32_t dtype, int32_t start_pos, int32_t n_new,
                                  float rope_base, void *ev_start, void *ev_stop,
                                  tq_stream_t stream) {
  if (!desc || !codec_dev || !cache_dev) return TQ_EINVAL;
  if (!cache_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_EINVAL;
  if (start_pos < 0 || n_new < 0) return TQ_EINVAL;
  if (int64_t(start_pos) + int64_t(n_new) > int64_t(desc->capacity)) return TQ_ECAPACITY;
  if (n_new > 0 && (!k || (desc->bits_v > 0) != (v != nullptr))) return TQ_EINVAL;
  if (!std::isfinite(rope_base) || rope_base < 0.0f) return TQ_EINVAL;
  // the kernels read K and V rows with 16-byte vector loads
  if ((reinterpret_cast<uintptr_t>(k) & 15) != 0 || (reinterpret_cast<uintptr_t>(v) & 15) != 0) return TQ_EINVAL;
  const int d = desc->d;
  const bool small = (d == 64 || d == 128);
  const bool large = (d == 256 || d == 512 || d == 1024 || d == 1536 || d == 2048);
  if (!small && !(large && desc->bits_v == 0)) return TQ_EUNSUPPORTED;
  if (large && rope_base != 0.0f) return TQ_EUNSUPPORTED;
  if (n_new == 0) return TQ_OK;
  if (desc->m > 0 && (desc->m % 32) != 0) return TQ_EUNSUPPORTED;
  QuantArgs a;
  a.cp = codec_ptrs(codec_dev, d, desc->bits_k, desc->bits_v, desc->m);
  a.ch = cache_ptrs(cache_dev, *desc);
  a.k = k;
  a.v = v;
  a.start = start_pos;
  a.n_new = n_new;
  a.capacity = desc->capacity;
  a.bits_k = desc->bits_k;
  a.bits_v = desc->bits_v;
  a.m = desc->m;
  a.units = desc->batch * desc->kv_heads;
  a.rope_base = rope_base;
  a.sqrt_b = std::sqrt(double(a.cp.block));
  a.inv_sqrt_b = 1.0 / a.sqrt_b;
  if (rope_base != 0.0f && small) {
    for (int j = 0; j < d / 2; ++j) {
      const double th = std::pow(double(rope_base), -2.0 * double(j) / double(d));
      a.rf.theta[j] = th;
      a.rf.c[j] = std::cos(th);
      a.rf.s[j] = std::sin(th);
    }
  }
  hipStream_t s = hipStream_t(stream);
  if (ev_start && hipEventRecord(hipEvent_t(ev_start), s) != hipSuccess) return TQ_EDEVICE;
  if (small) {
    const int first_tile = start_pos / kValueTile;
    const int end_tile = (start_pos + n_new + kValueTile - 1) / kValueTile;
    const int windows = (end_tile - first_tile + 1) / 2;
    dim3 grid(windows, a.units);
    // 2-bit keys with 3-bit values (the 3 bits per value configuration) have their code
    // counts fixed at compile time; other widths take them from the descriptor
    const bool k2v3 = desc->bits_k == 2 && desc->bits_v == 3;
#define TQ_QKV(DD, TT)                                                                              \
  do {                                                                                              \
    if (desc->polar) hipLaunchKernelGGL((k_quantize_kv<DD, TT, 0, 0, true>), grid, dim3(256), 0, s, a); \
    else if (k2v3) hipLaunchKernelGGL((k_quantize_kv<DD, TT, 4, 8>), grid, dim3(256), 0, s, a);     \
    else hipLaunchKernelGGL((k_quantize_kv<DD, TT, 0, 0>), grid, dim3(256), 0, s, a);               \
  } while (0)
    if (d == 64) {
      if (dtype == TQ_F32) TQ_QKV(64, TQ_F32); else if (dtype == TQ_BF16) TQ_QKV(64, TQ_BF16); else TQ_QKV(64, TQ_F16);
    } else {
      if (dtype == TQ_F32) TQ_QKV(128, TQ_F32); else if (dtype == TQ_BF16) TQ_QKV(128, TQ_BF16); else TQ_QKV(128, TQ_F16);
    }
#undef TQ_QKV
  } else {
#define TQ_QDB(CC, EE, TT)                                                                     \
  do {                                                                                         \
    const dim3 grid((n_new + db_group(CC) - 1) / db_group(CC), a.units);                       \
    const size_t shm = db_lds_bytes(CC);                                                       \
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_quantize_db<CC, EE, TT>),         \
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(shm)) != hipSuccess) \
      return TQ_EDEVICE;                                                                       \
    hipLaunchKernelGGL((k_quantize_db<CC, EE, TT>), grid, dim3(64 * kDbWaves), shm, s, a);     \
  } while (0)
#define TQ_QDB_T(CC, EE) \
  do { if (dtype == TQ_F32) TQ_QDB(CC, EE, TQ_F32); else if (dtype == TQ_BF16) TQ_QDB(CC, EE, TQ_BF16); else TQ_QDB(CC, EE, TQ_F16); } while (0)
    switch (d) {
      case 256: TQ_QDB_T(4, 4); break;
      case 512: TQ_QDB_T(8, 8); break;
      case 1024: TQ_QDB_T(16, 16); break;
      case 1536: TQ_QDB_T(24, 8); break;
      default: TQ_QDB_T(32, 32); break;
    }
#undef TQ_QDB_T
#undef TQ_QDB
  }
  const tq_status st = launch_status();
  if (ev_stop && hipEventRecord(hipEvent_t(ev_stop), s) != hipSuccess) return TQ_EDEVICE;
  return st;
}

tq_status tq_quantize_kv(const tq_cache_desc *desc, const void *codec_dev, void *cache_dev,
                         const void *k, const void *v, int32_t dtype, int32_t start_pos,
                         int32_t n_new, float rope_base, tq_stream_t stream) {
  return tq_quantize_kv_profiled(desc, codec_dev, cache_dev, k, v, dtype, start_pos, n_new,
                                 rope_base, nullptr, nullptr, stream);
}

size_t tq_decode_workspace_bytes_splits(const tq_cache_desc *desc, int32_t q_heads,
                                        int32_t splits) {
  if (!desc || !cache_desc_valid(*desc) || q_heads < 1 || splits < 1) return 0;
  return decode_ws(*desc, q_heads, splits);
}

int32_t tq_decode_splits(const tq_cache_desc *desc, int32_t q_heads, int32_t length) {
  if (!desc || !cache_desc_valid(*desc) || q_heads < 1 || length < 0) return 0;
  return default_splits(*desc, length);
}

size_t tq_decode_workspace_bytes(const tq_cache_desc *desc, int32_t q_heads, int32_t length) {
  if (!desc || !cache_desc_valid(*desc) || q_heads < 1 || length < 0) return 0;
  return decode_ws(*desc, q_heads, default_splits(*desc, length));
}

namespace {
struct WindowIn {
  const void *k, *v;
  int32_t dtype;
  int len, cap;            // tokens attended (including an appended one), buffer rows
  const void *nk, *nv;     // decode step: the token appended at row len - 1, or null
  void *ak, *av;           // decode step: writable window buffers
  bool flush;              // decode step: rows [0, cap) go to the packed cache first
};
}  // namespace

static tq_status decode_impl(const tq_cache_desc *desc, const void *codec_dev,
                             const void *cache_dev, int32_t length, const WindowIn *win,
                             const void *q, int32_t dtype, int32_t q_heads, int32_t q_pos,
                             float rope_base, float scale, float *out, float *scores,
                             int32_t splits, void *ws, size_t ws_bytes,
                             void *ev_start, void *ev_stop, tq_stream_t stream) {
  // out == NULL asks for the logits only (scores required)
  if (!desc || !codec_dev || !cache_dev || !q || (!out && !scores) || !ws) return TQ_EINVAL;
  if (!cache_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_EINVAL;
  if (q_heads < 1 || q_heads % desc->kv_heads != 0) return TQ_EINVAL;
  if (q_heads / desc->kv_heads > kMaxG) return TQ_EUNSUPPORTED;
  if (length < 0 || splits < 0 || q_pos < 0) return TQ_EINVAL;
  if (length > desc->capacity) return TQ_ECAPACITY;
  if (!std::isfinite(rope_base) || rope_base < 0.0f || !std::isfinite(scale)) return TQ_EINVAL;
  if (!decode_supported(*desc)) return TQ_EUNSUPPORTED;
  if (desc->m > 512) return TQ_EUNSUPPORTED;
  const int wlen = win ? win->len : 0;
  if (win) {
    if (win->len < 0 || win->cap < win->len || win->cap > kMaxWindow) return TQ_EINVAL;
    if (win->len > 0 && (!win->k || !win->v)) return TQ_EINVAL;
    if (win->dtype != TQ_F32 && win->dtype != TQ_BF16 && win->dtype != TQ_F16) return TQ_EINVAL;
    if (desc->d != 64 && desc->d != 128) return TQ_EUNSUPPORTED;
    if (desc->bits_v == 0) return TQ_EUNSUPPORTED;
    // the window kernel reads and writes rows with 16-byte vectors
    for (const void *p : {win->k, win->v, win->nk, win->nv, static_cast<const void *>(win->ak),
                          static_cast<const void *>(win->av)})
      if ((reinterpret_cast<uintptr_t>(p) & 15) != 0) return TQ_EINVAL;
  }
  const int S = splits == 0 ? default_splits(*desc, length) : splits;
  // the window's 64-token chunks over at most kWinMaxSplits blocks per unit, one partial each
  const int wchunks = (wlen + 63) / 64;
  const int wcpb = wchunks > 0 ? (wchunks + kWinMaxSplits - 1) / kWinMaxSplits : 1;
  const int wsplit = (wchunks + wcpb - 1) / wcpb;   // the window's partials follow the packed splits
  if (ws_bytes < decode_ws(*desc, q_heads, S + wsplit)) return TQ_ENOSPACE;
  const int d = desc->d, m = desc->m;
  const int rows = desc->batch * q_heads;
  hipStream_t s = hipStream_t(stream);
  if (length == 0 && wlen == 0) {
    if (!out) return TQ_OK;   // no tokens, no logits
    // a fill kernel rather than a memset node, so the call can be captured in a graph
    const size_t n = size_t(rows) * d;
    hipLaunchKernelGGL(k_fill_zero, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, out, n);
    return launch_status();
  }
  const CodecPtrs cp = codec_ptrs(codec_dev, d, desc->bits_k, desc->bits_v, m);
  if (win && cp.block != d) return TQ_EUNSUPPORTED;   // the window rotates with one d-point block
  // NSN caches decode on the MFMA path only (its kernels carry the mean terms); PolarQuant
  // caches on their own kernel (8 head slots, m = d QJL rows)
  if (desc->nsn && !decode_mfma_path(*desc, q_heads)) return TQ_EUNSUPPORTED;
  if (desc->polar && (q_heads / desc->kv_heads > 8 || desc->m != desc->d)) return TQ_EUNSUPPORTED;
  if (win && win->flush) {
    // the full window becomes packed tokens [length - cap, length) before anything reads them
    if (length < win->cap) return TQ_EINVAL;
    const tq_status st = tq_quantize_kv_profiled(desc, codec_dev, const_cast<void *>(cache_dev), win->k, win->v,
                                                 win->dtype, length - win->cap, win->cap, rope_base, nullptr,
                                                 nullptr, stream);
    if (st != TQ_OK) return st;
  }
  float *qp = static_cast<float *>(ws);
  const int qstride = d + m + 2;
  const int units = desc->batch * desc->kv_heads;
  uint8_t *qpack = static_cast<uint8_t *>(ws) + align256(size_t(rows) * qstride * 4);
  float *part = reinterpret_cast<float *>(qpack + align256(size_t(units) * qpack_unit_bytes(d)));
  const int G = q_heads / desc->kv_heads;
  const float sc = scale == 0.0f ? float(1.0 / std::sqrt(double(d))) : scale;
  const bool mfma = decode_mfma_path(*desc, q_heads);
  // groups of at most 4 query heads at d = 128 (plain caches, with an output): key scores
  // on the 16-row MFMA form (k_decode_lds16), whose digit rows the query prep lays out
  const bool l16 = mfma && out && d == 128 && m == 128 && !desc->nsn && q_heads / desc->kv_heads <= 4;
  // the int8 digit rows: the MFMA path's key and QJL scores, PolarQuant's QJL sums
  const bool with_qpack = mfma || desc->polar;
  // odd key codebook on the MFMA path: c[code] = c0 + a weighted sum of bit planes
  const int bk = desc->bits_k;
  const int score_stride = length + wlen;
  int used_splits = 0;
  const CachePtrs ch = cache_ptrs(const_cast<void *>(cache_dev), *desc);
  if (length > 0) {
  if (d == m && (d == 64 || d == 128) && cp.block == d) {
    QueryRope qr;
    for (int j = 0; j < d / 2; ++j) {
      if (rope_base != 0.0f) {
        const double ang = double(q_pos) * std::pow(double(rope_base), -2.0 * double(j) / double(d));
        qr.c[j] = float(std::cos(ang));
        qr.s[j] = float(std::sin(ang));
      } else {
        qr.c[j] = 1.0f;
        qr.s[j] = 0.0f;
      }
    }
    if (d == 64)
      hipLaunchKernelGGL(k_qprep_fast<64>, dim3(rows), dim3(256), 0, s, q, int(dtype), qr, cp, qp, qstride,
                         q_heads, G, bk, with_qpack ? qpack : nullptr, ch.nsn, 0);
    else
      hipLaunchKernelGGL(k_qprep_fast<128>, dim3(rows), dim3(256), 0, s, q, int(dtype), qr, cp, qp, qstride,
                         q_heads, G, bk, with_qpack ? qpack : nullptr, ch.nsn, l16 ? 1 : 0);
  } else {
    hipLaunchKernelGGL(k_qprep_pack, dim3(rows), dim3(256), size_t(d + m + (m > 1024 ? m : 1024)) * 4, s, q,
                       int(dtype), d, m, q_pos, rope_base, cp, qp, qstride, q_heads, G, bk,
                       with_qpack ? qpack : nullptr, ch.nsn);
  }
  used_splits = S;
  if (mfma) {
    const int chunk = split_chunk(length, S);
    used_splits = (length + chunk - 1) / chunk;
    MfmaArgs ma;
    ma.kbits = ch.kbits;
    ma.knorm = ch.knorm;
    ma.vcodes = ch.vcodes;
    ma.vnorm = ch.vnorm;
    ma.cv = cp.cv;
    ma.qpack = qpack;
    ma.part = part;
    ma.scores = scores;
    ma.nsn = ch.nsn;
    ma.kbytes = ch.kbytes;
    ma.tiles = ch.tiles;
    ma.capacity = desc->capacity;
    ma.length = length;
    ma.chunk = chunk;
    ma.splits = used_splits + wsplit;
    ma.score_stride = score_stride;
    ma.kv_heads = desc->kv_heads;
    ma.q_heads = q_heads;
    ma.G = G;
    ma.scale_log2 = sc * 1.4426950408889634f;
    ma.inv_scale_log2 = 1.0f / ma.scale_log2;
    if (!out) {
      // logits only: 4-wave blocks, about four per CU unless the caller fixed the splits
      const int by_len = (length + 127) / 128;
      int ls = splits != 0 ? splits : (kLogitsBlocks + units - 1) / units;
      ls = std::max(1, std::min(ls, by_len));
      const int lchunk = ((length + ls - 1) / ls + 127) / 128 * 128;
      ma.chunk = lchunk;
      const int lsplits = (length + lchunk - 1) / lchunk;
      const dim3 lgrid(units, lsplits);
      if (ev_start && hipEventRecord(hipEvent_t(ev_start), s) != hipSuccess) return TQ_EDEVICE;
      if (desc->nsn)
        launch_mfma<true, true>(d, bk, lgrid, dim3(256), s, ma);
      else
        launch_mfma<true, false>(d, bk, lgrid, dim3(256), s, ma);
      if (ev_stop && hipEventRecord(hipEvent_t(ev_stop), s) != hipSuccess) return TQ_EDEVICE;
      used_splits = 0;   // no partials: only the window (if any) still writes scores
    }
    if (out) {
    dim3 grid(units, used_splits);
    if (ev_start && hipEventRecord(hipEvent_t(ev_start), s) != hipSuccess) return TQ_EDEVICE;
    const dim3 blk(64 * kDecWaves);
    if (l16)
      launch_mfma16(bk, grid, blk, s, ma);
    else if (desc->nsn)
      launch_mfma<false, true>(d, bk, grid, blk, s, ma);
    else
      launch_mfma<false, false>(d, bk, grid, blk, s, ma);
    if (ev_stop && hipEventRecord(hipEvent_t(ev_stop), s) != hipSuccess) return TQ_EDEVICE;
    }
  } else if (desc->polar) {
    const int pchunk = (((length + S - 1) / S) + 63) / 64 * 64;
    used_splits = (length + pchunk - 1) / pchunk;
    PolarArgs pa;
    pa.krec = ch.kbits;
    pa.knorm = ch.knorm;
    pa.vrec = reinterpret_cast<const uint8_t *>(ch.vcodes);
    pa.vnorm = ch.vnorm;
    pa.qp = qp;
    pa.qpack = qpack;
    pa.pcs = cp.pcs;
    pa.part = part;
    pa.scores = scores;
    pa.kb = ch.kbytes;
    pa.capacity = desc->capacity;
    pa.length = length;
    pa.chunk = pchunk;
    pa.splits = used_splits + wsplit;
    pa.kv_heads = desc->kv_heads;
    pa.q_heads = q_heads;
    pa.G = G;
    pa.m = m;
    pa.qstride = qstride;
    pa.score_stride = score_stride;
    pa.scale_log2 = sc * 1.4426950408889634f;
    const dim3 grid(units, used_splits);
    if (ev_start && hipEventRecord(hipEvent_t(ev_start), s) != hipSuccess) return TQ_EDEVICE;
    if (d == 64)
      hipLaunchKernelGGL(k_decode_polar<64>, grid, dim3(64 * kPolarWaves), 0, s, pa);
    else
      hipLaunchKernelGGL(k_decode_polar<128>, grid, dim3(64 * kPolarWaves), 0, s, pa);
    if (ev_stop && hipEventRecord(hipEvent_t(ev_stop), s) != hipSuccess) return TQ_EDEVICE;
  } else {
    DecodeArgs a;
    a.cp = cp;
    a.kbits = ch.kbits;
    a.knorm = ch.knorm;
    a.vcodes = ch.vcodes;
    a.vnorm = ch.vnorm;
    a.kbytes = ch.kbytes;
    a.tiles = ch.tiles;
    a.capacity = desc->capacity;
    a.bits_k = desc->bits_k;
    a.bits_v = desc->bits_v;
    a.m = m;
    a.kv_heads = desc->kv_heads;
    a.q_heads = q_heads;
    a.G = G;
    a.length = length;
    a.splits = S + wsplit;
    a.chunk = (length + S - 1) / S;
    a.score_stride = score_stride;
    a.scale = sc;
    a.qp = qp;
    a.qstride = qstride;
    a.part = part;
    a.scores = scores;
    const size_t shm = (size_t(kMaxG) * d + size_t(kMaxG) * m + size_t(kMaxG) * kDecThreads +
                        4 * kMaxG) * 4;
    dim3 grid(units, S);
    if (ev_start && hipEventRecord(hipEvent_t(ev_start), s) != hipSuccess) return TQ_EDEVICE;
    if (d == 64)
      hipLaunchKernelGGL(k_decode_split<64>, grid, dim3(kDecThreads), shm, s, a);
    else
      hipLaunchKernelGGL(k_decode_split<128>, grid, dim3(kDecThreads), shm, s, a);
    if (ev_stop && hipEventRecord(hipEvent_t(ev_stop), s) != hipSuccess) return TQ_EDEVICE;
  }
  }   // length > 0
  if (wlen > 0) {
    WindowArgs wa;
    wa.k = win->k;
    wa.v = win->v;
    wa.nk = win->nk;
    wa.nv = win->nv;
    wa.ak = win->ak;
    wa.av = win->av;
    wa.q = q;
    wa.Dsg = cp.D;
    wa.part = part;
    wa.scores = scores;
    wa.dtype = int(win->dtype);
    wa.qdtype = int(dtype);
    wa.len = wlen;
    wa.cap = win->cap;
    wa.length = length;
    wa.q_pos = q_pos;
    wa.kv_heads = desc->kv_heads;
    wa.q_heads = q_heads;
    wa.G = G;
    wa.splits_total = used_splits + wsplit;
    wa.split_idx = used_splits;
    wa.chunks_per_block = wcpb;
    wa.score_stride = score_stride;
    wa.rope_base = rope_base;
    wa.scale_log2 = sc * 1.4426950408889634f;
    wa.inv_sqrt_block = cp.inv_sqrt_block;
    const bool f32 = win->dtype == TQ_F32;
    const dim3 wgrid(units, wsplit);
    if (d == 64) {
      if (G <= 8) {
        if (f32) hipLaunchKernelGGL((k_window<64, 4, 8>), wgrid, dim3(256), 0, s, wa);
        else hipLaunchKernelGGL((k_window<64, 2, 8>), wgrid, dim3(256), 0, s, wa);
      } else {
        if (f32) hipLaunchKernelGGL((k_window<64, 4, 16>), wgrid, dim3(256), 0, s, wa);
        else hipLaunchKernelGGL((k_window<64, 2, 16>), wgrid, dim3(256), 0, s, wa);
      }
    } else {
      if (G <= 8) {
        if (f32) hipLaunchKernelGGL((k_window<128, 4, 8>), wgrid, dim3(256), 0, s, wa);
        else hipLaunchKernelGGL((k_window<128, 2, 8>), wgrid, dim3(256), 0, s, wa);
      } else {
        if (f32) hipLaunchKernelGGL((k_window<128, 4, 16>), wgrid, dim3(256), 0, s, wa);
        else hipLaunchKernelGGL((k_window<128, 2, 16>), wgrid, dim3(256), 0, s, wa);
      }
    }
  }
  if (!out) return launch_status();   // logits only: the scores are written, no merge
  used_splits += wsplit;
  if ((d == 64 || d == 128) && cp.block == d) {
    const dim3 mg(unsigned((rows + 3) / 4));
    if (d == 64)
      hipLaunchKernelGGL(k_decode_merge_wave<64>, mg, dim3(256), 0, s, part, used_splits, rows, cp, out);
    else
      hipLaunchKernelGGL(k_decode_merge_wave<128>, mg, dim3(256), 0, s, part, used_splits, rows, cp, out);
  } else {
    hipLaunchKernelGGL(k_decode_merge, dim3(rows), dim3(256), size_t(used_splits + d + 256 + d) * 4, s, part,
                       used_splits, d, cp, out);
  }
  return launch_status();
}

tq_status tq_decode_attend_profiled(const tq_cache_desc *desc, const void *codec_dev,
                                    const void *cache_dev, int32_t length, const void *q,
                                    int32_t dtype, int32_t q_heads, int32_t q_pos,
                                    float rope_base, float scale, float *out, float *scores,
                                    int32_t splits, void *ws, size_t ws_bytes,
                                    void *ev_start, void *ev_stop, tq_stream_t stream) {
  return decode_impl(desc, codec_dev, cache_dev, length, nullptr, q, dtype, q_heads, q_pos, rope_base,
                     scale, out, scores, splits, ws, ws_bytes, ev_start, ev_stop, stream);
}

size_t tq_decode_window_workspace_bytes(const tq_cache_desc *desc, int32_t q_heads, int32_t length) {
  if (!desc || !cache_desc_valid(*desc) || q_heads < 1 || length < 0) return 0;
  return decode_ws(*desc, q_heads, default_splits(*desc, length) + kWinMaxSplits);
}

tq_status tq_decode_attend_window(const tq_cache_desc *desc, const void *codec_dev,
                                  const void *cache_dev, int32_t length, const void *win_k,
                                  const void *win_v, int32_t win_dtype, int32_t win_len,
                                  int32_t win_cap, const void *q, int32_t dtype, int32_t q_heads,
                                  int32_t q_pos, float rope_base, float scale, float *out,
                                  float *scores, void *ws, size_t ws_bytes, tq_stream_t stream) {
  const WindowIn w{win_k, win_v, win_dtype, win_len, win_cap, nullptr, nullptr, nullptr, nullptr, false};
  return decode_impl(desc, codec_dev, cache_dev, length, &w, q, dtype, q_heads, q_pos, rope_base, scale,
                     out, scores, 0, ws, ws_bytes, nullptr, nullptr, stream);
}

tq_status tq_decode_step(const tq_cache_desc *desc, const void *codec_dev, void *cache_dev,
                         int32_t *length, void *win_k, void *win_v, int32_t win_dtype,
                         int32_t *win_len, int32_t win_cap, const void *new_k, const void *new_v,
                         const void *q, int32_t dtype, int32_t q_heads, int32_t q_pos,
                         float rope_base, float scale, float *out, float *scores, void *ws,
                         size_t ws_bytes, tq_stream_t stream) {
  if (!length || !win_len || !win_k || !win_v || !new_k || !new_v) return TQ_EINVAL;
  if (*length < 0 || win_cap < 1 || *win_len < 0 || *win_len > win_cap) return TQ_EINVAL;
  const bool flush = *win_len == win_cap;
  const int64_t packed = int64_t(*length) + (flush ? win_cap : 0);
  if (packed > INT32_MAX) return TQ_ECAPACITY;
  const int n_win = (flush ? 0 : *win_len) + 1;
  const WindowIn w{win_k, win_v, win_dtype, n_win, win_cap, new_k, new_v, win_k, win_v, flush};
  const tq_status st = decode_impl(desc, codec_dev, cache_dev, int32_t(packed), &w, q, dtype, q_heads, q_pos,
                                   rope_base, scale, out, scores, 0, ws, ws_bytes, nullptr, nullptr, stream);
  if (st == TQ_OK) {
    *length = int32_t(packed);
    *win_len = n_win;
  }
  return st;
}

size_t tq_nsn_means_workspace_bytes(const tq_cache_desc *desc, int32_t n) {
  if (!desc || !cache_desc_valid(*desc) || !desc->nsn || n < 1) return 0;
  const int units = desc->batch * desc->kv_heads;
  return size_t(units) * size_t(nsn_slices(n, units)) * 2 * size_t(desc->d) * sizeof(double);
}

tq_status tq_nsn_set_means(const tq_cache_desc *desc, const void *codec_dev, void *cache_dev,
                           const void *k, const void *v, int32_t dtype, int32_t start_pos,
                           int32_t n, float rope_base, void *ws, size_t ws_bytes,
                           tq_stream_t stream) {
  if (!desc || !codec_dev || !cache_dev || !k || !v || !ws) return TQ_EINVAL;
  if (!cache_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  if (!desc->nsn) return TQ_EINVAL;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_EINVAL;
  if (n < 1 || start_pos < 0) return TQ_EINVAL;
  if (!std::isfinite(rope_base) || rope_base < 0.0f) return TQ_EINVAL;
  if (ws_bytes < tq_nsn_means_workspace_bytes(desc, n)) return TQ_ENOSPACE;
  const int units = desc->batch * desc->kv_heads, d = desc->d;
  const int S = nsn_slices(n, units);
  NsnArgs na;
  na.k = k;
  na.v = v;
  na.part = static_cast<double *>(ws);
  na.n = n;
  na.start = start_pos;
  na.slices = S;
  na.per = (n + S - 1) / S;
  na.rope_base = rope_base;
  const CodecPtrs cp = codec_ptrs(codec_dev, d, desc->bits_k, desc->bits_v, desc->m);
  const CachePtrs ch = cache_ptrs(cache_dev, *desc);
  hipStream_t s = hipStream_t(stream);
  const dim3 grid(units, S);
#define TQ_NSN(DD, DT)                                                                    \
  if (d == DD && dtype == DT) hipLaunchKernelGGL((k_nsn_partial<DD, DT>), grid, dim3(256), 0, s, na);
  TQ_NSN(64, TQ_F32)
  TQ_NSN(64, TQ_BF16)
  TQ_NSN(64, TQ_F16)
  TQ_NSN(128, TQ_F32)
  TQ_NSN(128, TQ_BF16)
  TQ_NSN(128, TQ_F16)
#undef TQ_NSN
  if (d == 64)
    hipLaunchKernelGGL(k_nsn_final<64>, dim3(units), dim3(256), 0, s, na.part, S, n, cp.D, ch.nsn);
  else
    hipLaunchKernelGGL(k_nsn_final<128>, dim3(units), dim3(256), 0, s, na.part, S, n, cp.D, ch.nsn);
  return launch_status();
}

tq_status tq_decode_attend_splits(const tq_cache_desc *desc, const void *codec_dev,
                                  const void *cache_dev, int32_t length, const void *q,
                                  int32_t dtype, int32_t q_heads, int32_t q_pos,
                                  float rope_base, float scale, float *out, float *scores,
                                  int32_t splits, void *ws, size_t ws_bytes,
                                  tq_stream_t stream) {
  return tq_decode_attend_profiled(desc, codec_dev, cache_dev, length, q, dtype, q_heads, q_pos,
                                   rope_base, scale, out, scores, splits, ws, ws_bytes, nullptr,
                                   nullptr, stream);
}

tq_status tq_decode_attend(const tq_cache_desc *desc, const void *codec_dev, const void *cache_dev,
                           int32_t length, const void *q, int32_t dtype, int32_t q_heads,
                           int32_t q_pos, float rope_base, float scale, float *out, float *scores,
                           void *ws, size_t ws_bytes, tq_stream_t stream) {
  return tq_decode_attend_splits(desc, codec_dev, cache_dev, length, q, dtype, q_heads, q_pos,
                                 rope_base, scale, out, scores, 0, ws, ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free decode
// tq_decode_attend_noalloc keeps the decode workspace (query pack and split partials) in
// this file-scope device array instead of a caller buffer.  Every GPU the library runs on
// holds its own copy until the process ends.  On the host the array's name is only a
// stand-in symbol, never a device address: host code uses the address hipGetSymbolAddress
// returns, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `s` (the current device for the
// null stream).
tq_status scratch_for_stream(hipStream_t s, void **out) {
  int dev = -1;
  if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return TQ_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return TQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return TQ_EDEVICE;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return TQ_EDEVICE;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return TQ_EDEVICE;
    if (e != hipSuccess || !p) return TQ_EDEVICE;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return TQ_OK;
}
}  // namespace

extern "C" {

tq_status tq_decode_attend_noalloc(const tq_cache_desc *desc, const void *codec_dev,
                                   const void *cache_dev, int32_t length, const void *q,
                                   int32_t dtype, int32_t q_heads, int32_t q_pos, float rope_base,
                                   float scale, float *out, float *scores, tq_stream_t stream) {
  // the workspace tq_decode_attend would take for this shape, at the library's split count
  const bool shaped = desc && cache_desc_valid(*desc) && q_heads >= 1 && length >= 0;
  const size_t need = shaped ? decode_ws(*desc, q_heads, default_splits(*desc, length)) : 0;
  if (need > TQ_NOALLOC_SCRATCH_BYTES) return TQ_ENOSPACE;
  // an unshaped call fails decode_impl's argument checks before anything reads the
  // workspace, so the scratch is looked up only for calls that can run
  void *ws = reinterpret_cast<void *>(uintptr_t(256));
  if (shaped) {
    const tq_status st = scratch_for_stream(hipStream_t(stream), &ws);
    if (st != TQ_OK) return st;
  }
  return decode_impl(desc, codec_dev, cache_dev, length, nullptr, q, dtype, q_heads, q_pos, rope_base, scale,
                     out, scores, 0, ws, TQ_NOALLOC_SCRATCH_BYTES, nullptr, nullptr, stream);
}

size_t tq_search_workspace_bytes(const tq_cache_desc *db, int32_t n_db, int32_t nq, int32_t k) {
  if (!db || !cache_desc_valid(*db) || n_db < 0 || nq < 0 || k < 1 || k > 64) return 0;
  const size_t qstride = size_t(db->d) + db->m + 2;
  const size_t cand = size_t(nq) * search_tiles(n_db) * k;
  return align256(size_t(nq) * qstride * 4) + align256(cand * 4) + align256(cand * 4) + 256;
}

tq_status tq_search_topk(const tq_cache_desc *db, const void *codec_dev, const void *db_cache,
                         int32_t n_db, const float *queries, int32_t nq, int32_t k,
                         int32_t *idx_out, float *score_out, void *ws, size_t ws_bytes,
                         tq_stream_t stream) {
  if (!db || !codec_dev || !db_cache || !idx_out || !score_out || !ws) return TQ_EINVAL;
  if (!cache_desc_valid(*db)) return TQ_EUNSUPPORTED;
  if (db->nsn || db->polar) return TQ_EUNSUPPORTED;   // database vectors use the plain codec
  if (db->batch != 1 || db->kv_heads != 1 || db->bits_v != 0) return TQ_EINVAL;
  if (n_db < 0 || nq < 0 || k < 1 || k > 64) return TQ_EINVAL;
  if (n_db > db->capacity) return TQ_ECAPACITY;
  if (nq > 0 && !queries) return TQ_EINVAL;
  const int d = db->d, m = db->m;
  if (d % 64 != 0 || d > 2048 || hadamard_block(d) < 64) return TQ_EUNSUPPORTED;
  if ((size_t(kSearchQ) * (d + m + kSearchTile)) * 4 > 160 * 1024) return TQ_EUNSUPPORTED;
  if (ws_bytes < tq_search_workspace_bytes(db, n_db, nq, k)) return TQ_ENOSPACE;
  if (nq == 0) return TQ_OK;
  hipStream_t s = hipStream_t(stream);
  const CodecPtrs cp = codec_ptrs(codec_dev, d, db->bits_k, 0, m);
  const int qstride = d + m + 2;
  float *qp = static_cast<float *>(ws);
  const int ntiles = search_tiles(n_db);
  const size_t cand = size_t(nq) * ntiles * k;
  uint8_t *wb = static_cast<uint8_t *>(ws);
  float *cand_s = reinterpret_cast<float *>(wb + align256(size_t(nq) * qstride * 4));
  int *cand_i = reinterpret_cast<int *>(wb + align256(size_t(nq) * qstride * 4) + align256(cand * 4));
  hipLaunchKernelGGL(k_qprep_pack, dim3(nq), dim3(256), size_t(d + m + (m > 1024 ? m : 1024)) * 4, s,
                     static_cast<const void *>(queries), int(TQ_F32), d, m, 0, 0.0f, cp, qp, qstride,
                     nq, 1, db->bits_k, static_cast<uint8_t *>(nullptr), nullptr);
  // MFMA path: 3-bit codes with m = d, whole 128-coordinate groups, k <= 16.  The codec's
  // codebooks are exactly symmetric by construction.
  const bool mfma = db->bits_k == 3 && m == d && d % 128 == 0 && d <= 2048 && k <= kSmTopMax;
  if (n_db > 0 && mfma) {
    const int qgroups = (nq + kSmQ - 1) / kSmQ;
    // about one block per CU (256 on MI355X), at most one slice per 256-vector tile of the
    // workspace's candidate layout
    int slices = std::max(1, 256 / qgroups);
    slices = std::min(slices, ntiles);
    int per = (n_db + slices - 1) / slices;
    per = (per + 31) / 32 * 32;
    slices = (n_db + per - 1) / per;
    SearchMfmaArgs sa;
    const CachePtrs ch = cache_ptrs(const_cast<void *>(db_cache), *db);
    sa.kbits = ch.kbits;
    sa.knorm = ch.knorm;
    sa.ck = cp.ck;
    sa.qp = qp;
    sa.cand_s = cand_s;
    sa.cand_i = cand_i;
    sa.kbytes = ch.kbytes;
    sa.d = d;
    sa.n_db = n_db;
    sa.nq = nq;
    sa.k = k;
    sa.slices = slices;
    sa.per = per;
    sa.qstride = qstride;
    sa.qjl_scale = cp.qjl_scale;
    const size_t shm = size_t(d / 32) * 2048 + size_t(kSmWaves) * kSmQ * kSmTopMax * 8;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_search_mfma),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(shm)) != hipSuccess)
      return TQ_EDEVICE;
    hipLaunchKernelGGL(k_search_mfma, dim3(qgroups, slices), dim3(512), shm, s, sa);
    hipLaunchKernelGGL(k_search_merge, dim3(nq), dim3(256), 0, s, cand_s, cand_i, slices, k, idx_out, score_out);
    return launch_status();
  }
  if (n_db > 0) {
    SearchArgs a;
    const CachePtrs ch = cache_ptrs(const_cast<void *>(db_cache), *db);
    a.cp = cp;
    a.kbits = ch.kbits;
    a.knorm = ch.knorm;
    a.kbytes = ch.kbytes;
    a.d = d;
    a.m = m;
    a.bits_k = db->bits_k;
    a.n_db = n_db;
    a.nq = nq;
    a.k = k;
    a.ntiles = ntiles;
    a.qp = qp;
    a.qstride = qstride;
    a.cand_s = cand_s;
    a.cand_i = cand_i;
    const size_t shm = size_t(kSearchQ) * (d + m + kSearchTile) * 4;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_search_tile),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(shm)) != hipSuccess)
      return TQ_EDEVICE;
    hipLaunchKernelGGL(k_search_tile, dim3(ntiles, (nq + kSearchQ - 1) / kSearchQ),
                       dim3(kSearchTile), shm, s, a);
  }
  hipLaunchKernelGGL(k_search_merge, dim3(nq), dim3(256), 0, s, cand_s, cand_i,
                     n_db > 0 ? ntiles : 0, k, idx_out, score_out);
  return launch_status();
}

}  // extern "C"
