// Device half of libtq: HIP kernels for gfx950 and the C entry points that launch them.
//
// Kernels (the step of the method each one carries out is named at its definition):
//   k_cache_init        header of a packed cache
//   k_quantize_kv       RoPE -> seeded-sign FWHT -> norm -> Lloyd-Max codes -> bit planes
//                       -> residual -> QJL sign bits (MFMA), 4 lanes per token, d in {64, 128}
//   k_quantize_db       the same for database vectors of large d (one wave per vector)
//   k_qprep             query RoPE, rotation Pi q, S q_rot and their sums
//   k_decode_split      split-K decode: scores from the packed keys, online softmax,
//                       accumulation of dequantized values in the rotated basis
//   k_decode_combine    merge of the splits, normalisation, inverse rotation Pi^T
//   k_search_tile       packed database scores for a query tile + per-tile top-k
//   k_search_merge      per-query top-k over the tile candidates

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

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

// fp32 -> fp16 bits, round to nearest even; values that would round to infinity are
// stored as 65504 and reported through *over.
__device__ __forceinline__ uint16_t f16_sat_bits(float x, bool *over) {
  if (!(x < 65520.0f)) {  // also catches +inf / NaN norms
    *over = true;
    return 0x7BFF;
  }
  _Float16 h = (_Float16)x;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
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
  p.kbytes = L.kbytes;
  p.tiles = L.tiles;
  return p;
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
    default: v = 0;
  }
  hdr[i] = v;
}

// ------------------------------------------------------------------ quantize
struct QuantArgs {
  CodecPtrs cp;
  CachePtrs ch;
  const void *k, *v;
  int start, n_new, capacity, bits_k, bits_v, m, units;
  float rope_base;
};

typedef float v16f __attribute__((ext_vector_type(16)));
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

// Seeded-sign FWHT of one vector spread over the 4 lanes of a group: lane q holds chunk A
// (coordinates q*HC + e) and chunk B (D/2 + q*HC + e), e < HC.  Coordinate bits below
// HC are in-lane, the next two bits select the lane, the top bit selects the chunk.
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
#pragma unroll
  for (int dist = 1; dist <= 2; dist <<= 1) {
#pragma unroll
    for (int e = 0; e < 2 * HC; ++e) {
      const double o = __shfl_xor(x[e], dist, 64);
      x[e] = (q & dist) ? (o - x[e]) : (x[e] + o);
    }
  }
}

__device__ __forceinline__ double group4_sum(double v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  return v;
}

__device__ __forceinline__ uint32_t group4_or(uint32_t v) {
  v |= __shfl_xor(v, 1, 64);
  v |= __shfl_xor(v, 2, 64);
  return v;
}

// One workgroup (4 waves) per 64-token window aligned to value tiles; 4 lanes per token.
// Keys: RoPE (fp64 angles from an LDS table built by the fp64 rotation recurrence),
// signs, FWHT, norm, codes and residual all in fp64; the QJL projection z = S r runs
// on fp32 MFMA (v_mfma_f32_32x32x2f32) over the window's 64 residuals.  Values: signs,
// FWHT, norm, codes in fp64, then the window's codes are packed into value tiles.
template <int D, int DT>
__global__ __launch_bounds__(256, 2) void k_quantize_kv(QuantArgs a) {
  constexpr int H = D / 2;
  constexpr int HC = D / 8;     // coordinates per chunk
  constexpr int C = 2 * HC;     // coordinates per lane
  constexpr int W = D / 32;     // dwords per plane
  constexpr int RS = D + 1;     // padded residual row (floats)
  constexpr int ROPE_BYTES = 64 * H * 16;
  constexpr int R_BYTES = 64 * RS * 4;
  constexpr int U_BYTES = ROPE_BYTES > R_BYTES ? ROPE_BYTES : R_BYTES;
  __shared__ __align__(16) unsigned char u_s[U_BYTES];   // RoPE table, later residuals
  __shared__ uint8_t vcode_s[64][D];
  __shared__ float cb_s[4][kMaxCodes];
  double2 *rope_s = reinterpret_cast<double2 *>(u_s);   // [64][H]
  float *r_s = reinterpret_cast<float *>(u_s);           // [64][RS]

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

  if (tid < kMaxCodes) {
    cb_s[0][tid] = a.cp.ck[tid];
    cb_s[1][tid] = a.cp.tk[tid];
    cb_s[2][tid] = a.cp.cv[tid];
    cb_s[3][tid] = a.cp.tv[tid];
  }
  const bool use_rope = a.rope_base != 0.0f;
  if (use_rope) {
    constexpr int nblk = 256 / H, per = 64 / nblk;
    const int j = tid % H, i0 = (tid / H) * per;
    const double theta = pow(double(a.rope_base), -2.0 * double(j) / double(D));
    double s, c, sd, cd;
    sincos(double(p0 + i0) * theta, &s, &c);
    sincos(theta, &sd, &cd);
    for (int i = 0; i < per; ++i) {
      rope_s[(i0 + i) * H + j] = make_double2(c, s);
      const double cn = c * cd - s * sd;
      s = s * cd + c * sd;
      c = cn;
    }
  }
  __syncthreads();

  const double inv_sqrt_b = 1.0 / sqrt(double(a.cp.block));
  auto coord = [&](int e) { return e < HC ? q * HC + e : H + q * HC + (e - HC); };

  // ------------------------------------------------------------ keys
  {
    double x[C];
#pragma unroll
    for (int e = 0; e < C; ++e) x[e] = valid ? load_d<DT>(a.k, row * D + coord(e)) : 0.0;
    if (use_rope) {
#pragma unroll
      for (int e = 0; e < HC; ++e) {
        const double2 cs = rope_s[slot * H + q * HC + e];
        const double x0 = x[e], x1 = x[HC + e];
        x[e] = x0 * cs.x - x1 * cs.y;
        x[HC + e] = x0 * cs.y + x1 * cs.x;
      }
    }
#pragma unroll
    for (int e = 0; e < C; ++e) x[e] *= double(a.cp.D[coord(e)]);
    fwht_group4<D>(x, q);
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      x[e] *= inv_sqrt_b;
      ss += x[e] * x[e];
    }
    const double n = sqrt(group4_sum(ss));
    const uint16_t n16b = f64_to_f16_sat(n, &over);
    const double n16 = double(f16_bits_to_float(n16b));
    const double inv = n > 0.0 ? 1.0 / n : 0.0;
    const int K = 1 << a.bits_k;
    uint32_t pl[4][W];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int w = 0; w < W; ++w) pl[pp][w] = 0u;
    double rr = 0.0;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      double chat;
      const int code = bucketize64(x[e] * inv, cb_s[1], cb_s[0], K, &chat);
      const int j = coord(e);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) pl[pp][j >> 5] |= uint32_t((code >> pp) & 1) << (j & 31);
      x[e] -= n16 * chat;   // residual against the stored fp16 norm
      rr += x[e] * x[e];
    }
    const uint16_t rn16b = f64_to_f16_sat(sqrt(group4_sum(rr)), &over);
    uint32_t *rec = reinterpret_cast<uint32_t *>(a.ch.kbits + (size_t(unit) * a.capacity + (valid ? p : 0)) * a.ch.kbytes);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const uint32_t v = group4_or(pl[pp][w]);
        if (valid && pp < a.bits_k && (w & 3) == q) rec[pp * W + w] = v;
      }
    }
    if (valid && q == 0)
      a.ch.knorm[size_t(unit) * a.capacity + p] = uint32_t(n16b) | (uint32_t(rn16b) << 16);
    __syncthreads();   // every wave is done with the RoPE table before residuals overwrite it
#pragma unroll
    for (int e = 0; e < C; ++e) r_s[slot * RS + coord(e)] = float(x[e]);
    __syncthreads();
    // z^T[m x 64 tokens] = S[m x D] . R^T[D x 64]: one 32 x 32 output tile per iteration
    const int mt_n = a.m / 32;
    for (int it = wv; it < 2 * mt_n; it += 4) {
      const int mt = it >> 1, tt = it & 1;
      v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const float *srow = a.cp.S + size_t(32 * mt + (lane & 31)) * D + (lane >> 5);
      const float *rrow = r_s + (32 * tt + (lane & 31)) * RS + (lane >> 5);
#pragma unroll 8
      for (int j0 = 0; j0 < D; j0 += 2)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(srow[j0], rrow[j0], acc, 0, 0, 0);
      uint32_t bits = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        bits |= uint32_t(acc[r] >= 0.0f) << (8 * (r >> 2) + 4 * (lane >> 5) + (r & 3));
      bits |= __shfl_xor(bits, 32, 64);
      const int ts = 32 * tt + (lane & 31);
      const int pt = p0 + ts;
      if (lane < 32 && pt >= a.start && pt < end) {
        uint32_t *rt = reinterpret_cast<uint32_t *>(a.ch.kbits + (size_t(unit) * a.capacity + pt) * a.ch.kbytes);
        rt[a.bits_k * W + mt] = bits;
      }
    }
  }

  // ------------------------------------------------------------ values
  if (a.bits_v > 0) {
    double x[C];
#pragma unroll
    for (int e = 0; e < C; ++e)
      x[e] = valid ? load_d<DT>(a.v, row * D + coord(e)) * double(a.cp.D[coord(e)]) : 0.0;
    fwht_group4<D>(x, q);
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      x[e] *= inv_sqrt_b;
      ss += x[e] * x[e];
    }
    const double n = sqrt(group4_sum(ss));
    const uint16_t n16b = f64_to_f16_sat(n, &over);
    const double inv = n > 0.0 ? 1.0 / n : 0.0;
    const int K = 1 << a.bits_v;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      double chat;
      vcode_s[slot][coord(e)] = uint8_t(bucketize64(x[e] * inv, cb_s[3], cb_s[2], K, &chat));
    }
    if (valid && q == 0) a.ch.vnorm[size_t(unit) * a.capacity + p] = n16b;
    __syncthreads();
    // value tiles: one (tile, coordinate) word per thread; tokens outside the written
    // range keep their previous bits
    const int bv = a.bits_v;
    const uint32_t mask = (1u << bv) - 1u;
    for (int wi = tid; wi < 2 * D; wi += 256) {
      const int tloc = wi / D, j = wi % D;
      const int tile = first_tile + 2 * int(blockIdx.x) + tloc;
      const int tstart = tile * kValueTile;
      if (tstart >= end || tile >= a.ch.tiles) continue;
      uint32_t *wp = a.ch.vcodes + ((size_t(unit) * a.ch.tiles + tile) * D + j) * bv;
      uint32_t word[4] = {0u, 0u, 0u, 0u};
      const bool full = tstart >= a.start && tstart + kValueTile <= end;
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
// z = S r on fp32 MFMA (v_mfma_f32_16x16x4f32), S streamed from L2.
constexpr int kLargeGroup = 16;

template <int C, int E, int DT>
__global__ __launch_bounds__(256) void k_quantize_db(QuantArgs a) {
  constexpr int NB = C / E;
  constexpr int B = 64 * E;
  constexpr int Dm = C * 64;
  constexpr int RS = Dm + 4;
  extern __shared__ float r_s[];   // [16][RS]
  __shared__ float cb_s[2][kMaxCodes];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int unit = blockIdx.y;
  const int g0 = a.start + int(blockIdx.x) * kLargeGroup;
  const int end = a.start + a.n_new;
  if (tid < kMaxCodes) {
    cb_s[0][tid] = a.cp.ck[tid];
    cb_s[1][tid] = a.cp.tk[tid];
  }
  __syncthreads();
  const double inv_sqrt_b = 1.0 / sqrt(double(B));
  const int K = 1 << a.bits_k;
  const int dbytes = Dm / 8;
  for (int vi = wv; vi < kLargeGroup; vi += 4) {
    const int p = g0 + vi;
    const bool valid = p < end;
    const size_t row = size_t(unit) * size_t(a.n_new) + size_t(valid ? p - a.start : 0);
    double x[C];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = b * B + E * lane + e;
        x[b * E + e] = valid ? load_d<DT>(a.k, row * Dm + j) * double(a.cp.D[j]) : 0.0;
      }
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
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < E; ++e) r_s[vi * RS + b * B + E * lane + e] = float(x[b * E + e]);
    if (valid && lane == 0) {
      a.ch.knorm[size_t(unit) * a.capacity + p] = uint32_t(n16b) | (uint32_t(rn16b) << 16);
      if (over) atomicOr(a.ch.flags, 1u);
    }
  }
  __syncthreads();
  // z^T[m x 16] = S[m x Dm] . R^T[Dm x 16], 16-row output tiles spread over the waves
  const int mt_n = a.m / 16;
  for (int mt = wv; mt < mt_n; mt += 4) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    const float *srow = a.cp.S + size_t(16 * mt + (lane & 15)) * Dm + (lane >> 4);
    const float *rrow = r_s + (lane & 15) * RS + (lane >> 4);
#pragma unroll 8
    for (int j0 = 0; j0 < Dm; j0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(srow[j0], rrow[j0], acc, 0, 0, 0);
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

// ------------------------------------------------------------------ query preparation
// One block per query row: q_rot = Pi RoPE(q, q_pos) (LDS FWHT), sq = S q_rot,
// sums sum_j q_rot_j and sum_i sq_i.  Output row layout: [q_rot d][sq m][sum_q, sum_sq].
__global__ __launch_bounds__(256) void k_qprep(const void *q, int dtype, int d, int m,
                                               int q_pos, float rope_base, CodecPtrs cp,
                                               float *out, int out_stride) {
  extern __shared__ float qs[];  // d floats
  const int rowi = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t base = size_t(rowi) * d;
  const int h = d / 2;
  if (rope_base != 0.0f) {
    for (int j = tid; j < h; j += blockDim.x) {
      const double theta = pow(double(rope_base), -2.0 * double(j) / double(d));
      double s, c;
      sincos(double(q_pos) * theta, &s, &c);
      const float x0 = load_elem(q, base + j, dtype), x1 = load_elem(q, base + j + h, dtype);
      qs[j] = (x0 * float(c) - x1 * float(s)) * cp.D[j];
      qs[j + h] = (x0 * float(s) + x1 * float(c)) * cp.D[j + h];
    }
  } else {
    for (int j = tid; j < d; j += blockDim.x) qs[j] = load_elem(q, base + j, dtype) * cp.D[j];
  }
  __syncthreads();
  const int B = cp.block;
  for (int hh = 1; hh < B; hh <<= 1) {
    for (int k = tid; k < d / 2; k += blockDim.x) {
      // butterfly k of this stage: pairs (i, i + hh) inside each block
      const int blk = k / (B / 2), kk = k % (B / 2);
      const int i = blk * B + (kk / hh) * 2 * hh + (kk % hh);
      const float x0 = qs[i], x1 = qs[i + hh];
      qs[i] = x0 + x1;
      qs[i + hh] = x0 - x1;
    }
    __syncthreads();
  }
  float *o = out + size_t(rowi) * out_stride;
  float part = 0.0f;
  for (int j = tid; j < d; j += blockDim.x) {
    const float v = qs[j] * cp.inv_sqrt_block;
    o[j] = v;
    part += v;
  }
  __syncthreads();
  for (int j = tid; j < d; j += blockDim.x) qs[j] *= cp.inv_sqrt_block;
  __syncthreads();
  float part2 = 0.0f;
  for (int i = tid; i < m; i += blockDim.x) {
    float z = 0.0f;
    for (int j = 0; j < d; ++j) z = fmaf(cp.S[size_t(i) * d + j], qs[j], z);
    o[d + i] = z;
    part2 += z;
  }
  __shared__ float red[2][8];
  part = wave_sum(part);
  part2 = wave_sum(part2);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = part;
    red[1][tid >> 6] = part2;
  }
  __syncthreads();
  if (tid == 0) {
    float s0 = 0.0f, s1 = 0.0f;
    for (int w = 0; w < int(blockDim.x) / 64; ++w) {
      s0 += red[0][w];
      s1 += red[1][w];
    }
    o[d + m] = s0;
    o[d + m + 1] = s1;
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
  float *scores;     // optional [B][Hq][length]
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
          if (a.scores) a.scores[(size_t(b) * a.q_heads + hq0 + h) * a.length + t] = score;
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

// Merge of the splits and inverse rotation: out = D .* (H o) / sqrt(B) = Pi^T o.
__global__ __launch_bounds__(256) void k_decode_combine(const float *part, int splits, int d,
                                                        CodecPtrs cp, float *out) {
  extern __shared__ float os[];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float *pr = part + size_t(row) * splits * (d + 2);
  float Mx = -INFINITY;
  for (int s = 0; s < splits; ++s) Mx = fmaxf(Mx, pr[size_t(s) * (d + 2) + d]);
  float L = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const float ms = pr[size_t(s) * (d + 2) + d];
    if (ms != -INFINITY) L += pr[size_t(s) * (d + 2) + d + 1] * __expf(ms - Mx);
  }
  const float invL = L > 0.0f ? 1.0f / L : 0.0f;
  for (int j = tid; j < d; j += blockDim.x) {
    float v = 0.0f;
    for (int s = 0; s < splits; ++s) {
      const float ms = pr[size_t(s) * (d + 2) + d];
      if (ms != -INFINITY) v += pr[size_t(s) * (d + 2) + j] * __expf(ms - Mx);
    }
    os[j] = v * invL;
  }
  __syncthreads();
  const int B = cp.block;
  for (int hh = 1; hh < B; hh <<= 1) {
    for (int k = tid; k < d / 2; k += blockDim.x) {
      const int blk = k / (B / 2), kk = k % (B / 2);
      const int i = blk * B + (kk / hh) * 2 * hh + (kk % hh);
      const float x0 = os[i], x1 = os[i + hh];
      os[i] = x0 + x1;
      os[i + hh] = x0 - x1;
    }
    __syncthreads();
  }
  for (int j = tid; j < d; j += blockDim.x) out[size_t(row) * d + j] = os[j] * cp.inv_sqrt_block * cp.D[j];
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

// ------------------------------------------------------------------ host-side helpers
tq_status launch_status() {
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EDEVICE;
}

bool decode_supported(const tq_cache_desc &c) {
  return (c.d == 64 || c.d == 128) && c.bits_v > 0;
}

int default_splits(const tq_cache_desc &c, int length) {
  if (length <= 0) return 1;
  const int units = c.batch * c.kv_heads;
  const int by_len = (length + 255) / 256;
  const int want = (4096 + units - 1) / units;
  int s = by_len < want ? by_len : want;
  if (s < 1) s = 1;
  if (s > 4096) s = 4096;
  return s;
}

size_t decode_ws(const tq_cache_desc &c, int q_heads, int splits) {
  const size_t rows = size_t(c.batch) * q_heads;
  const size_t qstride = size_t(c.d) + c.m + 2;
  return align256(rows * qstride * 4) + align256(rows * size_t(splits) * (c.d + 2) * 4);
}

int search_tiles(int n_db) { return (n_db + kSearchTile - 1) / kSearchTile; }

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_cache_init(const tq_cache_desc *desc, void *cache_dev, tq_stream_t stream) {
  if (!desc || !cache_dev) return TQ_EINVAL;
  if (!cache_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  hipLaunchKernelGGL(k_cache_init, dim3(1), dim3(64), 0, hipStream_t(stream),
                     static_cast<uint32_t *>(cache_dev), *desc);
  return launch_status();
}

tq_status tq_quantize_kv_profiled(const tq_cache_desc *desc, const void *codec_dev,
                                  void *cache_dev, const void *k, const void *v,
                                  tq_dtype dtype, int32_t start_pos, int32_t n_new,
                                  float rope_base, void *ev_start, void *ev_stop,
                                  tq_stream_t stream) {
  if (!desc || !codec_dev || !cache_dev) return TQ_EINVAL;
  if (!cache_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_EINVAL;
  if (start_pos < 0 || n_new < 0) return TQ_EINVAL;
  if (int64_t(start_pos) + int64_t(n_new) > int64_t(desc->capacity)) return TQ_ECAPACITY;
  if (n_new > 0 && (!k || (desc->bits_v > 0) != (v != nullptr))) return TQ_EINVAL;
  if (!std::isfinite(rope_base) || rope_base < 0.0f) return TQ_EINVAL;
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
  hipStream_t s = hipStream_t(stream);
  if (ev_start && hipEventRecord(hipEvent_t(ev_start), s) != hipSuccess) return TQ_EDEVICE;
  if (small) {
    const int first_tile = start_pos / kValueTile;
    const int end_tile = (start_pos + n_new + kValueTile - 1) / kValueTile;
    const int windows = (end_tile - first_tile + 1) / 2;
    dim3 grid(windows, a.units);
#define TQ_QKV(DD, TT) hipLaunchKernelGGL((k_quantize_kv<DD, TT>), grid, dim3(256), 0, s, a)
    if (d == 64) {
      if (dtype == TQ_F32) TQ_QKV(64, TQ_F32); else if (dtype == TQ_BF16) TQ_QKV(64, TQ_BF16); else TQ_QKV(64, TQ_F16);
    } else {
      if (dtype == TQ_F32) TQ_QKV(128, TQ_F32); else if (dtype == TQ_BF16) TQ_QKV(128, TQ_BF16); else TQ_QKV(128, TQ_F16);
    }
#undef TQ_QKV
  } else {
    dim3 grid((n_new + kLargeGroup - 1) / kLargeGroup, a.units);
    const size_t shm = size_t(kLargeGroup) * (d + 4) * 4;
#define TQ_QDB(CC, EE, TT)                                                                     \
  do {                                                                                         \
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_quantize_db<CC, EE, TT>),         \
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(shm)) != hipSuccess) \
      return TQ_EDEVICE;                                                                       \
    hipLaunchKernelGGL((k_quantize_db<CC, EE, TT>), grid, dim3(256), shm, s, a);               \
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
                         const void *k, const void *v, tq_dtype dtype, int32_t start_pos,
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

tq_status tq_decode_attend_profiled(const tq_cache_desc *desc, const void *codec_dev,
                                    const void *cache_dev, int32_t length, const void *q,
                                    tq_dtype dtype, int32_t q_heads, int32_t q_pos,
                                    float rope_base, float scale, float *out, float *scores,
                                    int32_t splits, void *ws, size_t ws_bytes,
                                    void *ev_start, void *ev_stop, tq_stream_t stream) {
  if (!desc || !codec_dev || !cache_dev || !q || !out || !ws) return TQ_EINVAL;
  if (!cache_desc_valid(*desc)) return TQ_EUNSUPPORTED;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_EINVAL;
  if (q_heads < 1 || q_heads % desc->kv_heads != 0) return TQ_EINVAL;
  if (q_heads / desc->kv_heads > kMaxG) return TQ_EUNSUPPORTED;
  if (length < 0 || splits < 0 || q_pos < 0) return TQ_EINVAL;
  if (length > desc->capacity) return TQ_ECAPACITY;
  if (!std::isfinite(rope_base) || rope_base < 0.0f || !std::isfinite(scale)) return TQ_EINVAL;
  if (!decode_supported(*desc)) return TQ_EUNSUPPORTED;
  if (desc->m > 512) return TQ_EUNSUPPORTED;
  const int S = splits == 0 ? default_splits(*desc, length) : splits;
  if (ws_bytes < decode_ws(*desc, q_heads, S)) return TQ_ENOSPACE;
  const int d = desc->d, m = desc->m;
  const int rows = desc->batch * q_heads;
  hipStream_t s = hipStream_t(stream);
  if (length == 0) {
    if (hipMemsetAsync(out, 0, size_t(rows) * d * 4, s) != hipSuccess) return TQ_EDEVICE;
    return TQ_OK;
  }
  const CodecPtrs cp = codec_ptrs(codec_dev, d, desc->bits_k, desc->bits_v, m);
  float *qp = static_cast<float *>(ws);
  const int qstride = d + m + 2;
  float *part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + align256(size_t(rows) * qstride * 4));
  hipLaunchKernelGGL(k_qprep, dim3(rows), dim3(256), d * 4, s, q, int(dtype), d, m, q_pos,
                     rope_base, cp, qp, qstride);
  DecodeArgs a;
  const CachePtrs ch = cache_ptrs(const_cast<void *>(cache_dev), *desc);
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
  a.G = q_heads / desc->kv_heads;
  a.length = length;
  a.splits = S;
  a.chunk = (length + S - 1) / S;
  a.scale = scale == 0.0f ? float(1.0 / std::sqrt(double(d))) : scale;
  a.qp = qp;
  a.qstride = qstride;
  a.part = part;
  a.scores = scores;
  const size_t shm = (size_t(kMaxG) * d + size_t(kMaxG) * m + size_t(kMaxG) * kDecThreads +
                      4 * kMaxG) * 4;
  // the value-phase partial sums reuse the p region: (256 / d) * kMaxG * d floats
  const size_t shm_all = shm;
  dim3 grid(desc->batch * desc->kv_heads, S);
  if (ev_start && hipEventRecord(hipEvent_t(ev_start), s) != hipSuccess) return TQ_EDEVICE;
  if (d == 64)
    hipLaunchKernelGGL(k_decode_split<64>, grid, dim3(kDecThreads), shm_all, s, a);
  else
    hipLaunchKernelGGL(k_decode_split<128>, grid, dim3(kDecThreads), shm_all, s, a);
  if (ev_stop && hipEventRecord(hipEvent_t(ev_stop), s) != hipSuccess) return TQ_EDEVICE;
  hipLaunchKernelGGL(k_decode_combine, dim3(rows), dim3(128), d * 4, s, part, S, d, cp, out);
  return launch_status();
}

tq_status tq_decode_attend_splits(const tq_cache_desc *desc, const void *codec_dev,
                                  const void *cache_dev, int32_t length, const void *q,
                                  tq_dtype dtype, int32_t q_heads, int32_t q_pos,
                                  float rope_base, float scale, float *out, float *scores,
                                  int32_t splits, void *ws, size_t ws_bytes,
                                  tq_stream_t stream) {
  return tq_decode_attend_profiled(desc, codec_dev, cache_dev, length, q, dtype, q_heads, q_pos,
                                   rope_base, scale, out, scores, splits, ws, ws_bytes, nullptr,
                                   nullptr, stream);
}

tq_status tq_decode_attend(const tq_cache_desc *desc, const void *codec_dev, const void *cache_dev,
                           int32_t length, const void *q, tq_dtype dtype, int32_t q_heads,
                           int32_t q_pos, float rope_base, float scale, float *out, float *scores,
                           void *ws, size_t ws_bytes, tq_stream_t stream) {
  return tq_decode_attend_splits(desc, codec_dev, cache_dev, length, q, dtype, q_heads, q_pos,
                                 rope_base, scale, out, scores, 0, ws, ws_bytes, stream);
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
  hipLaunchKernelGGL(k_qprep, dim3(nq), dim3(256), d * 4, s, static_cast<const void *>(queries),
                     int(TQ_F32), d, m, 0, 0.0f, cp, qp, qstride);
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
