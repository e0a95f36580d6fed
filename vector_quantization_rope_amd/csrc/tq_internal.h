// Internal declarations shared by the host part (tq_host.cpp) and the device part
// (tq_device.hip) of libtq.  Not installed; the public interface is include/tq.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr uint32_t kCacheMagic = 0x564B5154u;  // "TQKV"
constexpr uint32_t kCodecMagic = 0x44435154u;  // "TQCD"
constexpr uint32_t kFormatVersion = 1;
constexpr size_t kHeaderBytes = 256;
constexpr int kValueTile = 32;   // tokens per value-code tile
constexpr int kMaxCodes = 16;    // 2^4 centroids at most
constexpr int64_t kMaxUnits = 65535;         // batch x kv_heads of one cache
constexpr int32_t kMaxCapacity = 1 << 30;    // token slots per unit

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Largest power of two dividing d: the Hadamard block size.
inline int hadamard_block(int d) { return d & (-d); }

struct CacheLayout {
  size_t kbits = 0, knorm = 0, vcodes = 0, vnorm = 0, nsn = 0, total = 0;
  int kbytes = 0;   // bytes of one key record (planes + sign bits)
  int knrec = 4;    // bytes of one key norm record (8 with NSN: + fp16 s1, padding)
  int vnrec = 2;    // bytes of one value norm record (4 with NSN: + fp16 s1)
  int tiles = 0;    // value tiles per unit
  int vwords = 0;   // dwords per (tile, coordinate) = bits_v
};

// PolarQuant angle grids: levels 1..kPolarLevels, up to kPolarCodes cells per level.
constexpr int kPolarLevels = 11;
constexpr int kPolarCodes = 16;

struct CodecLayout {
  // byte offsets inside the codec table
  size_t ck = 0, tk = 0, cv = 0, tv = 0, D = 0, S = 0, ST = 0, total = 0;
  size_t Sh[3] = {0, 0, 0};   // S = Sh[0] + Sh[1] + Sh[2], fp16 parts (exact for |S| >= 1/2)
  size_t pcs = 0;   // fp32 [kPolarLevels][kPolarCodes][2]: cos, sin of each angle centroid
  size_t pt = 0;    // fp64 [kPolarLevels][kPolarCodes]: angle boundaries (level l at l - 1)
  int block = 0;
};

// Host-side header of the codec table (first 256 bytes).
struct CodecHeader {
  uint32_t magic, version;
  int32_t d, bits_k, bits_v, m;
  uint64_t seed;
  int32_t block;
  float qjl_scale;       // sqrt(pi/2) / m (0 if m == 0)
  float inv_sqrt_block;  // 1 / sqrt(block)
  uint32_t reserved[53];
};
static_assert(sizeof(CodecHeader) == 256, "codec header is 256 bytes");

struct CacheHeader {
  uint32_t magic, version, flags, zero;
  int32_t batch, kv_heads, d, capacity, bits_k, bits_v, m, nsn, polar;
  uint32_t reserved[51];
};
static_assert(sizeof(CacheHeader) == 256, "cache header is 256 bytes");

bool codec_desc_valid(const tq_codec_desc &c);
bool cache_desc_valid(const tq_cache_desc &c);
CacheLayout cache_layout(const tq_cache_desc &c);
CodecLayout codec_layout(int d, int bits_k, int bits_v, int m);

// PolarQuant grid of one level in fp64: level 1, 16 centroids and 15 boundaries; level
// l >= 2, 4 centroids and 3 boundaries.
void polar_grid(int level, double *c, double *t);

// fp64 -> fp16 (round to nearest even); returns the fp16 value as a double and its bits.
double round_fp16(double x, uint16_t *bits_out = nullptr);

}  // namespace tq
