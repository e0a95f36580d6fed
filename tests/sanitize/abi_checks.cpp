// Host-side checks of libtq run under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built by tests/test_sanitize_host.py from the library's own sources with the sanitizers
// on the host half only (the device code is compiled but never launched: every device
// entry point called here fails its host-side validation first, so no GPU is needed).
// Every buffer the library writes is sized exactly, so a write past its end is an ASan
// report; integer overflow in the layout arithmetic is a UBSan report.  The process exit
// status is the number of failed checks.

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/tq.h"

static int g_checks = 0, g_fail = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    ++g_checks;                                                            \
    if (!(cond)) {                                                         \
      ++g_fail;                                                            \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
    }                                                                      \
  } while (0)

static void codebooks() {
  const int dims[] = {8, 64, 128, 1536, 4096};
  for (int d : dims) {
    for (int bits = 1; bits <= 4; ++bits) {
      const int K = 1 << bits;
      std::vector<float> c(K), t(K - 1 > 0 ? K - 1 : 1);
      CHECK(tq_make_codebook(d, bits, c.data(), t.data()) == TQ_OK);
      for (int k = 0; k < K; ++k) CHECK(c[K - 1 - k] == -c[k]);
      for (int k = 0; k + 1 < K; ++k) CHECK(c[k] < t[k] && t[k] < c[k + 1]);
      std::vector<double> c64(K), t64(K - 1 > 0 ? K - 1 : 1);
      CHECK(tq_make_codebook_f64(d, bits, c64.data(), t64.data()) == TQ_OK);
    }
  }
  float c[16], t[16];
  CHECK(tq_make_codebook(4, 2, c, t) == TQ_EUNSUPPORTED);
  CHECK(tq_make_codebook(4097, 2, c, t) == TQ_EUNSUPPORTED);
  CHECK(tq_make_codebook(64, 5, c, t) == TQ_EUNSUPPORTED);
  CHECK(tq_make_codebook(64, 0, c, t) == TQ_EUNSUPPORTED);
  CHECK(tq_make_codebook(64, 2, nullptr, t) == TQ_EINVAL);
  CHECK(tq_make_codebook(INT_MIN, 2, c, t) == TQ_EUNSUPPORTED);
  for (int lv = 1; lv <= 11; ++lv) {
    const int K = lv == 1 ? 16 : 4;
    std::vector<double> pc(K), pt(K - 1);
    CHECK(tq_make_polar_grid(lv, pc.data(), pt.data()) == TQ_OK);
    for (int k = 0; k + 1 < K; ++k) CHECK(pc[k] < pt[k] && pt[k] < pc[k + 1]);
  }
  double pc[16], pt[16];
  CHECK(tq_make_polar_grid(0, pc, pt) == TQ_EUNSUPPORTED);
  CHECK(tq_make_polar_grid(12, pc, pt) == TQ_EUNSUPPORTED);
}

static void codec_tables() {
  const tq_codec_desc descs[] = {{64, 2, 3, 64, 0},     {128, 2, 3, 128, 7}, {128, 3, 3, 96, 12345},
                                 {1536, 3, 0, 1536, 0}, {8, 1, 1, 32, 1},    {4096, 4, 4, 0, 3}};
  for (const tq_codec_desc &cd : descs) {
    const size_t n = tq_codec_bytes(&cd);
    CHECK(n > 0);
    std::vector<uint8_t> buf(n);                      // exactly the reported size
    CHECK(tq_codec_build(&cd, buf.data(), n) == TQ_OK);
    CHECK(tq_codec_build(&cd, buf.data(), n - 1) == TQ_ENOSPACE);
  }
  const tq_codec_desc bad[] = {{100, 2, 3, 128, 0}, {128, 5, 3, 128, 0}, {128, 2, 3, 100, 0},
                               {128, 2, -1, 128, 0}, {128, 2, 3, 4096, 0}, {INT_MAX, 2, 3, 128, 0}};
  uint8_t tiny[16];
  for (const tq_codec_desc &cd : bad) {
    CHECK(tq_codec_bytes(&cd) == 0);
    CHECK(tq_codec_build(&cd, tiny, sizeof(tiny)) == TQ_EUNSUPPORTED);
  }
  CHECK(tq_codec_bytes(nullptr) == 0);
  CHECK(tq_codec_build(&descs[0], nullptr, 1 << 20) == TQ_EINVAL);
}

static void cache_sizes() {
  const tq_cache_desc ok[] = {
      {1, 1, 128, 1024, 2, 3, 128, 0, 0},  {3, 5, 64, 100, 2, 3, 64, 0, 0},
      {1, 1, 1536, 1000, 3, 0, 1536, 0, 0}, {2, 2, 128, 33, 4, 1, 32, 0, 0},
      {1, 1, 128, 1024, 2, 3, 128, 1, 0},  {1, 1, 128, 1024, 3, 3, 128, 0, 1},
      {1, 1, 128, 0, 2, 3, 128, 0, 0},     {255, 257, 128, 1 << 30, 4, 4, 2048, 0, 0},
      {65535, 1, 4096, 1 << 30, 4, 4, 2048, 0, 0}};
  for (const tq_cache_desc &c : ok) {
    const size_t n = tq_cache_bytes(&c);
    CHECK(n >= 256 && n % 256 == 0);
    // at least the key records of every slot
    const double slots = double(c.batch) * c.kv_heads * c.capacity;
    CHECK(double(n) >= slots * ((c.bits_k * c.d + c.m) / 8));
  }
  const tq_cache_desc bad[] = {
      {0, 1, 128, 64, 2, 3, 128, 0, 0},        {1, 1, 128, -1, 2, 3, 128, 0, 0},
      {1, 1, 128, INT_MAX, 2, 3, 128, 0, 0},   {1, 1, 128, (1 << 30) + 1, 2, 3, 128, 0, 0},
      {65536, 1, 128, 64, 2, 3, 128, 0, 0},    {INT_MAX, INT_MAX, 128, 64, 2, 3, 128, 0, 0},
      {256, 256, 128, 64, 2, 3, 128, 0, 0},    {1, 1, 128, 64, 2, 3, 128, 2, 0},
      {1, 1, 128, 64, 2, 0, 128, 1, 0},        {1, 1, 128, 64, 2, 3, 128, 0, 1},
      {1, 1, 256, 64, 3, 0, 256, 0, 1},        {1, 1, 128, 64, 3, 3, 128, 1, 1}};
  for (const tq_cache_desc &c : bad) CHECK(tq_cache_bytes(&c) == 0);
  CHECK(tq_cache_bytes(nullptr) == 0);
}

static void device_entry_validation() {
  // none of these calls gets past its host-side checks, so the fake pointer is never used
  void *P = reinterpret_cast<void *>(uintptr_t(0x1000));
  float *F = static_cast<float *>(P);
  const tq_cache_desc good{1, 1, 128, 64, 2, 3, 128, 0, 0};
  const tq_cache_desc bad_d{1, 1, 100, 64, 2, 3, 128, 0, 0};
  const tq_cache_desc huge{INT_MAX, INT_MAX, 128, 64, 2, 3, 128, 0, 0};
  const tq_cache_desc nsn{1, 1, 128, 64, 2, 3, 128, 1, 0};
  const tq_cache_desc db{1, 1, 128, 64, 3, 0, 128, 0, 0};
  const size_t big = size_t(1) << 30;

  CHECK(tq_cache_init(&good, nullptr, nullptr) == TQ_EINVAL);
  CHECK(tq_cache_init(&huge, P, nullptr) == TQ_EUNSUPPORTED);

  CHECK(tq_quantize_kv(&good, nullptr, P, P, P, TQ_F32, 0, 1, 0.0f, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&good, P, P, P, P, TQ_F32, 60, 5, 0.0f, nullptr) == TQ_ECAPACITY);
  CHECK(tq_quantize_kv(&good, P, P, P, P, TQ_F32, INT_MAX, INT_MAX, 0.0f, nullptr) == TQ_ECAPACITY);
  CHECK(tq_quantize_kv(&good, P, P, P, nullptr, TQ_F32, 0, 1, 0.0f, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&good, P, P, P, P, 7, 0, 1, 0.0f, nullptr) == TQ_EINVAL);
  CHECK(tq_decode_attend(&good, P, P, 10, P, -1, 1, 0, 0.f, 0.f, F, nullptr, P, big, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&good, P, P, P, P, TQ_F32, 0, -1, 0.0f, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&good, P, P, P, P, TQ_F32, -1, 1, 0.0f, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&good, P, P, P, P, TQ_F32, 0, 1, NAN, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&good, P, P, P, P, TQ_F32, 0, 1, -1.0f, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&good, P, P, static_cast<char *>(P) + 4, P, TQ_F32, 0, 1, 0.0f, nullptr) == TQ_EINVAL);
  CHECK(tq_quantize_kv(&bad_d, P, P, P, P, TQ_F32, 0, 1, 0.0f, nullptr) == TQ_EUNSUPPORTED);
  CHECK(tq_quantize_kv(&huge, P, P, P, P, TQ_F32, 0, 1, 0.0f, nullptr) == TQ_EUNSUPPORTED);

  CHECK(tq_decode_attend(&good, P, P, 65, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P, big, nullptr) == TQ_ECAPACITY);
  CHECK(tq_decode_attend(&good, P, P, -1, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P, big, nullptr) != TQ_OK);
  CHECK(tq_decode_attend(&good, P, P, 10, nullptr, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P, big, nullptr) == TQ_EINVAL);
  CHECK(tq_decode_attend(&good, P, P, 10, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P, 16, nullptr) == TQ_ENOSPACE);
  CHECK(tq_decode_attend(&good, P, P, 10, P, TQ_F32, 32, 0, 0.f, 0.f, F, nullptr, P, big, nullptr) ==
        TQ_EUNSUPPORTED);
  CHECK(tq_decode_attend(&good, P, P, 10, P, TQ_F32, INT_MAX, 0, 0.f, 0.f, F, nullptr, P, big, nullptr) != TQ_OK);
  CHECK(tq_decode_attend(&good, P, P, 10, P, TQ_F32, 1, 0, 0.f, 0.f, nullptr, nullptr, P, big, nullptr) ==
        TQ_EINVAL);
  CHECK(tq_decode_attend(&huge, P, P, 10, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P, big, nullptr) != TQ_OK);
  const tq_cache_desc two{1, 2, 128, 64, 2, 3, 128, 0, 0};
  CHECK(tq_decode_attend_splits(&two, P, P, 10, P, TQ_F32, 3, 0, 0.f, 0.f, F, nullptr, 0, P, big, nullptr) ==
        TQ_EINVAL);
  CHECK(tq_decode_attend_splits(&good, P, P, 10, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, -3, P, big, nullptr) !=
        TQ_OK);

  // workspace queries: zero for invalid shapes, no overflow for extreme valid ones
  CHECK(tq_decode_workspace_bytes(&huge, 8, 64) == 0);
  CHECK(tq_decode_workspace_bytes(&good, 0, 64) == 0);
  CHECK(tq_decode_workspace_bytes(&good, 1, -5) == 0);
  const tq_cache_desc wide{255, 257, 128, 1 << 30, 2, 3, 128, 0, 0};
  CHECK(tq_decode_workspace_bytes(&wide, 257 * 16, 1 << 30) > 0);
  CHECK(tq_decode_splits(&wide, 257 * 16, 1 << 30) >= 1);
  CHECK(tq_decode_workspace_bytes_splits(&good, 1, 1 << 20) > tq_decode_workspace_bytes_splits(&good, 1, 1));
  (void)tq_decode_workspace_bytes_splits(&wide, 257 * 16, INT_MAX);   // size arithmetic only
  CHECK(tq_decode_window_workspace_bytes(&huge, 8, 64) == 0);
  CHECK(tq_search_workspace_bytes(&huge, 10, 4, 10) == 0);
  CHECK(tq_nsn_means_workspace_bytes(&good, 5000) == 0);
  CHECK(tq_nsn_means_workspace_bytes(&nsn, 5000) > 0);
  CHECK(tq_nsn_means_workspace_bytes(&nsn, INT_MAX) > 0);

  // window and step
  int32_t len = 10, wl = 0;
  CHECK(tq_decode_attend_window(&good, P, P, 10, P, P, TQ_BF16, 5, 4, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P,
                                big, nullptr) == TQ_EINVAL);   // win_len > win_cap
  CHECK(tq_decode_attend_window(&good, P, P, 10, P, P, TQ_BF16, 5, 8192, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr,
                                P, big, nullptr) != TQ_OK);    // cap beyond 4096
  CHECK(tq_decode_attend_window(&db, P, P, 10, P, P, TQ_BF16, 5, 8, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P,
                                big, nullptr) != TQ_OK);       // no values
  CHECK(tq_decode_step(&good, P, P, nullptr, P, P, TQ_BF16, &wl, 8, P, P, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr,
                       P, big, nullptr) == TQ_EINVAL);
  wl = 9;
  CHECK(tq_decode_step(&good, P, P, &len, P, P, TQ_BF16, &wl, 8, P, P, P, TQ_F32, 1, 0, 0.f, 0.f, F, nullptr, P,
                       big, nullptr) != TQ_OK);
  CHECK(len == 10 && wl == 9);                                  // untouched on error

  // NSN means
  CHECK(tq_nsn_set_means(&good, P, P, P, P, TQ_BF16, 0, 10, 0.f, P, big, nullptr) == TQ_EINVAL);
  CHECK(tq_nsn_set_means(&nsn, P, P, P, P, TQ_BF16, 0, 0, 0.f, P, big, nullptr) == TQ_EINVAL);
  CHECK(tq_nsn_set_means(&nsn, P, P, P, P, TQ_BF16, 0, 10, 0.f, P, 8, nullptr) == TQ_ENOSPACE);

  // search
  int32_t *I = static_cast<int32_t *>(P);
  CHECK(tq_search_topk(&good, P, P, 10, F, 4, 10, I, F, P, big, nullptr) == TQ_EINVAL);
  CHECK(tq_search_topk(&db, P, P, 65, F, 4, 10, I, F, P, big, nullptr) == TQ_ECAPACITY);
  CHECK(tq_search_topk(&db, P, P, 10, F, 4, 65, I, F, P, big, nullptr) == TQ_EINVAL);
  CHECK(tq_search_topk(&db, P, P, 10, F, 4, 0, I, F, P, big, nullptr) == TQ_EINVAL);
  CHECK(tq_search_topk(&db, P, P, 10, F, 4, 10, I, F, P, 8, nullptr) == TQ_ENOSPACE);
  CHECK(tq_search_topk(&db, P, P, 10, F, -1, 10, I, F, P, big, nullptr) != TQ_OK);
}

int main() {
  codebooks();
  codec_tables();
  cache_sizes();
  device_entry_validation();
  for (int s = 0; s <= 6; ++s) CHECK(tq_status_str(s) != nullptr);
  CHECK(tq_status_str(99) != nullptr && tq_status_str(-1) != nullptr);
  CHECK(tq_version() != nullptr);
  std::printf("abi_checks: %d checks, %d failed\n", g_checks, g_fail);
  return g_fail;
}
