// Host-side checks of the C ABI layer (flash_attn.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU: the device launchers are replaced by
// stubs that record their arguments. Every entry point is called with known good
// and bad arguments and then with random ones (sizes at the int64 and int32 limits,
// extreme and negative strides, NaN / inf / negative scales, unaligned and
// overlapping fake addresses, which the library never dereferences on the host).
// Any sanitizer report aborts the process with a non-zero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "bwd_kernel.h"
#include "flash_attn.h"
#include "fp8_kernel.h"
#include "fwd_kernel.h"

// ---- stubs of the device side ----
namespace {
int g_launches = 0;
int g_kernel = 0;  // forward kernel of the last unsplit launch (FA_FWD_KERNEL_*)
int g_fp8_d = 0;   // head dimension of the last FP8 launch
int g_fwd_d = 0;   // instance width of the last ping-pong launch
fa::FwdArgs g_fwd;
}  // namespace

namespace fa {
int rows_per_workgroup() { return 256; }
int keys_per_tile() { return 64; }
int device_cus() { return 256; }
hipError_t launch_fwd(const FwdArgs& a, bool, int d, bool, hipStream_t) {
  if (d != 64 && d != 128 && d != 256) std::abort();
  if (d == 256 && a.splits > 1) std::abort();  // no key split at the wide instance
  g_fwd_d = d;
  if (a.splits <= 1) g_kernel = FA_FWD_KERNEL_PINGPONG;
  g_fwd = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_sp(const FwdArgs& a, bool, int d, bool, hipStream_t) {
  if (d != 64 && d != 80 && d != 96 && d != 128) std::abort();
  g_kernel = FA_FWD_KERNEL_PIPELINED;
  g_fwd = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdArgs&, bool, int, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_quant_fp8(const QuantArgs&, bool, int, bool, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_fp8(const Fp8Args&, int d, bool, bool, bool, hipStream_t) {
  if (d != 64 && d != 128) std::abort();
  g_fp8_d = d;
  ++g_launches;
  return hipSuccess;
}
}  // namespace fa

namespace {

int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return g_rng;
}

int64_t any_size() {
  static const int64_t edge[] = {0, 1, 2, 3, 7, 8, 63, 64, 65, 255, 256, 257, 4096, 4099, 16384, 1 << 20,
                                 INT32_MAX - 1, INT32_MAX, (int64_t)INT32_MAX + 1, (int64_t)1 << 40,
                                 INT64_MAX / 2, INT64_MAX, -1, -2, INT64_MIN};
  const uint64_t r = next();
  if (r % 3 == 0) return edge[(r >> 8) % (sizeof(edge) / sizeof(edge[0]))];
  if (r % 3 == 1) return (int64_t)((r >> 8) % 5000);
  return (int64_t)(r >> 1) * ((r & 1) ? 1 : -1);
}

int64_t any_d() {
  static const int64_t ds[] = {0, 8, 16, 24, 40, 56, 64, 72, 80, 88, 96, 120, 128, 136, 256, -64, 65, 127};
  return ds[next() % (sizeof(ds) / sizeof(ds[0]))];
}

float any_scale() {
  static const float s[] = {0.125f, 1.0f, 0.0f, -0.5f, 1e-30f, 1e30f, std::numeric_limits<float>::infinity(),
                            std::numeric_limits<float>::quiet_NaN(), std::numeric_limits<float>::denorm_min()};
  return s[next() % (sizeof(s) / sizeof(s[0]))];
}

void* any_ptr() {
  const uint64_t r = next();
  if (r % 7 == 0) return nullptr;
  uint64_t p = (r >> 4) & 0x0000FFFFFFFFFFF0ull;
  if (r % 5 == 0) p += (r >> 60);  // occasionally misaligned
  return reinterpret_cast<void*>(p);
}

int any_small(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }

void known_cases() {
  char* base = reinterpret_cast<char*>(0x100000000ull);
  const uint64_t GB = 1ull << 30;
  void *q = base, *k = base + GB, *v = base + 2 * GB, *o = base + 3 * GB;
  float* lse = reinterpret_cast<float*>(base + 4 * GB);
  CHECK(flash_attn_abi_version() == 9);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 2, 32, 4096, 128, 1, 0.088f, nullptr, FA_BF16) == FA_OK);
  CHECK(g_kernel == FA_FWD_KERNEL_PINGPONG && flash_attn_fwd_kernel(4096, 128, 1) == FA_FWD_KERNEL_PINGPONG);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 1, 32, 16384, 128, 1, 0.088f, nullptr, FA_BF16) == FA_OK);
  CHECK(g_kernel == FA_FWD_KERNEL_PINGPONG && flash_attn_fwd_kernel(16384, 128, 1) == FA_FWD_KERNEL_PINGPONG);
  CHECK(flash_attn_fwd_kernel(300, 80, 1) == FA_FWD_KERNEL_PIPELINED);
  CHECK(flash_attn_fwd_kernel(-1, 128, 1) == FA_ERR_SHAPE && flash_attn_fwd_kernel(1, 130, 1) == FA_ERR_HEADDIM);
  CHECK(flash_attn_fwd_kernel(1, 128, 2) == FA_ERR_ARG);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 2, 32, 4096, 128, 1, 0.088f, nullptr, FA_BF16) == FA_OK);
  CHECK(g_fwd.bh == 64 && g_fwd.n == 4096 && g_fwd.q_tiles == 16 && g_fwd.xcd_grouped == 1);
  CHECK(g_fwd.q_ext == 4096u * 128u * 2u && g_fwd.k_sh == 4096 * 128);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 1, 1, 0, 128, 0, 0.1f, nullptr, FA_BF16) == FA_OK);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 1, 1, 16, 96, 0, 0.1f, nullptr, FA_BF16) == FA_ERR_HEADDIM);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 2, 32, 4096, 256, 1, 0.0625f, nullptr, FA_BF16) == FA_OK);
  CHECK(g_fwd_d == 256 && g_kernel == FA_FWD_KERNEL_PINGPONG && g_fwd.d_real == 256 && g_fwd.v_col0 == 0);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 1, 1, 16, 192, 0, 0.1f, nullptr, FA_BF16) == FA_ERR_HEADDIM);
  CHECK(flash_attn_fwd_kernel(300, 200, 0) == FA_FWD_KERNEL_PINGPONG && flash_attn_fwd_kernel(1, 264, 0) == FA_ERR_HEADDIM);
  CHECK(flash_attn_fwd_splitkv(q, k, v, o, lse, 1, 4, 4096, 256, 1, 0.1f, 4, base + 6 * GB, GB, nullptr, FA_BF16) ==
        FA_ERR_HEADDIM);
  CHECK(flash_attn_fwd(q, k, v, q, lse, 1, 1, 16, 64, 0, 0.1f, nullptr, FA_BF16) == FA_ERR_ALIAS);
  CHECK(flash_attn_fwd(q, k, v, o, lse, 1, 1, 16, 64, 0, NAN, nullptr, FA_BF16) == FA_ERR_SCALE);
  CHECK(flash_attn_fwd(q, k, v, o, lse, (int64_t)1 << 40, 1, 16, 64, 0, 0.1f, nullptr, FA_BF16) == FA_ERR_SHAPE);
  // strided: packed qkv [B, N, 3, H, d] and [B, N, H, d] output at d = 80
  const int64_t B = 2, H = 4, N = 300, d = 80;
  const int64_t qs[3] = {N * 3 * H * d, d, 3 * H * d}, os[3] = {N * H * d, d, H * d}, ls[2] = {H * N, N};
  CHECK(flash_attn_fwd_strided(q, (char*)q + d * 2 * H, (char*)q + 2 * d * 2 * H, o, lse, B, H, N, d, qs, qs, qs,
                               os, ls, 1, 0.11f, nullptr, FA_FP16) == FA_OK);
  CHECK(g_fwd.d_real == 80 && g_fwd.q_sn == 3 * H * d);
  const int64_t bad[3] = {N * 3 * H * d, d, 3 * H * d + 4};
  CHECK(flash_attn_fwd_strided(q, k, v, o, lse, B, H, N, d, bad, qs, qs, os, ls, 0, 0.1f, nullptr, FA_BF16) ==
        FA_ERR_STRIDE);
  const int64_t self_overlap[3] = {0, d, H * d};
  CHECK(flash_attn_fwd_strided(q, k, v, o, lse, B, H, N, d, qs, qs, qs, self_overlap, ls, 0, 0.1f, nullptr,
                               FA_BF16) == FA_ERR_STRIDE);
  // key split: plan, size, call
  CHECK(flash_attn_fwd_splitkv_plan(1, 4, 4096, 128, 1, 256) == 4);
  const int64_t ws = flash_attn_fwd_splitkv_workspace_size(1, 4, 4096, 128, 1, 4);
  CHECK(ws == 4LL * 4 * 4096 * 129 * 4);
  CHECK(flash_attn_fwd_splitkv(q, k, v, o, lse, 1, 4, 4096, 128, 1, 0.1f, 4, base + 6 * GB, (uint64_t)ws, nullptr,
                               FA_BF16) == FA_OK);
  CHECK(g_fwd.splits == 4);
  CHECK(flash_attn_fwd_splitkv(q, k, v, o, lse, 1, 4, 4096, 128, 1, 0.1f, 4, base + 6 * GB, (uint64_t)ws - 1,
                               nullptr, FA_BF16) == FA_ERR_WORKSPACE);
  // fp8 and backward
  int32_t* se = reinterpret_cast<int32_t*>(base + 7 * GB);
  CHECK(flash_attn_quantize_fp8(q, o, se, 1, 2, 100, 128, FA_FP8_KEYS_T, nullptr, FA_BF16, FA_FP8_E5M2) == FA_OK);
  CHECK(flash_attn_quantize_fp8(q, o, se, 1, 2, 100, 128, FA_FP8_KEYS_T, nullptr, FA_BF16, 3) == FA_ERR_ARG);
  CHECK(flash_attn_fwd_fp8(q, k, v, se, se + 64, se + 128, o, lse, 1, 2, 100, 128, 1, 0.1f, nullptr, FA_BF16,
                           FA_FP8_E4M3) == FA_OK);
  CHECK(g_fp8_d == 128);
  CHECK(flash_attn_fwd_fp8(q, k, v, se, se + 64, se + 128, o, lse, 1, 2, 100, 64, 0, 0.1f, nullptr, FA_FP16,
                           FA_FP8_E5M2) == FA_OK);
  CHECK(g_fp8_d == 64);
  CHECK(flash_attn_fwd_fp8(q, k, v, se, se + 64, se + 128, o, lse, 1, 2, 100, 96, 0, 0.1f, nullptr, FA_FP16,
                           FA_FP8_E5M2) == FA_ERR_HEADDIM);
  float* delta = reinterpret_cast<float*>(base + 8 * GB);
  CHECK(flash_attn_bwd(q, k, v, o, base + 5 * GB, lse, base + 9 * GB, base + 10 * GB, base + 11 * GB, delta, 2, 32,
                       4096, 128, 1, 0.088f, nullptr, FA_BF16) == FA_OK);
  for (int st = -20; st <= 5; ++st) CHECK(flash_attn_strerror(st) != nullptr);
}

void fuzz(int rounds) {
  for (int r = 0; r < rounds; ++r) {
    // a third of the rounds are plausible calls (small shapes, valid head dims and
    // flags, buffers 1 TiB apart) so that the code past the checks runs too
    const bool plausible = r % 3 == 0;
    const int64_t B = plausible ? any_small(1, 8) : any_size(), H = plausible ? any_small(1, 40) : any_size();
    const int64_t N = plausible ? any_small(1, 20000) : any_size();
    const int64_t d = plausible ? (int64_t)(8 * any_small(1, 16)) : any_d();
    const int causal = plausible ? any_small(0, 1) : any_small(-1, 2);
    const int dtype = plausible ? any_small(0, 1) : any_small(-1, 2);
    const float scale = plausible ? 0.125f : any_scale();
    auto buf = [&](int i) { return plausible ? reinterpret_cast<void*>((uint64_t)(i + 1) << 40) : any_ptr(); };
    void *q = buf(0), *k = buf(1), *v = buf(2), *o = buf(3);
    float* lse = static_cast<float*>(buf(4));
    flash_attn_fwd_validate(q, k, v, o, lse, B, H, N, d, causal, scale, nullptr, dtype);
    g_kernel = 0;
    const int fst = flash_attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, nullptr, dtype);
    const int kern = flash_attn_fwd_kernel(N, d, causal);
    // a call that launched ran the kernel the query names
    if (fst == FA_OK && g_kernel != 0) CHECK(g_kernel == kern);
    if (fst == FA_OK && B > 0 && H > 0 && N > 0) CHECK(g_kernel == kern);
    int64_t s4[4][3], ls[2];
    for (auto& t : s4)
      for (auto& x : t) x = any_size();
    ls[0] = any_size();
    ls[1] = any_size();
    if (next() % 2) {  // plausible strides more often
      for (auto& t : s4) {
        t[2] = d + 8 * (int64_t)(next() % 4);
        t[1] = t[2] * (N > 0 && N < 100000 ? N : 1);
        t[0] = t[1] * (H > 0 && H < 1000 ? H : 1);
      }
    }
    flash_attn_fwd_strided_validate(q, k, v, o, lse, B, H, N, d, s4[0], s4[1], s4[2], s4[3], ls, causal, scale,
                                    nullptr, dtype);
    flash_attn_fwd_strided(q, k, v, o, lse, B, H, N, d, s4[0], s4[1], s4[2], s4[3], ls, causal, scale, nullptr,
                           dtype);
    const int splits = any_small(-2, 40);
    const uint64_t wsb = next() >> (next() % 64);
    void* ws = plausible ? buf(5) : any_ptr();
    flash_attn_fwd_splitkv_validate(q, k, v, o, lse, B, H, N, d, causal, scale, splits, ws, wsb, nullptr, dtype);
    flash_attn_fwd_splitkv(q, k, v, o, lse, B, H, N, d, causal, scale, splits, ws, wsb, nullptr, dtype);
    flash_attn_fwd_splitkv_plan(B, H, N, d, causal, any_small(-1, 1024));
    flash_attn_fwd_splitkv_workspace_size(B, H, N, d, causal, splits);
    flash_attn_bwd_validate(q, k, v, o, buf(5), lse, buf(6), buf(7), buf(8), static_cast<float*>(buf(9)), B, H, N,
                            d, causal, scale, nullptr, dtype);
    flash_attn_bwd(q, k, v, o, buf(5), lse, buf(6), buf(7), buf(8), static_cast<float*>(buf(9)), B, H, N, d, causal,
                   scale, nullptr, dtype);
    const int layout = plausible ? any_small(0, 1) : any_small(-1, 2);
    const int fmt = plausible ? any_small(0, 1) : any_small(-1, 2);
    int32_t* se = static_cast<int32_t*>(buf(10));
    flash_attn_quantize_fp8_validate(q, o, se, B, H, N, d, layout, nullptr, dtype, fmt);
    flash_attn_quantize_fp8(q, o, se, B, H, N, d, layout, nullptr, dtype, fmt);
    int32_t *ks = static_cast<int32_t*>(buf(11)), *vs = static_cast<int32_t*>(buf(12));
    flash_attn_fwd_fp8_validate(q, k, v, se, ks, vs, o, lse, B, H, N, d, causal, scale, nullptr, dtype, fmt);
    flash_attn_fwd_fp8(q, k, v, se, ks, vs, o, lse, B, H, N, d, causal, scale, nullptr, dtype, fmt);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 20000;
  known_cases();
  fuzz(rounds);
  std::printf("abi_fuzz: %d fuzz rounds, %d stub launches, %d failed checks\n", rounds, g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
