// FP8 (E4M3 or E5M2) block quantization for the FP8 attention forward on gfx950.
//
// "FlashAttention: IO-Aware Tiling, Online Softmax Mathematics, Memory Hierarchy
// Dynamics, and Kernel Evolution", section on FlashAttention-3, runs attention in
// 8-bit floating point with block-level quantization and dynamic scaling factors.
// Here a block is 64 consecutive rows of one (batch, head) slice; its scale is the
// power of two 2^e with e the smallest integer such that the block's largest
// magnitude a satisfies a <= F * 2^e (F the format's largest finite value: 448 for
// E4M3, 57344 for E5M2; e = 0 for an all-zero block; e limited to the E8M0 range
// [-127, 127]), and each value is stored as FP8(x / 2^e), rounded to nearest even by
// v_cvt_pk_fp8_f32 (E4M3) or v_cvt_pk_bf8_f32 (E5M2). The division by 2^e is exact
// in fp32. The scale is kept as its E8M0 code e + 127, the form the scaled matrix
// instructions take.
//
// One workgroup of 256 lanes per block: 16-byte loads, a maximum reduction, then
// either row-major E4M3 (queries, keys) or the keys-transposed layout of values,
// written through an LDS copy of the block: row c of the output block holds
// column c of V for the 64 keys in the order the attention kernel's P operand
// uses (see fp8_kernel.h), so that its P V product needs no transposing read.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fp8_kernel.h"
#include "gfx950_ops.h"
#include "launch_log.h"

namespace fa {
namespace fp8q {

using namespace ::fa::ops;

constexpr int kThreads = 256;

__device__ __forceinline__ void unpack8(const u32x4 w, bool fp16, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i];
    if (fp16) {
      const f16x2 h = __builtin_bit_cast(f16x2, x);
      f[2 * i] = (float)h[0];
      f[2 * i + 1] = (float)h[1];
    } else {
      f[2 * i] = __uint_as_float(x << 16);
      f[2 * i + 1] = __uint_as_float(x & 0xffff0000u);
    }
  }
}

// four E4M3 (E5 false) or E5M2 (E5 true) codes, rounded to nearest even: a in byte
// 0 ... d in byte 3
template <bool E5>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  if constexpr (E5)
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false), true);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false), true);
}

// smallest e with amax <= F * 2^e, F the format's largest finite value (exact: 448 =
// 0.875 * 2^9, 57344 = 0.875 * 2^16), in [-127, 127]
template <bool E5>
__device__ __forceinline__ int block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = frexpf(amax, &E);  // amax = m * 2^E, m in [0.5, 1)
  constexpr int kTop = E5 ? 16 : 9;
  int e = (m > 0.875f) ? E - kTop + 1 : E - kTop;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

template <bool FP16, int D, bool VT, bool E5>
__global__ __launch_bounds__(kThreads) void quant_fp8(QuantArgs a) {
  constexpr int kChunks = kFp8Block * D / 8;          // 16-byte input chunks per block
  constexpr int kPer = kChunks / kThreads;             // per lane
  constexpr int kCpr = D / 8;                          // chunks per row
  __shared__ float tile[VT ? kFp8Block : 1][D + 1];
  __shared__ float wmax[kThreads / 64];
  const int bh = blockIdx.x / a.t64, t = blockIdx.x % a.t64;
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)t * kFp8Block;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x) + ((int64_t)bh * a.n + row0) * D;

  float v[kPer][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + kThreads * i, r = c / kCpr, c8 = c % kCpr;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row0 + r < a.n) w = *reinterpret_cast<const u32x4*>(x + (int64_t)r * D + c8 * 8);
    unpack8(w, FP16, v[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = block_exp<E5>(amax);
  const float inv = ldexpf(1.0f, -e);
  if (tid == 0) a.se[(int64_t)bh * a.t64 + t] = e + 127;

  if constexpr (!VT) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + kThreads * i, r = c / kCpr, c8 = c % kCpr;
      if (row0 + r < a.n) {
        const float* f = v[i];
        const u32x2 w = {pack4<E5>(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                         pack4<E5>(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv)};
        *reinterpret_cast<u32x2*>(a.x8 + ((int64_t)bh * a.n + row0 + r) * D + c8 * 8) = w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + kThreads * i, r = c / kCpr, c8 = c % kCpr;
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[r][c8 * 8 + j] = v[i][j] * inv;
    }
    __syncthreads();
    // output block: D rows of 64 positions; a lane writes groups of 16 positions
    constexpr int kGroups = D * 4 / kThreads;
    uint8_t* out = a.x8 + ((int64_t)bh * a.t64 + t) * D * kFp8Block;
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const int g = tid + kThreads * gi, col = g / 4, g4 = g % 4;
      // positions p = 16 g4 + i hold key 32 (g4 % 2) + 8 (i / 4) + 4 (g4 / 2) + i % 4
      const int kb = 32 * (g4 & 1) + 4 * (g4 >> 1);
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = pack4<E5>(tile[kb + 8 * q + 0][col], tile[kb + 8 * q + 1][col], tile[kb + 8 * q + 2][col],
                         tile[kb + 8 * q + 3][col]);
      *reinterpret_cast<u32x4*>(out + (int64_t)col * kFp8Block + 16 * g4) = w;
    }
  }
}

template <bool FP16, int D, bool E5>
hipError_t launch2(const QuantArgs& a, bool vt, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.bh * a.t64));
  if (vt) hipLaunchKernelGGL((quant_fp8<FP16, D, true, E5>), grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL((quant_fp8<FP16, D, false, E5>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool E5>
hipError_t launch_fmt(const QuantArgs& a, bool fp16, int d, bool vt, hipStream_t stream) {
  if (fp16) return d == 64 ? launch2<true, 64, E5>(a, vt, stream) : launch2<true, 128, E5>(a, vt, stream);
  return d == 64 ? launch2<false, 64, E5>(a, vt, stream) : launch2<false, 128, E5>(a, vt, stream);
}

}  // namespace fp8q

hipError_t launch_quant_fp8(const QuantArgs& a, bool fp16, int d, bool keys_transposed, bool e5m2,
                            hipStream_t stream) {
  using namespace fp8q;
  launch_log("quant_fp8<%s, %d, %s, %s> grid %lld x %d", dtype_name(fp16), d, keys_transposed ? "keys-transposed" : "rows",
             e5m2 ? "E5M2" : "E4M3", (long long)a.bh * a.t64, kThreads);
  return e5m2 ? launch_fmt<true>(a, fp16, d, keys_transposed, stream)
              : launch_fmt<false>(a, fp16, d, keys_transposed, stream);
}

}  // namespace fa
