// Exact attention forward for gfx950 (MI355X): bf16/fp16 in, fp32 accumulate.
//
// Method ("FlashAttention: optimize data movement before counting FLOPs",
// section 02): for each key tile with scores s and values V keep the running row
// maximum m, denominator l and unnormalised numerator u,
//     m' = max(m, max s),  l' = e^(m-m') l + sum e^(s-m'),  u' = e^(m-m') u + sum e^(s-m') V,
// and finish with O = u / l. The loop order is the one the IO-aware survey
// ("FlashAttention: IO-Aware Tiling, Online Softmax Mathematics, Memory Hierarchy
// Dynamics, and Kernel Evolution", FlashAttention-2 section) describes: query
// tiles on the grid, key/value tiles streamed in the inner loop, the accumulator
// kept on chip and divided once at the end. The log-sum-exp m + ln l is stored
// for a backward pass (same survey, "Backward Pass Recomputation").
//
// gfx950 mapping (one workgroup = 4 wave64s = 128 query rows; one key tile = 64 rows):
//  * Each wave owns 32 query rows. Scores are computed transposed, S^T = K Q^T,
//    with v_mfma_f32_32x32x16 (A = K rows from LDS, B = the wave's Q rows held in
//    registers). In the 32x32 accumulator layout a lane holds one query column
//    and 16 key rows, so the row max and row sum are mostly in-lane; the two
//    32-lane halves that share a query are combined with v_permlane32_swap.
//  * The probabilities stay in registers: the S^T accumulator, rounded to the
//    16-bit input type, is exactly the B operand of O^T = V^T P^T. The V^T
//    operand is read from a row-major V tile with ds_read_b64_tr_b16 (gfx950's
//    transposing LDS read), so no transpose pass is needed anywhere.
//  * O^T accumulates in registers: each lane owns one query, so the rescale by
//    e^(m-m') is a per-lane multiply, skipped when no row of the wave moved its max.
//  * Exponentials use exp2 with scale*log2(e) folded into one FMA per score.
//  * K/V tiles are double-buffered in LDS; the next tile is fetched into
//    registers while the current one is consumed; one barrier per tile.
//  * Causal: key tiles past the workgroup's last row are never visited, waves
//    whose rows all precede a tile skip its math, and only tiles that straddle
//    the diagonal or the end of the sequence evaluate the mask.
//  * Workgroup order: heaviest causal query tiles first, and all query tiles of
//    one (batch, head) on the same XCD (workgroups go round-robin over 8 XCDs)
//    so that K/V tiles are shared through that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_kernel.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // key rows per tile
constexpr int kThreads = 64 * kWaves;

template <int D>
struct Layout {
  // LDS row strides in bytes. K rows (read 16 bytes per lane, 32 rows per
  // instruction) are padded by 16 bytes so consecutive rows start 4 banks apart.
  // V rows (read 8 bytes per lane by the transposing read, 4 rows x 16 dwords
  // per half-wave) are padded so those 4 rows land in disjoint 16-bank windows.
  static constexpr int kStride = D * 2 + 16;
  static constexpr int vStride = D * 2 + 64;
  static constexpr int kBytes = kBN * kStride;
  static constexpr int vBytes = kBN * vStride;
  static constexpr int stageBytes = kBytes + vBytes;
  static constexpr int chunksPerRow = D / 8;                 // 16-byte chunks
  static constexpr int chunksPerThread = kBN * chunksPerRow / kThreads;
  static_assert(kBN * chunksPerRow % kThreads == 0, "tile load must split evenly");
};

template <bool FP16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (FP16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// Two fp32 values rounded to nearest-even 16-bit floats, packed low|high
// (one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <bool FP16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if constexpr (FP16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
}

// Value of x held by the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0..31 receive the upper half's value in r[1]; lanes 32..63 in r[0]
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 lds_read16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <bool FP16, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdArgs a) {
  using L = Layout<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::stageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;    // which half of the wave
  const int l32 = lane & 31;  // query column within the wave's 32

  // ---- workgroup -> (batch*head, query tile) ----
  const int bid = blockIdx.x;
  const int bh_count = a.bh;
  int bh, rank;
  if (a.xcd_grouped) {
    const int hpx = bh_count / 8;  // heads per XCD
    const int xcd = bid & 7, t = bid >> 3;
    rank = t / hpx;
    bh = xcd * hpx + t % hpx;
  } else {
    rank = bid / bh_count;
    bh = bid % bh_count;
  }
  const int qtile = CAUSAL ? (a.q_tiles - 1 - rank) : rank;
  const int N = a.n;
  const int q0 = qtile * kBM;
  const int64_t head_off = (int64_t)bh * N * D;

  const uint16_t* __restrict__ qg = reinterpret_cast<const uint16_t*>(a.q) + head_off;
  const uint16_t* __restrict__ kg = reinterpret_cast<const uint16_t*>(a.k) + head_off;
  const uint16_t* __restrict__ vg = reinterpret_cast<const uint16_t*>(a.v) + head_off;

  // ---- Q rows of this lane's query, as B operands (k-slots d = 16*ks + 8*h + 0..7) ----
  const int qrow = q0 + wave * 32 + l32;
  u32x4 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qreg[ks] = (qrow < N) ? *reinterpret_cast<const u32x4*>(qg + (int64_t)qrow * D + ks * 16 + h * 8)
                          : u32x4{0, 0, 0, 0};
  }

  // ---- key tiles this workgroup visits ----
  const int kv_tiles_all = (N + kBN - 1) / kBN;
  int n_tiles = kv_tiles_all;
  if (CAUSAL) {
    const int last_row = min(q0 + kBM, N) - 1;
    n_tiles = min(kv_tiles_all, last_row / kBN + 1);
  }
  const int wave_first_row = q0 + wave * 32;
  const int wave_last_row = wave_first_row + 31;

  // global -> register staging of one K/V tile (16-byte chunks, coalesced rows)
  u32x4 kstage[L::chunksPerThread], vstage[L::chunksPerThread];
  auto fetch = [&](int tile) {
    const int kv0 = tile * kBN;
#pragma unroll
    for (int i = 0; i < L::chunksPerThread; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / L::chunksPerRow, col = (c % L::chunksPerRow) * 8;
      const bool ok = kv0 + row < N;
      const int64_t off = (int64_t)(kv0 + row) * D + col;
      kstage[i] = ok ? *reinterpret_cast<const u32x4*>(kg + off) : u32x4{0, 0, 0, 0};
      vstage[i] = ok ? *reinterpret_cast<const u32x4*>(vg + off) : u32x4{0, 0, 0, 0};
    }
  };
  auto stash = [&](int buf) {
    char* ks = smem + buf * L::stageBytes;
    char* vs = ks + L::kBytes;
#pragma unroll
    for (int i = 0; i < L::chunksPerThread; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / L::chunksPerRow, colb = (c % L::chunksPerRow) * 16;
      *reinterpret_cast<u32x4*>(ks + row * L::kStride + colb) = kstage[i];
      *reinterpret_cast<u32x4*>(vs + row * L::vStride + colb) = vstage[i];
    }
  };

  // per-lane offsets inside a stage
  const int k_off = l32 * L::kStride + h * 16;  // K row l32 (+32 for the second block), d-slot 8h
  // transposing V read: this lane sources row 4h + (lane%16)/4 (+8, +16t) and
  // columns 16*((lane/16)%2) + 4*(lane%4) (+32 per d block)
  const int v_off = (4 * h + ((lane & 15) >> 2)) * L::vStride + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  const float sc = a.scale_log2;  // scale * log2(e)
  float m_run = -INFINITY;        // running max of scale*log2(e)*s for this lane's query
  float l_run = 0.f;              // running denominator (this half's keys only)
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  if (n_tiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < n_tiles;
    if (more) fetch(j + 1);

    const int kv0 = j * kBN;
    const bool active = wave_first_row < N && (!CAUSAL || kv0 <= wave_last_row);
    if (active) {
      const char* ks = smem + buf * L::stageBytes;
      const char* vs = ks + L::kBytes;

      // ---- S^T = K Q^T for 64 keys x 32 queries ----
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 k0 = lds_read16(ks + k_off + kk * 32);
        const u32x4 k1 = lds_read16(ks + k_off + 32 * L::kStride + kk * 32);
        s[0] = mfma32<FP16>(k0, qreg[kk], s[0]);
        s[1] = mfma32<FP16>(k1, qreg[kk], s[1]);
      }

      // ---- mask keys past the end and (causal) keys after the query ----
      const bool edge = (kv0 + kBN > N) || (CAUSAL && kv0 + kBN - 1 > wave_first_row);
      if (edge) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + b * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool dead = key >= N || (CAUSAL && key > qrow);
            s[b][r] = dead ? -INFINITY : s[b][r];
          }
      }

      // ---- running max (in log2 units) ----
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = fmaxf(mx, other_half(mx));
      const float m_new = fmaxf(m_run, mx * sc);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;  // no -inf - -inf
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);

      // ---- p = 2^(s*sc - m'), partial row sum, 16-bit P operands ----
      float psum = 0.f;
      u32x4 pb[4];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], sc, -m_ref));
          psum += p[r];
        }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          pb[2 * b + t2] = u32x4{pack2<FP16>(p[8 * t2 + 0], p[8 * t2 + 1]), pack2<FP16>(p[8 * t2 + 2], p[8 * t2 + 3]),
                                 pack2<FP16>(p[8 * t2 + 4], p[8 * t2 + 5]), pack2<FP16>(p[8 * t2 + 6], p[8 * t2 + 7])};
        }
      }
      l_run = alpha * l_run + psum;
      m_run = m_new;

      // ---- u <- alpha * u (skipped when no query of the wave raised its max) ----
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      }

      // ---- u += P V: O^T = V^T P^T over 4 groups of 16 keys ----
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const char* p0 = vs + v_off + (16 * t) * L::vStride + db * 64;
          const u32x2 lo = lds_read_tr16(p0);
          const u32x2 hi = lds_read_tr16(p0 + 8 * L::vStride);
          acc[db] = mfma32<FP16>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[t], acc[db]);
        }
      }
    }

    if (more) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = u / l, LSE = (m + log2 l) * ln 2 ----
  const float l_tot = l_run + other_half(l_run);
  if (qrow < N) {
    const float inv = 1.0f / l_tot;
    uint16_t* og = reinterpret_cast<uint16_t*>(a.o) + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack2<FP16>(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                         pack2<FP16>(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(og + db * 32 + 8 * g + 4 * h) = w;
      }
    if (h == 0) a.lse[(int64_t)bh * N + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
  }
}

template <bool FP16, int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<FP16, D, CAUSAL>), dim3(a.grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int rows_per_workgroup() { return kBM; }

hipError_t launch_fwd(const FwdArgs& a, bool fp16, int d, bool causal, hipStream_t stream) {
  if (fp16) {
    if (d == 64) return causal ? launch_one<true, 64, true>(a, stream) : launch_one<true, 64, false>(a, stream);
    return causal ? launch_one<true, 128, true>(a, stream) : launch_one<true, 128, false>(a, stream);
  }
  if (d == 64) return causal ? launch_one<false, 64, true>(a, stream) : launch_one<false, 64, false>(a, stream);
  return causal ? launch_one<false, 128, true>(a, stream) : launch_one<false, 128, false>(a, stream);
}

}  // namespace fa
