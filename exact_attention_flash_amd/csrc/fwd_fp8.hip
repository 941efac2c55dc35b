// Exact attention forward on FP8 (E4M3 or E5M2) inputs for gfx950, d = 64 or 128, bf16/fp16 out.
//
// "FlashAttention: IO-Aware Tiling, Online Softmax Mathematics, Memory Hierarchy
// Dynamics, and Kernel Evolution", section on FlashAttention-3: attention in 8-bit
// floating point with block-level quantization and dynamic scaling factors. The
// inputs come from fp8_quant.hip: Q and K as row-major E4M3 with one power-of-two
// scale per 64 rows of a (batch, head) slice, V in the keys-transposed layout with
// one scale per 64 keys. The result is attention on the dequantized inputs; the
// online softmax is the one of fwd_kernel.hip ("FlashAttention: optimize data
// movement before counting FLOPs", section 02): running maximum m, denominator l,
// unnormalised u, O = u / l and LSE = m + ln l at the end.
//
// Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (the inputs' format for Q, K
// and V, E4M3 for P; fp32 accumulate) with the blocks' E8M0 scales as the
// instruction's operand scales,
// so every score and every P V contribution is exact in scale:
//  * S^T = K Q^T: A = 32 key rows of the K tile (LDS), B = the wave's 32 query
//    rows (registers), d / 64 k-steps of 64 over d; scales = the K tile's and the Q
//    block's exponents.
//  * O^T += V^T P^T: A = 32 rows (head-dimension columns) of the V^T tile (LDS),
//    B = P^T packed to E4M3 in registers from the S^T accumulator; the byte order
//    of the V^T rows (fixed by the quantizer) is the accumulator's key order, so no
//    transposing read is needed. One k-step of 64 keys per 32 columns.
//  * P is rounded to E4M3 as p' = 2^(s' - r) with the reference r 8 below the row
//    maximum (log2 units), moved only when the maximum rises by more than 0.8: p' <=
//    2^8.8 < 448, E4M3's largest value, and E4M3's range reaches down to 2^-17 of the
//    row maximum. l sums the same unrounded p', so the reference cancels in u / l and
//    r + log2 l is still the log-sum-exp.
// Schedule as in fwd_kernel.hip: persistent workgroups of 8 waves over items of
// 256 query rows, snake order, a slice's items on one XCD, a 3-stage K/V ring
// filled by buffer_load ... lds one tile ahead across items, Q by the same path one
// item ahead. Unlike the 16-bit kernel, the two waves of a SIMD run their phases in
// step (matrix work, then softmax): the FP8 products of a tile take half the time of
// the 16-bit ones and cannot hide a softmax, while two waves in their softmax at once
// issue VALU work faster than one (measured: 6-11% faster than the ping-pong order).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp8_kernel.h"
#include "fwd_kernel.h"
#include "gfx950_ops.h"
#include "launch_log.h"

namespace fa {
namespace f8 {

using namespace ::fa::ops;

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // query rows per item
constexpr int kBN = kFp8Block;     // keys per tile = rows per quantization block
constexpr int kStages = 3;
constexpr int kAhead = kStages - 2;
constexpr int kScale = 256;  // one tile scale replicated by the 64 lanes of a load

// 16-byte chunk swizzles: rows of 8 chunks (K and Q at d = 128) and of 4 chunks (K
// and Q at d = 64, V^T), so that 16 consecutive rows read at one logical chunk hit
// every LDS bank once
__device__ __forceinline__ int swz8(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

// Sizes for head dimension D (64 or 128).
template <int D>
struct Geo8 {
  static constexpr int kRow = D;                   // bytes of a K or Q row
  static constexpr int kChunks = D / 16;           // 16-byte chunks of a K or Q row
  static constexpr int kTile = kBN * kRow;         // K tile bytes (= V^T tile bytes: D rows of 64)
  static constexpr int kStage = 2 * kTile + 2 * kScale;
  static constexpr int kQBytes = kBM * kRow;
  static constexpr int kBlocks = kTile / 1024;     // 1 KiB blocks of the K tile (and of the V^T tile)
  // every wave loads one block of K and one of V^T (D = 128), or one block of either
  // (D = 64: waves 0-3 K, waves 4-7 V^T)
  static constexpr int kTileLoads = 2 * kBlocks / kWaves;
  static constexpr int kQLoads = kQBytes / 1024 / kWaves + 1;  // Q blocks + the Q scales
  static constexpr int kSteps = D / 32;            // products of S (and of P V) per tile
  static_assert(D == 64 || D == 128, "FP8 instances: d = 64 or 128");
  static_assert(kTileLoads == 1 || kTileLoads == 2, "whole 1 KiB blocks per wave");
  __device__ static __forceinline__ int swz(int row) { return D == 128 ? swz8(row) : swz4(row); }
};

// FA (A operand) and FB (B operand) select the instruction's operand formats: 0 =
// E4M3, 1 = E5M2
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma8(const u32x4 a0, const u32x4 a1, const i32x8 b, f32x16 c, int sa, int sb) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

__device__ __forceinline__ int pack4(float a, float b, float c, float d) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false), true);
}

template <bool FP16OUT, bool CAUSAL, bool E5, int kD>
__global__ __launch_bounds__(kThreads, 1) void fwd_fp8(Fp8Args a) {
  using G = Geo8<kD>;
  constexpr int kRow = G::kRow, kTile = G::kTile, kStage = G::kStage, kQBytes = G::kQBytes;
  constexpr int kIn = E5 ? 1 : 0;  // format code of Q, K and V; P is always E4M3
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage + kQBytes + kScale];
  char* const qsm = smem + kStages * kStage;
  char* const qscale = qsm + kQBytes;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, h = lane >> 5, l32 = lane & 31;

  // ---- persistent schedule (as fwd_kernel.hip) ----
  const int bid = blockIdx.x;
  int wg_k, wg_n, hpx, bh_base;
  if (a.xcd_grouped) {
    hpx = a.bh >> 3;
    wg_k = bid >> 3;
    wg_n = (int)gridDim.x >> 3;
    bh_base = (bid & 7) * hpx;
  } else {
    hpx = a.bh;
    wg_k = bid;
    wg_n = (int)gridDim.x;
    bh_base = 0;
  }
  const int n_items = hpx * a.q_tiles;
  const int N = a.n;
  const int T = a.t64;
  const int tiles_all = (N + kBN - 1) / kBN;
  auto item_index = [&](int r) {
    const int j = r * wg_n + ((r & 1) ? wg_n - 1 - wg_k : wg_k);
    return j < n_items ? j : -1;
  };
  auto item_bh = [&](int j) { return bh_base + j % hpx; };
  auto item_q0 = [&](int j) { return (CAUSAL ? (a.q_tiles - 1 - j / hpx) : j / hpx) * kBM; };
  auto item_tiles = [&](int q0) { return CAUSAL ? min(tiles_all, (min(q0 + kBM, N) - 1) / kBN + 1) : tiles_all; };
  const int wave_rows = 32 * (grp == 0 ? (wave & 3) : 7 - (wave & 3));

  // DMA offsets: block blk of the K tile and of the V^T tile (D = 128: blk = wave,
  // both tiles; D = 64: wave w < 4 loads K block w, wave w >= 4 V^T block w - 4)
  const int blk = G::kTileLoads == 2 ? wave : (wave & 3);
  // wave-uniform choice of the one tile a wave loads at D = 64 (a scalar branch)
  const bool loads_k = __builtin_amdgcn_readfirstlane(wave) < 4;
  const int kp = 64 * blk + lane;
  const uint32_t k_ld = (uint32_t)(kp / G::kChunks) * kRow +
                        (uint32_t)(((kp % G::kChunks) ^ G::swz(kp / G::kChunks)) * 16);
  const uint32_t v_ld = (uint32_t)(kp / 4) * kBN + (uint32_t)(((kp % 4) ^ swz4(kp / 4)) * 16);

  int c_r = 0, c_j = item_index(0), c_t = 0, c_n = 0, c_g = 0, c_bh = 0;
  auto cursor_item = [&]() {
    if (c_j < 0) return;
    c_bh = item_bh(c_j);
    c_n = item_tiles(item_q0(c_j));
    c_t = 0;
  };
  cursor_item();
  auto issue_next = [&]() {
    if (c_j < 0) return false;
    const uint8_t* kb = a.k8 + ((int64_t)c_bh * N + (int64_t)c_t * kBN) * kRow;
    const uint8_t* vb = a.v8t + ((int64_t)c_bh * T + c_t) * kTile;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kb, (uint32_t)(N - c_t * kBN) * kRow);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vb, (uint32_t)kTile);
    const __amdgpu_buffer_rsrc_t ksr = buffer_rsrc(a.k_se + (int64_t)c_bh * T + c_t, 4u);
    const __amdgpu_buffer_rsrc_t vsr = buffer_rsrc(a.v_se + (int64_t)c_bh * T + c_t, 4u);
    char* st = smem + (c_g % kStages) * kStage;
    if constexpr (G::kTileLoads == 2) {
      buffer_load16_lds(kr, k_ld, st + 1024 * blk);
      buffer_load16_lds(vr, v_ld, st + kTile + 1024 * blk);
    } else if (loads_k) {
      buffer_load16_lds(kr, k_ld, st + 1024 * blk);
    } else {
      buffer_load16_lds(vr, v_ld, st + kTile + 1024 * blk);
    }
    buffer_load4_lds(ksr, 0u, st + 2 * kTile);
    buffer_load4_lds(vsr, 0u, st + 2 * kTile + kScale);
    ++c_g;
    if (++c_t == c_n) {
      c_j = item_index(++c_r);
      cursor_item();
    }
    return true;
  };
  if (c_j < 0) return;

  // Q rows of an item (and the exponents of its four 64-row blocks) into LDS
  auto issue_q = [&](int j) {
    const int q0 = item_q0(j), bh = item_bh(j);
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(a.q8 + ((int64_t)bh * N + q0) * kRow, (uint32_t)(N - q0) * kRow);
    int lw = lane + 64 * wave;
    asm volatile("" : "+v"(lw));
#pragma unroll
    for (int i = 0; i < kQBytes / 1024 / kWaves; ++i) {
      const int p = lw + 64 * kWaves * i;
      const int row = p / G::kChunks;
      buffer_load16_lds(qr, (uint32_t)row * kRow + (uint32_t)(((p % G::kChunks) ^ G::swz(row)) * 16),
                        qsm + 1024 * (wave + kWaves * i));
    }
    const int b0 = q0 / kBN;
    const __amdgpu_buffer_rsrc_t qsr = buffer_rsrc(a.q_se + (int64_t)bh * T + b0, (uint32_t)(min(4, T - b0) * 4));
    buffer_load4_lds(qsr, (uint32_t)(lane * 4), qscale);
  };
  i32x8 qreg[kD / 64];
  int q_sc = 0;
  auto read_q = [&]() {
    int row = wave_rows + l32;
    asm volatile("" : "+v"(row));
#pragma unroll
    for (int kk = 0; kk < kD / 64; ++kk) {
      const u32x4 lo = lds_read16(qsm + row * kRow + (((4 * kk + 2 * h) ^ G::swz(row)) * 16));
      const u32x4 hi = lds_read16(qsm + row * kRow + (((4 * kk + 2 * h + 1) ^ G::swz(row)) * 16));
      qreg[kk] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    q_sc = *reinterpret_cast<const int*>(qscale + 4 * (wave_rows / kBN));
  };

  const int first_j = c_j;
  issue_q(first_j);
#pragma unroll
  for (int t = 0; t < kAhead; ++t) issue_next();
  bool first = true;

  // per-lane LDS offsets: K row l32 (+32 rows for the second key block), logical
  // chunks 4 kk + 2 h + {0, 1}; V^T row 32 db + l32, logical chunks 2 h + {0, 1}
  int k_off[2][kD / 64][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int kk = 0; kk < kD / 64; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * b + l32;
        k_off[b][kk][i] = row * kRow + (((4 * kk + 2 * h + i) ^ G::swz(row)) * 16);
      }
  int v_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) v_off[i] = l32 * kBN + (((2 * h + i) ^ swz4(l32)) * 16);  // rows 32 db + l32: same swizzle

  const float sc = a.scale_log2;
  const int one = a.e8m0_one;  // E8M0 code of 1.0, as a run-time value
  float m_run, l_run;
  f32x16 acc[kD / 32];
  f32x16 s[2] = {f32x16{}, f32x16{}};
  i32x8 pb = {0, 0, 0, 0, 0, 0, 0, 0};

  int it_r = 0, it_j = first_j;
  int row0 = 0, qrow = 0, n_tiles = 0, g0 = 0;
  auto active = [&](int t) { return row0 < N && (!CAUSAL || t * kBN <= row0 + 31); };

  // matrix phase of tile i: S^T(i) (D/32 MFMAs: key block st % 2, k-step st / 2) and
  // u += P(i-1) V(i-1) (D/32 MFMAs: columns 32 st ..), interleaved; operand reads one
  // step ahead
  auto mfma_steps = [&](auto do_s_c, auto do_p_c, int i) {
    constexpr bool DO_S = decltype(do_s_c)::value;
    constexpr bool DO_P = decltype(do_p_c)::value;
    const char* kt = smem + ((g0 + i) % kStages) * kStage;
    const char* vt = smem + ((g0 + i + kStages - 1) % kStages) * kStage + kTile;
    const int ks = DO_S ? *reinterpret_cast<const int*>(kt + 2 * kTile) : 0;
    const int vs = DO_P ? *reinterpret_cast<const int*>(vt + kTile + kScale) : 0;
    if constexpr (DO_S) {
      s[0] = f32x16{};
      s[1] = f32x16{};
    }
    u32x4 ka[2][2], va[2][2];
    auto issue = [&](int st) {
      if constexpr (DO_S) {
        const int b = st & 1, kk = st >> 1;
        ka[st & 1][0] = lds_read16(kt + k_off[b][kk][0]);
        ka[st & 1][1] = lds_read16(kt + k_off[b][kk][1]);
      }
      if constexpr (DO_P) {
        va[st & 1][0] = lds_read16(vt + 32 * st * kBN + v_off[0]);
        va[st & 1][1] = lds_read16(vt + 32 * st * kBN + v_off[1]);
      }
    };
    issue(0);
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) {
      if (st + 1 < G::kSteps) issue(st + 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DO_S) s[st & 1] = mfma8<kIn, kIn>(ka[st & 1][0], ka[st & 1][1], qreg[st >> 1], s[st & 1], ks, q_sc);
      if constexpr (DO_P) acc[st] = mfma8<kIn, 0>(va[st & 1][0], va[st & 1][1], pb, acc[st], vs, one);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto mfma_phase = [&](int i) {
    const bool do_s = i < n_tiles && active(i);
    const bool do_p = i >= 1 && active(i - 1);
    __builtin_amdgcn_s_setprio(1);
    if (do_s && do_p) mfma_steps(std::true_type{}, std::true_type{}, i);
    else if (do_s) mfma_steps(std::true_type{}, std::false_type{}, i);
    else if (do_p) mfma_steps(std::false_type{}, std::true_type{}, i);
    __builtin_amdgcn_s_setprio(0);
  };

  // online softmax of S(t) against the exact running maximum; p' = 2^(s' - (m - 8))
  auto softmax_phase = [&](int t) {
    if (!(t >= 0 && t < n_tiles && active(t))) return;
    const int kv0 = t * kBN;
    if ((kv0 + kBN > N) || (CAUSAL && kv0 + kBN - 1 > row0)) {
      int lim = N - 1 - kv0;
      if (CAUSAL) lim = min(lim, qrow - kv0);
      lim -= 4 * h;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = (32 * b + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[b][r];
    }
    float mc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& v = s[c >> 1];
      const int o = 8 * (c & 1);
      mc[c] = __builtin_fmaxf(__builtin_fmaxf(v[o], v[o + 1]), v[o + 2]);
#pragma unroll
      for (int r = 3; r < 8; ++r) mc[c] = __builtin_fmaxf(mc[c], v[o + r]);
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(mc[0], mc[1]), __builtin_fmaxf(mc[2], mc[3]));
    mx = __builtin_fmaxf(mx, other_half(mx)) * sc;
    // reference: 8 below the row maximum, moved only when the maximum rises by more than
    // 0.8 (so p' <= 2^8.8 < 448, E4M3's largest value)
    const float m_new = (mx > m_run + 8.8f) ? mx - 8.f : m_run;
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    float pr[32], ps[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& v = s[c >> 1];
      const int o = 8 * (c & 1);
#pragma unroll
      for (int r = 0; r < 8; ++r) pr[8 * c + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[o + r], sc, -m_ref));
      const float* p = pr + 8 * c;
      ps[c] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) pb[w] = pack4(pr[4 * w], pr[4 * w + 1], pr[4 * w + 2], pr[4 * w + 3]);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    l_run = alpha * l_run + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) acc[db] *= alpha;
    }
  };

  for (;;) {
    if (first) wait_vmcnt<0>();
    first = false;
    __syncthreads();
    read_q();
    const int bh = item_bh(it_j);
    row0 = item_q0(it_j) + wave_rows;
    qrow = row0 + l32;
    n_tiles = item_tiles(item_q0(it_j));
    const int next_j = item_index(it_r + 1);
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) acc[db] = f32x16{};
    __syncthreads();
    for (int i = 0; i <= n_tiles; ++i) {
      if (i < n_tiles) issue_next();
      const bool q_in_flight = i == 0 && next_j >= 0;
      if (q_in_flight) issue_q(next_j);
      // every wave: the matrix work of tile i (S(i), P V of tile i-1), then the softmax
      // of tile i, the two waves of a SIMD in step (see the header)
      mfma_phase(i);
      softmax_phase(i);
      if (i + 1 < n_tiles) {
        if (q_in_flight) wait_vmcnt<G::kQLoads>();
        else wait_vmcnt<0>();
        __syncthreads();
      }
    }

    wait_vmcnt<0>();
    const float l_tot = l_run + other_half(l_run);
    if (qrow < N) {
      const float inv = 1.0f / l_tot;
      uint16_t* og = reinterpret_cast<uint16_t*>(a.o) + ((int64_t)bh * N + qrow) * kD;
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = {pack2<FP16OUT>(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                           pack2<FP16OUT>(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(og + db * 32 + 8 * g + 4 * h) = w;
        }
      if (h == 0) a.lse[(int64_t)bh * N + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
    }
    if (next_j < 0) break;
    g0 += n_tiles;
    it_j = next_j;
    ++it_r;
  }
}

}  // namespace f8

template <bool E5, int D>
hipError_t launch_fmt(const Fp8Args& a, int grid, bool fp16_out, bool causal, hipStream_t stream) {
  using namespace f8;
  if (fp16_out) {
    if (causal) hipLaunchKernelGGL((fwd_fp8<true, true, E5, D>), dim3(grid), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((fwd_fp8<true, false, E5, D>), dim3(grid), dim3(kThreads), 0, stream, a);
  } else {
    if (causal) hipLaunchKernelGGL((fwd_fp8<false, true, E5, D>), dim3(grid), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((fwd_fp8<false, false, E5, D>), dim3(grid), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Args& args, int d, bool fp16_out, bool causal, bool e5m2, hipStream_t stream) {
  using namespace f8;
  Fp8Args a = args;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int64_t items = (int64_t)a.bh * a.q_tiles;
  int grid = items < cus ? (int)items : cus;
  if (a.xcd_grouped) {
    grid &= ~7;
    if (grid < 8) grid = 8;
  }
  launch_log("fwd_fp8<%s out, %d, %s, %s> grid %d x %d", dtype_name(fp16_out), d, causal ? "causal" : "full",
             e5m2 ? "E5M2" : "E4M3", grid, kThreads);
  if (d == 64)
    return e5m2 ? launch_fmt<true, 64>(a, grid, fp16_out, causal, stream)
                : launch_fmt<false, 64>(a, grid, fp16_out, causal, stream);
  return e5m2 ? launch_fmt<true, 128>(a, grid, fp16_out, causal, stream)
              : launch_fmt<false, 128>(a, grid, fp16_out, causal, stream);
}

}  // namespace fa
