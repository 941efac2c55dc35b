// Exact attention backward for gfx950 (MI355X): bf16/fp16 in and out, fp32 math.
//
// Method ("6.1 FlashAttention V1 in detail", §6; "FlashAttention: IO-Aware
// Tiling, Online Softmax Mathematics, Memory Hierarchy Dynamics, and Kernel
// Evolution", section "Backward Pass Recomputation"): the forward keeps only O
// and the row statistic L = m + ln l; the backward rebuilds each tile of
// P = exp(S - L) from Q, K and L and forms
//     dV = P^T dO,  dP = dO V^T,  dS = P ∘ (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
// with D_i = rowsum(dO ∘ O)_i (the identity rowsum(dP ∘ P) = rowsum(dO ∘ O) of
// V1 §6.1). Three kernels run in order on one stream:
//  1. bwd_delta: D = rowsum(dO ∘ O) in fp32, one value per query row.
//  2. bwd_dq: a workgroup owns 256 query rows (8 waves of 32) and streams key
//     tiles of 64 rows through LDS, like the forward pass. Per tile each wave
//     forms S^T = K Q^T and dP^T = V dO^T (MFMA, operands K and V rows from LDS,
//     Q and dO rows in registers), P^T = exp2(S^T scale log2 e - L log2 e),
//     dS^T = P^T ∘ (dP^T - D), and accumulates dQ^T += K^T dS^T with K^T read
//     through the transposing LDS read and dS^T rounded to 16 bits as the B
//     operand without leaving registers.
//  3. bwd_dkdv: a workgroup owns 128 keys (4 waves of 32, one wave per SIMD, so
//     each wave has the whole register file) and streams query tiles of 64 rows
//     (Q, dO, L and D) through LDS. Per tile each wave forms S = Q K^T and
//     dP = dO V^T (K and V rows of its keys in registers), P and dS as above,
//     and accumulates dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T through the
//     transposing read).
// All MFMAs are v_mfma_f32_32x32x16 on 16-bit operands with fp32 accumulation;
// P and dS are rounded to the input dtype only as MFMA operands. Tiles are
// loaded straight into LDS (buffer_load ... lds) into 4-stage rings with the
// same XOR chunk swizzle as the forward pass, so every operand read hits every
// LDS bank once. Rows past N read as zeros through the buffer descriptor range;
// their contributions vanish because their K, V (dQ kernel) or Q, dO (dK/dV
// kernel) rows are zero, and keys past N are masked in the dQ kernel so that no
// overflowing exponent can reach a valid row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bwd_kernel.h"
#include "gfx950_ops.h"
#include "launch_log.h"

namespace fa {
namespace bwd {

using namespace ::fa::ops;

constexpr int kStages = 4;
constexpr int kAhead = 2;
constexpr int kTile = 64;  // rows of a streamed tile (keys in bwd_dq, queries in bwd_dkdv)
constexpr float kLog2e = 1.4426950408889634074f;

// Row-major 64-row tile of D-element rows in LDS (16-byte chunks swizzled by row).
template <int D>
struct Tile {
  static constexpr int rowBytes = D * 2;
  static constexpr int chunksPerRow = D / 8;
  static constexpr int bytes = kTile * rowBytes;
  static constexpr int blocks = bytes / 1024;  // 1 KiB per wave-instruction
  // lane `lane` of 1 KiB block b lands at chunk position 64 b + lane = (row, physical
  // chunk) and fetches the logical chunk physical ^ swizzle(row) of that row
  __device__ static __forceinline__ uint32_t src_offset(int b, int lane) {
    const int p = 64 * b + lane;
    const int row = p / chunksPerRow, phys = p % chunksPerRow;
    return (uint32_t)row * rowBytes + (uint32_t)((phys ^ chunk_swizzle<D>(row)) * 16);
  }
  // row-operand read (MFMA A operand, 32-row block): lane (l32, h) reads logical
  // chunk 2 kk + h of row l32, i.e. elements 16 kk + 8 h .. + 7 of that row
  __device__ static __forceinline__ int row_offset(int l32, int h, int kk) {
    return l32 * rowBytes + (((2 * kk + h) ^ chunk_swizzle<D>(l32)) * 16);
  }
  // transposing read (MFMA A operand M^T, d block db of 32 columns, 16-row step t):
  // source row 16 t + 8 half + 4 h + (lane % 16) / 4, logical chunk
  // 4 db + 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2) in the chunk.
  // The 16 rows of step t come out in the order in which a 32x32 accumulator's
  // rows are packed into the B operand of k-step t (see pack_b).
  __device__ static __forceinline__ int tr_offset(int lane, int half, int db) {
    const int h = lane >> 5;
    const int row = 8 * half + 4 * h + ((lane & 15) >> 2);
    const int logical = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return row * rowBytes + ((logical ^ chunk_swizzle<D>(row)) * 16) + 8 * (lane & 1);
  }
};

// Products of the dK/dV kernel with the register file of each operand fixed. One
// wave per SIMD holds K and V rows (B operands written once), the dK and dV
// accumulators and a tile of S and dP: more than the 256 vector registers, so K,
// V, dK and dV live in the accumulation registers (AGPRs), which MFMA reads and
// writes directly, and S and dP, which the VALU works on, in vector registers.
// The compiler's hazard checks do not see an MFMA inside an asm statement, so the
// wait states they would insert are explicit: two before a product whose operand
// the VALU may just have written (mfma32_aa), mfma_wait() before the first VALU
// access of an S or dP block, and mfma_drain_a() before the accumulators are read.
// c (AGPR) += a (VGPR) b (VGPR), after two wait states
template <bool FP16>
__device__ __forceinline__ void mfma32_aa(u32x4 a, u32x4 b, f32x16& c) {
  if constexpr (FP16)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// c (VGPR) = a (VGPR) b (AGPR), the first k-step of a product
template <bool FP16>
__device__ __forceinline__ f32x16 mfma32_va0(u32x4 a, u32x4 b) {
  f32x16 c;
  if constexpr (FP16)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
  return c;
}
// c (VGPR) += a (VGPR) b (AGPR)
template <bool FP16>
__device__ __forceinline__ void mfma32_va(u32x4 a, u32x4 b, f32x16& c) {
  if constexpr (FP16)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
// wait states between a 32x32x16 product and a VALU access of its result, when at
// least two more products were issued in between (the result passes through the
// statement, so no access of it is scheduled before it)
__device__ __forceinline__ void mfma_wait(f32x16& x, f32x16& y) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(x), "+v"(y));
}
template <int N>
__device__ __forceinline__ void mfma_drain_a(f32x16 (&x)[N], f32x16 (&y)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(x[i]), "+a"(y[i]));
}

// B operand of k-step c (16 rows) from two 32x32 accumulators covering 64 rows:
// elements 8 (c % 2) .. + 7 of accumulator c / 2, rounded to 16 bits
template <bool FP16>
__device__ __forceinline__ u32x4 pack_b(const f32x16 (&x)[2], int c) {
  const f32x16& v = x[c >> 1];
  const int o = 8 * (c & 1);
  return u32x4{pack2<FP16>(v[o], v[o + 1]), pack2<FP16>(v[o + 2], v[o + 3]), pack2<FP16>(v[o + 4], v[o + 5]),
               pack2<FP16>(v[o + 6], v[o + 7])};
}

// Store a d x 32 accumulator set (one lane per column = output row) to a row of
// the output, times `mul`: element 4 g + r of block db is column 32 db + 8 g + 4 h + r.
template <bool FP16, int D>
__device__ __forceinline__ void store_rows(uint16_t* row_ptr, const f32x16 (&acc)[D / 32], float mul, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = {pack2<FP16>(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul),
                       pack2<FP16>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      *reinterpret_cast<u32x2*>(row_ptr + db * 32 + 8 * g + 4 * h) = w;
    }
}

// ------------------------------------------------------------------------------
// 1. D = rowsum(dO ∘ O): 16-byte chunks, D/8 lanes per row, fp32 products and sums.
template <bool FP16, int D>
__global__ __launch_bounds__(256) void bwd_delta(BwdArgs a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int64_t rows = (int64_t)a.bh * a.n;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int part = threadIdx.x % kLanesPerRow;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.dout) + row * D + part * 8);
    const u32x4 y = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.o) + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x0, x1, y0, y1;
      if constexpr (FP16) {
        // element copies first: a bit cast applied to a vector element expression
        // directly has been compiled as a cast of element 0
        const uint32_t xi = x[i], yi = y[i];
        const f16x2 xv = __builtin_bit_cast(f16x2, xi), yv = __builtin_bit_cast(f16x2, yi);
        x0 = (float)xv[0]; x1 = (float)xv[1]; y0 = (float)yv[0]; y1 = (float)yv[1];
      } else {
        x0 = __uint_as_float(x[i] << 16); x1 = __uint_as_float(x[i] & 0xffff0000u);
        y0 = __uint_as_float(y[i] << 16); y1 = __uint_as_float(y[i] & 0xffff0000u);
      }
      acc = __builtin_fmaf(x0, y0, acc);
      acc = __builtin_fmaf(x1, y1, acc);
    }
  }
#pragma unroll
  for (int m = 1; m < kLanesPerRow; m <<= 1) acc += __shfl_xor(acc, m, kLanesPerRow);
  if (row < rows && part == 0) a.delta[row] = acc;
}

// ------------------------------------------------------------------------------
// 2. dQ: 8 waves x 32 query rows, key tiles of 64 streamed through LDS.
constexpr int kDqWaves = 8;
constexpr int kDqRows = 32 * kDqWaves;

template <bool FP16, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kDqWaves, 1) void bwd_dq(BwdArgs a) {
  using T = Tile<D>;
  constexpr int kStage = 2 * T::bytes;  // K then V
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, h = lane >> 5, l32 = lane & 31;

  // workgroup -> (slice, query tile): heaviest causal tiles first; with
  // xcd_grouped all query tiles of a slice on one XCD (shared K/V in its L2)
  const int bid = blockIdx.x;
  int bh, rank;
  if (a.xcd_grouped) {
    const int hpx = a.bh / 8;
    const int t = bid >> 3;
    rank = t / hpx;
    bh = (bid & 7) * hpx + t % hpx;
  } else {
    rank = bid / a.bh;
    bh = bid % a.bh;
  }
  const int q_tiles = (a.n + kDqRows - 1) / kDqRows;
  const int qtile = CAUSAL ? (q_tiles - 1 - rank) : rank;
  const int N = a.n;
  const int q0 = qtile * kDqRows;
  const int64_t head = (int64_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const uint16_t* kg = reinterpret_cast<const uint16_t*>(a.k) + head;
  const uint16_t* vg = reinterpret_cast<const uint16_t*>(a.v) + head;

  // rows of this wave: block wave%4 (waves 0-3) or 7 - wave%4 (waves 4-7), so that
  // causal work on the diagonal tiles is spread over the SIMDs
  const int row0 = q0 + 32 * (grp == 0 ? (wave & 3) : 7 - (wave & 3));
  const int qrow = row0 + l32;
  const int tiles_all = (N + kTile - 1) / kTile;
  const int n_tiles = CAUSAL ? min(tiles_all, (min(q0 + kDqRows, N) - 1) / kTile + 1) : tiles_all;

  uint32_t ld_off[T::blocks / kDqWaves];
#pragma unroll
  for (int i = 0; i < T::blocks / kDqWaves; ++i) ld_off[i] = T::src_offset(wave + kDqWaves * i, lane);
  auto issue_tile = [&](int t) {
    const uint32_t skip = (uint32_t)t * kTile * T::rowBytes;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kg + (int64_t)t * kTile * D, head_bytes - skip);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vg + (int64_t)t * kTile * D, head_bytes - skip);
    char* st = smem + (t % kStages) * kStage;
#pragma unroll
    for (int i = 0; i < T::blocks / kDqWaves; ++i) {
      buffer_load16_lds(kr, ld_off[i], st + 1024 * (wave + kDqWaves * i));
      buffer_load16_lds(vr, ld_off[i], st + T::bytes + 1024 * (wave + kDqWaves * i));
    }
  };
  constexpr int kLoads = 2 * T::blocks / kDqWaves;

  issue_tile(0);
  if (n_tiles > 1) issue_tile(1);
  // Q and dO rows of this lane's query (B operands, k-slots d = 16 kk + 8 h + 0..7),
  // L and D of the query (rows past N read as zeros and are never stored)
  u32x4 qreg[D / 16], doreg[D / 16];
  {
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(reinterpret_cast<const uint16_t*>(a.q) + head, head_bytes);
    const __amdgpu_buffer_rsrc_t dr = buffer_rsrc(reinterpret_cast<const uint16_t*>(a.dout) + head, head_bytes);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qreg[kk] = buffer_load16(qr, (uint32_t)qrow * T::rowBytes + kk * 32 + h * 16);
      doreg[kk] = buffer_load16(dr, (uint32_t)qrow * T::rowBytes + kk * 32 + h * 16);
    }
  }
  const bool row_ok = qrow < N;
  const float lse2 = row_ok ? a.lse[(int64_t)bh * N + qrow] * kLog2e : 0.f;
  const float dlt = row_ok ? a.delta[(int64_t)bh * N + qrow] : 0.f;
  const float c = a.scale_log2;
  wait_vmcnt<0>();
  __syncthreads();

  int k_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = T::row_offset(l32, h, kk);
  int t_off[2][D / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) t_off[half][db] = T::tr_offset(lane, half, db);

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  for (int i = 0; i < n_tiles; ++i) {
    if (i + kAhead < n_tiles) issue_tile(i + kAhead);
    const bool active = row0 < N && (!CAUSAL || i * kTile <= row0 + 31);
    if (active) {
      const char* kt = smem + (i % kStages) * kStage;
      const char* vt = kt + T::bytes;
      // S^T = K Q^T and dP^T = V dO^T: two key blocks of 32, D/16 k-steps each
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int st = 0; st < D / 8; ++st) {
        const int kk = st >> 1, b = st & 1;
        const u32x4 ka = lds_read16(kt + k_off[kk] + b * 32 * T::rowBytes);
        const u32x4 va = lds_read16(vt + k_off[kk] + b * 32 * T::rowBytes);
        s[b] = mfma32<FP16>(ka, qreg[kk], s[b]);
        dp[b] = mfma32<FP16>(va, doreg[kk], dp[b]);
      }
      // P^T and dS^T; key = 32 b + 8 (r / 4) + 4 h + r % 4 within the tile
      const int kv0 = i * kTile;
      const bool masked = (kv0 + kTile > N) || (CAUSAL && kv0 + kTile - 1 > row0);
      int lim = N - 1 - kv0;
      if (CAUSAL) lim = min(lim, qrow - kv0);
      lim -= 4 * h;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -lse2));
          if (masked && 32 * b + 8 * (r >> 2) + (r & 3) > lim) p = 0.f;
          s[b][r] = p * (dp[b][r] - dlt);
        }
      u32x4 dsb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) dsb[t] = pack_b<FP16>(s, t);
      // dQ^T += K^T dS^T
#pragma unroll
      for (int st = 0; st < D / 8; ++st) {
        const int t = st / (D / 32), db = st % (D / 32);
        const u32x2 lo = lds_read_tr16(kt + t_off[0][db] + 16 * t * T::rowBytes);
        const u32x2 hi = lds_read_tr16(kt + t_off[1][db] + 16 * t * T::rowBytes);
        dq[db] = mfma32<FP16>(u32x4{lo[0], lo[1], hi[0], hi[1]}, dsb[t], dq[db]);
      }
    }
    if (i + 1 < n_tiles) {
      if (i + kAhead < n_tiles) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
      __syncthreads();
    }
  }

  if (row_ok) store_rows<FP16, D>(reinterpret_cast<uint16_t*>(a.dq) + head + (int64_t)qrow * D, dq, a.scale, h);
}

// ------------------------------------------------------------------------------
// 3. dK, dV: 4 waves x 32 keys, query tiles of 64 (Q, dO, L, D) streamed through LDS.
constexpr int kKvWaves = 4;
constexpr int kLookBwd = 3;  // LDS operand reads issued this many product steps ahead
constexpr int kKvRows = 32 * kKvWaves;

template <bool FP16, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kKvWaves, 1) void bwd_dkdv(BwdArgs a) {
  using T = Tile<D>;
  constexpr int kStat = kTile * 4;                        // L or D of the tile's rows
  constexpr int kStage = 2 * T::bytes + 2 * kStat;        // Q, dO, L, D
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // workgroup -> (slice, key block): key blocks in increasing order, so under a
  // causal mask the heaviest blocks (most query tiles) start first
  const int bid = blockIdx.x;
  const int k_blocks = (a.n + kKvRows - 1) / kKvRows;
  int bh, kb;
  if (a.xcd_grouped) {
    const int hpx = a.bh / 8;
    const int t = bid >> 3;
    kb = t / hpx;
    bh = (bid & 7) * hpx + t % hpx;
  } else {
    kb = bid / a.bh;
    bh = bid % a.bh;
  }
  (void)k_blocks;
  const int N = a.n;
  const int k0 = kb * kKvRows;
  const int key0 = k0 + 32 * wave;  // this wave's first key
  const int key = key0 + l32;       // this lane's key (B-operand column)
  const int64_t head = (int64_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const uint16_t* qg = reinterpret_cast<const uint16_t*>(a.q) + head;
  const uint16_t* og = reinterpret_cast<const uint16_t*>(a.dout) + head;
  const float* lg = a.lse + (int64_t)bh * N;
  const float* dg = a.delta + (int64_t)bh * N;

  // query tiles that can see this workgroup's keys
  const int tiles_all = (N + kTile - 1) / kTile;
  const int t_first = CAUSAL ? k0 / kTile : 0;
  const int n_tiles = tiles_all - t_first;

  uint32_t ld_off[T::blocks / kKvWaves];
#pragma unroll
  for (int i = 0; i < T::blocks / kKvWaves; ++i) ld_off[i] = T::src_offset(wave + kKvWaves * i, lane);
  // every wave loads the tile's L and D rows (the same bytes to the same place), so
  // that all waves issue the same number of loads per tile
  // The kLoads loads of tile j, one at a time: load n < kLoads - 2 is Q block n / 2
  // (even n) or dO block n / 2 (odd n) of this wave's share, then L and D.
  struct TileSrc {
    __amdgpu_buffer_rsrc_t q, o, l, d;
    char* st;
  };
  auto tile_src = [&](int j) {
    const int t = t_first + j;
    const uint32_t skip = (uint32_t)t * kTile * T::rowBytes;
    const uint32_t sskip = (uint32_t)t * kTile * 4;
    return TileSrc{buffer_rsrc(qg + (int64_t)t * kTile * D, head_bytes - skip),
                   buffer_rsrc(og + (int64_t)t * kTile * D, head_bytes - skip),
                   buffer_rsrc(lg + t * kTile, (uint32_t)N * 4 - sskip),
                   buffer_rsrc(dg + t * kTile, (uint32_t)N * 4 - sskip), smem + (j % kStages) * kStage};
  };
  constexpr int kLoads = 2 * T::blocks / kKvWaves + 2;
  auto issue_load = [&](const TileSrc& ts, int n) {
    if (n < kLoads - 2) {
      const int i = n >> 1;
      if ((n & 1) == 0) buffer_load16_lds(ts.q, ld_off[i], ts.st + 1024 * (wave + kKvWaves * i));
      else buffer_load16_lds(ts.o, ld_off[i], ts.st + T::bytes + 1024 * (wave + kKvWaves * i));
    } else if (n == kLoads - 2) {
      buffer_load4_lds(ts.l, lane * 4, ts.st + 2 * T::bytes);
    } else {
      buffer_load4_lds(ts.d, lane * 4, ts.st + 2 * T::bytes + kStat);
    }
  };
  auto issue_tile = [&](int j) {
    const TileSrc ts = tile_src(j);
#pragma unroll
    for (int n = 0; n < kLoads; ++n) issue_load(ts, n);
  };

  issue_tile(0);
  if (n_tiles > 1) issue_tile(1);
  // K and V rows of this lane's key (B operands, k-slots d = 16 kk + 8 h + 0..7)
  u32x4 kreg[D / 16], vreg[D / 16];
  {
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(reinterpret_cast<const uint16_t*>(a.k) + head, head_bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(reinterpret_cast<const uint16_t*>(a.v) + head, head_bytes);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kreg[kk] = buffer_load16(kr, (uint32_t)key * T::rowBytes + kk * 32 + h * 16);
      vreg[kk] = buffer_load16(vr, (uint32_t)key * T::rowBytes + kk * 32 + h * 16);
    }
  }
  const float c = a.scale_log2;
  wait_vmcnt<0>();
  __syncthreads();

  int r_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) r_off[kk] = T::row_offset(l32, h, kk);
  int t_off[2][D / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) t_off[half][db] = T::tr_offset(lane, half, db);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  for (int j = 0; j < n_tiles; ++j) {
    // dK and dV stay in the accumulation registers across iterations (without this
    // the loop-carried copy lands in vector registers and is copied every tile)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
    // tile j + kAhead: loaded one instruction per step of the dV/dK products (a
    // load that waits for the address unit then holds up no product), or all at
    // once here by a wave with no work in this tile
    const bool load_next = j + kAhead < n_tiles;
    const int qt0 = (t_first + j) * kTile;  // first query row of the tile
    // queries below this wave's first key see none of its keys (causal)
    const bool active = key0 < N && (!CAUSAL || qt0 + kTile - 1 >= key0);
    if (!active && load_next) issue_tile(j + kAhead);
    if (active) {
      const char* qt = smem + (j % kStages) * kStage;
      const char* ot = qt + T::bytes;
      const float* lt = reinterpret_cast<const float*>(qt + 2 * T::bytes);
      const float* dt = reinterpret_cast<const float*>(qt + 2 * T::bytes + kStat);
      // The tile's 64 query rows form two blocks of 32. Products of block 0 run
      // first; the VALU work of block 0 (P, dS and their 16-bit B operands) is
      // interleaved with the S and dP products of block 1, and that of block 1
      // with the dV and dK products of block 0, so that the exponentials run
      // under matrix work instead of between its phases.
      constexpr int kSd = D / 16;  // k-steps of one block's S (and dP) product
      f32x16 s[2], dp[2];
      u32x4 pb[4], dsb[4];
      // P and dS in place for query rows 32 b + 8 g + 4 h + r (r = 0..3)
      const bool masked = CAUSAL && qt0 < key0 + 31;
      auto p_ds = [&](int b, int g) {
        const int row = 32 * b + 8 * g + 4 * h;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + row);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + row);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][e], c, -l4[r] * kLog2e));
          if (masked && qt0 + row + r < key) p = 0.f;
          s[b][e] = p;
          dp[b][e] = p * (dp[b][e] - d4[r]);
        }
      };
      // VALU job j of block b: 0..3 P and dS of one row group, 4 and 5 the B operands
      auto valu_job = [&](int b, int j) {
        if (j < 4) {
          p_ds(b, j);
        } else if (j == 4) {
          pb[2 * b] = pack_b<FP16>(s, 2 * b);
          pb[2 * b + 1] = pack_b<FP16>(s, 2 * b + 1);
        } else {
          dsb[2 * b] = pack_b<FP16>(dp, 2 * b);
          dsb[2 * b + 1] = pack_b<FP16>(dp, 2 * b + 1);
        }
      };
      // the jobs of a block run after steps 1 .. kSd - 1 of the next product phase;
      // the first reads accumulators that the products just before may still be
      // writing: mfma_wait() supplies the wait states (the results pass through it,
      // so no read is scheduled earlier)
      auto jobs_after_step = [&](int b, int k) {
        if (k == 1) mfma_wait(s[b], dp[b]);
#pragma unroll
        for (int jj = 0; jj < 6; ++jj)
          if ((jj + 1 < kSd ? jj + 1 : kSd - 1) == k) valu_job(b, jj);
      };
      // S = Q K^T and dP = dO V^T, block 0 then block 1, D/16 k-steps each; operand
      // reads from LDS are issued kLookBwd steps ahead of their products
      {
        u32x4 qa[kLookBwd + 1], oa[kLookBwd + 1];
        auto issue = [&](int st) {
          const int kk = st % kSd, b = st / kSd;
          qa[st % (kLookBwd + 1)] = lds_read16(qt + r_off[kk] + b * 32 * T::rowBytes);
          oa[st % (kLookBwd + 1)] = lds_read16(ot + r_off[kk] + b * 32 * T::rowBytes);
        };
#pragma unroll
        for (int st = 0; st < kLookBwd; ++st) issue(st);
#pragma unroll
        for (int st = 0; st < 2 * kSd; ++st) {
          if (st + kLookBwd < 2 * kSd) issue(st + kLookBwd);
          __builtin_amdgcn_sched_barrier(0);
          const int kk = st % kSd, b = st / kSd, sl = st % (kLookBwd + 1);
          if (kk == 0) {
            s[b] = mfma32_va0<FP16>(qa[sl], kreg[kk]);
            dp[b] = mfma32_va0<FP16>(oa[sl], vreg[kk]);
          } else {
            mfma32_va<FP16>(qa[sl], kreg[kk], s[b]);
            mfma32_va<FP16>(oa[sl], vreg[kk], dp[b]);
          }
          if (b == 1) jobs_after_step(0, kk);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS: k-steps t = 0, 1 take block 0's rows
      // (the first kSd steps), t = 2, 3 block 1's
      {
        u32x2 olo[kLookBwd + 1], ohi[kLookBwd + 1], qlo[kLookBwd + 1], qhi[kLookBwd + 1];
        static_assert(kLoads <= D / 8, "one tile load per dV/dK step");
        const TileSrc ts = tile_src(load_next ? j + kAhead : j);
        auto issue = [&](int st) {
          const int t = st / (D / 32), db = st % (D / 32), sl = st % (kLookBwd + 1);
          olo[sl] = lds_read_tr16(ot + t_off[0][db] + 16 * t * T::rowBytes);
          ohi[sl] = lds_read_tr16(ot + t_off[1][db] + 16 * t * T::rowBytes);
          qlo[sl] = lds_read_tr16(qt + t_off[0][db] + 16 * t * T::rowBytes);
          qhi[sl] = lds_read_tr16(qt + t_off[1][db] + 16 * t * T::rowBytes);
        };
#pragma unroll
        for (int st = 0; st < kLookBwd; ++st) issue(st);
#pragma unroll
        for (int st = 0; st < D / 8; ++st) {
          if (st + kLookBwd < D / 8) issue(st + kLookBwd);
          __builtin_amdgcn_sched_barrier(0);
          const int t = st / (D / 32), db = st % (D / 32), sl = st % (kLookBwd + 1);
          mfma32_aa<FP16>(u32x4{olo[sl][0], olo[sl][1], ohi[sl][0], ohi[sl][1]}, pb[t], dv[db]);
          mfma32_aa<FP16>(u32x4{qlo[sl][0], qlo[sl][1], qhi[sl][0], qhi[sl][1]}, dsb[t], dk[db]);
          if (st < kLoads && load_next) issue_load(ts, st);
          if (st < kSd) jobs_after_step(1, st);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (j + 1 < n_tiles) {
      if (j + kAhead < n_tiles) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
      __syncthreads();
    }
  }

  mfma_drain_a<D / 32>(dk, dv);
  if (key < N) {
    store_rows<FP16, D>(reinterpret_cast<uint16_t*>(a.dk) + head + (int64_t)key * D, dk, a.scale, h);
    store_rows<FP16, D>(reinterpret_cast<uint16_t*>(a.dv) + head + (int64_t)key * D, dv, 1.0f, h);
  }
}

template <bool FP16, int D, bool CAUSAL>
hipError_t launch_all(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.bh * a.n;
  constexpr int kRowsPerBlock = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_delta<FP16, D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int q_tiles = (a.n + kDqRows - 1) / kDqRows;
  const int k_blocks = (a.n + kKvRows - 1) / kKvRows;
  launch_log("bwd_delta<%s, %d> grid %lld x 256; bwd_dq<%s, %d, %s> grid %d x %d; bwd_dkdv<%s, %d, %s> grid %d x %d",
             dtype_name(FP16), D, (long long)((rows + kRowsPerBlock - 1) / kRowsPerBlock), dtype_name(FP16), D,
             CAUSAL ? "causal" : "full", a.bh * q_tiles, 64 * kDqWaves, dtype_name(FP16), D,
             CAUSAL ? "causal" : "full", a.bh * k_blocks, 64 * kKvWaves);
  hipLaunchKernelGGL((bwd_dq<FP16, D, CAUSAL>), dim3(a.bh * q_tiles), dim3(64 * kDqWaves), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv<FP16, D, CAUSAL>), dim3(a.bh * k_blocks), dim3(64 * kKvWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bwd

hipError_t launch_bwd(const BwdArgs& a, bool fp16, int d, bool causal, hipStream_t stream) {
  using namespace bwd;
  if (fp16) {
    if (d == 64) return causal ? launch_all<true, 64, true>(a, stream) : launch_all<true, 64, false>(a, stream);
    return causal ? launch_all<true, 128, true>(a, stream) : launch_all<true, 128, false>(a, stream);
  }
  if (d == 64) return causal ? launch_all<false, 64, true>(a, stream) : launch_all<false, 64, false>(a, stream);
  return causal ? launch_all<false, 128, true>(a, stream) : launch_all<false, 128, false>(a, stream);
}

}  // namespace fa
