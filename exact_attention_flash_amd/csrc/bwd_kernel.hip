// Exact attention backward for gfx950 (MI355X): bf16/fp16 in and out, fp32 math.
//
// Method ("6.1 FlashAttention V1 in detail", §6; "FlashAttention: IO-Aware
// Tiling, Online Softmax Mathematics, Memory Hierarchy Dynamics, and Kernel
// Evolution", section "Backward Pass Recomputation"): the forward keeps only O
// and the row statistic L = m + ln l; the backward rebuilds each tile of
// P = exp(S - L) from Q, K and L and forms
//     dV = P^T dO,  dP = dO V^T,  dS = P ∘ (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
// with D_i = rowsum(dO ∘ O)_i (the identity rowsum(dP ∘ P) = rowsum(dO ∘ O) of
// V1 §6.1). Two kernels run in order on one stream:
//  1. bwd_dq: a workgroup owns 256 query rows (4 waves of 64, one wave per SIMD)
//     and streams key sub-tiles of 32 rows through LDS. Per sub-tile each wave
//     forms S^T = K Q^T and dP^T = V dO^T for its two 32-row query blocks (MFMA,
//     operands K and V rows from LDS, each read serving both blocks; Q and dO
//     rows in registers), P^T = exp2(S^T scale log2 e - L log2 e),
//     dS^T = P^T ∘ (dP^T - D), and accumulates dQ^T += K^T dS^T with K^T read
//     through the transposing LDS read and dS^T rounded to 16 bits as the B
//     operand without leaving registers; software-pipelined like bwd_dkdv. It
//     first forms D for its rows in fp32 (from the dO rows it holds and the O
//     rows it loads) and stores it for bwd_dkdv.
//  2. bwd_dkdv: a workgroup owns 128 keys (4 waves of 32, one wave per SIMD, so
//     each wave has the whole register file) and streams query tiles of 64 rows
//     (Q, dO, L and D) through LDS. Per tile each wave forms S = Q K^T and
//     dP = dO V^T (K and V rows of its keys in registers), P and dS as above,
//     and accumulates dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T through the
//     transposing read). The tile loop is software-pipelined: the S/dP products
//     of tile j and the dV/dK products of tile j - 1 each run with half of a
//     tile's P/dS work placed between them, one element per product or two.
// All MFMAs are v_mfma_f32_32x32x16 on 16-bit operands with fp32 accumulation;
// P and dS are rounded to the input dtype only as MFMA operands. Tiles are
// loaded straight into LDS (buffer_load ... lds) into 4-stage rings with the
// same XOR chunk swizzle as the forward pass, so every operand read hits every
// LDS bank once. Rows past N read as zeros through the buffer descriptor range;
// their contributions vanish because their K, V (dQ kernel) or Q, dO (dK/dV
// kernel) rows are zero, and keys past N (sub-tiles past the end included) are
// masked in the dQ kernel so that no overflowing exponent can reach a valid row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "bwd_kernel.h"
#include "gfx950_ops.h"
#include "launch_log.h"

namespace fa {
namespace bwd {

using namespace ::fa::ops;

// The 4-byte load straight to LDS with a scalar LDS byte address, under the rules of
// buffer_load16_lds_s (one wait state after a scalar write of M0; neither M0 nor the
// descriptor written by a VALU instruction within five).
__device__ __forceinline__ void buffer_load4_lds_s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr) : "memory");
}

constexpr int kStages = 4;
constexpr int kAhead = 2;
constexpr int kTile = 64;  // rows of a streamed tile (keys in bwd_dq, queries in bwd_dkdv)
constexpr float kLog2e = 1.4426950408889634074f;

// Row-major tile of ROWS D-element rows in LDS (16-byte chunks swizzled by row).
template <int D, int ROWS = kTile>
struct Tile {
  static constexpr int rowBytes = D * 2;
  static constexpr int chunksPerRow = D / 8;
  static constexpr int bytes = ROWS * rowBytes;
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

// x of lane N of the lane's 16-lane row (DPP row_newbcast:N), for the VALU
// instruction that consumes it: the compiler folds the move into a two-operand
// subtraction (v_subrev_f32_dpp)
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, true));
}

// f(std::integral_constant<int, i>) for i = 0 .. N - 1 in order: code generated per i,
// with i a constant expression (no loop for the compiler to unroll)
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------------------------
// 1. dQ (and D): 4 waves x 64 query rows (one wave per SIMD), key sub-tiles of 32 streamed
// through LDS.
//
// Each wave owns two 32-row query blocks, so every K, V or K^T operand it reads
// from LDS serves two products (one per block): half the LDS bytes per product of
// one block per wave. The blocks' Q and dO rows (the B operands of S^T and dP^T)
// and the dQ^T accumulators fill the accumulation registers; with S^T = K Q^T the
// lane is the query, so L and D are per-lane constants. The sub-tile loop is
// software-pipelined like the dK/dV kernel's tile loop:
//   phase A(j): S^T and dP^T of sub-tile j (both blocks)  | P, dS of sub-tile j - 1, block 1
//   phase B(j): dQ^T of sub-tile j - 1 (both blocks)       | P, dS of sub-tile j, block 0
constexpr int kDqWaves = 4;
constexpr int kDqRows = 64 * kDqWaves;
constexpr int kSub = 32;        // keys per sub-tile
constexpr int kDqStages = 4;
constexpr int kDqItems = 18;    // softmax items of one block: 16 elements, 2 packed dS operands

// Per-sub-tile values of one wave: S^T and dP^T of its two query blocks (dS^T
// replaces dP^T in place) and dS^T rounded to 16 bits as the B operands of the two
// 16-key k-steps of the dQ^T product.
struct DqSub {
  f32x16 s[2], dp[2];
  u32x4 dsb[2][2];
};

// One 16-bit value of a 32-bit word (half 0: low bits) widened to fp32.
template <bool FP16>
__device__ __forceinline__ float widen16(uint32_t w, int half) {
  const uint32_t bits = half ? (w >> 16) : (w & 0xffffu);
  if constexpr (FP16) return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  else return __uint_as_float(bits << 16);
}

// Sum of the 8 products of two 16-byte vectors of 16-bit values, in fp32, each
// value widened from its 32-bit word with integer operations. (Widening an element
// of the vector through a bit cast to a two-element fp16 vector made the compiler
// read element 0 for every element, fused into v_dot2c_f32_f16 or not: the sum held
// one quarter of the products four times.)
template <bool FP16>
__device__ __forceinline__ float dot8(u32x4 x, u32x4 y) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t xw = x[i], yw = y[i];
    acc = __builtin_fmaf(widen16<FP16>(xw, 0), widen16<FP16>(yw, 0), acc);
    acc = __builtin_fmaf(widen16<FP16>(xw, 1), widen16<FP16>(yw, 1), acc);
  }
  return acc;
}

template <bool FP16>
__device__ __forceinline__ u32x4 pack_b1(const f32x16& v, int t) {
  const int o = 8 * t;
  return u32x4{pack2<FP16>(v[o], v[o + 1]), pack2<FP16>(v[o + 2], v[o + 3]), pack2<FP16>(v[o + 4], v[o + 5]),
               pack2<FP16>(v[o + 6], v[o + 7])};
}

template <bool FP16, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kDqWaves, 1) void bwd_dq(BwdArgs a) {
  using T = Tile<D, kSub>;
  constexpr int kStage = 2 * T::bytes;  // K then V
  constexpr int kSd = D / 16;           // k-steps of S^T (and dP^T)
  constexpr int kSlotsA = 4 * kSd;      // S^T, dP^T products of both blocks
  constexpr int kSlotsB = 4 * (D / 32); // dQ^T products: 2 k-steps x D/32 blocks x 2 query blocks
  constexpr int kLoads = 2 * T::blocks / kDqWaves;
  static_assert(T::blocks % kDqWaves == 0 && kLoads <= kSlotsB, "tile loads");
  __shared__ __attribute__((aligned(1024))) char smem[kDqStages * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

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

  // query blocks of this wave: 32-row blocks wave and 7 - wave of the tile, so that
  // the causal diagonal's masked work is spread evenly over the waves
  int qrow[2];
  qrow[0] = q0 + 32 * wave + l32;
  qrow[1] = q0 + 32 * (2 * kDqWaves - 1 - wave) + l32;

  // key sub-tiles: those any row of the tile can see; from sub-tile m0 on some
  // element needs the mask (causal diagonal, keys past N)
  const int subs_all = (N + kSub - 1) / kSub;
  const int n_sub = CAUSAL ? (min(q0 + kDqRows, N) + kSub - 1) / kSub : subs_all;
  const int m0 = CAUSAL ? q0 / kSub : (N % kSub == 0 ? n_sub : n_sub - 1);

  // sub-tile loads: this wave's share of K and V (1 KiB blocks); a sub-tile past the
  // last one reads zeros through an empty range (its keys are masked)
  uint32_t ld_off[T::blocks / kDqWaves];
#pragma unroll
  for (int i = 0; i < T::blocks / kDqWaves; ++i) ld_off[i] = T::src_offset(wave + kDqWaves * i, lane);
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(1024u * (uint32_t)wave);
  struct SubSrc {
    __amdgpu_buffer_rsrc_t k, v;
    uint32_t st;
  };
  auto sub_src = [&](int j) {
    const bool in = j < subs_all;
    const uint32_t skip = (uint32_t)j * kSub * T::rowBytes;
    const uint32_t rows = in ? head_bytes - skip : 0u;
    return SubSrc{buffer_rsrc(kg + (int64_t)j * kSub * D, rows), buffer_rsrc(vg + (int64_t)j * kSub * D, rows),
                  (uint32_t)(uintptr_t)smem + (uint32_t)((j % kDqStages) * kStage) + lds_w};
  };
  auto issue_load = [&](const SubSrc& ss, int n) {
    const int i = n >> 1;
    const uint32_t dst = ss.st + 1024u * kDqWaves * i + ((n & 1) ? (uint32_t)T::bytes : 0u);
    buffer_load16_lds_s((n & 1) ? ss.v : ss.k, ld_off[i], dst);
  };
  auto issue_sub = [&](int j) {
    const SubSrc ss = sub_src(j);
#pragma unroll
    for (int n = 0; n < kLoads; ++n) issue_load(ss, n);
  };

  issue_sub(0);
  issue_sub(1);
  // Q and dO rows of this lane's queries (B operands, k-slots d = 16 kk + 8 h + 0..7),
  // L log2 e of the queries, and D = rowsum(dO ∘ O): each lane of a query holds half
  // its dO row and loads the same half of its O row, and the two halves meet with one
  // lane swap. D is stored for the dK/dV kernel (rows past N read as zeros and are
  // never stored).
  u32x4 qreg[2][kSd], oreg[2][kSd];
  float lse2[2], dlt[2];
  {
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(reinterpret_cast<const uint16_t*>(a.q) + head, head_bytes);
    const __amdgpu_buffer_rsrc_t dr = buffer_rsrc(reinterpret_cast<const uint16_t*>(a.dout) + head, head_bytes);
    const __amdgpu_buffer_rsrc_t orr = buffer_rsrc(reinterpret_cast<const uint16_t*>(a.o) + head, head_bytes);
    u32x4 orow[2][kSd];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int kk = 0; kk < kSd; ++kk) {
        qreg[qb][kk] = buffer_load16(qr, (uint32_t)qrow[qb] * T::rowBytes + kk * 32 + h * 16);
        oreg[qb][kk] = buffer_load16(dr, (uint32_t)qrow[qb] * T::rowBytes + kk * 32 + h * 16);
        orow[qb][kk] = buffer_load16(orr, (uint32_t)qrow[qb] * T::rowBytes + kk * 32 + h * 16);
      }
      const bool ok = qrow[qb] < N;
      lse2[qb] = ok ? a.lse[(int64_t)bh * N + qrow[qb]] * kLog2e : 0.f;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float part = 0.f;
#pragma unroll
      for (int kk = 0; kk < kSd; ++kk) part += dot8<FP16>(oreg[qb][kk], orow[qb][kk]);
      dlt[qb] = part + other_half(part);
      if (h == 0 && qrow[qb] < N) a.delta[(int64_t)bh * N + qrow[qb]] = dlt[qb];
    }
    // the B operands move into the accumulation registers here, before the first
    // product reads them (the statement fixes where the copies happen)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < kSd; ++kk) asm volatile("" : "+a"(qreg[qb][kk]), "+a"(oreg[qb][kk]));
  }
  const float c = a.scale_log2;
  wait_vmcnt<0>();
  __syncthreads();

  int k_off[kSd];
#pragma unroll
  for (int kk = 0; kk < kSd; ++kk) k_off[kk] = T::row_offset(l32, h, kk);
  int t_off[2][D / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) t_off[half][db] = T::tr_offset(lane, half, db);

  // dQ^T accumulators (one lane per query), zeroed in the accumulation registers
  // before the first product
  f32x16 dq[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      dq[qb][db] = f32x16{};
      asm volatile("" : "+a"(dq[qb][db]));
    }

  auto stage = [&](int j) -> const char* { return smem + (j % kDqStages) * kStage; };
  // the last key a query row of block qb may see (causal), or the last key
  const int lim0 = CAUSAL ? min(qrow[0], N - 1) : N - 1;
  const int lim1 = CAUSAL ? min(qrow[1], N - 1) : N - 1;

  // Softmax item i of block qb of sub-tile j in x: items 0-7 and 9-16 are elements
  // 0-7 and 8-15 (key 8 g + 4 h + r of the sub-tile for element 4 g + r): P =
  // exp2(S scale log2 e - L log2 e), zero for keys past the row's last (MASK), and
  // dS = P (dP - D) in place; items 8 and 17 pack dS of elements 0-7 (8-15) into the
  // B operand of k-step 0 (1). lim = last visible key - first key of the sub-tile -
  // 4 h: element 4 g + r is masked when 8 g + r > lim.
  auto item = [&](auto mask, DqSub& x, int qb, int i, int lim) {
    if (i == 8 || i == 17) {
      x.dsb[qb][i / 17] = pack_b1<FP16>(x.dp[qb], i / 17);
    } else {
      const int e = i < 8 ? i : i - 1, g = e >> 2, r = e & 3;
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x.s[qb][e], c, -lse2[qb]));
      if constexpr (decltype(mask)::value) p = (8 * g + r > lim) ? 0.f : p;
      x.dp[qb][e] = p * (x.dp[qb][e] - dlt[qb]);
    }
  };
  // slot after which item i runs in a phase of `slots` products, from product
  // `first` on: phase A's items (a sub-tile finished a phase earlier) start after
  // two products; phase B's read block 0's products, the last of which ends a few
  // products before phase A does, so they start after four
  auto item_slot = [](int i, int slots, int first) { return first + (i * (slots - first)) / kDqItems; };

  // Phase A(j): S^T and dP^T of sub-tile j into cur (MFMA) | items of block 1 of
  // sub-tile j - 1 in prev (VALU). Product m: k-step m / 4; m % 4 = S^T of block 0,
  // of block 1, dP^T of block 0, of block 1. The K row read of a k-step serves its
  // two S^T products, the V row read its two dP^T products.
  constexpr int kLookRA = 3;  // operand reads issued this many reads ahead
  auto phase_a = [&](auto mfma, auto valu, auto mask, int j, DqSub& cur, DqSub& prev) {
    constexpr bool kM = decltype(mfma)::value, kV = decltype(valu)::value;
    const char* kt = stage(j);
    const char* vt = kt + T::bytes;
    u32x4 opa[kLookRA + 1];
    auto rd = [&](int r) {  // read r: k-step r / 2, K (even) or V (odd)
      opa[r % (kLookRA + 1)] = lds_read16(((r & 1) ? vt : kt) + k_off[r >> 1]);
    };
    if constexpr (kM) {
#pragma unroll
      for (int r = 0; r < kLookRA; ++r) rd(r);
    }
    const int lim = (kV ? lim1 : 0) - (j - 1) * kSub - 4 * h;
#pragma unroll
    for (int m = 0; m < kSlotsA; ++m) {
      if constexpr (kM) {
        if ((m & 1) == 0 && m / 2 + kLookRA < 2 * kSd) rd(m / 2 + kLookRA);
        __builtin_amdgcn_sched_barrier(0);
        const int kk = m >> 2, qb = m & 1;
        const u32x4 op = opa[(m >> 1) % (kLookRA + 1)];
        if (m & 2) {
          if (kk == 0) cur.dp[qb] = mfma32_va0<FP16>(op, oreg[qb][0]);
          else mfma32_va<FP16>(op, oreg[qb][kk], cur.dp[qb]);
        } else {
          if (kk == 0) cur.s[qb] = mfma32_va0<FP16>(op, qreg[qb][0]);
          else mfma32_va<FP16>(op, qreg[qb][kk], cur.s[qb]);
        }
      }
      if constexpr (kV) {
#pragma unroll
        for (int i = 0; i < kDqItems; ++i)
          if (kM ? item_slot(i, kSlotsA, 2) == m : m == 0) item(mask, prev, 1, i, lim);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Phase B(j): dQ^T of sub-tile j - 1 from prev (MFMA) | items of block 0 of
  // sub-tile j in cur (VALU) | the loads of sub-tile j + 2. Product m: operand pair
  // m / 2 (k-step t, d block db) read through the transposing read, serving
  // block m % 2.
  constexpr int kLookRB = 2;  // transposing read pairs issued this many pairs ahead
  auto phase_b = [&](auto mfma, auto valu, auto mask, int j, DqSub& cur, DqSub& prev, bool loads) {
    constexpr bool kM = decltype(mfma)::value, kV = decltype(valu)::value;
    const char* kp = stage(j - 1);
    u32x2 lo[kLookRB + 1], hi[kLookRB + 1];
    auto rd = [&](int s) {
      const int t = s / (D / 32), db = s % (D / 32), sl = s % (kLookRB + 1);
      lo[sl] = lds_read_tr16(kp + t_off[0][db] + 16 * t * T::rowBytes);
      hi[sl] = lds_read_tr16(kp + t_off[1][db] + 16 * t * T::rowBytes);
    };
    if constexpr (kM) {
#pragma unroll
      for (int s = 0; s < kLookRB; ++s) rd(s);
    }
    const int lim = (kV ? lim0 : 0) - j * kSub - 4 * h;
    const SubSrc ss = sub_src(j + 2);
#pragma unroll
    for (int m = 0; m < kSlotsB; ++m) {
      if constexpr (kM) {
        if ((m & 1) == 0 && m / 2 + kLookRB < kSlotsB / 2) rd(m / 2 + kLookRB);
        __builtin_amdgcn_sched_barrier(0);
        const int s = m >> 1, t = s / (D / 32), db = s % (D / 32), sl = s % (kLookRB + 1), qb = m & 1;
        mfma32_aa<FP16>(u32x4{lo[sl][0], lo[sl][1], hi[sl][0], hi[sl][1]}, prev.dsb[qb][t], dq[qb][db]);
      }
      if (loads && m < kLoads) issue_load(ss, m);
      if constexpr (kV) {
#pragma unroll
        for (int i = 0; i < kDqItems; ++i)
          if (kM ? item_slot(i, kSlotsB, 4) == m : m == 0) item(mask, cur, 0, i, lim);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using Y_ = std::true_type;
  using N_ = std::false_type;
  auto sub_end = [&]() {
    wait_vmcnt<kLoads>();
    __syncthreads();
  };
  auto trip = [&](auto mask, int j, DqSub& cur, DqSub& prev) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) asm volatile("" : "+a"(dq[qb][db]));
    phase_a(Y_{}, Y_{}, mask, j, cur, prev);
    phase_b(Y_{}, Y_{}, mask, j, cur, prev, true);
    sub_end();
  };
  // the last sub-tile (in x): its block-1 items, then its dQ^T products
  auto finish = [&](int j, DqSub& x) {
    wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends
    mfma_wait(x.s[1], x.dp[1]);
    phase_a(N_{}, Y_{}, Y_{}, j + 1, x, x);
    phase_b(Y_{}, N_{}, Y_{}, j + 1, x, x, false);
  };

  DqSub X, Y;
  // sub-tile 0: its products, then its block-0 items with nothing to overlap
  phase_a(Y_{}, N_{}, N_{}, 0, X, Y);
  mfma_wait(X.s[0], X.dp[0]);
  phase_b(N_{}, Y_{}, Y_{}, 0, X, Y, true);
  sub_end();
  // Trips in pairs (sub-tiles j in Y, j + 1 in X), at least one pair, so that the
  // last sub-tile is always in X; sub-tiles past the end are masked. A pair whose
  // items (sub-tiles 2 p .. 2 p + 2) all precede m0 needs no mask.
  const int pairs = max(1, n_sub >> 1);
  const int p_u = min(pairs, max(0, (m0 - 1) / 2));
  int p = 0;
  for (; p < p_u; ++p) {
    trip(N_{}, 2 * p + 1, Y, X);
    trip(N_{}, 2 * p + 2, X, Y);
  }
  for (; p < pairs; ++p) {
    trip(Y_{}, 2 * p + 1, Y, X);
    trip(Y_{}, 2 * p + 2, X, Y);
  }
  finish(2 * pairs, X);

  mfma_drain_a<D / 32>(dq[0], dq[1]);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
    if (qrow[qb] < N)
      store_rows<FP16, D>(reinterpret_cast<uint16_t*>(a.dq) + head + (int64_t)qrow[qb] * D, dq[qb], a.scale, h);
}

// ------------------------------------------------------------------------------
// 2. dK, dV: 4 waves x 32 keys, query tiles of 64 (Q, dO, L, D) streamed through LDS.
//
// One wave per SIMD, so nothing but the wave's own instruction order overlaps its
// matrix work with its VALU work. The loop is software-pipelined over tiles: the
// products of tile j (S and dP) and those of tile j - 1 (dV and dK) each run with
// half of tile j's or tile j - 1's softmax work (P, dS and their 16-bit operands)
// spread between them, one element or one packed operand after every product or
// two. Per tile j the wave runs
//   phase A(j): S and dP of tile j          | P, dS of tile j - 1, query block 1
//   phase B(j): dV and dK of tile j - 1     | P, dS of tile j, query block 0
// so that every VALU item reads products finished a phase earlier, and the LDS
// ring holds tiles j - 1 (read by the dV/dK products), j, j + 1 and j + 2 (in
// flight). Two register sets of per-tile values alternate between consecutive
// tiles (the loop runs two tiles per trip), which keeps loop-carried values in
// place without copies.
constexpr int kKvWaves = 4;
constexpr int kKvRows = 32 * kKvWaves;
constexpr int kLookA = 4;  // row-operand reads of the S and dP products issued this many products ahead
constexpr int kLookB = 3;  // transposing reads of the dV and dK products issued this many products ahead
constexpr int kItems = 20;  // softmax items of one 32-row query block (16 elements, 4 packed operands)

// Per-tile values of one wave: S and dP of the tile's two 32-row query blocks (P
// and dS replace them in place), and P and dS rounded to 16 bits as the B operands
// of the four 16-row k-steps of the dV and dK products.
struct KvTile {
  f32x16 s[2], dp[2];
  u32x4 pb[4], dsb[4];
};

template <bool FP16, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kKvWaves, 1) void bwd_dkdv(BwdArgs a) {
  using T = Tile<D>;
  constexpr int kStat = kTile * 4;                        // L or D of the tile's rows
  constexpr int kStage = 2 * T::bytes + 2 * kStat;        // Q, dO, L, D
  constexpr int kSd = D / 16;                             // k-steps of one block's S (and dP) product
  constexpr int kSlots = 4 * kSd;                         // products per phase (S/dP or dV/dK)
  static_assert(kSlots == 8 * (D / 32), "both phases hold the same number of products");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // workgroup -> (slice, key block): key blocks in increasing order, so under a
  // causal mask the heaviest blocks (most query tiles) start first
  const int bid = blockIdx.x;
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

  // query tiles that can see this workgroup's keys (the first one starts at k0,
  // a multiple of the tile height, under a causal mask)
  const int tiles_all = (N + kTile - 1) / kTile;
  const int t_first = CAUSAL ? k0 / kTile : 0;
  const int n_tiles = tiles_all - t_first;

  // Tile loads: this wave's share of Q and dO (1 KiB blocks) and the tile's L and D
  // rows (every wave loads them, the same bytes to the same place, so that all
  // waves issue the same number of loads per tile). A tile past the last one is
  // "loaded" through an empty buffer range (zeros into a free stage), which keeps
  // the count of loads in flight the same on every trip.
  uint32_t ld_off[T::blocks / kKvWaves];
#pragma unroll
  for (int i = 0; i < T::blocks / kKvWaves; ++i) ld_off[i] = T::src_offset(wave + kKvWaves * i, lane);
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(1024u * (uint32_t)wave);
  struct TileSrc {
    __amdgpu_buffer_rsrc_t q, o, l, d;
    uint32_t st;  // LDS byte address of the tile's stage
  };
  auto tile_src = [&](int j) {
    const int t = t_first + j;
    const bool in = t < tiles_all;
    const uint32_t skip = (uint32_t)t * kTile * T::rowBytes;
    const uint32_t sskip = (uint32_t)t * kTile * 4;
    const uint32_t rows = in ? head_bytes - skip : 0u, stats = in ? (uint32_t)N * 4 - sskip : 0u;
    return TileSrc{buffer_rsrc(qg + (int64_t)t * kTile * D, rows), buffer_rsrc(og + (int64_t)t * kTile * D, rows),
                   buffer_rsrc(lg + t * kTile, stats), buffer_rsrc(dg + t * kTile, stats),
                   (uint32_t)(uintptr_t)smem + (uint32_t)((j % kStages) * kStage)};
  };
  constexpr int kLoads = 2 * T::blocks / kKvWaves + 2;
  static_assert(kLoads <= kSlots, "one tile load per dV/dK product at most");
  auto issue_load = [&](const TileSrc& ts, int n) {
    if (n < kLoads - 2) {
      const int i = n >> 1;
      const uint32_t dst = ts.st + lds_w + 1024u * kKvWaves * i + ((n & 1) ? (uint32_t)T::bytes : 0u);
      buffer_load16_lds_s((n & 1) ? ts.o : ts.q, ld_off[i], dst);
    } else if (n == kLoads - 2) {
      buffer_load4_lds_s(ts.l, lane * 4, ts.st + 2 * T::bytes);
    } else {
      buffer_load4_lds_s(ts.d, lane * 4, ts.st + 2 * T::bytes + kStat);
    }
  };
  auto issue_tile = [&](int j) {
    const TileSrc ts = tile_src(j);
#pragma unroll
    for (int n = 0; n < kLoads; ++n) issue_load(ts, n);
  };

  issue_tile(0);
  issue_tile(1);
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
  const float inv_scale = 1.f / a.scale;
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

  // dK and dV accumulators, zeroed in the accumulation registers before the first
  // product (the statement fixes where the zeroing happens)
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
    asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
  }

  auto stage = [&](int j) -> const char* { return smem + (j % kStages) * kStage; };

  // Softmax item i (0 .. kItems - 1) of query block b of tile j, held in x: items
  // 0-7 and 10-17 are the elements 0-7 and 8-15 (rows 32 b + 8 g + 4 h + r for
  // element 4 g + r): P = exp2(S scale log2 e - L log2 e), zero where the query
  // precedes the key (MASK), and dS = P (dP - D) in place; items 8, 9 (18, 19) pack
  // P and dS of elements 0-7 (8-15) into the B operand of k-step 2 b (2 b + 1).
  // lim = key - (first query row of the tile) - 4 h: element 4 g + r is masked when
  // 32 b + 8 g + r < lim. A row's L / scale and D come from the block's compact
  // registers cl, cd (lane k of each 16-lane row holds row 16 q + k + 4 h of the
  // block, q = g / 2) by a broadcast of lane 8 (g % 2) + r into the subtraction
  // (S - L / scale) scale log2 e, whose operands no VALU instruction has just written.
  auto item = [&](auto mask, KvTile& x, int b, auto ic, const float (&cl)[2], const float (&cd)[2], int lim) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i == 8 || i == 18) {
      x.pb[2 * b + i / 18] = pack_b<FP16>(x.s, 2 * b + i / 18);
    } else if constexpr (i == 9 || i == 19) {
      x.dsb[2 * b + i / 19] = pack_b<FP16>(x.dp, 2 * b + i / 19);
    } else {
      constexpr int e = i < 8 ? i : i - 2, g = e >> 2, r = e & 3, n = 8 * (g & 1) + r;
      float p = __builtin_amdgcn_exp2f((x.s[b][e] - row_bcast<n>(cl[g >> 1])) * c);
      if constexpr (decltype(mask)::value) p = (32 * b + 8 * g + r < lim) ? 0.f : p;
      x.s[b][e] = p;
      x.dp[b][e] = p * (x.dp[b][e] - row_bcast<n>(cd[g >> 1]));
    }
  };
  // slot (product index within a phase) after which item i runs: the items start a
  // few products into the phase (their L and D reads are then in) and spread evenly
  auto item_slot = [](int i) constexpr {
    constexpr int first = kSlots >= 32 ? 2 : 1;
    return first + (i * (kSlots - first)) / kItems;
  };
  // the block's compact L / scale and D registers (see item); the row index is
  // clamped to the tile (the lanes past row 63 feed no element)
  auto read_stats = [&](const char* st, int b, float (&cl)[2], float (&cd)[2]) {
    const float* lt = reinterpret_cast<const float*>(st + 2 * T::bytes);
    const float* dt = reinterpret_cast<const float*>(st + 2 * T::bytes + kStat);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = min(32 * b + 16 * q + (lane & 15) + 4 * h, kTile - 1);
      cl[q] = lt[row] * inv_scale;
      cd[q] = dt[row];
    }
  };

  // Phase A(j): S and dP of tile j into cur (MFMA) | items of query block 1 of tile
  // j - 1 in prev (VALU).
  auto phase_a = [&](auto mfma, auto valu, auto mask, int j, KvTile& cur, KvTile& prev) {
    constexpr bool kM = decltype(mfma)::value, kV = decltype(valu)::value;
    const char* qt = stage(j);
    const char* ot = qt + T::bytes;
    u32x4 opa[kLookA + 1];
    auto rd = [&](int m) {
      const int b = m / (2 * kSd), kk = (m >> 1) % kSd;
      opa[m % (kLookA + 1)] = lds_read16(((m & 1) ? ot : qt) + r_off[kk] + b * 32 * T::rowBytes);
    };
    if constexpr (kM) {
#pragma unroll
      for (int m = 0; m < kLookA; ++m) rd(m);
    }
    float l4[2], d4[2];
    int lim = 0;
    if constexpr (kV) {
      read_stats(stage(j - 1), 1, l4, d4);
      lim = key - (t_first + j - 1) * kTile - 4 * h;
    }
    static_for<kSlots>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (kM) {
        if constexpr (m + kLookA < kSlots) rd(m + kLookA);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int b = m / (2 * kSd), kk = (m >> 1) % kSd;
        const u32x4 op = opa[m % (kLookA + 1)];
        if constexpr (m & 1) {
          if constexpr (kk == 0) cur.dp[b] = mfma32_va0<FP16>(op, vreg[0]);
          else mfma32_va<FP16>(op, vreg[kk], cur.dp[b]);
        } else {
          if constexpr (kk == 0) cur.s[b] = mfma32_va0<FP16>(op, kreg[0]);
          else mfma32_va<FP16>(op, kreg[kk], cur.s[b]);
        }
      }
      if constexpr (kV) {
        static_for<kItems>([&](auto ic) {
          if constexpr (kM ? item_slot(decltype(ic)::value) == m : m == 0) item(mask, prev, 1, ic, l4, d4, lim);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Phase B(j): dV and dK of tile j - 1 from prev (MFMA) | items of query block 0
  // of tile j in cur (VALU) | the loads of tile j + 2.
  auto phase_b = [&](auto mfma, auto valu, auto mask, int j, KvTile& cur, KvTile& prev, bool loads) {
    constexpr bool kM = decltype(mfma)::value, kV = decltype(valu)::value;
    const char* qp = stage(j - 1);
    const char* op = qp + T::bytes;
    u32x2 lo[kLookB + 1], hi[kLookB + 1];
    auto rd = [&](int m) {
      const int s = m >> 1, t = s / (D / 32), db = s % (D / 32), sl = m % (kLookB + 1);
      const char* src = (m & 1) ? qp : op;
      lo[sl] = lds_read_tr16(src + t_off[0][db] + 16 * t * T::rowBytes);
      hi[sl] = lds_read_tr16(src + t_off[1][db] + 16 * t * T::rowBytes);
    };
    if constexpr (kM) {
#pragma unroll
      for (int m = 0; m < kLookB; ++m) rd(m);
    }
    float l4[2], d4[2];
    int lim = 0;
    if constexpr (kV) {
      read_stats(stage(j), 0, l4, d4);
      lim = key - (t_first + j) * kTile - 4 * h;
    }
    const TileSrc ts = tile_src(j + 2);
    static_for<kSlots>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (kM) {
        if constexpr (m + kLookB < kSlots) rd(m + kLookB);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int s = m >> 1, t = s / (D / 32), db = s % (D / 32), sl = m % (kLookB + 1);
        const u32x4 opnd = u32x4{lo[sl][0], lo[sl][1], hi[sl][0], hi[sl][1]};
        if constexpr (m & 1) mfma32_aa<FP16>(opnd, prev.dsb[t], dk[db]);
        else mfma32_aa<FP16>(opnd, prev.pb[t], dv[db]);
      }
      if constexpr (m < kLoads) {
        if (loads) issue_load(ts, m);
      }
      if constexpr (kV) {
        static_for<kItems>([&](auto ic) {
          if constexpr (kM ? item_slot(decltype(ic)::value) == m : m == 0) item(mask, cur, 0, ic, l4, d4, lim);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  using Y_ = std::true_type;
  using N_ = std::false_type;
  using MaskT = std::integral_constant<bool, CAUSAL>;
  auto tile_end = [&]() {
    wait_vmcnt<kLoads>();
    __syncthreads();
  };
  // one pipelined trip: tile j into cur, tile j - 1 (in prev) finished
  auto trip = [&](auto mask_a, auto mask_b, int j, KvTile& cur, KvTile& prev) {
    // dK and dV stay in the accumulation registers across trips
#pragma unroll
    for (int db = 0; db < D / 32; ++db) asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
    phase_a(Y_{}, Y_{}, mask_a, j, cur, prev);
    phase_b(Y_{}, Y_{}, mask_b, j, cur, prev, true);
    tile_end();
  };
  // the last tile (in x): its block-1 items, then its dV and dK products
  auto finish = [&](int j, KvTile& x) {
    // no load may still be writing LDS when the workgroup ends
    wait_vmcnt<0>();
    mfma_wait(x.s[1], x.dp[1]);
    phase_a(N_{}, Y_{}, MaskT{}, j + 1, x, x);
    phase_b(Y_{}, N_{}, MaskT{}, j + 1, x, x, false);
  };

  KvTile X, Y;
  // tile 0: its S and dP products, then its block-0 items with nothing to overlap
  phase_a(Y_{}, N_{}, N_{}, 0, X, Y);
  mfma_wait(X.s[0], X.dp[0]);
  phase_b(N_{}, Y_{}, MaskT{}, 0, X, Y, true);
  tile_end();
  // Trips run in pairs (tiles j in Y, j + 1 in X), at least one pair, so that the
  // last tile is always in X and the code has a single path: tiles past the end
  // (one for an even tile count, two for a single tile) read Q, dO, L and D as
  // zeros (P = 1, dS = 0, dO = 0: they add exactly nothing). Under a causal mask the
  // items of tiles 0 and 1 (the first pair) need the mask; from tile 2 on every
  // query of a tile follows every key of the block.
  const int pairs = max(1, n_tiles >> 1);
  trip(MaskT{}, MaskT{}, 1, Y, X);
  trip(MaskT{}, N_{}, 2, X, Y);
  for (int p = 1; p < pairs; ++p) {
    trip(N_{}, N_{}, 2 * p + 1, Y, X);
    trip(N_{}, N_{}, 2 * p + 2, X, Y);
  }
  finish(2 * pairs, X);

  mfma_drain_a<D / 32>(dk, dv);
  if (key < N) {
    store_rows<FP16, D>(reinterpret_cast<uint16_t*>(a.dk) + head + (int64_t)key * D, dk, a.scale, h);
    store_rows<FP16, D>(reinterpret_cast<uint16_t*>(a.dv) + head + (int64_t)key * D, dv, 1.0f, h);
  }
}

template <bool FP16, int D, bool CAUSAL>
hipError_t launch_all(const BwdArgs& a, hipStream_t stream) {
  // D = rowsum(dO ∘ O) is formed by bwd_dq (each workgroup for its own rows) and
  // stored for bwd_dkdv, which runs after it on the same stream
  const int q_tiles = (a.n + kDqRows - 1) / kDqRows;
  const int k_blocks = (a.n + kKvRows - 1) / kKvRows;
  launch_log("bwd_dq<%s, %d, %s> grid %d x %d; bwd_dkdv<%s, %d, %s> grid %d x %d", dtype_name(FP16), D,
             CAUSAL ? "causal" : "full", a.bh * q_tiles, 64 * kDqWaves, dtype_name(FP16), D,
             CAUSAL ? "causal" : "full", a.bh * k_blocks, 64 * kKvWaves);
  hipLaunchKernelGGL((bwd_dq<FP16, D, CAUSAL>), dim3(a.bh * q_tiles), dim3(64 * kDqWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
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
