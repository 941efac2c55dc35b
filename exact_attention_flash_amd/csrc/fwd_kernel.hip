// Exact attention forward for gfx950 (MI355X): bf16/fp16 in, fp32 accumulate.
//
// Method ("FlashAttention: optimize data movement before counting FLOPs",
// section 02): per key tile with scores s and values V, keep the running row
// maximum m, denominator l and unnormalised numerator u,
//     m' = max(m, max s),  l' = e^(m-m') l + sum e^(s-m'),  u' = e^(m-m') u + sum e^(s-m') V,
// and finish with O = u / l and LSE = m + ln l ("FlashAttention: IO-Aware Tiling,
// Online Softmax Mathematics, Memory Hierarchy Dynamics, and Kernel Evolution",
// sections on FlashAttention-2 and on backward recomputation). Query tiles sit on
// the grid, key/value tiles stream through LDS, the accumulator stays in registers
// and is divided once at the end.
//
// Persistent workgroups (one per compute unit) of 8 wave64s walk a list of work
// items, each 256 query rows of one (batch, head); keys stream in 64-key tiles.
//  * Each wave owns 32 query rows and computes S^T = K Q^T and O^T = V^T P^T with
//    v_mfma_f32_32x32x16 (bf16 or fp16 in, fp32 out). In the 32x32 accumulator
//    layout a lane holds one query and 16 keys, so row max and row sum are in-lane
//    plus one v_permlane32_swap, and the S^T accumulator rounded to 16 bits is the
//    B operand of the P V product without leaving registers. V^T is read from the
//    row-major V tile with ds_read_b64_tr_b16.
//  * Ping-pong: waves 0-3 (group A) and 4-7 (group B) land on the four SIMDs in
//    pairs. In every iteration group A first issues its matrix work (S of tile i
//    and P V of tile i-1) and then runs the softmax of tile i, while group B runs
//    the softmax of tile i-1 first and then issues its matrix work, so the MFMA
//    and VALU streams of the two waves sharing a SIMD overlap. One barrier per
//    iteration publishes the next K/V tile.
//  * K/V tiles are loaded straight into LDS with buffer_load ... lds (no staging
//    registers; the LDS address in M0 formed by the scalar unit from a per-wave
//    offset) into a 3-stage ring, one tile ahead of use; the tile stream runs
//    across work items, so the next item's first tile is in flight while the
//    current item finishes. Q rows of an item take the same path into a fourth
//    LDS region one item ahead (160 KiB of LDS in all). Rows past the end of the
//    sequence read as zeros through the buffer descriptor's range. Tiles are
//    stored unpadded with 16-byte chunks XOR-swizzled by row, chosen so that the
//    K and Q reads (16 lanes, 16 rows) and the transposing V reads (32 lanes, 4
//    rows) hit every LDS bank once.
//  * The pair of waves on SIMD k owns row blocks k and 7-k of the workgroup's eight
//    blocks of 32 rows, so under a causal mask every SIMD has the same amount of
//    work on the diagonal tiles and late diagonal tiles cost half an iteration.
//  * Exponentials use exp2 with scale*log2(e) folded into one FMA per score.
//  * Layout: q, k, v and o are addressed through (batch, head, row) strides with
//    the head dimension contiguous. A head dimension d below the instance's D
//    (64, 128 or 256) is masked the way "6.1 FlashAttention V1 in detail", §8.3
//    masks BLOCK_D > D: chunks past d are loaded from an offset outside the buffer
//    descriptor's range, which writes zeros into LDS, so they add nothing to the
//    scores, and output columns past d are not stored.
//  * The 256-wide instance forms the scores over all 256 columns but P V for one
//    128-column half of V and O per launch (the host launches it once per half),
//    and loads Q straight into registers, since 256 wide Q rows do not fit in LDS
//    beside the K/V ring.
//  * Causal: tiles past the workgroup's last row are never loaded; waves skip the
//    math of tiles entirely after their rows; only tiles on the diagonal or at the
//    end of the sequence evaluate the mask.
//  * Item order: heaviest causal query tiles first, dealt to the workgroups in
//    snake order so that every workgroup gets the same causal work; all query
//    tiles of one (batch, head) on one XCD so K/V tiles are shared through its L2.
//  * Key split (shapes with fewer work items than compute units): the key tiles a
//    query tile visits are cut into S contiguous ranges, each its own work item.
//    An item's rows end with the range's own (m, l, u); it stores u / l and
//    m + ln l in fp32, and merge_splits combines the S partials of a row with the
//    two-block rule of the IO-aware tiling page ("Online Softmax Mathematics"):
//    m = max m_k, l = sum e^(m_k - m) l_k, O = sum (l_k e^(m_k - m) / l) O_k,
//    written with the identity l_k e^(m_k - m) / l = e^(LSE_k - LSE). A causal
//    row that ends before its range starts has l = 0 there and stores O = 0 and
//    LSE = -inf (weight zero in the merge).
//
// Reference maximum. The rescaling identity of "6.1 FlashAttention V1 in detail",
// §3.3 holds for any per-row reference r: with p = 2^(s' - r) (s' the score in
// log2 units), u / l and r + log2 l do not depend on r, as long as no p
// overflows. fp16 keeps r equal to the running row maximum (p <= 1). bf16 keeps
// the reference of the previous tile and skips the row maximum: the tile's
// probabilities are computed against it directly, and only if there is no
// reference yet (first tile) or some partial row sum exceeds 2^15 is the tile
// redone with the exact running maximum. bf16 P carries 8 bits at any magnitude, so
// probabilities up to 2^15 lose nothing, and the bound keeps the fp32 accumulator
// finite for N * max|v| < 2^113 (the value range the interface states).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "fwd_kernel.h"
#include "gfx950_ops.h"
#include "launch_log.h"

namespace fa {
namespace pp {

using namespace ::fa::ops;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kStages = 3;        // LDS ring depth (tiles)
constexpr int kAhead = kStages - 2;  // tiles in flight ahead of use

// partial row sums above this send a bf16 tile back through the exact maximum
constexpr float kBig = 0x1p15f;

// load offset of a masked head-dimension chunk: past every descriptor's range (the
// host keeps slice extents below 2^31 bytes), so the load writes zeros to LDS
constexpr uint32_t kMaskedOffset = 0x80000000u;

// Instance width D: the head dimension of Q and K (the scores). D = 64 and 128 cover
// V and O whole; the wide instance D = 256 covers one 128-column half of V and O per
// launch (the host launches it once per half, each launch recomputing the scores),
// and takes Q straight into registers, since a Q region of 256 wide rows would not
// fit in LDS beside the ring.
template <int D>
struct Geo {
  static constexpr bool wide = D > 128;
  static constexpr int DV = wide ? 128 : D;             // columns of V and O per launch
  static constexpr int rowBytes = D * 2;                // a K (and Q) row
  static constexpr int chunksPerRow = D / 8;            // 16-byte chunks of a K row
  static constexpr int vRowBytes = DV * 2;              // a V row (its half, for the wide instance)
  static constexpr int vChunksPerRow = DV / 8;
  static constexpr int tileBytes = kBN * rowBytes;      // K tile
  static constexpr int vTileBytes = kBN * vRowBytes;    // V tile
  static constexpr int stageBytes = tileBytes + vTileBytes;  // K then V
  static constexpr int qBytes = wide ? 0 : kBM * rowBytes;   // the Q rows of one item (LDS)
  static constexpr int blocksPerTile = tileBytes / 1024;     // 1 KiB per wave-instruction
  static constexpr int vBlocksPerTile = vTileBytes / 1024;
  static constexpr int qLoadsPerWave = qBytes / 1024 / kWaves;  // Q instructions per wave per item
  static_assert(blocksPerTile % kWaves == 0 && vBlocksPerTile % kWaves == 0,
                "tile must split into whole 1 KiB blocks per wave");
  // The XOR swizzle of a 16-byte chunk acts on the low four bits of its index; a
  // 256-wide K row is two 128-wide halves with the same pattern.
  __device__ static __forceinline__ int swz(int row) { return chunk_swizzle<(D > 128 ? 128 : D)>(row); }
  __device__ static __forceinline__ int vswz(int row) { return chunk_swizzle<DV>(row); }
};

// The kernel's argument block, read from the kernel-argument segment where a field
// is used rather than kept in scalar registers for the whole kernel: the layout
// fields read through it are needed only when a work item starts or ends, and the
// scalar registers are needed by the tile loop.
using KArgs = const __attribute__((address_space(4))) FwdArgs;
__device__ __forceinline__ KArgs* kargs() {
  KArgs* p = (KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  return p;
}

template <bool FP16, int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void fwd_pingpong(FwdArgs a) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * G::stageBytes + G::qBytes];
  char* const qsm = smem + kStages * G::stageBytes;  // Q rows of the current item

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // ---- persistent schedule ----
  // Work items are (slice, query tile) pairs. With xcd_grouped, the workgroups of
  // XCD x (blockIdx % 8 == x) own slices [x*hpx, (x+1)*hpx), so all query tiles of
  // a slice share K/V through one L2. Workgroup k of a group of size G takes the
  // items k, 2G-1-k, 2G+k, 4G-1-k, ... of its group's list (snake order). The list
  // is slice-major when a.slice_major is set (no key split): the items a group's
  // workgroups run at the same time cover one or two slices, whose K/V then stay in
  // the XCD's L2, and the snake pairs causal ranks i and q_tiles - 1 - i; the host
  // sets it only when those pairs fill whole rounds (or without a mask). Otherwise
  // the list is rank-major (every slice's rank 0, then rank 1, ...): the heaviest
  // causal query tiles first, balanced by the snake over whole rounds.
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
  const int splits = SPLIT ? a.splits : 1;
  const int n_items = hpx * a.q_tiles * splits;
  const int N = a.n;
  // slice base (elements) of item slice bh in a tensor with batch/head strides sb, sh
  auto slice_off = [&](int bh, int64_t sb, int64_t sh) {
    const int heads = kargs()->heads;
    return (int64_t)(bh / heads) * sb + (bh % heads) * sh;
  };
  const int tiles_all = (N + kBN - 1) / kBN;
  // r-th item of this workgroup, or -1 past the end of its list
  auto item_index = [&](int r) {
    const int j = r * wg_n + ((r & 1) ? wg_n - 1 - wg_k : wg_k);
    return j < n_items ? j : -1;
  };
  // item j, slice-major: slice j / q_tiles, rank j % q_tiles. Rank-major: slice
  // j % hpx; query-tile rank and key split from j / hpx (the splits of one query
  // tile are adjacent in the list). Causal rank 0 is the last, heaviest query tile.
  const bool slice_major = !SPLIT && a.slice_major != 0;
  auto item_bh = [&](int j) { return bh_base + (slice_major ? j / a.q_tiles : j % hpx); };
  auto item_rank = [&](int j) {
    return slice_major ? j % a.q_tiles : SPLIT ? (j / hpx) / splits : j / hpx;
  };
  auto item_split = [&](int j) { return SPLIT ? (j / hpx) % splits : 0; };
  auto item_q0 = [&](int j) { return (CAUSAL ? (a.q_tiles - 1 - item_rank(j)) : item_rank(j)) * kBM; };
  // key tiles visited by a query tile starting at q0 (causal: up to its last row)
  auto item_tiles = [&](int q0) {
    return CAUSAL ? min(tiles_all, (min(q0 + kBM, N) - 1) / kBN + 1) : tiles_all;
  };
  // key tiles [item_first, item_last) of item j: split s of the query tile's nt
  // tiles is [s nt / S, (s + 1) nt / S), never empty because S <= nt
  auto item_first = [&](int j) { return SPLIT ? item_split(j) * item_tiles(item_q0(j)) / splits : 0; };
  auto item_last = [&](int j) {
    return SPLIT ? (item_split(j) + 1) * item_tiles(item_q0(j)) / splits : item_tiles(item_q0(j));
  };
  // this wave's block of 32 rows: block wave%4 (group A) or 7 - wave%4 (group B)
  const int wave_rows = 32 * (grp == 0 ? (wave & 3) : 7 - (wave & 3));

  // ---- direct-to-LDS tile loads: this wave fills blocks wave + 8*i of K and of V ----
  // lane `lane` of block b lands at chunk position 64*b + lane = (row, physical chunk);
  // it fetches the logical chunk physical ^ swz(row) of that row.
  // (V: of the launch's columns v_col0 .. v_col0 + DV - 1)
  uint32_t k_ld[G::blocksPerTile / kWaves], v_ld[G::vBlocksPerTile / kWaves];
#pragma unroll
  for (int i = 0; i < G::blocksPerTile / kWaves; ++i) {
    const int p = 64 * (wave + kWaves * i) + lane;
    const int row = p / G::chunksPerRow, logical = (p % G::chunksPerRow) ^ G::swz(row);
    const bool live = logical * 8 < a.d_real;
    k_ld[i] = live ? (uint32_t)row * (uint32_t)(2 * a.k_sn) + (uint32_t)(logical * 16) : kMaskedOffset;
  }
#pragma unroll
  for (int i = 0; i < G::vBlocksPerTile / kWaves; ++i) {
    const int p = 64 * (wave + kWaves * i) + lane;
    const int row = p / G::vChunksPerRow, col = (G::wide ? a.v_col0 : 0) + 8 * ((p % G::vChunksPerRow) ^ G::vswz(row));
    const bool live = col < a.d_real;
    v_ld[i] = live ? (uint32_t)row * (uint32_t)(2 * a.v_sn) + (uint32_t)(col * 2) : kMaskedOffset;
  }
  // LDS byte address of this wave's first 1 KiB block relative to a region, in a
  // scalar register: the load addresses (M0) are then formed by the scalar unit
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(1024u * (uint32_t)wave);
  // The workgroup's key tiles form one stream over its items; tile g of the stream
  // lives in ring stage g % kStages. A cursor walks the stream kAhead tiles ahead
  // of the matrix work, so the first tiles of the next item are in flight while the
  // current item finishes.
  // (c_st: byte offset of the ring stage the cursor's tile goes to)
  int c_r = 0, c_j = item_index(0), c_t = 0, c_n = 0, c_st = 0;
  const uint16_t *c_k = nullptr, *c_v = nullptr;
  auto cursor_item = [&]() {
    if (c_j < 0) return;
    KArgs* ka = kargs();
    c_k = reinterpret_cast<const uint16_t*>(ka->k) + slice_off(item_bh(c_j), ka->k_sb, ka->k_sh);
    c_v = reinterpret_cast<const uint16_t*>(ka->v) + slice_off(item_bh(c_j), ka->v_sb, ka->v_sh);
    c_n = item_last(c_j);
    c_t = item_first(c_j);
  };
  cursor_item();
  // issue the cursor's tile and advance; false once the stream is exhausted
  auto issue_next = [&]() {
    if (c_j < 0) return false;
    // byte offsets of the tile in its slice (below the 32-bit extents)
    const uint32_t k0 = (uint32_t)c_t * (uint32_t)(kBN * 2 * a.k_sn);
    const uint32_t v0 = (uint32_t)c_t * (uint32_t)(kBN * 2 * a.v_sn);
    const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(reinterpret_cast<const char*>(c_k) + k0, a.k_ext - k0);
    const __amdgpu_buffer_rsrc_t vr = uniform_rsrc(reinterpret_cast<const char*>(c_v) + v0, a.v_ext - v0);
    const uint32_t st = (uint32_t)(uintptr_t)smem + (uint32_t)c_st + lds_w;
#pragma unroll
    for (int i = 0; i < G::blocksPerTile / kWaves; ++i) {
      buffer_load16_lds_s(kr, k_ld[i], st + 1024 * kWaves * i);
      if (i < G::vBlocksPerTile / kWaves)
        buffer_load16_lds_s(vr, v_ld[i], st + G::tileBytes + 1024 * kWaves * i);
    }
    c_st = c_st + G::stageBytes == kStages * G::stageBytes ? 0 : c_st + G::stageBytes;
    if (++c_t == c_n) {
      c_j = item_index(++c_r);
      cursor_item();
    }
    return true;
  };
  if (c_j < 0) return;  // no work for this workgroup

  // Q rows of an item go to LDS like K tiles (same chunk swizzle, 256 rows); at the
  // start of the item every lane reads its query's row into the B operands
  // (k-slots d = 16*kk + 8*h + 0..7), and once every wave has done so the next
  // item's Q is loaded while this item runs.
  auto issue_q = [&](int j) {
    const int q0 = item_q0(j);
    KArgs* ka = kargs();
    const int q_sn = ka->q_sn;
    const __amdgpu_buffer_rsrc_t qr =
        uniform_rsrc(reinterpret_cast<const uint16_t*>(ka->q) + slice_off(item_bh(j), ka->q_sb, ka->q_sh) +
                        (int64_t)q0 * q_sn,
                    ka->q_ext - (uint32_t)((int64_t)q0 * q_sn * 2));
    const int d_real = ka->d_real;
    int lw = lane + 64 * wave;
    asm volatile("" : "+v"(lw));  // recomputed per call rather than kept live
#pragma unroll
    for (int i = 0; i < G::qLoadsPerWave; ++i) {
      const int p = lw + 64 * kWaves * i;
      const int row = p / G::chunksPerRow, logical = (p % G::chunksPerRow) ^ G::swz(row);
      const uint32_t off = logical * 8 < d_real
                               ? (uint32_t)row * (uint32_t)(2 * q_sn) + (uint32_t)(logical * 16)
                               : kMaskedOffset;
      buffer_load16_lds_s(qr, off, (uint32_t)(uintptr_t)qsm + lds_w + 1024 * kWaves * i);
    }
  };
  u32x4 qreg[D / 16];
  // wide instance: the wave's Q rows straight from memory into the B operands (rows
  // past N and columns past d read as zeros); issued while the previous item drains
  auto load_q_regs = [&](int j) {
    const int q0 = item_q0(j);
    KArgs* ka = kargs();
    const int q_sn = ka->q_sn;
    const __amdgpu_buffer_rsrc_t qr =
        uniform_rsrc(reinterpret_cast<const uint16_t*>(ka->q) + slice_off(item_bh(j), ka->q_sb, ka->q_sh) +
                        (int64_t)q0 * q_sn,
                    ka->q_ext - (uint32_t)((int64_t)q0 * q_sn * 2));
    const int d_real = ka->d_real;
    const uint32_t rowoff = (uint32_t)(wave_rows + l32) * (uint32_t)(2 * q_sn);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int col = 16 * kk + 8 * h;
      qreg[kk] = buffer_load16(qr, col < d_real ? rowoff + (uint32_t)(2 * col) : kMaskedOffset);
    }
  };
  auto read_q = [&]() {
    int row = wave_rows + l32;
    asm volatile("" : "+v"(row));  // recomputed per call rather than kept live
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qreg[kk] = lds_read16(qsm + row * G::rowBytes + (((2 * kk + h) ^ G::swz(row)) * 16));
  };

  // prologue: the first item's Q and the first kAhead tiles of the stream (the
  // cursor may move past the first item while doing so)
  const int first_j = c_j;
  if constexpr (G::wide) load_q_regs(first_j);
  else issue_q(first_j);
#pragma unroll
  for (int t = 0; t < kAhead; ++t) issue_next();
  bool first = true;

  // ---- per-lane LDS offsets (within a stage) ----
  // K: row l32 (+32 for the second block of keys), logical chunk 2*kk + h
  const int krow_sw = G::swz(l32);
  const int k_lane = l32 * G::rowBytes;
  // V (transposing read): source row 16t + 8*half + 4h + (lane%16)/4, logical chunk
  // 4*db + 2*((lane/16)%2) + (lane%4)/2, byte 8*(lane%2) inside the chunk
  const int vk = (lane & 15) >> 2;
  const int vrow_base = 4 * h + vk;
  int v_lane[2][G::DV / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < G::DV / 32; ++db) {
      const int row = 8 * half + vrow_base;
      const int logical = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      v_lane[half][db] = row * G::vRowBytes + ((logical ^ G::vswz(row)) * 16) + 8 * (lane & 1);
    }

  const float sc = a.scale_log2;
  float m_run;  // reference maximum (log2 units) of this lane's query
  float l_run;  // denominator over this half-wave's keys
  f32x16 acc[G::DV / 32];
  f32x16 s[2] = {f32x16{}, f32x16{}};
  u32x4 pb[4] = {u32x4{}, u32x4{}, u32x4{}, u32x4{}};

  // the current item: its first row, this wave's rows, its key tiles and the
  // stream index of its tile 0
  // (with a key split, tile i of the item is key tile t_base + i)
  int it_r = 0, it_j = first_j;
  int row0 = 0, qrow = 0, n_tiles = 0, g0 = 0, t_base = 0;
  auto key_tile = [&](int t) { return SPLIT ? t_base + t : t; };
  auto active = [&](int t) { return row0 < N && (!CAUSAL || key_tile(t) * kBN <= row0 + 31); };

  // per-lane K offsets: row l32 (the second block of 32 keys adds 32 rows), logical
  // chunk 2*kk + h; in a 256-wide row, chunk 16 + c sits 256 bytes after chunk c
  constexpr int kOffs = D / 16 < 8 ? D / 16 : 8;
  int k_off[kOffs];
#pragma unroll
  for (int kk = 0; kk < kOffs; ++kk) k_off[kk] = k_lane + (((2 * kk + h) ^ krow_sw) * 16);
  auto koff = [&](int kk) { return k_off[kk % kOffs] + (kk / kOffs) * 256; };

  // Matrix phase of tile i: S^T(i) = K_i Q^T (D/8 MFMAs) and u += P(i-1) V(i-1)
  // (DV/8 MFMAs), one P V product after every kRatio S products. Operand reads from
  // LDS are issued kLook steps ahead of their MFMA so that LDS latency hides behind
  // matrix work; the scheduling fences keep the compiler from regrouping reads next
  // to their uses.
  constexpr int kSteps = D / 8;
  constexpr int kRatio = D / G::DV;
#ifdef FA_LOOKAHEAD
  constexpr int kLook = FA_LOOKAHEAD;
#else
  // (measured: 4 at D = 64 is 5% faster than 3; at D = 128, 3 and 4 are within 1%)
  // (the wide instance looks two steps ahead: three would spill)
  constexpr int kLook = D == 64 ? 4 : D > 128 ? 2 : 3;
#endif
  auto mfma_steps = [&](auto do_s_c, auto do_p_c, int i) {
    constexpr bool DO_S = decltype(do_s_c)::value;
    constexpr bool DO_P = decltype(do_p_c)::value;
    const char* kt = smem + ((g0 + i) % kStages) * G::stageBytes;
    const char* vt = smem + ((g0 + i + kStages - 1) % kStages) * G::stageBytes + G::tileBytes;
    u32x4 kop[kLook + 1];
    u32x2 vlo[kLook + 1], vhi[kLook + 1];
    auto issue = [&](int st) {
      if constexpr (DO_S) kop[st % (kLook + 1)] = lds_read16(kt + koff(st >> 1) + (st & 1) * 32 * G::rowBytes);
      if constexpr (DO_P) {
        if (st % kRatio == 0) {
          const int pst = st / kRatio, t = pst / (G::DV / 32), db = pst % (G::DV / 32);
          vlo[pst % (kLook + 1)] = lds_read_tr16(vt + v_lane[0][db] + 16 * t * G::vRowBytes);
          vhi[pst % (kLook + 1)] = lds_read_tr16(vt + v_lane[1][db] + 16 * t * G::vRowBytes);
        }
      }
    };
    if constexpr (DO_S) {
      s[0] = f32x16{};
      s[1] = f32x16{};
    }
#pragma unroll
    for (int st = 0; st < kLook; ++st) issue(st);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (st + kLook < kSteps) issue(st + kLook);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DO_S) s[st & 1] = mfma32<FP16>(kop[st % (kLook + 1)], qreg[st >> 1], s[st & 1]);
      if constexpr (DO_P) {
        if (st % kRatio == 0) {
          const int pst = st / kRatio, t = pst / (G::DV / 32), db = pst % (G::DV / 32);
          const int slot = pst % (kLook + 1);
          acc[db] = mfma32<FP16>(u32x4{vlo[slot][0], vlo[slot][1], vhi[slot][0], vhi[slot][1]}, pb[t], acc[db]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the matrix phase runs at raised issue priority so that, when both waves of a
  // SIMD have an instruction ready, the matrix pipe is fed first
  auto mfma_phase = [&](int i) {
    const bool do_s = i < n_tiles && active(i);
    const bool do_p = i >= 1 && active(i - 1);
    __builtin_amdgcn_s_setprio(1);
    if (do_s && do_p) mfma_steps(std::true_type{}, std::true_type{}, i);
    else if (do_s) mfma_steps(std::true_type{}, std::false_type{}, i);
    else if (do_p) mfma_steps(std::false_type{}, std::true_type{}, i);
    __builtin_amdgcn_s_setprio(0);
  };

  // online softmax of S(t): reference, p, l, rescale of u, 16-bit P. Maximum and
  // sum run as four independent chains to keep the VALU pipeline full.
  auto softmax_phase = [&](int t) {
    if (!(t >= 0 && t < n_tiles && active(t))) return;
    const int kv0 = key_tile(t) * kBN;
    if ((kv0 + kBN > N) || (CAUSAL && kv0 + kBN - 1 > row0)) {
      // key = kv0 + c(b, r) + 4h with c(b, r) = 32b + 8(r/4) + r%4; a key is dead
      // past the sequence end or (causal) after the query: c(b, r) > lim
      int lim = N - 1 - kv0;
      if (CAUSAL) lim = min(lim, qrow - kv0);
      lim -= 4 * h;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = (32 * b + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[b][r];
    }
    // probabilities of this tile against the reference m_ref and their row sum
    float pr[32];
    auto exps = [&](float m_ref) {
      float ps[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x16& v = s[c >> 1];
        const int o = 8 * (c & 1);
#pragma unroll
        for (int r = 0; r < 8; ++r) pr[8 * c + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[o + r], sc, -m_ref));
        const float* p = pr + 8 * c;
        ps[c] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      }
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    // maximum of this lane's query over the tile (in-lane, then the other half-wave)
    auto row_max = [&]() {
      float mc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x16& v = s[c >> 1];
        const int o = 8 * (c & 1);
        mc[c] = __builtin_fmaxf(__builtin_fmaxf(v[o], v[o + 1]), v[o + 2]);
#pragma unroll
        for (int r = 3; r < 8; ++r) mc[c] = __builtin_fmaxf(mc[c], v[o + r]);
      }
      const float mx = __builtin_fmaxf(__builtin_fmaxf(mc[0], mc[1]), __builtin_fmaxf(mc[2], mc[3]));
      return __builtin_fmaxf(mx, other_half(mx)) * sc;
    };
    float m_new = m_run, m_ref = m_run, lt = 0.f;
    bool exact = true;
    if constexpr (!FP16) {
      exact = __any(m_run == -INFINITY);
      if (!exact) {
        lt = exps(m_run);
        exact = __any(lt > kBig);
      }
    }
    if (exact) {
      const float mx = row_max();
      m_new = (mx > m_run) ? mx : m_run;
      m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      lt = exps(m_ref);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float* p = pr + 8 * c;
      pb[c] = u32x4{pack2<FP16>(p[0], p[1]), pack2<FP16>(p[2], p[3]), pack2<FP16>(p[4], p[5]),
                    pack2<FP16>(p[6], p[7])};
    }
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    l_run = alpha * l_run + lt;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < G::DV / 32; ++db) acc[db] *= alpha;
    }
  };

  for (;;) {
    // the item's Q and first tile were issued during the previous item and waited
    // for before its epilogue (for the first item: in the prologue), so the
    // previous item's stores may still be in flight here
    if (first) wait_vmcnt<0>();
    first = false;
    __syncthreads();
    if constexpr (!G::wide) read_q();
    const int bh = item_bh(it_j);
    row0 = item_q0(it_j) + wave_rows;
    qrow = row0 + l32;
    if constexpr (SPLIT) {
      t_base = item_first(it_j);
      n_tiles = item_last(it_j) - t_base;
    } else {
      n_tiles = item_tiles(item_q0(it_j));
    }
    const int next_j = item_index(it_r + 1);
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < G::DV / 32; ++db) acc[db] = f32x16{};

    // once every wave holds its Q rows (this barrier), the next item's Q may be
    // loaded; it is issued after the first tile load so that the wait for that tile
    // can leave it in flight for another iteration
    __syncthreads();
    for (int i = 0; i <= n_tiles; ++i) {
      // one stream tile per iteration keeps the cursor kAhead tiles ahead; its stage
      // last held the tile kStages - kAhead before it, read before the last barrier
      // A wave stalls at a load instruction until the address unit takes it, and the
      // unit takes about one 1 KiB block per 11-12 cycles per compute unit: with
      // every wave issuing at the top of the iteration the last ones wait for
      // hundreds of cycles. Group A issues at the top; group B issues after its
      // softmax, when the queue has drained (tile first, then the next item's Q, so
      // that the wait below can leave only Q in flight).
      const bool q_in_flight = !G::wide && i == 0 && next_j >= 0;
      // wide instance: the next item's Q goes straight to registers in the last
      // iteration, which has no score product left (its loads land by the epilogue)
      if constexpr (G::wide)
        if (i == n_tiles && next_j >= 0) load_q_regs(next_j);
      // A: matrix work of tile i, then its softmax; B: softmax of tile i-1, then
      // matrix work of tile i
      // (the raised issue priority of the matrix phase starts before the loads, so
      // that the cursor work of the wave about to feed the matrix pipe is not held
      // up by the other wave's softmax)
      // Only the softmax calls sit under the group test: the compiler cannot tell
      // that it is uniform per wave, and the stream cursor must be updated outside
      // such branches to stay in scalar registers.
      if (grp != 0) softmax_phase(i - 1);
      __builtin_amdgcn_s_setprio(1);
      if (i < n_tiles) issue_next();
      if constexpr (!G::wide)
        if (q_in_flight) issue_q(next_j);
      mfma_phase(i);
      if (grp == 0) softmax_phase(i);
      // tile i+1 must have landed (every wave waits for its own loads) before the
      // barrier that publishes it; only the next item's Q may still be in flight
      if (i + 1 < n_tiles) {
        if (q_in_flight) wait_vmcnt<G::qLoadsPerWave>();
        else wait_vmcnt<0>();
        __syncthreads();
      }
    }

    // ---- epilogue: O = u / l, LSE = (m + log2 l) * ln 2 ----
    // the next item's Q and first tile are the only loads in flight: wait for them
    // here, before the stores, so that the next item need not wait for the stores
    wait_vmcnt<0>();
    const float l_tot = l_run + other_half(l_run);
    if constexpr (SPLIT) {
      static_assert(!G::wide, "no key split for the wide instance");
      if (qrow < N) {
      // partial of this key range: u / l and m + ln l in fp32 (a row with no
      // visible key in the range has l = 0: O = 0, LSE = -inf)
      const int64_t prow = ((int64_t)item_split(it_j) * a.bh + bh) * N + qrow;
      const bool live = l_tot > 0.f;
      const float inv = live ? 1.0f / l_tot : 0.f;
      KArgs* ka = kargs();
      float* po = ka->part_o + prow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(po + db * 32 + 8 * g + 4 * h) =
              f32x4{acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                    acc[db][4 * g + 3] * inv};
      if (h == 0)
        ka->part_lse[prow] = live ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f : -INFINITY;
      }
    } else {
      // Rounded output in 16-byte pieces: a lane holds four columns of each group of
      // eight and the lane 32 away the other four of the same row, so one swap of
      // the two halves' words gives the lower half all eight columns of an even
      // group and the upper half all eight of the odd group after it.
      const float inv = 1.0f / l_tot;
      u32x4 w[G::DV / 16];
#pragma unroll
      for (int db = 0; db < G::DV / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; g += 2) {
          const uint32_t e0 = pack2<FP16>(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv);
          const uint32_t e1 = pack2<FP16>(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
          const uint32_t o0 = pack2<FP16>(acc[db][4 * g + 4] * inv, acc[db][4 * g + 5] * inv);
          const uint32_t o1 = pack2<FP16>(acc[db][4 * g + 6] * inv, acc[db][4 * g + 7] * inv);
          const auto s0 = __builtin_amdgcn_permlane32_swap(e0, o0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(e1, o1, false, false);
          w[db * 2 + g / 2] = u32x4{s0[0], s1[0], s0[1], s1[1]};
        }
      if (qrow < N) {
        KArgs* ka = kargs();
        // columns v_col0 .. v_col0 + DV - 1 of which the first d_real - v_col0 exist
        const int d_real = ka->d_real - (G::wide ? ka->v_col0 : 0);
        uint16_t* og = reinterpret_cast<uint16_t*>(ka->o) + slice_off(bh, ka->o_sb, ka->o_sh) +
                       (int64_t)qrow * ka->o_sn + (G::wide ? ka->v_col0 : 0) + 8 * h;
        if (d_real >= G::DV) {
#pragma unroll
          for (int k = 0; k < G::DV / 16; ++k) *reinterpret_cast<u32x4*>(og + 16 * k) = w[k];
        } else {
          // d_real is a multiple of 8: each piece is wholly inside or outside
#pragma unroll
          for (int k = 0; k < G::DV / 16; ++k)
            if (16 * k + 8 * h < d_real) *reinterpret_cast<u32x4*>(og + 16 * k) = w[k];
        }
        // (both launches of the wide instance form the same LSE; the first stores it)
        if (h == 0 && (!G::wide || ka->v_col0 == 0))
          ka->lse[slice_off(bh, ka->l_sb, ka->l_sh) + qrow] =
              (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
      }
    }
    if (next_j < 0) break;
    g0 += n_tiles;
    it_j = next_j;
    ++it_r;
  }
}

// Merge of the key-split partials of every row (memory bound): D/4 lanes per row,
// four fp32 columns per lane. LSE = M + ln sum_k e^(LSE_k - M) with M = max_k LSE_k
// (finite: split 0 holds key 0, which every row sees), O = sum_k e^(LSE_k - LSE) O_k,
// rounded to the output dtype.
template <bool FP16, int D>
__global__ __launch_bounds__(256) void merge_splits(FwdArgs a) {
  constexpr int kLanes = D / 4;
  constexpr int kRows = 256 / kLanes;
  const int64_t rows = (int64_t)a.bh * a.n;
  const int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes;
  const int c = threadIdx.x % kLanes;
  if (row >= rows) return;
  const int S = a.splits;
  float mx = -INFINITY;
  for (int k = 0; k < S; ++k) mx = fmaxf(mx, a.part_lse[k * rows + row]);
  float den = 0.f;
  for (int k = 0; k < S; ++k) den += expf(a.part_lse[k * rows + row] - mx);
  const float lse = mx + logf(den);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < S; ++k) {
    const float w = expf(a.part_lse[k * rows + row] - lse);
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.part_o + (k * rows + row) * D + 4 * c);
    o += w * x;
  }
  uint16_t* og = reinterpret_cast<uint16_t*>(a.o) + row * D + 4 * c;
  *reinterpret_cast<u32x2*>(og) = u32x2{pack2<FP16>(o[0], o[1]), pack2<FP16>(o[2], o[3])};
  if (c == 0) a.lse[row] = lse;
}

template <bool FP16, int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  launch_log("fwd_pingpong<%s, %d, %s, %s> grid %d x %d, %d splits, %s order, columns from %d", dtype_name(FP16),
             D, CAUSAL ? "causal" : "full", a.splits > 1 ? "split" : "whole", a.grid, kThreads, a.splits,
             a.slice_major ? "slice-major" : "rank-major", a.v_col0);
  if constexpr (D > 128) {
    // the wide instance: one launch per 128-column half of V and O (no key split)
    if (a.splits > 1) return hipErrorInvalidValue;
    for (int c0 = 0; c0 < a.d_real; c0 += 128) {
      FwdArgs h = a;
      h.v_col0 = c0;
      hipLaunchKernelGGL((fwd_pingpong<FP16, D, CAUSAL, false>), dim3(a.grid), dim3(kThreads), 0, stream, h);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  } else if (a.splits > 1) {
    hipLaunchKernelGGL((fwd_pingpong<FP16, D, CAUSAL, true>), dim3(a.grid), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kRows = 256 / (D / 4);
    const int64_t rows = (int64_t)a.bh * a.n;
    launch_log("merge_splits<%s, %d> grid %lld x 256", dtype_name(FP16), D, (long long)((rows + kRows - 1) / kRows));
    hipLaunchKernelGGL((merge_splits<FP16, D>), dim3((unsigned)((rows + kRows - 1) / kRows)), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fwd_pingpong<FP16, D, CAUSAL, false>), dim3(a.grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// compute units of the current device, queried once per device
int cached_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace pp

int rows_per_workgroup() { return pp::kBM; }
int keys_per_tile() { return pp::kBN; }
int device_cus() { return pp::cached_cus(); }

hipError_t launch_fwd(const FwdArgs& args, bool fp16, int d, bool causal, hipStream_t stream) {
  using namespace pp;
  // persistent grid: one workgroup per compute unit (the LDS ring admits one per
  // CU), never more than there are items; a multiple of 8 when slices are grouped
  // by XCD so that every XCD gets the same number of workgroups
  FwdArgs a = args;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int64_t items = (int64_t)a.bh * a.q_tiles * (a.splits > 1 ? a.splits : 1);
  int grid = items < cus ? (int)items : cus;
  if (a.xcd_grouped) {
    grid &= ~7;
    if (grid < 8) grid = 8;
  }
  a.grid = grid;
  // slice-major item order (unsplit only) where the snake's causal pairs fill whole
  // rounds of the schedule group
  const int64_t group_wgs = a.xcd_grouped ? grid >> 3 : grid;
  const int64_t group_items = (int64_t)(a.xcd_grouped ? a.bh >> 3 : a.bh) * a.q_tiles;
  a.slice_major = a.splits <= 1 && (!causal || ((2 * group_wgs) % a.q_tiles == 0 &&
                                                group_items % (2 * group_wgs) == 0));
  if (fp16) {
    if (d == 64) return causal ? launch_one<true, 64, true>(a, stream) : launch_one<true, 64, false>(a, stream);
    if (d == 256) return causal ? launch_one<true, 256, true>(a, stream) : launch_one<true, 256, false>(a, stream);
    return causal ? launch_one<true, 128, true>(a, stream) : launch_one<true, 128, false>(a, stream);
  }
  if (d == 64) return causal ? launch_one<false, 64, true>(a, stream) : launch_one<false, 64, false>(a, stream);
  if (d == 256) return causal ? launch_one<false, 256, true>(a, stream) : launch_one<false, 256, false>(a, stream);
  return causal ? launch_one<false, 128, true>(a, stream) : launch_one<false, 128, false>(a, stream);
}

}  // namespace fa
