// Exact attention forward for gfx950 (MI355X), software-pipelined per wave.
//
// Same method as the ping-pong kernel ("FlashAttention: optimize data movement
// before counting FLOPs", section 02: per key tile keep the running row maximum m,
// denominator l and unnormalised numerator u, finish with O = u / l and
// LSE = m + ln l), same work items (256 query rows of one (batch, head)), same
// persistent schedule, LDS chunk swizzle and matrix-instruction layouts. What
// differs is how a wave orders its work.
//
// Each wave owns 32 query rows and walks the workgroup's stream of key tiles
// (all tiles of all its items, back to back). In iteration g it issues
//   S(g+1) = K_{g+1} Q^T            (D/8 v_mfma_f32_32x32x16)
//   P(g)   = 2^(S(g) scale log2 e - r)   (the softmax of the scores computed in
//                                         the previous iteration, on the VALU)
//   u     += V_{g-1}^T P(g-1)^T     (D/8 v_mfma_f32_32x32x16)
// None of the three depends on another within the iteration, so the matrix
// products and the softmax arithmetic are interleaved instruction by instruction
// in one stream: the VALU work of a score hides under the 32-cycle matrix
// instructions, and the two waves of a SIMD fill each other's gaps. Scores and
// packed probabilities are double-buffered in registers (the loop is unrolled by
// two so the buffers never move). The softmax of the ping-pong design (two waves
// per SIMD in opposite phases, matrix phase against softmax phase) stalled each
// half on the slower one and on the tile loads.
//
// K and V live in separate 3-stage LDS rings: K_{g+3} and V_{g+1} are loaded in
// iteration g (K two tiles ahead of V, since S needs K one iteration before P V
// needs V), straight from global memory into LDS with buffer_load ... lds, spread
// over the iteration. One barrier per iteration publishes K_{g+2} and V_g. Q rows
// of the next item are loaded into a fourth region one item ahead (160 KiB of LDS
// at d = 128).
//
// Reference maximum ("6.1 FlashAttention V1 in detail", §3.3: u / l and r + log l
// do not depend on the per-row reference r as long as nothing overflows): a tile's
// probabilities are computed against the reference kept from an earlier tile unless
// one of its scores lies more than a slack above it (log2 units; the tile's maximum is
// taken first), or it is an item's first tile (no reference yet); then the reference
// becomes the exact running maximum and u and l are rescaled by 2^(r_old - r_new).
// The slack is 15 for bf16 and 0 for fp16 (the exact running maximum, as in §5.1 of
// that page), so every probability is at most 2^15 (bf16 P keeps its full relative
// precision at that size), l stays below N 2^15 and |u| below N 2^15 max|v|.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>
#include <utility>

#include "fwd_kernel.h"
#include "gfx950_ops.h"
#include "launch_log.h"

namespace fa {
namespace sp {

using namespace ::fa::ops;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per item
constexpr int kBN = 64;           // keys per tile
constexpr int kStages = 3;        // depth of each of the K and V rings

// load offset of a masked head-dimension chunk: past every descriptor's range (the
// host keeps slice extents below 2^31 bytes), so the load writes zeros to LDS
constexpr uint32_t kMaskedOffset = 0x80000000u;

template <int D>
struct Geo {
  static constexpr int rowBytes = D * 2;
  static constexpr int chunksPerRow = D / 8;  // 16-byte chunks
  static constexpr int tileBytes = kBN * rowBytes;
  static constexpr int qBytes = kBM * rowBytes;
  static constexpr int blocksPerTile = tileBytes / 1024;       // 1 KiB per wave-instruction
  static constexpr int perWave = blocksPerTile / kWaves;       // K (and V) blocks per wave per tile
  static constexpr int qLoadsPerWave = qBytes / 1024 / kWaves;  // Q blocks per wave per item
  static constexpr int vRing = kStages * tileBytes;
  static constexpr int qRegion = 2 * kStages * tileBytes;
  static constexpr int ldsBytes = 2 * kStages * tileBytes + qBytes;
  static_assert(blocksPerTile % kWaves == 0, "tile must split into whole 1 KiB blocks per wave");
  __device__ static __forceinline__ int swz(int row) { return chunk_swizzle<D>(row); }
};

// Division by a run-time invariant divisor d >= 1 of dividends below 2^31 with a
// multiply-high, an add and a shift: the round-up method of Granlund and Montgomery
// ("Division by invariant integers using multiplication", 1994). With
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (below 2^32),
// n / d = (mulhi(m, n) + n) >> l; n < 2^31 keeps the sum inside 32 bits.
struct FastDiv {
  uint32_t mul, shift;
};
constexpr FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t{1} << l) < d) ++l;
  return FastDiv{(uint32_t)(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1), l};
}
__host__ __device__ constexpr uint32_t fastdiv(uint32_t n, uint32_t mul, uint32_t shift) {
  return ((uint32_t)(((uint64_t)n * mul) >> 32) + n) >> shift;
}
constexpr bool fastdiv_selfcheck() {
  const uint32_t ns[] = {0u, 1u, 2u, 3u, 7u, 63u, 64u, 65u, 255u, 1000u, 4095u, 65535u, 65536u, 1u << 20,
                         (1u << 24) + 17u, 123456789u, (1u << 30) + 3u, 2147483646u, 2147483647u};
  for (uint32_t d = 1; d <= 600; ++d) {
    const FastDiv f = make_fastdiv(d);
    for (uint32_t n : ns)
      if (fastdiv(n, f.mul, f.shift) != n / d) return false;
    for (uint32_t k = 1; k < 40; ++k) {  // around multiples of d
      const uint32_t n = d * k * 977u;
      if (n < 2147483647u && (fastdiv(n, f.mul, f.shift) != n / d || fastdiv(n - 1, f.mul, f.shift) != (n - 1) / d))
        return false;
    }
  }
  const uint32_t big[] = {1000003u, 65537u, 2147483647u, 1u << 30, 46341u};
  for (uint32_t d : big) {
    const FastDiv f = make_fastdiv(d);
    for (uint32_t n : ns)
      if (fastdiv(n, f.mul, f.shift) != n / d) return false;
  }
  return true;
}
static_assert(fastdiv_selfcheck(), "fast division");

using KArgs = const __attribute__((address_space(4))) FwdArgs;
__device__ __forceinline__ KArgs* kargs() {
  KArgs* p = (KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  return p;
}

// s_waitcnt vmcnt(n) for a run-time n (the instruction takes an immediate)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    default: wait_vmcnt<12>(); break;
  }
}

// workgroup barrier without a memory fence: tile loads into LDS are awaited
// explicitly with s_waitcnt before it, and every LDS read of the iteration has
// been consumed by then
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
using ic = std::integral_constant<int, N>;

// Order of the products in an iteration: S and P V alternate (S first); S products
// take all 16-column steps of the first 32-key half before the second half, so the
// first half of the new scores is complete halfway through.
// Order of one block's products: 2 KS S products (two 32-key halves of KS steps of 16
// columns) and 4 NB P V products (four 16-key chunks of NB blocks of 32 output
// columns). The S products sit in a leading region with the P V products spread
// evenly between them; the block ends with nP/2 - 1 P V products only, so that both
// halves of the new scores are complete several products before the end and their
// lane maxima are taken in the VALU slots of those last products.
template <int KS, int NB>
struct Sched {
  static constexpr int nS = 2 * KS, nP = 4 * NB, kSteps = nS + nP;
  static constexpr int tailP = nP / 2 - 1;
  static constexpr int region = kSteps - tailP;
  bool is_s[kSteps];
  int idx[kSteps];       // index of the step's product among those of its kind
  int last_s[2];         // step of the last S product of each 32-key half
  constexpr Sched() : is_s{}, idx{}, last_s{} {
    const int m = nP - tailP;
    bool p_at[kSteps] = {};
    for (int i = 0; i < m; ++i) p_at[(2 * i + 1) * region / (2 * m)] = true;
    for (int st = region; st < kSteps; ++st) p_at[st] = true;
    int ns = 0, np = 0;
    for (int st = 0; st < kSteps; ++st) {
      is_s[st] = !p_at[st];
      idx[st] = p_at[st] ? np++ : ns++;
      if (!p_at[st]) last_s[idx[st] / (nS / 2)] = st;
    }
  }
  constexpr bool valid() const {
    int ns = 0, np = 0;
    for (int st = 0; st < kSteps; ++st) (is_s[st] ? ns : np) += 1;
    return ns == nS && np == nP && last_s[1] + 2 < kSteps && last_s[0] < last_s[1];
  }
};
static_assert(Sched<8, 4>().valid() && Sched<6, 3>().valid() && Sched<5, 3>().valid() && Sched<4, 2>().valid(),
              "block schedule");

// f(integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time (a loop
// the unroller might leave rolled would index the register arrays dynamically)
template <typename F, int... Is>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// The lane index, computed where it is used: values derived from it for rarely taken
// paths (item starts, epilogues) are then not hoisted out of the tile loop and kept
// live (or spilled) across it.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// keeps a value's computation at this point of the instruction stream
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

template <bool FP16, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_sp(FwdArgs a) {
  // LDS and load layout: rows of DL = 64 or 128 columns (a power-of-two chunk count
  // for the swizzle, whole 1 KiB blocks per wave); arithmetic: KS = D/16 steps of 16
  // columns per S half and NB = ceil(D/32) blocks of 32 output columns (D = 80 and 96
  // skip the padding columns a 128-wide instance would multiply)
  constexpr int DL = D <= 64 ? 64 : 128;
  constexpr int KS = D / 16, NB = (D + 31) / 32;
  static_assert(D % 16 == 0 && D <= DL, "head dimension of an instance");
  using G = Geo<DL>;
  __shared__ __attribute__((aligned(1024))) char smem[G::ldsBytes];
  char* const kring = smem;
  char* const vring = smem + G::vRing;
  char* const qsm = smem + G::qRegion;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // waves w and w + 4 share a SIMD: they own 32-row blocks w and 7 - w, so under a
  // causal mask every SIMD has the same work on the diagonal tiles
  const int wave_rows = 32 * (wave < 4 ? wave : 11 - wave);

  // ---- persistent schedule (a group's slices in turn, each slice's query tiles
  // heaviest causal tile first, dealt in snake order over the group's workgroups; a
  // group is one XCD's share of the slices when B*H % 8 == 0, else all of them) ----
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
  const int tiles_all = (N + kBN - 1) / kBN;
  auto slice_off = [&](int bh, int64_t sb, int64_t sh) {
    const int heads = kargs()->heads;
    const int b = (int)fastdiv((uint32_t)bh, a.heads_mul, a.heads_shift);
    return (int64_t)b * sb + (int64_t)(bh - b * heads) * sh;
  };
  auto item_index = [&](int r) {
    const int j = r * wg_n + ((r & 1) ? wg_n - 1 - wg_k : wg_k);
    return j < n_items ? j : -1;
  };
  // Item j of a schedule group. Slice-major order (slice j / q_tiles, query tile
  // rank j % q_tiles): consecutive items -- those the group's workgroups run at the
  // same time -- cover one or two slices, whose K/V tiles they then share through
  // the XCD's L2. Under a causal mask the snake then gives each workgroup ranks i
  // and q_tiles - 1 - i only when q_tiles divides twice the group's workgroups and
  // the items fill whole pairs of rounds, so other causal shapes keep rank-major
  // order (rank j / hpx, slice j % hpx: every slice's heaviest tiles first). Causal
  // rank 0 is the last, heaviest tile.
  const bool slice_major = a.slice_major != 0;
  auto item_split = [&](int j, int& slice, int& rank) {
    const int qd = (int)fastdiv((uint32_t)j, a.grp_mul, a.grp_shift);
    const int rem = j - qd * (slice_major ? a.q_tiles : hpx);
    slice = slice_major ? qd : rem;
    rank = slice_major ? rem : qd;
  };
  auto item_bh = [&](int j) {
    int slice, rank;
    item_split(j, slice, rank);
    return bh_base + slice;
  };
  auto item_q0 = [&](int j) {
    int slice, rank;
    item_split(j, slice, rank);
    return (CAUSAL ? (a.q_tiles - 1 - rank) : rank) * kBM;
  };
  auto item_tiles = [&](int q0) {
    return CAUSAL ? min(tiles_all, (min(q0 + kBM, N) - 1) / kBN + 1) : tiles_all;
  };
  // this wave's rows of an item starting at q0 see key tile t / need the mask there
  auto act = [&](int q0, int t) {
    const int r0 = q0 + wave_rows;
    return r0 < N && (!CAUSAL || t * kBN <= r0 + 31);
  };
  auto masked = [&](int q0, int t) {
    return (t * kBN + kBN > N) || (CAUSAL && t * kBN + kBN - 1 > q0 + wave_rows);
  };

  const int first_j = item_index(0);
  if (first_j < 0) return;  // no work for this workgroup

  // ---- direct-to-LDS tile loads: this wave fills blocks wave + 8 i of a tile ----
  // lane `lane` of block b lands at chunk position 64 b + lane = (row, physical
  // chunk); it fetches the logical chunk physical ^ swz(row) of that row
  uint32_t k_ld[G::perWave], v_ld[G::perWave];
#pragma unroll
  for (int i = 0; i < G::perWave; ++i) {
    const int p = 64 * (wave + kWaves * i) + lane;
    const int row = p / G::chunksPerRow, logical = (p % G::chunksPerRow) ^ G::swz(row);
    const bool live = logical * 8 < a.d_real;
    k_ld[i] = live ? (uint32_t)row * (uint32_t)(2 * a.k_sn) + (uint32_t)(logical * 16) : kMaskedOffset;
    v_ld[i] = live ? (uint32_t)row * (uint32_t)(2 * a.v_sn) + (uint32_t)(logical * 16) : kMaskedOffset;
  }

  // Tile-stream cursors of the K and V loads: item rank r, item j (-1 once the
  // stream is exhausted), tile t of the item's n, the address of tile t and the bytes
  // from there to the end of the slice (the load descriptor's range), and the bytes
  // per tile. Rebuilt (and made wave-uniform) when the cursor enters an item,
  // advanced by one tile step otherwise.
  struct Cursor {
    int r, j, t, n;
    const char* base;
    uint32_t rem, step;
  };
  auto cursor_item = [&](Cursor& c, bool is_k) {
    if (c.j < 0) return;
    KArgs* ka = kargs();
    const char* b;
    if (is_k) {
      b = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(ka->k) +
                                        slice_off(item_bh(c.j), ka->k_sb, ka->k_sh));
      c.rem = ka->k_ext;
      c.step = (uint32_t)(kBN * 2 * ka->k_sn);
    } else {
      b = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(ka->v) +
                                        slice_off(item_bh(c.j), ka->v_sb, ka->v_sh));
      c.rem = ka->v_ext;
      c.step = (uint32_t)(kBN * 2 * ka->v_sn);
    }
    c.base = uniform_ptr(b);
    c.rem = __builtin_amdgcn_readfirstlane(c.rem);
    c.step = __builtin_amdgcn_readfirstlane(c.step);
    c.t = 0;
    c.n = __builtin_amdgcn_readfirstlane(item_tiles(item_q0(c.j)));
  };
  auto cursor_advance = [&](Cursor& c, bool is_k) {
    if (++c.t == c.n) {
      c.j = item_index(++c.r);
      cursor_item(c, is_k);
    } else {
      c.base += c.step;
      c.rem -= c.step;
    }
  };
  // one tile step with no item check, and the item check on its own
  auto cursor_step = [&](Cursor& c) {
    ++c.t;
    c.base += c.step;
    c.rem -= c.step;
  };
  auto cursor_settle = [&](Cursor& c, bool is_k) {
    if (c.t == c.n) {
      c.j = item_index(++c.r);
      cursor_item(c, is_k);
    }
  };
  auto cursor_rsrc = [&](const Cursor& c) { return buffer_rsrc(c.base, c.rem); };
  Cursor kc{0, first_j, 0, 0, nullptr, 0, 0}, vc{0, first_j, 0, 0, nullptr, 0, 0};
  cursor_item(kc, true);
  cursor_item(vc, false);
  // issue all of this wave's blocks of the cursor's tile into ring stage `st`
  auto issue_tile = [&](Cursor& c, bool is_k, char* ring, int st) {
    const __amdgpu_buffer_rsrc_t r = cursor_rsrc(c);
    char* dst = ring + st * G::tileBytes;
#pragma unroll
    for (int i = 0; i < G::perWave; ++i)
      buffer_load16_lds(r, is_k ? k_ld[i] : v_ld[i], dst + 1024 * (wave + kWaves * i));
  };

  // Q rows of an item go to LDS like K tiles (same chunk swizzle, 256 rows)
  auto issue_q = [&](int j) {
    const int q0 = item_q0(j);
    KArgs* ka = kargs();
    const int q_sn = ka->q_sn;
    const __amdgpu_buffer_rsrc_t qr =
        uniform_rsrc(reinterpret_cast<const uint16_t*>(ka->q) + slice_off(item_bh(j), ka->q_sb, ka->q_sh) +
                         (int64_t)q0 * q_sn,
                     ka->q_ext - (uint32_t)((int64_t)q0 * q_sn * 2));
    const int d_real = ka->d_real;
    const int lw = lane_here() + 64 * wave;
#pragma unroll
    for (int i = 0; i < G::qLoadsPerWave; ++i) {
      const int p = lw + 64 * kWaves * i;
      const int row = p / G::chunksPerRow, logical = (p % G::chunksPerRow) ^ G::swz(row);
      const uint32_t off = logical * 8 < d_real ? (uint32_t)row * (uint32_t)(2 * q_sn) + (uint32_t)(logical * 16)
                                                : kMaskedOffset;
      buffer_load16_lds(qr, off, qsm + 1024 * (wave + kWaves * i));
    }
  };
  // every lane reads its query's row into the B operands (k-slots d = 16 kk + 8 h + 0..7)
  u32x4 qreg[KS];
  auto read_q = [&]() {
    int row = wave_rows + l32;
    asm volatile("" : "+v"(row));
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qreg[kk] = lds_read16(qsm + row * G::rowBytes + (((2 * kk + h) ^ G::swz(row)) * 16));
  };

  // ---- per-lane LDS operand offsets ----
  // K (A operand of S^T = K Q^T): row l32 (+32 for the second half of the keys),
  // logical chunk 2 kk + h, i.e. byte l32 rowBytes + ((2 kk + h) ^ swz(l32)) 16. The
  // chunk field lies below the row and 2 kk shares no bit with h, so this equals
  // kbase ^ 32 kk with kbase the kk = 0 offset.
  // V (transposing read, A operand of O^T = V^T P^T): source row 16 t + 8 half + 4 h
  // + (lane % 16) / 4, logical chunk 4 db + 2 ((lane / 16) % 2) + (lane % 4) / 2, byte
  // 8 (lane % 2) inside the chunk; the 16 rows of step t come out in the order in which
  // the 32x32 accumulator's rows are packed into the B operand of step t. Likewise the
  // offset is vbase[half] ^ 64 db (plus 16 t rows).
  const int kbase = l32 * G::rowBytes + ((h ^ G::swz(l32)) * 16);
  int vbase[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 8 * half + 4 * h + ((lane & 15) >> 2);
    const int lc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    vbase[half] = row * G::rowBytes + ((lc ^ G::swz(row)) * 16) + 8 * (lane & 1);
  }

  const float sc = a.scale_log2;
  // How far (log2 units) a score may lie above the kept reference. bf16: 15, so a
  // probability stays below 2^15 and the reference moves only on large rises. fp16: 0,
  // the exact running maximum: the dominant probability of a row is then exactly 1,
  // while a kept reference would round it to 11 bits in P (the numerator) against the
  // unrounded fp32 sum l (the denominator) -- a relative error of up to 2^-12 of the
  // row's largest |v|, too much for fp16 inputs with a dominant key and |v| ~ 30.
  constexpr float kSlack = FP16 ? 0.0f : 15.0f;
  f32x16 sb[2][2];    // S^T accumulators [buffer][32-key half]: lane = query, 16 keys each
  u32x4 pb[2][4];     // 16-bit P as B operands [buffer][16-key chunk]
  f32x16 acc[NB];  // u^T: 32 columns of the head dimension per block
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    sb[b][0] = sb[b][1] = f32x16{};
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[b][t] = u32x4{};
  }
#pragma unroll
  for (int db = 0; db < NB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // reference (log2 units) of this lane's query
  float l_run = 0.f;        // denominator over this half-wave's keys
  // a finished item's statistics: x_* once the softmax leaves the item, e_* once its
  // epilogue is scheduled (the next item may finish in between)
  float x_m = 0.f, x_l = 1.f, e_m = 0.f, e_l = 1.f;

  // key of element r of half b of the S^T accumulator for lane half h:
  // 32 b + 8 (r / 4) + 4 h + r % 4

  // ---- building blocks ----
  // operand reads: S product j covers 32-key half j / (D/16) and 16-column step
  // j % (D/16) (all steps of half 0 first, so that half's accumulator is complete
  // early); P V product j covers 16-key chunk j / (D/32) and 32-column block j % (D/32)
  constexpr int kHalfSteps = KS;
  // kx, vx0, vx1: this iteration's stage offsets (multiples of the tile size, so
  // above every bit the XOR touches) plus the lane bases
  auto k_read = [&](int kx, int j) {
    const int half = j / kHalfSteps, kk = j % kHalfSteps;
    return lds_read16(smem + ((kx ^ (32 * kk)) + half * 32 * G::rowBytes));
  };
  auto v_read = [&](int vx0, int vx1, int j) {
    const int t = j / NB, db = j % NB;
    const u32x2 lo = lds_read_tr16(smem + ((vx0 ^ (64 * db)) + 16 * t * G::rowBytes));
    const u32x2 hi = lds_read_tr16(smem + ((vx1 ^ (64 * db)) + 16 * t * G::rowBytes));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // dead keys of a tile (past the sequence end or, causal, after the query) to -inf
  auto apply_mask = [&](auto pc, int kv0, int q0) {
    constexpr int P = decltype(pc)::value;
    int lim = N - 1 - kv0;
    if (CAUSAL) lim = min(lim, q0 + wave_rows + l32 - kv0);
    lim -= 4 * h;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[P][b][r] = (32 * b + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : sb[P][b][r];
  };
  // maximum of this lane's 32 scores of S^T(buffer P), unscaled
  auto lane_max = [&](auto pc) {
    constexpr int P = decltype(pc)::value;
    float mc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& v = sb[P][c >> 1];
      const int o = 8 * (c & 1);
      mc[c] = __builtin_fmaxf(__builtin_fmaxf(v[o], v[o + 1]), v[o + 2]);
#pragma unroll
      for (int r = 3; r < 8; ++r) mc[c] = __builtin_fmaxf(mc[c], v[o + r]);
    }
    return __builtin_fmaxf(__builtin_fmaxf(mc[0], mc[1]), __builtin_fmaxf(mc[2], mc[3]));
  };

  // One iteration's arithmetic as a single instruction stream: S(g+1) into sb[P],
  // the softmax of sb[P^1] against `ref` into pb[P^1] (returns the lane's sum of the
  // unrounded fp32 probabilities), u += V^T P^T from pb[P], the lane maximum of the
  // new scores sb[P] (unmasked, unscaled) into `lmx`, and this wave's share of the
  // tile loads (K_{g+3} from descriptor kr into kdst, V_{g+1} from vr into vdst).
  // Products follow Sched<KS, NB>; each carries one score's softmax work (two at D = 64),
  // split into three stages two ticks apart so that no instruction waits on the one
  // before it; the operand of each product is read two products ahead.
  auto block = [&](auto pc, float ref, int kst, int vst, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                   char* kdst, char* vdst, float& lmx) {
    constexpr int P = decltype(pc)::value;
    constexpr int Q = P ^ 1;
    constexpr Sched<KS, NB> kS{};
    constexpr int kSteps = Sched<KS, NB>::kSteps;
    const int kx = kst + kbase, vx0 = vst + vbase[0], vx1 = vst + vbase[1];
    auto operand = [&](auto stc) -> u32x4 {
      constexpr int st = decltype(stc)::value;
      if constexpr (kS.is_s[st]) return k_read(kx, kS.idx[st]);
      else return v_read(vx0, vx1, kS.idx[st]);
    };
    u32x4 op[3];
    op[0] = operand(std::integral_constant<int, 0>{});
    op[1] = operand(std::integral_constant<int, 1>{});
    float x[4];
    float sum = 0.f;
    // (each result passes through an empty volatile asm statement: instruction
    // selection would otherwise gather the pure arithmetic after the last product or
    // sink it into later blocks, and the scheduling fences only act after it)
    // tick e: x = s_e sc - ref; tick e + 1: x = 2^x; tick e + 2: add to the lane's sum
    // (one add per product, so the serial chain costs nothing) and pack the pair into
    // the P operand
    auto tick = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < 32) {
        constexpr int e = k;
        x[e & 3] = __builtin_fmaf(sb[Q][e >> 4][e & 15], sc, -ref);
        pin(x[e & 3]);
      }
      if constexpr (k >= 1 && k - 1 < 32) {
        constexpr int e = k - 1;
        x[e & 3] = __builtin_amdgcn_exp2f(x[e & 3]);
        pin(x[e & 3]);
      }
      if constexpr (k >= 2 && k - 2 < 32) {
        constexpr int e = k - 2;
        sum = e == 0 ? x[0] : sum + x[e & 3];
        pin(sum);
        if constexpr (e & 1) {
          pb[Q][e >> 3][(e & 7) >> 1] = pack2<FP16>(x[(e - 1) & 3], x[e & 3]);
          pin(pb[Q][e >> 3]);
        }
      }
    };
    // ticks of step st: [first_tick(st), first_tick(st + 1)). With 32 / kSteps whole
    // (D = 128: 1, D = 64: 2) the two extra ticks that drain the three-stage skew go to
    // the first two steps; otherwise the 34 ticks are spread evenly.
    constexpr int kTps = 32 / kSteps;
    auto first_tick = [](int st) {
      if (32 % kSteps == 0) return st * kTps + (st < 2 ? st : 2);
      return st * 34 / kSteps;
    };
    // lane maximum of each half of sb[P]: eight max operations per half (a chain of
    // 3-input maxima over its 16 values), from two products after the half's last S
    // product, spread over the steps left
    float mh[2];
    auto max_op = [&](int half, int o) {
      const f32x16& v = sb[P][half];
      if (o == 0) mh[half] = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
      else if (o < 7) mh[half] = __builtin_fmaxf(__builtin_fmaxf(mh[half], v[2 * o + 1]), v[2 * o + 2]);
      else mh[half] = __builtin_fmaxf(mh[half], v[15]);
      pin(mh[half]);
    };
    auto max_step = [](int half, int o) {
      const int start = kS.last_s[half] + 2;
      const int avail = kSteps - start < 8 ? kSteps - start : 8;
      return start + o * avail / 8;
    };
    // this wave's K blocks, then its V blocks, at evenly spread products
    constexpr int kLoads = 2 * G::perWave;
    auto maybe_load = [&](auto stc) {
      constexpr int st = decltype(stc)::value;
      static_for<kLoads>([&](auto ic_) {
        constexpr int i = decltype(ic_)::value;
        if constexpr (st == (2 * i + 1) * kSteps / (2 * kLoads)) {
          if constexpr (i < G::perWave) {
            buffer_load16_lds(kr, k_ld[i], kdst + 1024 * (wave + kWaves * i));
          } else {
            constexpr int iv = i - G::perWave;
            buffer_load16_lds(vr, v_ld[iv], vdst + 1024 * (wave + kWaves * iv));
          }
        }
      });
    };
    // The two waves of a SIMD run the same stream at the same time; the issue
    // arbiter favours the older one (waves 0-3), which would finish its products
    // early and wait at the barrier while the other runs alone. Waves 4-7 get the
    // higher issue priority for the first half of the products, waves 0-3 for the
    // second. (The choice is made inside the asm statement so that the compiler sees
    // no branch on the wave index.)
    asm volatile("s_cmp_lt_u32 %0, 4\n\ts_cbranch_scc1 .Lprio_a%=\n\ts_setprio 1\n.Lprio_a%=:" ::"s"(wave) : "scc");
    static_for<kSteps>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      if constexpr (st == kSteps / 2) {
        asm volatile("s_setprio 1\n\ts_cmp_lt_u32 %0, 4\n\ts_cbranch_scc1 .Lprio_b%=\n\ts_setprio 0\n.Lprio_b%=:" ::"s"(wave)
                     : "scc");
      }
      if constexpr (st + 2 < kSteps) op[(st + 2) % 3] = operand(std::integral_constant<int, st + 2>{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kS.is_s[st]) {
        constexpr int j = kS.idx[st];
        constexpr int half = j / KS, kk = j % KS;
        sb[P][half] = mfma32<FP16>(op[st % 3], qreg[kk], kk == 0 ? f32x16{} : sb[P][half]);
      } else {
        constexpr int j = kS.idx[st];
        constexpr int t = j / NB, db = j % NB;
        acc[db] = mfma32<FP16>(op[st % 3], pb[P][t], acc[db]);
      }
      static_for<first_tick(st + 1) - first_tick(st)>(
          [&](auto qc) { tick(std::integral_constant<int, first_tick(st) + decltype(qc)::value>{}); });
      static_for<16>([&](auto oc) {
        constexpr int half = decltype(oc)::value / 8, o = decltype(oc)::value % 8;
        if constexpr (max_step(half, o) == st) max_op(half, o);
      });
      maybe_load(stc);
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_setprio(0);
    lmx = __builtin_fmaxf(mh[0], mh[1]);
    return sum;
  };

  // ---- epilogue of a finished item: O = u / l, LSE = (m + log2 l) ln 2 ----
  auto epilogue = [&](int bh, int q0) {
    const float l_tot = e_l + other_half(e_l);
    const float inv = 1.0f / l_tot;
    const int qrow = q0 + wave_rows + l32;
    // a lane holds four columns of each group of eight and the lane 32 away the other
    // four of the same row: one swap gives the lower half all eight columns of an even
    // group and the upper half all eight of the odd group after it
    u32x4 w[2 * NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
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
      const int d_real = ka->d_real;
      uint16_t* og =
          reinterpret_cast<uint16_t*>(ka->o) + slice_off(bh, ka->o_sb, ka->o_sh) + (int64_t)qrow * ka->o_sn + 8 * h;
      if (d_real == 32 * NB) {
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) *reinterpret_cast<u32x4*>(og + 16 * k) = w[k];
      } else {
        // d_real is a multiple of 8: each piece is wholly inside or outside (the lane's
        // column offset is recomputed here rather than kept per piece across the loop)
        int c8 = 8 * h;
        asm volatile("" : "+v"(c8));
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k)
          if (c8 < d_real - 16 * k) *reinterpret_cast<u32x4*>(og + 16 * k) = w[k];
      }
      if (h == 0)
        ka->lse[slice_off(bh, ka->l_sb, ka->l_sh) + qrow] =
            (e_m + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
    }
#pragma unroll
    for (int db = 0; db < NB; ++db) acc[db] = f32x16{};
  };

  // ---- the compute slots' items: cur holds tile g (the first item before g = 0),
  // prv the item before it, nxt the one after ----
  // Last tile t of an item (starting at q0, n tiles) whose iteration is steady: every
  // wave active for S(t+1) and no wave masked at t (non-causal: t + 1 < n and no
  // ragged end; causal: tile t + 1 does not pass row q0 + 31); 0 when some wave has
  // no rows in the item.
  auto fast_last = [&](int q0, int n) {
    if (q0 + kBM - 32 >= N) return 0;
    return CAUSAL ? q0 / kBN - 1 : min(N / kBN - 1, n - 2);
  };
  int g = -1;
  int c_r = 0, c_j = first_j, c_start = 0, c_q0 = item_q0(first_j), c_n = item_tiles(c_q0);
  int c_fl = fast_last(c_q0, c_n);
  int n_j = item_index(1);
  int n_q0 = item_q0(n_j >= 0 ? n_j : 0);
  int p_j = 0, p_q0 = 0, p_n = 0;
  bool p_ok = false;
  // epilogue owed at the top of the next iteration (item slice and first row)
  bool pend = false;
  int e_bh = 0, e_q0 = 0;
  int c3 = 0;  // K ring stage read in this iteration; V is read from (c3 + 1) % 3

  // The rings start zeroed: dummy products of slots without work (see the
  // iteration) then only ever read finite values. Q of the first item and K tiles 0
  // and 1 follow; wait for Q and K_0.
  {
    constexpr int kPer = 2 * kStages * G::tileBytes / (16 * kThreads);
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4*>(smem + 16 * (tid + kThreads * i)) = u32x4{};
    __syncthreads();
  }
  issue_q(first_j);
  issue_tile(kc, true, kring, 0);
  cursor_advance(kc, true);
  int k_pending = 0;
  if (kc.j >= 0) {
    issue_tile(kc, true, kring, 1);
    cursor_advance(kc, true);
    k_pending = G::perWave;
  }
  wait_vm(k_pending);
  barrier();

  // ---- the iteration's plan ----
  // Everything an iteration needs that does not depend on LDS contents published by
  // the barrier that starts it is worked out at the end of the iteration before,
  // ahead of that barrier: the waves of a SIMD leave their products at different
  // times, so one wave's planning overlaps the other's products, and after the
  // barrier both go straight to their products. Only the epilogue, the next item's Q
  // load and reading Q (once per item) come after the barrier.
  // Steady iterations (every wave computes all three slots, no mask, no item
  // boundary, no epilogue, not an item's first two tiles) skip the slot logic.
  // lane maximum of the scores the last block computed (before any mask)
  float lmx_blk = -INFINITY;
  bool pl_stop = false, pl_do_m = false, pl_do_s = false, pl_do_p = false, pl_first = false, pl_exact = false;
  bool pl_need_q = false, pl_q_issue = false, pl_q_keep = false;
  float pl_ref = INFINITY, pl_m = -INFINITY, pl_alpha = 1.0f;
  auto plan = [&](auto pc) {
    constexpr int P = decltype(pc)::value;
    constexpr int Q = P ^ 1;
    const int m_t = g - c_start;
    const bool steady = c_j >= 0 && m_t >= 2 && m_t <= c_fl;
    bool do_s = true, do_m = true, do_p = true, first = false, mask_m = false;
    pl_stop = pl_need_q = pl_q_issue = pl_q_keep = false;
    if (!steady) {
      pl_stop = c_j < 0 && g >= c_start + 1;
      // slots: S(g+1), softmax(g), P V(g-1)
      const bool s_in_cur = c_j >= 0 && g + 1 < c_start + c_n;
      const bool s_ok = s_in_cur || (c_j >= 0 && n_j >= 0);
      const int s_q0 = s_in_cur ? c_q0 : n_q0;
      const int s_t = s_in_cur ? g + 1 - c_start : 0;
      pl_need_q = s_ok && s_t == 0;
      const bool m_ok = c_j >= 0 && g >= c_start;
      first = m_ok && m_t == 0;
      const bool pin_cur = c_j >= 0 && g - 1 >= c_start;
      const bool pv_ok = pin_cur || (g >= 1 && p_ok);
      const int pv_q0 = pin_cur ? c_q0 : p_q0;
      const int pv_t = pin_cur ? g - 1 - c_start : p_n - 1;
      // Q of the item after cur: loaded once every wave holds cur's Q; with a one-tile
      // item it is needed at once; otherwise it may stay in flight past this
      // iteration unless it is read in the next
      pl_q_issue = first && n_j >= 0;
      pl_q_keep = pl_q_issue && c_n > 2;
      do_s = s_ok && act(s_q0, s_t);
      do_m = m_ok && act(c_q0, m_t);
      do_p = pv_ok && act(pv_q0, pv_t);
      mask_m = do_m && masked(c_q0, m_t);
    }
    // The tile's probabilities keep the reference unless some score lies more than
    // kSlack (log2 units) above it; an item's first tile has no reference yet. A slot
    // this wave has no work in runs as harmless dummy work in the same instruction
    // stream: no softmax -> reference +inf (P = 0, nothing accumulated); no P V -> P = 0.
    float ref = INFINITY, m_new = m_run, alpha = 1.0f;
    bool exact_m = false;
    if (do_m) {
      float lmx = lmx_blk;
      if (mask_m) {
        apply_mask(ic<Q>{}, m_t * kBN, c_q0);
        lmx = lane_max(ic<Q>{});
      }
      exact_m = first || __any(lmx * sc > m_run + kSlack);
      if (exact_m) {
        const float mx = __builtin_fmaxf(lmx, other_half(lmx)) * sc;
        m_new = mx > m_run ? mx : m_run;
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run = -inf
      }
      ref = m_new;
    }
    if (!do_p) {
#pragma unroll
      for (int t = 0; t < 4; ++t) pb[P][t] = u32x4{};
    }
    pl_do_s = do_s;
    pl_do_m = do_m;
    pl_do_p = do_p;
    pl_first = first;
    pl_exact = exact_m;
    pl_ref = ref;
    pl_m = m_new;
    pl_alpha = alpha;
  };

  // One iteration of the stream (parity P of g + 1, planned); false once it is done.
  auto iteration = [&](auto pc) -> bool {
    constexpr int P = decltype(pc)::value;
    if (pend) {
      epilogue(e_bh, e_q0);
      pend = false;
    }
    if (pl_stop) return false;
    if (pl_q_issue) {
      issue_q(n_j);
      if (c_n == 1) {
        wait_vm(0);
        barrier();
      }
    }
    if (pl_need_q) read_q();
    // tile loads of this iteration: K_{g+3} into stage (c3 + 2) % 3, V_{g+1} into c3
    const bool ld_k = kc.j >= 0, ld_v = vc.j >= 0;
    const int c3w = c3 == 0 ? 2 : c3 - 1;
    const int c3v = c3 == 2 ? 0 : c3 + 1;
    char* const kdst = kring + c3w * G::tileBytes;
    char* const vdst = vring + c3 * G::tileBytes;
    const int kst = c3 * G::tileBytes;              // K read stage (offset in LDS)
    const int vst = G::vRing + c3v * G::tileBytes;  // V read stage
    // (an exhausted cursor gets an empty range: its loads write zeros to the free stage)
    const __amdgpu_buffer_rsrc_t kr = ld_k ? cursor_rsrc(kc) : buffer_rsrc(a.k, 0);
    const __amdgpu_buffer_rsrc_t vr = ld_v ? cursor_rsrc(vc) : buffer_rsrc(a.v, 0);
    const bool q_keep = pl_q_keep;
    if (pl_do_s || pl_do_m || pl_do_p) {
      const float sum = block(pc, pl_ref, kst, vst, kr, vr, kdst, vdst, lmx_blk);
      if (pl_do_m) {
        l_run = pl_alpha * l_run + sum;
        m_run = pl_m;
        // u holds the tiles up to g - 1 against the old reference (on an item's first
        // tile u belongs to the previous item, awaiting its epilogue)
        if (pl_exact && !pl_first) {
#pragma unroll
          for (int db = 0; db < NB; ++db) acc[db] *= pl_alpha;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < G::perWave; ++i) {
        buffer_load16_lds(kr, k_ld[i], kdst + 1024 * (wave + kWaves * i));
        buffer_load16_lds(vr, v_ld[i], vdst + 1024 * (wave + kWaves * i));
      }
    }
    // the previous item's last P V ran in this iteration: its epilogue is next
    if (p_ok && g == c_start) {
      pend = true;
      e_bh = item_bh(p_j);
      e_q0 = p_q0;
      e_m = x_m;
      e_l = x_l;
    }
    if (c_j >= 0 && g + 1 == c_start + c_n) {
      // the softmax is done with cur: keep its statistics for the epilogue
      x_m = m_run;
      x_l = l_run;
      m_run = -INFINITY;
      l_run = 0.f;
      p_ok = true;
      p_j = c_j;
      p_n = c_n;
      p_q0 = c_q0;
      c_start += c_n;
      ++c_r;
      c_j = n_j;
      c_q0 = n_q0;
      if (c_j >= 0) {
        c_n = item_tiles(c_q0);
        c_fl = fast_last(c_q0, c_n);
        n_j = item_index(c_r + 1);
        n_q0 = item_q0(n_j >= 0 ? n_j : 0);
      }
    }
    if (ld_k) cursor_advance(kc, true);
    if (ld_v) cursor_advance(vc, false);
    c3 = c3v;
    ++g;
    plan(ic<P ^ 1>{});
    // K_{g+2} and V_g (loaded in the previous iteration) must have landed before the
    // barrier that publishes them; this iteration's loads (always 2 perWave, empty
    // ranges included), and the next item's Q when it is not read in the next
    // iteration, may stay in flight (Q is issued first)
    if (q_keep) wait_vmcnt<2 * G::perWave + G::qLoadsPerWave>();
    else wait_vmcnt<2 * G::perWave>();
    barrier();
    return true;
  };

  // ---- steady runs ----
  // Runs of steady iterations, two at a time (buffer parity 0 then 1), without the
  // slot logic: m-slot tiles t of the current item with 2 <= t <= n - 2 (the S slot
  // stays in the item; tile 0 needs the exact maximum, tile 1's P V follows the
  // previous item's epilogue). Every wave computes every slot. A tile that needs the
  // mask (causal diagonal, ragged end) gets it before its lane maximum, and a tile
  // wholly masked for a wave then gives it P = 0 by itself: its scores are all -inf,
  // the reference stays at the (finite) running one and nothing is accumulated.
  // The load cursors step without the item check while the K loads (three tiles
  // ahead) stay in the item, t <= n - 4; the last iterations (K entering the next
  // item) use the checked advance, and an exhausted stream loads an empty range as in
  // the general iteration. The plan of each next iteration (mask, reference choice
  // from the lane maximum of the new scores) is taken before the barrier; the
  // iteration after the run is planned in full.
  auto steady_iter = [&](auto pc, auto crossc) {
    constexpr int P = decltype(pc)::value;
    constexpr bool kCross = decltype(crossc)::value;
    const int c3w = c3 == 0 ? 2 : c3 - 1;
    const int c3v = c3 == 2 ? 0 : c3 + 1;
    const bool ld_k = !kCross || kc.j >= 0, ld_v = !kCross || vc.j >= 0;
    const __amdgpu_buffer_rsrc_t kr = ld_k ? cursor_rsrc(kc) : buffer_rsrc(a.k, 0);
    const __amdgpu_buffer_rsrc_t vr = ld_v ? cursor_rsrc(vc) : buffer_rsrc(a.v, 0);
    const float sum = block(pc, pl_ref, c3 * G::tileBytes, G::vRing + c3v * G::tileBytes, kr, vr,
                            kring + c3w * G::tileBytes, vring + c3 * G::tileBytes, lmx_blk);
    l_run = pl_alpha * l_run + sum;
    m_run = pl_m;
    if (pl_exact) {
#pragma unroll
      for (int db = 0; db < NB; ++db) acc[db] *= pl_alpha;
    }
    if constexpr (kCross) {
      if (ld_k) cursor_advance(kc, true);
      if (ld_v) cursor_advance(vc, false);
    } else {
      cursor_step(kc);
      cursor_step(vc);
    }
    c3 = c3v;
    ++g;
    // plan of the next iteration (all slots): sb[P] holds its scores
    const int mt = g - c_start;
    float lmx = lmx_blk;
    if (masked(c_q0, mt)) {
      apply_mask(ic<P>{}, mt * kBN, c_q0);
      lmx = lane_max(ic<P>{});
    }
    pl_exact = __any(lmx * sc > m_run + kSlack);
    pl_m = m_run;
    pl_alpha = 1.0f;
    if (pl_exact) {
      const float mx = __builtin_fmaxf(lmx, other_half(lmx)) * sc;
      pl_m = mx > m_run ? mx : m_run;
      pl_alpha = __builtin_amdgcn_exp2f(m_run - pl_m);
    }
    pl_ref = pl_m;
    wait_vmcnt<2 * G::perWave>();
    barrier();
  };
  auto steady_run = [&]() {
    const int t0 = g - c_start;
    const int t_last = c_n - 2;
    if (!(c_j >= 0 && t0 >= 2 && t0 + 1 <= t_last)) return;
    // the planned iteration is steady (not an item's first two tiles): pl_* hold its
    // reference choice
    int t = t0;
    const int t_step = c_n - 4;
    while (t + 1 <= t_step) {
      steady_iter(ic<0>{}, std::false_type{});
      steady_iter(ic<1>{}, std::false_type{});
      t += 2;
    }
    cursor_settle(kc, true);
    cursor_settle(vc, false);
    while (t + 1 <= t_last) {
      steady_iter(ic<0>{}, std::true_type{});
      steady_iter(ic<1>{}, std::true_type{});
      t += 2;
    }
    plan(ic<0>{});
  };

  plan(ic<0>{});
  for (;;) {
    if (!iteration(ic<0>{})) break;
    if (!iteration(ic<1>{})) break;
    steady_run();
  }
  wait_vmcnt<0>();
}

template <bool FP16, int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_sp<FP16, D, CAUSAL>), dim3(a.grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sp

hipError_t launch_fwd_sp(const FwdArgs& args, bool fp16, int d, bool causal, hipStream_t stream) {
  using namespace sp;
  // persistent grid: one workgroup per compute unit (the LDS footprint admits one),
  // never more than there are items; a multiple of 8 when slices are grouped by XCD
  FwdArgs a = args;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int64_t items = (int64_t)a.bh * a.q_tiles;
  int grid = items < cus ? (int)items : cus;
  if (a.xcd_grouped) {
    grid &= ~7;
    if (grid < 8) grid = 8;
  }
  a.grid = grid;
  // slice-major order pairs each workgroup's causal ranks i and q_tiles - 1 - i only
  // when q_tiles divides twice the group's workgroups and the group's items fill
  // whole pairs of rounds; otherwise rank-major order (heaviest tiles of every slice
  // first) balances better
  const int group_wgs = a.xcd_grouped ? grid >> 3 : grid;
  const int64_t group_items = (int64_t)(a.xcd_grouped ? a.bh >> 3 : a.bh) * a.q_tiles;
  a.slice_major =
      (!causal || ((2 * group_wgs) % a.q_tiles == 0 && group_items % (2 * group_wgs) == 0)) ? 1 : 0;
  const FastDiv grp =
      make_fastdiv((uint32_t)(a.slice_major ? a.q_tiles : (a.xcd_grouped ? a.bh >> 3 : a.bh)));
  const FastDiv heads = make_fastdiv((uint32_t)a.heads);
  a.grp_mul = grp.mul;
  a.grp_shift = grp.shift;
  a.heads_mul = heads.mul;
  a.heads_shift = heads.shift;
  launch_log("fwd_sp<%s, %d, %s> grid %d x %d, %lld items, %d workgroups per schedule group, %s order, d_real %d",
             dtype_name(fp16), d, causal ? "causal" : "full", grid, kThreads, (long long)items, group_wgs,
             a.slice_major ? "slice-major" : "rank-major", a.d_real);
  auto pick = [&](auto fp16c) -> hipError_t {
    constexpr bool F = decltype(fp16c)::value;
    switch (d) {
      case 64: return causal ? launch_one<F, 64, true>(a, stream) : launch_one<F, 64, false>(a, stream);
      case 80: return causal ? launch_one<F, 80, true>(a, stream) : launch_one<F, 80, false>(a, stream);
      case 96: return causal ? launch_one<F, 96, true>(a, stream) : launch_one<F, 96, false>(a, stream);
      case 128: return causal ? launch_one<F, 128, true>(a, stream) : launch_one<F, 128, false>(a, stream);
      default: return hipErrorInvalidValue;
    }
  };
  return fp16 ? pick(std::true_type{}) : pick(std::false_type{});
}

}  // namespace fa
