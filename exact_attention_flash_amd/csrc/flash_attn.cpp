// C ABI of the attention forward: host-side validation and dispatch.
// Every check runs before anything touches the GPU, so the error paths can be
// exercised on a machine without one.
#include "flash_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "bwd_kernel.h"
#include "fp8_kernel.h"
#include "fwd_kernel.h"

namespace {

bool overlaps(const void* a, uint64_t an, const void* b, uint64_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Forward kernel of a call without a key split. The software-pipelined kernel
// (fwd_sp.hip) overlaps each wave's softmax with its own products; the ping-pong
// kernel (fwd_kernel.hip) overlaps the two waves of a SIMD and starts work items
// more cheaply. Measured on one MI355X (same-process A/B over 28 shapes), the
// ping-pong kernel is 2-15% faster wherever a work item spans fewer than 4096 keys
// (the causal B2 H32 N4096 d128 workload included) and level (within +-2%, either
// way) on longer ones, so it serves head dimensions up to 64 and 97..128 (its 64-
// and 128-wide instances). Head dimensions 65..96 take the pipelined kernel's 80- and
// 96-wide instances rather than the ping-pong kernel's 128-wide one with its
// zero-padded columns. FLASH_ATTN_FWD_KERNEL=pipelined or =pingpong forces one
// (read at every call; the ping-pong kernel serves d = 65..96 with its 128-wide
// instance). inst is the smallest instance width (64, 80, 96 or 128) that holds the
// real head dimension.
int pick_unsplit(int inst) {
  if (inst > 128) return FA_FWD_KERNEL_PINGPONG;  // the wide instance exists only there
  const char* e = std::getenv("FLASH_ATTN_FWD_KERNEL");
  if (e != nullptr && std::strcmp(e, "pingpong") == 0) return FA_FWD_KERNEL_PINGPONG;
  if (e != nullptr && std::strcmp(e, "pipelined") == 0) return FA_FWD_KERNEL_PIPELINED;
  return inst == 64 || inst == 128 ? FA_FWD_KERNEL_PINGPONG : FA_FWD_KERNEL_PIPELINED;
}

int instance_width(int64_t d) { return d <= 64 ? 64 : d <= 80 ? 80 : d <= 96 ? 96 : d <= 128 ? 128 : 256; }

// Calls with a key split always use the ping-pong kernel's split instance.
hipError_t launch_unsplit(const fa::FwdArgs& a, bool fp16, int inst, bool causal, hipStream_t stream) {
  return pick_unsplit(inst) == FA_FWD_KERNEL_PIPELINED
             ? fa::launch_fwd_sp(a, fp16, inst, causal, stream)
             : fa::launch_fwd(a, fp16, inst <= 64 ? 64 : inst <= 128 ? 128 : 256, causal, stream);
}

}  // namespace

extern "C" int flash_attn_abi_version(void) { return 9; }

extern "C" const char* flash_attn_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is negative or too large for the kernel's indexing";
    case FA_ERR_HEADDIM:
      return "head dimension d must be 64, 128 or 256 (strided calls: a multiple of 8 up to 256; key split and "
             "FP8 calls: 64 or 128)";
    case FA_ERR_DTYPE: return "dtype must be FA_BF16 or FA_FP16";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIGN: return "16-bit tensors must be 16-byte aligned and fp32 ones 4-byte aligned";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    case FA_ERR_ARG: return "causal must be 0 or 1, num_splits >= 0, and an FP8 layout or format one of those defined";
    case FA_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than the split needs";
    case FA_ERR_STRIDE:
      return "a stride is negative, not a multiple of 8 elements, a row stride is below d or too large, a slice "
             "spans 2 GiB or more, or an output overlaps itself";
    case FA_ERR_SCRATCH: return "the split needs more partial-result memory than the library's fixed array holds";
    default: return "unknown status";
  }
}

namespace {

// All host-side checks; on success fills the launch arguments.
int check_args(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
               int64_t N, int64_t d, int causal, float scale, int dtype, fa::FwdArgs* a, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }

  // indexing limits: a (batch, head) slice is addressed with 32-bit offsets,
  // workgroups with a 32-bit grid
  const int64_t rows = fa::rows_per_workgroup();
  if (N > (INT32_MAX - 1) / d) return FA_ERR_SHAPE;
  if (B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  const int64_t q_tiles = (N + rows - 1) / rows;
  if (bh > INT32_MAX / q_tiles) return FA_ERR_SHAPE;

  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  const uint64_t in_bytes = static_cast<uint64_t>(bh) * N * d * 2;
  const uint64_t lse_bytes = static_cast<uint64_t>(bh) * N * 4;
  if (overlaps(o, in_bytes, q, in_bytes) || overlaps(o, in_bytes, k, in_bytes) ||
      overlaps(o, in_bytes, v, in_bytes) || overlaps(lse, lse_bytes, q, in_bytes) ||
      overlaps(lse, lse_bytes, k, in_bytes) || overlaps(lse, lse_bytes, v, in_bytes) ||
      overlaps(o, in_bytes, lse, lse_bytes))
    return FA_ERR_ALIAS;

  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->lse = lse;
  a->bh = static_cast<int>(bh);
  a->n = static_cast<int>(N);
  a->q_tiles = static_cast<int>(q_tiles);
  a->grid = static_cast<int>(bh * q_tiles);
  a->xcd_grouped = (bh % 8 == 0) ? 1 : 0;
  a->scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  a->splits = 1;
  a->part_o = nullptr;
  a->part_lse = nullptr;
  // contiguous [B, H, N, d] layout
  a->heads = static_cast<int>(H);
  a->d_real = static_cast<int>(d);
  a->v_col0 = 0;
  a->q_sb = a->k_sb = a->v_sb = a->o_sb = H * N * d;
  a->q_sh = a->k_sh = a->v_sh = a->o_sh = N * d;
  a->q_sn = a->k_sn = a->v_sn = a->o_sn = static_cast<int>(d);
  a->l_sb = H * N;
  a->l_sh = N;
  a->q_ext = a->k_ext = a->v_ext = static_cast<uint32_t>(N * d * 2);
  return FA_OK;
}

// ---- strided layout ----

// Offset (elements) one past the last element of a [B, H, N, inner] view whose
// innermost dimension is contiguous; false if it does not fit comfortably in int64.
bool view_end(int64_t B, int64_t H, int64_t N, int64_t inner, int64_t sb, int64_t sh, int64_t sn, int64_t* end) {
  const __int128 e = static_cast<__int128>(B - 1) * sb + static_cast<__int128>(H - 1) * sh +
                     static_cast<__int128>(N - 1) * sn + inner;
  if (e > (static_cast<__int128>(1) << 60)) return false;
  *end = static_cast<int64_t>(e);
  return true;
}

// Sufficient condition for a view with a contiguous innermost dimension of `inner`
// elements to address every element once: taken in increasing stride order, each
// dimension of size > 1 steps past everything spanned by the dimensions inside it.
bool no_self_overlap(int64_t inner, const int64_t (&size)[3], const int64_t (&stride)[3]) {
  int idx[3] = {0, 1, 2};
  std::sort(idx, idx + 3, [&](int x, int y) { return stride[x] < stride[y]; });
  __int128 ext = inner;
  for (int t = 0; t < 3; ++t) {
    const int i = idx[t];
    if (size[i] <= 1) continue;
    if (stride[i] < ext) return false;
    ext += static_cast<__int128>(size[i] - 1) * stride[i];
  }
  return true;
}

int check_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                  int64_t N, int64_t d, const int64_t* qs, const int64_t* ks, const int64_t* vs, const int64_t* os,
                  const int64_t* ls, int causal, float scale, int dtype, fa::FwdArgs* a, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d < 8 || d > 256 || d % 8 != 0) return FA_ERR_HEADDIM;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!qs || !ks || !vs || !os || !ls) return FA_ERR_NULL;
  const int64_t rows = fa::rows_per_workgroup();
  if (N > INT32_MAX / 2) return FA_ERR_SHAPE;
  if (B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  const int64_t q_tiles = (N + rows - 1) / rows;
  if (bh > INT32_MAX / q_tiles) return FA_ERR_SHAPE;

  // 16-bit tensors: strides >= 0 and multiples of 8 elements (16-byte row starts),
  // row stride in [d, 2^23), one slice under 2 GiB
  const int64_t* st16[4] = {qs, ks, vs, os};
  for (const int64_t* t : st16) {
    for (int i = 0; i < 3; ++i)
      if (t[i] < 0 || t[i] % 8 != 0) return FA_ERR_STRIDE;
    if (t[2] < d || t[2] >= (int64_t{1} << 23)) return FA_ERR_STRIDE;
    if (((N - 1) * t[2] + d) * 2 >= (int64_t{1} << 31)) return FA_ERR_STRIDE;
  }
  if (ls[0] < 0 || ls[1] < 0) return FA_ERR_STRIDE;
  const int64_t size3[3] = {B, H, N};
  const int64_t o_str[3] = {os[0], os[1], os[2]};
  if (!no_self_overlap(d, size3, o_str)) return FA_ERR_STRIDE;
  const int64_t size2[3] = {B, H, 1};
  const int64_t l_str[3] = {ls[0], ls[1], 0};
  if (!no_self_overlap(N, size2, l_str)) return FA_ERR_STRIDE;

  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  int64_t qe, ke, ve, oe, le;
  if (!view_end(B, H, N, d, qs[0], qs[1], qs[2], &qe) || !view_end(B, H, N, d, ks[0], ks[1], ks[2], &ke) ||
      !view_end(B, H, N, d, vs[0], vs[1], vs[2], &ve) || !view_end(B, H, N, d, os[0], os[1], os[2], &oe) ||
      !view_end(B, H, 1, N, ls[0], ls[1], 0, &le))
    return FA_ERR_SHAPE;
  const uint64_t qb = qe * 2, kb = ke * 2, vb = ve * 2, ob = oe * 2, lb = le * 4;
  if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, vb) || overlaps(lse, lb, q, qb) ||
      overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, vb) || overlaps(o, ob, lse, lb))
    return FA_ERR_ALIAS;

  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->lse = lse;
  a->bh = static_cast<int>(bh);
  a->n = static_cast<int>(N);
  a->q_tiles = static_cast<int>(q_tiles);
  a->grid = static_cast<int>(bh * q_tiles);
  // slices of one XCD share K/V through its L2 only when they are distinct heads of
  // a contiguous layout; the grouping itself is valid for any layout
  a->xcd_grouped = (bh % 8 == 0) ? 1 : 0;
  a->scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  a->splits = 1;
  a->part_o = nullptr;
  a->part_lse = nullptr;
  a->heads = static_cast<int>(H);
  a->d_real = static_cast<int>(d);
  a->v_col0 = 0;
  a->q_sb = qs[0]; a->q_sh = qs[1]; a->q_sn = static_cast<int>(qs[2]);
  a->k_sb = ks[0]; a->k_sh = ks[1]; a->k_sn = static_cast<int>(ks[2]);
  a->v_sb = vs[0]; a->v_sh = vs[1]; a->v_sn = static_cast<int>(vs[2]);
  a->o_sb = os[0]; a->o_sh = os[1]; a->o_sn = static_cast<int>(os[2]);
  a->l_sb = ls[0]; a->l_sh = ls[1];
  a->q_ext = static_cast<uint32_t>(((N - 1) * qs[2] + d) * 2);
  a->k_ext = static_cast<uint32_t>(((N - 1) * ks[2] + d) * 2);
  a->v_ext = static_cast<uint32_t>(((N - 1) * vs[2] + d) * 2);
  return FA_OK;
}

// ---- key split ----
constexpr int kMaxSplits = 16;

// Largest split count for which no work item is empty: the fewest key tiles any
// query tile visits (causal: the first query tile's), capped at kMaxSplits.
int max_splits(int64_t N, int causal) {
  const int64_t bn = fa::keys_per_tile(), bm = fa::rows_per_workgroup();
  const int64_t tiles_all = (N + bn - 1) / bn;
  int64_t fewest = tiles_all;
  if (causal) {
    const int64_t first = ((N < bm ? N : bm) - 1) / bn + 1;
    if (first < fewest) fewest = first;
  }
  if (fewest > kMaxSplits) fewest = kMaxSplits;
  return fewest < 1 ? 1 : static_cast<int>(fewest);
}

int resolve_splits(int64_t N, int causal, int num_splits) {
  const int mx = max_splits(N, causal);
  return num_splits > mx ? mx : num_splits;
}

// Split count for a device with `cus` compute units: enough items to give every
// compute unit one, when the unsplit work has fewer items than compute units and
// the sequence spans at least kMinSplitTiles key tiles (below that an item is so
// short that the merge launch costs more than the split saves).
constexpr int kMinSplitTiles = 8;

int plan_splits(int64_t bh, int64_t N, int causal, int cus) {
  const int64_t items = bh * ((N + fa::rows_per_workgroup() - 1) / fa::rows_per_workgroup());
  if (items <= 0 || cus <= 0 || items >= cus) return 1;
  if ((N + fa::keys_per_tile() - 1) / fa::keys_per_tile() < kMinSplitTiles) return 1;
  const int64_t want = (cus + items - 1) / items;
  return resolve_splits(N, causal, want > kMaxSplits ? kMaxSplits : static_cast<int>(want));
}

uint64_t workspace_bytes_for(int64_t bh, int64_t N, int64_t d, int splits) {
  if (splits <= 1) return 0;
  return static_cast<uint64_t>(splits) * static_cast<uint64_t>(bh) * static_cast<uint64_t>(N) *
         static_cast<uint64_t>(d + 1) * 4u;
}

// Checks of the split call beyond those of the forward; fills the split fields.
// num_splits must already be resolved (>= 1).
int check_split(const void* q, const void* k, const void* v, const void* o, const float* lse, int64_t B,
                int64_t H, int64_t N, int64_t d, int splits, void* workspace, uint64_t workspace_bytes,
                fa::FwdArgs* a) {
  if (splits <= 1) return FA_OK;
  const int64_t bh = B * H;
  if (static_cast<int64_t>(a->q_tiles) * bh > INT32_MAX / splits) return FA_ERR_SHAPE;
  const uint64_t need = workspace_bytes_for(bh, N, d, splits);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const uint64_t in_bytes = static_cast<uint64_t>(bh) * N * d * 2;
  const uint64_t lse_bytes = static_cast<uint64_t>(bh) * N * 4;
  if (overlaps(workspace, need, q, in_bytes) || overlaps(workspace, need, k, in_bytes) ||
      overlaps(workspace, need, v, in_bytes) || overlaps(workspace, need, o, in_bytes) ||
      overlaps(workspace, need, lse, lse_bytes))
    return FA_ERR_ALIAS;
  a->splits = splits;
  a->part_o = static_cast<float*>(workspace);
  a->part_lse = static_cast<float*>(workspace) + static_cast<uint64_t>(splits) * bh * N * d;
  return FA_OK;
}

}  // namespace

extern "C" int flash_attn_fwd_validate(const void* q, const void* k, const void* v, void* o, float* lse,
                                       int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                       void* /*stream*/, int dtype) {
  fa::FwdArgs a;
  bool empty;
  return check_args(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, &a, &empty);
}

extern "C" int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                              void* stream, int dtype) {
  fa::FwdArgs a;
  bool empty;
  const int st = check_args(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, &a, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t err = launch_unsplit(a, dtype == FA_FP16, static_cast<int>(d), causal == 1,
                                        static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_fwd_strided_validate(const void* q, const void* k, const void* v, void* o, float* lse,
                                               int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* q_strides,
                                               const int64_t* k_strides, const int64_t* v_strides,
                                               const int64_t* o_strides, const int64_t* lse_strides, int causal,
                                               float scale, void* /*stream*/, int dtype) {
  fa::FwdArgs a;
  bool empty;
  return check_strided(q, k, v, o, lse, B, H, N, d, q_strides, k_strides, v_strides, o_strides, lse_strides, causal,
                       scale, dtype, &a, &empty);
}

extern "C" int flash_attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                      int64_t H, int64_t N, int64_t d, const int64_t* q_strides,
                                      const int64_t* k_strides, const int64_t* v_strides, const int64_t* o_strides,
                                      const int64_t* lse_strides, int causal, float scale, void* stream, int dtype) {
  fa::FwdArgs a;
  bool empty;
  const int st = check_strided(q, k, v, o, lse, B, H, N, d, q_strides, k_strides, v_strides, o_strides,
                               lse_strides, causal, scale, dtype, &a, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t err = launch_unsplit(a, dtype == FA_FP16, instance_width(d), causal == 1,
                                        static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_fwd_kernel(int64_t N, int64_t d, int causal) {
  if (N < 0) return FA_ERR_SHAPE;
  if (d < 8 || d > 256 || d % 8 != 0) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  return pick_unsplit(instance_width(d));
}

extern "C" int flash_attn_fwd_splitkv_plan(int64_t B, int64_t H, int64_t N, int64_t d, int causal, int cus) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) return 1;
  // the forward's indexing limits (also keep the item count below far from overflow)
  if (N > (INT32_MAX - 1) / d || B > INT32_MAX / H) return FA_ERR_SHAPE;
  return plan_splits(B * H, N, causal, cus);
}

extern "C" int64_t flash_attn_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                                         int num_splits) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if ((causal != 0 && causal != 1) || num_splits < 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) return 0;
  // the split forward's indexing limits: then the byte count stays far inside 64 bits
  if (N > (INT32_MAX - 1) / d || B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int splits = resolve_splits(N, causal, num_splits);
  const int64_t items = B * H * ((N + fa::rows_per_workgroup() - 1) / fa::rows_per_workgroup());
  if (items > INT32_MAX / splits) return FA_ERR_SHAPE;
  return static_cast<int64_t>(workspace_bytes_for(B * H, N, d, splits));
}

namespace {

int splitkv_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t N, int64_t d, int causal, float scale, int num_splits, void* workspace,
                   uint64_t workspace_bytes, int dtype, bool plan_on_device, fa::FwdArgs* a, bool* empty) {
  if (num_splits < 0) return FA_ERR_ARG;
  if (d > 128) return FA_ERR_HEADDIM;  // the key split has instances for d = 64 and 128
  const int st = check_args(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, a, empty);
  if (st != FA_OK || *empty) return st;
  int splits = num_splits;
  if (splits == 0) {
    if (!plan_on_device) return FA_OK;  // validation only: the split is chosen at launch
    splits = plan_splits(a->bh, N, causal, fa::device_cus());
  }
  splits = resolve_splits(N, causal, splits);
  return check_split(q, k, v, o, lse, B, H, N, d, splits, workspace, workspace_bytes, a);
}

}  // namespace

extern "C" int flash_attn_fwd_splitkv_validate(const void* q, const void* k, const void* v, void* o, float* lse,
                                               int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                               float scale, int num_splits, void* workspace,
                                               uint64_t workspace_bytes, void* /*stream*/, int dtype) {
  fa::FwdArgs a;
  bool empty;
  return splitkv_common(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, workspace, workspace_bytes, dtype,
                        false, &a, &empty);
}

extern "C" int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                      int64_t H, int64_t N, int64_t d, int causal, float scale, int num_splits,
                                      void* workspace, uint64_t workspace_bytes, void* stream, int dtype) {
  fa::FwdArgs a;
  bool empty;
  const int st = splitkv_common(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, workspace,
                                workspace_bytes, dtype, true, &a, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t err =
      a.splits > 1 ? fa::launch_fwd(a, dtype == FA_FP16, static_cast<int>(d), causal == 1,
                                    static_cast<hipStream_t>(stream))
                   : launch_unsplit(a, dtype == FA_FP16, static_cast<int>(d), causal == 1,
                                    static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---- FP8 ----

namespace {

int check_quant(const void* x, void* x8, int32_t* se, int64_t B, int64_t H, int64_t N, int64_t d, int layout,
                int dtype, int format, fa::QuantArgs* a, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_DTYPE;
  if (layout != FA_FP8_ROWS && layout != FA_FP8_KEYS_T) return FA_ERR_ARG;
  if (format != FA_FP8_E4M3 && format != FA_FP8_E5M2) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (N > (INT32_MAX - 1) / d || B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H, t64 = (N + fa::kFp8Block - 1) / fa::kFp8Block;
  if (bh > INT32_MAX / t64) return FA_ERR_SHAPE;
  if (!x || !x8 || !se) return FA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(se, 4)) return FA_ERR_ALIGN;
  const uint64_t xb = static_cast<uint64_t>(bh) * N * d * 2;
  const uint64_t x8b = layout == FA_FP8_ROWS ? static_cast<uint64_t>(bh) * N * d
                                             : static_cast<uint64_t>(bh) * t64 * d * fa::kFp8Block;
  const uint64_t seb = static_cast<uint64_t>(bh) * t64 * 4;
  if (overlaps(x8, x8b, x, xb) || overlaps(se, seb, x, xb) || overlaps(x8, x8b, se, seb)) return FA_ERR_ALIAS;
  a->x = x;
  a->x8 = static_cast<uint8_t*>(x8);
  a->se = se;
  a->bh = static_cast<int>(bh);
  a->n = static_cast<int>(N);
  a->t64 = static_cast<int>(t64);
  return FA_OK;
}

int check_fp8(const void* q8, const void* k8, const void* v8t, const int32_t* qs, const int32_t* ks,
              const int32_t* vs, void* o, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int causal,
              float scale, int out_dtype, int format, fa::Fp8Args* a, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (out_dtype != FA_BF16 && out_dtype != FA_FP16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (format != FA_FP8_E4M3 && format != FA_FP8_E5M2) return FA_ERR_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (N > (INT32_MAX - 1) / d || B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H, t64 = (N + fa::kFp8Block - 1) / fa::kFp8Block;
  const int64_t q_tiles = (N + fa::rows_per_workgroup() - 1) / fa::rows_per_workgroup();
  if (bh > INT32_MAX / t64) return FA_ERR_SHAPE;
  if (!q8 || !k8 || !v8t || !qs || !ks || !vs || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8t, 16) || !aligned(o, 16) || !aligned(qs, 4) ||
      !aligned(ks, 4) || !aligned(vs, 4) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  const uint64_t rb = static_cast<uint64_t>(bh) * N * d, vb = static_cast<uint64_t>(bh) * t64 * d * fa::kFp8Block;
  const uint64_t sb = static_cast<uint64_t>(bh) * t64 * 4, ob = rb * 2, lb = static_cast<uint64_t>(bh) * N * 4;
  const void* ins[6] = {q8, k8, v8t, qs, ks, vs};
  const uint64_t inb[6] = {rb, rb, vb, sb, sb, sb};
  for (int i = 0; i < 6; ++i)
    if (overlaps(o, ob, ins[i], inb[i]) || overlaps(lse, lb, ins[i], inb[i])) return FA_ERR_ALIAS;
  if (overlaps(o, ob, lse, lb)) return FA_ERR_ALIAS;
  a->q8 = static_cast<const uint8_t*>(q8);
  a->k8 = static_cast<const uint8_t*>(k8);
  a->v8t = static_cast<const uint8_t*>(v8t);
  a->q_se = qs;
  a->k_se = ks;
  a->v_se = vs;
  a->o = o;
  a->lse = lse;
  a->bh = static_cast<int>(bh);
  a->n = static_cast<int>(N);
  a->t64 = static_cast<int>(t64);
  a->q_tiles = static_cast<int>(q_tiles);
  a->xcd_grouped = (bh % 8 == 0) ? 1 : 0;
  a->scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  a->e8m0_one = 127;
  return FA_OK;
}

}  // namespace

extern "C" int flash_attn_quantize_fp8_validate(const void* x, void* x8, int32_t* scale_codes, int64_t B, int64_t H,
                                                int64_t N, int64_t d, int layout, void* /*stream*/, int dtype,
                                                int format) {
  fa::QuantArgs a;
  bool empty;
  return check_quant(x, x8, scale_codes, B, H, N, d, layout, dtype, format, &a, &empty);
}

extern "C" int flash_attn_quantize_fp8(const void* x, void* x8, int32_t* scale_codes, int64_t B, int64_t H,
                                       int64_t N, int64_t d, int layout, void* stream, int dtype, int format) {
  fa::QuantArgs a;
  bool empty;
  const int st = check_quant(x, x8, scale_codes, B, H, N, d, layout, dtype, format, &a, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t err = fa::launch_quant_fp8(a, dtype == FA_FP16, static_cast<int>(d), layout == FA_FP8_KEYS_T,
                                              format == FA_FP8_E5M2, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_fwd_fp8_validate(const void* q8, const void* k8, const void* v8t, const int32_t* q_scale,
                                           const int32_t* k_scale, const int32_t* v_scale, void* o, float* lse,
                                           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                           void* /*stream*/, int out_dtype, int format) {
  fa::Fp8Args a;
  bool empty;
  return check_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, o, lse, B, H, N, d, causal, scale, out_dtype, format, &a,
                   &empty);
}

extern "C" int flash_attn_fwd_fp8(const void* q8, const void* k8, const void* v8t, const int32_t* q_scale,
                                  const int32_t* k_scale, const int32_t* v_scale, void* o, float* lse, int64_t B,
                                  int64_t H, int64_t N, int64_t d, int causal, float scale, void* stream,
                                  int out_dtype, int format) {
  fa::Fp8Args a;
  bool empty;
  const int st = check_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, o, lse, B, H, N, d, causal, scale, out_dtype,
                           format, &a, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t err = fa::launch_fwd_fp8(a, static_cast<int>(d), out_dtype == FA_FP16, causal == 1,
                                            format == FA_FP8_E5M2, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// All host-side checks of the backward call; on success fills the launch arguments.
int check_bwd_args(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N, int64_t d,
                   int causal, float scale, int dtype, fa::BwdArgs* a, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  // a slice is addressed with 32-bit offsets; grids of bh * ceil(N / 128) workgroups
  if (N > (INT32_MAX - 1) / d) return FA_ERR_SHAPE;
  if (B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh > INT32_MAX / ((N + 127) / 128)) return FA_ERR_SHAPE;
  if (bh * N > INT32_MAX / 4) return FA_ERR_SHAPE;

  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return FA_ERR_ALIGN;
  const uint64_t t = static_cast<uint64_t>(bh) * N * d * 2;  // one 16-bit tensor
  const uint64_t r = static_cast<uint64_t>(bh) * N * 4;      // one fp32 row statistic
  const void* ins[] = {q, k, v, o, dout, lse};
  const uint64_t in_n[] = {t, t, t, t, t, r};
  const void* outs[] = {dq, dk, dv, delta};
  const uint64_t out_n[] = {t, t, t, r};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return FA_ERR_ALIAS;
  }

  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->dout = dout;
  a->lse = lse;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->delta = delta;
  a->bh = static_cast<int>(bh);
  a->n = static_cast<int>(N);
  a->xcd_grouped = (bh % 8 == 0) ? 1 : 0;
  a->scale = scale;
  a->scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  return FA_OK;
}

}  // namespace

extern "C" int flash_attn_bwd_validate(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                       const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B,
                                       int64_t H, int64_t N, int64_t d, int causal, float scale, void* /*stream*/,
                                       int dtype) {
  fa::BwdArgs a;
  bool empty;
  return check_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, &a, &empty);
}

extern "C" int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H,
                              int64_t N, int64_t d, int causal, float scale, void* stream, int dtype) {
  fa::BwdArgs a;
  bool empty;
  const int st =
      check_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, &a, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t err = fa::launch_bwd(a, dtype == FA_FP16, static_cast<int>(d), causal == 1,
                                        static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}
