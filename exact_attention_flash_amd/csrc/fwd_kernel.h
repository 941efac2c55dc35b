// Internal interface between the C ABI layer and the gfx950 forward kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int bh;           // B * H slices
  int n;            // sequence length
  int q_tiles;      // ceil(n / rows_per_workgroup())
  int grid;         // workgroups launched (persistent: at most one per CU)
  int xcd_grouped;  // 1 when bh % 8 == 0: keep each slice's tiles on one XCD
  float scale_log2; // scale * log2(e)
  // key split (splits > 1): every query tile's key tiles are cut into `splits`
  // contiguous ranges handled as separate work items; each writes its normalised
  // partial output and log-sum-exp (fp32) to part_o [splits, bh, n, d] and
  // part_lse [splits, bh, n], and a merge kernel forms o and lse from them
  int splits;
  float* part_o;
  float* part_lse;
  // layout: element (b, h, i, c) of q sits at q + b*q_sb + h*q_sh + i*q_sn + c
  // (likewise k, v, o; lse at b*l_sb + h*l_sh + i), with bh = b * heads + h. Only
  // columns c < d_real exist (the kernel instance's D >= d_real; columns past
  // d_real read as zeros and are never stored). *_ext: bytes from a slice's first
  // element to the end of its last row, ((n - 1) * row stride + d_real) * 2.
  int heads;
  int d_real;
  // first column of V and O that a launch covers: 0, or 128 for the second launch
  // of the wide (256) instance of the ping-pong kernel
  int v_col0;
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh, l_sb, l_sh;
  int q_sn, k_sn, v_sn, o_sn;
  uint32_t q_ext, k_ext, v_ext;
  // filled by the launchers: the item order (1: slice-major, 0: rank-major); and,
  // for the software-pipelined kernel, multiply-high / shift pairs that divide by
  // its group divisor (q_tiles, or the slices per group) and by heads
  int slice_major;
  uint32_t grp_mul, grp_shift, heads_mul, heads_shift;
};

// Query rows handled by one workgroup.
int rows_per_workgroup();

// Keys per streamed tile.
int keys_per_tile();

// Compute units of the current device (queried once per device), or 0 on error.
int device_cus();

// Enqueue the kernel instance for (dtype, d, causal); d is 64 or 128. Sizes the
// persistent grid from the current device's compute units. With a.splits > 1 the
// split instance runs and is followed by the merge kernel.
hipError_t launch_fwd(const FwdArgs& a, bool fp16, int d, bool causal, hipStream_t stream);

// Enqueue the software-pipelined forward (no key split: a.splits must be 1) for
// (dtype, d, causal); d is the instance width, 64, 80, 96 or 128 (a.d_real <= d
// columns exist). Sizes the persistent grid like launch_fwd.
hipError_t launch_fwd_sp(const FwdArgs& a, bool fp16, int d, bool causal, hipStream_t stream);

}  // namespace fa
