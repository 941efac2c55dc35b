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
};

// Query rows handled by one workgroup.
int rows_per_workgroup();

// Enqueue the kernel instance for (dtype, d, causal); d is 64 or 128. Sizes the
// persistent grid from the current device's compute units.
hipError_t launch_fwd(const FwdArgs& a, bool fp16, int d, bool causal, hipStream_t stream);

}  // namespace fa
