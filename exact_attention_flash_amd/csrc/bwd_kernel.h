// Internal interface between the C ABI layer and the gfx950 backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // forward output
  const void* dout;   // gradient of the loss with respect to o
  const float* lse;   // forward row statistic (natural log), [bh, n]
  void* dq;
  void* dk;
  void* dv;
  float* delta;       // workspace [bh, n]: rowsum(dout * o)
  int bh;             // B * H slices
  int n;              // sequence length
  int xcd_grouped;    // 1 when bh % 8 == 0: keep each slice's workgroups on one XCD
  float scale;        // logit multiplier
  float scale_log2;   // scale * log2(e)
};

// Enqueue the three backward kernels for (dtype, d, causal); d is 64 or 128.
hipError_t launch_bwd(const BwdArgs& a, bool fp16, int d, bool causal, hipStream_t stream);

}  // namespace fa
