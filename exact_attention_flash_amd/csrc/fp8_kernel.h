// Internal interface between the C ABI layer and the gfx950 FP8 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Rows of one quantization block (one scale each) = keys of one kernel tile.
constexpr int kFp8Block = 64;

// Block quantization of a contiguous [bh, n, d] 16-bit tensor to E4M3 or E5M2.
struct QuantArgs {
  const void* x;
  uint8_t* x8;      // rows layout: [bh, n, d]; keys-transposed layout: [bh, t64, d, 64]
  int32_t* se;      // [bh, t64]: E8M0 code (e + 127) of each block's scale 2^e
  int bh;
  int n;
  int t64;          // ceil(n / 64)
};

// Attention forward on quantized inputs (d = 64 or 128).
struct Fp8Args {
  const uint8_t* q8;     // [bh, n, d] FP8 (E4M3 or E5M2)
  const uint8_t* k8;     // [bh, n, d] FP8
  const uint8_t* v8t;    // [bh, t64, d, 64] FP8, keys-transposed layout
  const int32_t* q_se;   // [bh, t64] E8M0 codes of the blocks' scales
  const int32_t* k_se;
  const int32_t* v_se;
  void* o;               // [bh, n, d] bf16 or fp16
  float* lse;            // [bh, n]
  int bh;
  int n;
  int t64;
  int q_tiles;           // ceil(n / 256)
  int xcd_grouped;
  float scale_log2;      // scale * log2(e)
  int e8m0_one;          // 127: the E8M0 code of 1.0 (passed at run time: the scaled
                         // instruction does not take it as a literal)
};

// Enqueue the FP8 forward for head dimension d (64 or 128); sizes the persistent grid
// from the device's compute units. e5m2: q8, k8 and v8t hold E5M2 codes (else E4M3).
hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool fp16_out, bool causal, bool e5m2, hipStream_t stream);

// Keys-transposed layout: position p (0..63) of a block row holds key
// 32 * ((p % 32) / 16) + 8 * ((p % 16) / 4) + 4 * (p / 32) + p % 4 of the block.
// e5m2: quantize to E5M2 (largest finite 57344) instead of E4M3 (448).
hipError_t launch_quant_fp8(const QuantArgs& a, bool fp16, int d, bool keys_transposed, bool e5m2,
                            hipStream_t stream);

}  // namespace fa
