// Device-side arguments of the packing kernels (quantize.hip): pointers into
// one packed buffer laid out as archead_pack_layout describes, plus the dense
// inputs of the construction step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "archead.h"

namespace archead {

struct QuantArgs {
  // dense inputs: W [V][D] (bf16 or fp32, row stride W_stride elements)
  const void* W;
  int64_t W_stride;
  bool w_bf16;
  int64_t V, D;
  int r_c, r, g;  // r = r_c + r_r
  int nA;         // a_scales columns: (r_c > 0) + (r_r > 0)
  int64_t nb;     // 16-row blocks: V16 / 16
  // packed sections
  uint8_t* buf;
  uint8_t* r_codes;
  uint8_t* r_gcodes;
  uint16_t* r_rowscale;
  int8_t* a_codes;
  uint16_t* a_scales;
  int8_t* b_codes;
  uint16_t* b_scales;
  // optional fp32 [V][D] output: the residual left after SC4, fp32(R) - SC4(R)
  float* E;
  int64_t E_stride;
};

// The largest hidden size the residual kernel holds in registers, and the
// largest core rank whose dequantised factor rows it keeps in LDS.
constexpr int64_t kQuantMaxD = 8192;
constexpr int kQuantMaxCoreRank = 1024;

// Enqueue the whole packing step on `s`: zero the buffer (total_bytes, a
// multiple of 256), write the header, quantise A_c, B_c, compute the SC4
// residual, quantise A_w, B_w.  A_c [V][r_c], B_c [r_c][D], A_w [V][r_r],
// B_w [r_r][D] are dense fp32 device arrays.
hipError_t launch_quantize(const QuantArgs& q, const float* A_c, const float* B_c, const float* A_w,
                           const float* B_w, uint64_t total_bytes, hipStream_t s);

// The same in two phases: the zero fill, header, core factors and SC4
// residual (which writes E when q.E is set), then the correction factors.
hipError_t launch_quantize_core(const QuantArgs& q, const float* A_c, const float* B_c, uint64_t total_bytes,
                                hipStream_t s);
hipError_t launch_quantize_corr(const QuantArgs& q, const float* A_w, const float* B_w, hipStream_t s);

// Pointers of every section of a packed buffer laid out as L.
QuantArgs quant_args(const archead_dims* d, const archead_layout& L, void* packed, const void* W, int64_t W_stride,
                     bool w_bf16, float* E, int64_t E_stride);

}  // namespace archead
