// Host-side launchers of the device kernels, called by the C ABI after it has
// validated every argument. Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zyfa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;  // FP8 only
  const float* k_scale;
  const float* v_scale;
  uint16_t* o;
  float* lse;            // may be null
  int B, Hq, Hkv, S, Dqk, Dv;
  int scale_block;       // FP8 only
  float softmax_scale;
};

// lean: probabilities as linear e4m3 codes instead of rounded exponentials
hipError_t launch_attn_fwd_fp8(const AttnArgs& a, bool lean, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream);

struct QuantArgs {
  const void* x;
  int x_is_bf16;
  uint8_t* codes;
  float* scales;
  int B, H, S, D, scale_block, hadamard;
};

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream);

}  // namespace zyfa
