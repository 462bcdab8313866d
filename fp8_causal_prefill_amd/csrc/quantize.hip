// Quantization of Q, K or V to e4m3 with one power-of-two scale per (batch, head,
// token block), with an optional Hadamard rotation of each row over the head dimension.
//
// "ZYFA: Fast and Accurate FP8 Attention on AMD MI355X", section "FP8 Error in
// Full-Model Inference" and footnote 2: inputs are quantized in a pass of their own;
// a Hadamard rotation of Q and K over the head dimension, fused into that pass,
// spreads outlier channels. FP8 GEMM on CDNA4 blog, sections 2.2-2.3: absmax
// scaling with a zero guard, round-to-nearest-even. The scale is restricted to a
// power of two (the E8M0 form the scaled FP8 matrix instruction applies exactly):
// the e4m3 grid is the same in every binade, so normal values keep their relative
// precision, and the attention kernel can apply the V scale without rounding it
// into the probabilities.
//
// One workgroup per (batch, head, token block). Each thread owns chunks of 4 consecutive
// elements of a row, consecutive lanes holding consecutive chunks, so that every wave
// load is one contiguous 1 KiB run (fp32; 512 B for bf16) and every store of 4 codes a
// contiguous 256 B run; both carry the nontemporal hint (x is read once, the codes are
// read by a later kernel). The block stays in registers between the absmax reduction
// and the conversion, so HBM sees one read of x and one write of the codes. The
// rotation is a fast Walsh-Hadamard transform: 2 butterfly stages inside a thread, 5
// across the 32 lanes that hold one 128-wide row.
#include "device.h"
#include "launch.h"

namespace zyfa {

constexpr int kQThreads = 256;

template <int D, int BLOCK, bool BF16IN, bool HAD>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales, int S, int nb) {
  constexpr int CPR = D / 4;                                       // 4-element chunks per row
  constexpr int NCH = (BLOCK * CPR + kQThreads - 1) / kQThreads;  // chunks per thread
  static_assert(!HAD || D == 128, "rotation is defined for D = 128");
  static_assert(BLOCK * CPR % kQThreads == 0, "chunks split evenly over the threads");
  __shared__ float red[kQThreads / 64];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / nb;
  const int blk = blockIdx.x - bh * nb;
  const int t0 = blk * BLOCK;
  const int ntok = min(BLOCK, S - t0);
  const size_t base = ((size_t)bh * S + t0) * D;  // element offset of the block's first token

  float vals[NCH][4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * kQThreads;
    const int row = c / CPR;
    const int col = (c % CPR) * 4;
    if (row < ntok) {
      if constexpr (BF16IN) {
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        const v2u w = __builtin_nontemporal_load((const v2u*)((const uint16_t*)x + base + (size_t)row * D + col));
        vals[i][0] = __builtin_bit_cast(float, w[0] << 16);
        vals[i][1] = __builtin_bit_cast(float, w[0] & 0xFFFF0000u);
        vals[i][2] = __builtin_bit_cast(float, w[1] << 16);
        vals[i][3] = __builtin_bit_cast(float, w[1] & 0xFFFF0000u);
      } else {
        const v4f a = __builtin_nontemporal_load((const v4f*)((const float*)x + base + (size_t)row * D + col));
#pragma unroll
        for (int j = 0; j < 4; ++j) vals[i][j] = a[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) vals[i][j] = 0.0f;
    }
    if constexpr (HAD) {
      // stages 1, 2 inside the thread (Sylvester order: the upper index gets a - b)
#pragma unroll
      for (int s = 1; s < 4; s <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!(j & s)) {
            const float a = vals[i][j], b = vals[i][j + s];
            vals[i][j] = a + b;
            vals[i][j + s] = a - b;
          }
      // stages 4 .. 64 across the 32 lanes of the row (lane bit = element bit - 2)
#pragma unroll
      for (int s = 1; s < 32; s <<= 1) {
        const bool upper = (tid & s) != 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float other = __shfl_xor(vals[i][j], s, 64);
          vals[i][j] = upper ? other - vals[i][j] : vals[i][j] + other;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) vals[i][j] *= 0.08838834764831845f;  // 1 / sqrt(128)
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(vals[i][j]));
  }

  // block absmax
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) amax = fmaxf(amax, red[w]);

  // s = 2^k, the least power of two with amax <= 448 * 2^k (k >= -126), or 1 when
  // amax == 0. With amax = m * 2^E, m in [1, 2): 448 * 2^k = 1.75 * 2^(k + 8), so
  // k = E - 8, plus one when m > 1.75.
  int k = 0;
  if (amax > 0.0f) {
    int ex;
    const float fr = frexpf(amax, &ex);  // amax = fr * 2^ex, fr in [0.5, 1)
    k = max(ex - 9 + (fr > 0.875f ? 1 : 0), -126);
  }
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, k);

#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * kQThreads;
    const int row = c / CPR;
    const int col = (c % CPR) * 4;
    if (row < ntok) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(ldexpf(vals[i][j], -k), -448.0f), 448.0f);  // exact quotient
      const int w = cvt_pk_fp8<true>(y[2], y[3], cvt_pk_fp8<false>(y[0], y[1], 0));
      __builtin_nontemporal_store((unsigned)w, (unsigned*)(codes + base + (size_t)row * D + col));
    }
  }
}

template <int D, int BLOCK, bool BF16IN, bool HAD>
static hipError_t launch_q(const QuantArgs& a, hipStream_t stream) {
  const int nb = (a.S + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.B * a.H * nb;
  hipLaunchKernelGGL((quantize_kernel<D, BLOCK, BF16IN, HAD>), dim3((unsigned)grid), dim3(kQThreads), 0, stream,
                     a.x, a.codes, a.scales, a.S, nb);
  return hipGetLastError();
}

template <int D, int BLOCK>
static hipError_t launch_q_d(const QuantArgs& a, hipStream_t stream) {
  if (a.x_is_bf16) return a.hadamard ? launch_q<D, BLOCK, true, D == 128>(a, stream) : launch_q<D, BLOCK, true, false>(a, stream);
  return a.hadamard ? launch_q<D, BLOCK, false, D == 128>(a, stream) : launch_q<D, BLOCK, false, false>(a, stream);
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.scale_block == 64 ? launch_q_d<128, 64>(a, stream) : launch_q_d<128, 128>(a, stream);
  return a.scale_block == 64 ? launch_q_d<192, 64>(a, stream) : launch_q_d<192, 128>(a, stream);
}

}  // namespace zyfa
