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
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace zyfa {

constexpr int kQThreads = 256;

// threads per workgroup: the rotation keeps more live values per element, so its blocks are
// spread over twice the threads (fewer registers per thread, more waves in flight)
template <bool HAD>
constexpr int quant_threads() { return HAD ? 2 * kQThreads : kQThreads; }

template <int D, int BLOCK, bool BF16IN, bool HAD>
__global__ __launch_bounds__(quant_threads<HAD>()) void quantize_kernel(const void* __restrict__ x,
                                                                       uint8_t* __restrict__ codes,
                                                                       float* __restrict__ scales, int S, int nb) {
  constexpr int kQThreads = quant_threads<HAD>();
  constexpr int CPR = D / 4;                                       // 4-element chunks per row
  constexpr int NCH = (BLOCK * CPR + kQThreads - 1) / kQThreads;  // chunks per thread
  static_assert(!HAD || D == 128, "this kernel rotates D = 128 rows; D = 192 has quantize_rot192_kernel");
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
      auto stage = [&](auto s_tag) {
        constexpr int s = decltype(s_tag)::value;
        const bool upper = (tid & s) != 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float other = lane_xor<s>(vals[i][j]);
          vals[i][j] = upper ? other - vals[i][j] : vals[i][j] + other;
        }
      };
      stage(std::integral_constant<int, 1>{});
      stage(std::integral_constant<int, 2>{});
      stage(std::integral_constant<int, 4>{});
      stage(std::integral_constant<int, 8>{});
      stage(std::integral_constant<int, 16>{});
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

// ---- the rotation of order 192 (the MLA query-key dimension) ----
// H_192 = P_12 (x) H_16: Paley's first construction of order 12 over GF(11), Kronecker
// times Sylvester's matrix of order 16; row element e = 16 a + b (a < 12, b < 16) maps to
// y[16 a' + b'] = sum_a P[a][a'] (sum_b x[16 a + b] H16[b][b']) / sqrt(192).

// quadratic character of GF(11): 0 at 0, +1 on the nonzero squares, -1 elsewhere
constexpr int gf11_chi(int x) {
  x = ((x % 11) + 11) % 11;
  if (x == 0) return 0;
  for (int y = 1; y < 11; ++y)
    if ((y * y) % 11 == x) return 1;
  return -1;
}
// Paley's first construction: H = I + S, S zero at the corner, +1 along the rest of the
// first row, -1 down the rest of the first column, chi(j - i) elsewhere
constexpr int paley12(int i, int j) {
  if (i == j) return 1;
  if (i == 0) return 1;
  if (j == 0) return -1;
  return gf11_chi(j - i);
}

// One workgroup per (batch, head, token block); 16 lanes per row. Lane l = 4 A + C of a
// row holds the 3 x 4 elements a = 3 A + k (k < 3), b = 4 C + j (j < 4): three 16-byte
// chunks. H_16 acts on b: bits j in the thread, bits C across lanes l ^ 1, l ^ 2. P_12 acts
// on a: each lane forms the partial sums of its three a's for all twelve outputs, then a
// reduce-scatter across lanes l ^ 8 and l ^ 4 leaves it the full sums for a' = 3 A + k,
// the positions it loaded.
constexpr int kR192Threads = 1024;  // 64 rows at a time: 2 (or 1) rows per thread

template <int BLOCK, bool BF16IN>
__global__ __launch_bounds__(kR192Threads) void quantize_rot192_kernel(const void* __restrict__ x,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ scales, int S, int nb) {
  constexpr int D = 192;
  constexpr int NR = BLOCK / (kR192Threads / 16);  // rows per thread
  __shared__ float red[kR192Threads / 64];
  const int tid = threadIdx.x;
  const int l = tid & 15, A = l >> 2, C = l & 3;
  const int bh = blockIdx.x / nb;
  const int blk = blockIdx.x - bh * nb;
  const int t0 = blk * BLOCK;
  const int ntok = min(BLOCK, S - t0);
  const size_t base = ((size_t)bh * S + t0) * D;

  // this lane's Paley signs P[3 A + k][a'] (A differs between lanes)
  float sgn[3][12];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int ap = 0; ap < 12; ++ap) {
      const int s0 = paley12(k, ap), s1 = paley12(3 + k, ap), s2 = paley12(6 + k, ap), s3 = paley12(9 + k, ap);
      const int sv = A == 0 ? s0 : A == 1 ? s1 : A == 2 ? s2 : s3;
      sgn[k][ap] = (float)sv;
    }

  float v[NR][3][4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = (tid >> 4) + i * (kR192Threads / 16);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int col = 16 * (3 * A + k) + 4 * C;
      if (row < ntok) {
        if constexpr (BF16IN) {
          typedef unsigned v2u __attribute__((ext_vector_type(2)));
          const v2u w = __builtin_nontemporal_load((const v2u*)((const uint16_t*)x + base + (size_t)row * D + col));
          v[i][k][0] = __builtin_bit_cast(float, w[0] << 16);
          v[i][k][1] = __builtin_bit_cast(float, w[0] & 0xFFFF0000u);
          v[i][k][2] = __builtin_bit_cast(float, w[1] << 16);
          v[i][k][3] = __builtin_bit_cast(float, w[1] & 0xFFFF0000u);
        } else {
          const v4f a = __builtin_nontemporal_load((const v4f*)((const float*)x + base + (size_t)row * D + col));
#pragma unroll
          for (int j = 0; j < 4; ++j) v[i][k][j] = a[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][k][j] = 0.0f;
      }
      // H_16 over b = 4 C + j: stages on j inside the thread, on C across lanes
#pragma unroll
      for (int s = 1; s < 4; s <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!(j & s)) {
            const float a = v[i][k][j], b = v[i][k][j + s];
            v[i][k][j] = a + b;
            v[i][k][j + s] = a - b;
          }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float o1 = lane_xor<1>(v[i][k][j]);
        v[i][k][j] = (C & 1) ? o1 - v[i][k][j] : v[i][k][j] + o1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float o2 = lane_xor<2>(v[i][k][j]);
        v[i][k][j] = (C & 2) ? o2 - v[i][k][j] : v[i][k][j] + o2;
      }
    }
    // P_12 over a = 3 A + k, for each b
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float part[12];
#pragma unroll
      for (int ap = 0; ap < 12; ++ap)
        part[ap] = fmaf(v[i][0][j], sgn[0][ap], fmaf(v[i][1][j], sgn[1][ap], v[i][2][j] * sgn[2][ap]));
      // lanes A < 2 keep a' < 6, lanes A >= 2 keep a' >= 6; each receives its partner's
      // partial sums for the half it keeps
      const bool hi2 = A >= 2;
      float kept[6];
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const float keep = hi2 ? part[6 + u] : part[u];
        const float send = hi2 ? part[u] : part[6 + u];
        kept[u] = keep + lane_xor<8>(send);
      }
      const bool odd = (A & 1) != 0;
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const float keep = odd ? kept[3 + u] : kept[u];
        const float send = odd ? kept[u] : kept[3 + u];
        v[i][u][j] = (keep + lane_xor<4>(send)) * 0.07216878364870323f;  // 1 / sqrt(192)
      }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[i][k][j]));
  }

  // block absmax and the power-of-two scale, as in quantize_kernel
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kR192Threads / 64; ++w) amax = fmaxf(amax, red[w]);
  int ks = 0;
  if (amax > 0.0f) {
    int ex;
    const float fr = frexpf(amax, &ex);
    ks = max(ex - 9 + (fr > 0.875f ? 1 : 0), -126);
  }
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, ks);

#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = (tid >> 4) + i * (kR192Threads / 16);
    if (row < ntok) {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(ldexpf(v[i][k][j], -ks), -448.0f), 448.0f);
        const int w = cvt_pk_fp8<true>(y[2], y[3], cvt_pk_fp8<false>(y[0], y[1], 0));
        __builtin_nontemporal_store((unsigned)w,
                                    (unsigned*)(codes + base + (size_t)row * D + 16 * (3 * A + k) + 4 * C));
      }
    }
  }
}

template <int D, int BLOCK, bool BF16IN, bool HAD>
static hipError_t launch_q(const QuantArgs& a, hipStream_t stream) {
  const int nb = (a.S + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.B * a.H * nb;
  if constexpr (D == 192 && HAD) {
    hipLaunchKernelGGL((quantize_rot192_kernel<BLOCK, BF16IN>), dim3((unsigned)grid), dim3(kR192Threads), 0, stream, a.x,
                       a.codes, a.scales, a.S, nb);
  } else {
    hipLaunchKernelGGL((quantize_kernel<D, BLOCK, BF16IN, HAD>), dim3((unsigned)grid), dim3(quant_threads<HAD>()), 0, stream,
                       a.x, a.codes, a.scales, a.S, nb);
  }
  return hipGetLastError();
}

template <int D, int BLOCK>
static hipError_t launch_q_d(const QuantArgs& a, hipStream_t stream) {
  if (a.x_is_bf16) return a.hadamard ? launch_q<D, BLOCK, true, true>(a, stream) : launch_q<D, BLOCK, true, false>(a, stream);
  return a.hadamard ? launch_q<D, BLOCK, false, true>(a, stream) : launch_q<D, BLOCK, false, false>(a, stream);
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.scale_block == 64 ? launch_q_d<128, 64>(a, stream) : launch_q_d<128, 128>(a, stream);
  return a.scale_block == 64 ? launch_q_d<192, 64>(a, stream) : launch_q_d<192, 128>(a, stream);
}

}  // namespace zyfa
