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
// One workgroup of 512 threads per (batch, head, token block); 16 lanes per row, each
// lane holding chunks of 4 consecutive elements, so that a wave's load covers whole
// 64-byte runs of 4 rows (whole cache lines); loads and stores carry the nontemporal hint
// (x is read once, the codes are read by a later kernel). The block stays in registers
// between the absmax reduction and the conversion, so HBM sees one read of x and one write
// of the codes; full blocks load without per-row guards, and two or more workgroups share a
// CU so that one's loads overlap another's arithmetic. There are two kernels, one per head
// dimension (quantize_d128_kernel, quantize_d192_kernel), each with the rotation as a
// compile-time option: their lane layouts put the transforms' cross-lane steps on cheap
// lane exchanges.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace zyfa {

// The block's absmax (this thread's amax reduced over the workgroup of T threads; red holds
// T / 64 floats of LDS) and k, the exponent of the block scale 2^k: the least power of two
// with amax <= 448 * 2^k (k >= -126), or 1 when amax == 0. With amax = m * 2^E, m in
// [1, 2): 448 * 2^k = 1.75 * 2^(k + 8), so k = E - 8, plus one when m > 1.75.
template <int T>
__device__ __forceinline__ int block_scale_exponent(float amax, float* red) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) amax = fmaxf(amax, red[w]);
  int k = 0;
  if (amax > 0.0f) {
    int ex;
    const float fr = frexpf(amax, &ex);  // amax = fr * 2^ex, fr in [0.5, 1)
    k = max(ex - 9 + (fr > 0.875f ? 1 : 0), -126);
  }
  return k;
}

// ---- D = 128: plain, or the rotation of order 128 (Sylvester) ----
// y = x H_128 / sqrt(128) with H_128[e][e'] = (-1)^popcount(e & e'): one butterfly stage per
// bit of the element index, the element with the bit clear getting a + b and the other
// a - b. A row is held by 16 lanes, two chunks of four elements per lane (elements 4 c + j
// and 64 + 4 c + j, c < 16), so that element bits 0, 1 (j) and 6 (the chunk) are stages
// inside the thread and bits 2..5 (c) stages across lanes. The lanes holding c are chosen
// so that every exchange is cheap: c bits 0, 1 on lane bits 0, 1 (DPP quad permutations),
// c bit 2 on lane bit 3 (a DPP rotation of the 16-lane row by 8, which is lane ^ 8), c bit 3
// on lane bit 4 (v_permlane16_swap); lane bits 2 and 5 select one of four rows. A wave's
// load of a chunk then covers the same half of four consecutive rows (whole cache lines).
// A cross-lane butterfly is one fused multiply-add: new = s v + partner's v, with s = +1 in
// the lane whose element bit is clear and -1 in the other. The 1/sqrt(128) is applied with
// the power-of-two scale in one product, which rounds exactly as the two products would
// (multiplying by 2^-k is exact).
constexpr int kR128Threads = 512;

template <int BLOCK, bool BF16IN, bool HAD>
__global__ __launch_bounds__(kR128Threads) void quantize_d128_kernel(const void* __restrict__ x,
                                                                  uint8_t* __restrict__ codes,
                                                                  float* __restrict__ scales, int S, int nb) {
  constexpr int D = 128;
  constexpr int RPR = kR128Threads / 16;  // rows per round
  constexpr int NR = BLOCK / RPR;         // rounds
  constexpr int NV = 8 * NR;              // values per thread
  static_assert(BLOCK % RPR == 0, "rows split evenly over the rounds");
  __shared__ float red[kR128Threads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = (lane & 3) | ((lane >> 1) & 0xC);           // lane bits 0, 1, 3, 4 -> chunk bits 0..3
  const int rsub = ((lane >> 2) & 1) | ((lane >> 4) & 2);  // lane bits 2, 5 -> row within the wave's four
  const int bh = blockIdx.x / nb;
  const int blk = blockIdx.x - bh * nb;
  const int t0 = blk * BLOCK;
  const int ntok = min(BLOCK, S - t0);
  const size_t base = ((size_t)bh * S + t0) * D;
  auto row_of = [&](int i) { return (i * (kR128Threads / 64) + wave) * 4 + rsub; };

  // v[8 i + 4 hf + j]: element 64 hf + 4 c + j of row row_of(i)
  float v[NV];
  auto load = [&](int i, int hf, bool live) {
    const size_t off = base + (size_t)row_of(i) * D + 64 * hf + 4 * c;
    float* d = v + 8 * i + 4 * hf;
    if (!live) {
      d[0] = d[1] = d[2] = d[3] = 0.0f;
    } else if constexpr (BF16IN) {
      typedef unsigned v2u __attribute__((ext_vector_type(2)));
      const v2u w = __builtin_nontemporal_load((const v2u*)((const uint16_t*)x + off));
      d[0] = __builtin_bit_cast(float, w[0] << 16);
      d[1] = __builtin_bit_cast(float, w[0] & 0xFFFF0000u);
      d[2] = __builtin_bit_cast(float, w[1] << 16);
      d[3] = __builtin_bit_cast(float, w[1] & 0xFFFF0000u);
    } else {
      const v4f a = __builtin_nontemporal_load((const v4f*)((const float*)x + off));
      d[0] = a[0];
      d[1] = a[1];
      d[2] = a[2];
      d[3] = a[3];
    }
  };
  if (ntok == BLOCK) {  // (uniform) every row of a full block is loaded unguarded
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) load(i, hf, true);
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) load(i, hf, row_of(i) < ntok);
  }

  // Stages in order, each over all of the thread's values (independent neighbours, so the
  // cross-lane moves wait for nothing). Inside the thread: element bits 0, 1 (j), 6 (hf).
  constexpr float kNorm = HAD ? 0.08838834764831845f : 1.0f;  // 1/sqrt(128)
  if constexpr (HAD) {
#pragma unroll
  for (int sb = 1; sb <= 4; sb <<= 1)
#pragma unroll
    for (int e = 0; e < NV; ++e)
      if (!(e & sb)) {
        const float a = v[e], b = v[e + sb];
        v[e] = a + b;
        v[e + sb] = a - b;
      }
  // Across lanes: element bits 2, 3 (lane bits 0, 1: DPP quad permutations), 4 (lane bit 3:
  // the row rotation by 8), 5 (lane bit 4: ds_swizzle xor 16); new = s v + partner's v.
  auto stage = [&](auto m_tag, bool upper) {
    constexpr int M = decltype(m_tag)::value;
    const float sg = upper ? -1.0f : 1.0f;
    float p[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) p[e] = M == 16 ? lane_xor_swizzle<16>(v[e]) : lane_xor<M>(v[e]);
#pragma unroll
    for (int e = 0; e < NV; ++e) v[e] = fmaf(sg, v[e], p[e]);
  };
  stage(std::integral_constant<int, 1>{}, (lane & 1) != 0);
  stage(std::integral_constant<int, 2>{}, (lane & 2) != 0);
  stage(std::integral_constant<int, 8>{}, (lane & 8) != 0);
  stage(std::integral_constant<int, 16>{}, (lane & 16) != 0);
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < NV; ++e) amax = fmaxf(amax, fabsf(v[e]));

  // scale of the block: its absmax times 1/sqrt(128) when rotated (the maximum of the
  // rounded products is the rounded product of the maximum); codes of the exact quotients
  // (a power-of-two shift) within +-448
  const int k = block_scale_exponent<kR128Threads>(amax * kNorm, red);
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, k);
  const float f = ldexpf(kNorm, -k);  // (1/sqrt(128)) 2^-k, exact power-of-two shift

  auto store = [&](int i, int hf) {
    const float* d = v + 8 * i + 4 * hf;
    const int w = cvt_pk_fp8<true>(d[2] * f, d[3] * f, cvt_pk_fp8<false>(d[0] * f, d[1] * f, 0));
    __builtin_nontemporal_store((unsigned)w, (unsigned*)(codes + base + (size_t)row_of(i) * D + 64 * hf + 4 * c));
  };
#pragma unroll
  for (int i = 0; i < NR; ++i)
    if (ntok == BLOCK || row_of(i) < ntok) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) store(i, hf);
    }
}

// ---- D = 192 (the MLA query-key dimension): plain, or the rotation of order 192 ----
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
// row holds the 3 x 4 elements a = A + 4 k (k < 3), b = 4 C + j (j < 4): three 16-byte
// chunks, elements 64 k + 16 A + 4 C + j, so that a row's 16 lanes load 256 contiguous bytes
// per k. H_16 acts on b: bits j in the thread, bits C across lanes l ^ 1, l ^ 2. P_12 acts
// on a: each lane forms the partial sums of its three a's for all twelve outputs, then a
// reduce-scatter across lanes l ^ 8 (A ^ 2) and l ^ 4 (A ^ 1) leaves it the full sums for
// a' = A + 4 k, the positions it loaded. The lane's twelve partial sums are kept in an
// order of its own (its sign table is permuted to match): positions 0..5 are the outputs
// it keeps after the exchange with A ^ 2, 0..2 of them the ones it keeps after the exchange
// with A ^ 1, and positions 6..11 (then 3..5) what its partner keeps, so every exchange
// sends the same register in both lanes and no value is selected per lane.
constexpr int kR192Threads = 512;  // 32 rows at a time: 4 (or 2) rows per thread; two workgroups fit a CU

template <int BLOCK, bool BF16IN, bool HAD>
__global__ __launch_bounds__(kR192Threads) void quantize_d192_kernel(const void* __restrict__ x,
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

  float v[NR][3][4];
  auto load = [&](int i, bool live) {
    const int row = (tid >> 4) + i * (kR192Threads / 16);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const size_t off = base + (size_t)row * D + 64 * k + 16 * A + 4 * C;
      if (!live) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][k][j] = 0.0f;
      } else if constexpr (BF16IN) {
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        const v2u w = __builtin_nontemporal_load((const v2u*)((const uint16_t*)x + off));
        v[i][k][0] = __builtin_bit_cast(float, w[0] << 16);
        v[i][k][1] = __builtin_bit_cast(float, w[0] & 0xFFFF0000u);
        v[i][k][2] = __builtin_bit_cast(float, w[1] << 16);
        v[i][k][3] = __builtin_bit_cast(float, w[1] & 0xFFFF0000u);
      } else {
        const v4f a = __builtin_nontemporal_load((const v4f*)((const float*)x + off));
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][k][j] = a[j];
      }
    }
  };
  if (ntok == BLOCK) {  // (uniform) every row of a full block is loaded unguarded
#pragma unroll
    for (int i = 0; i < NR; ++i) load(i, true);
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i) load(i, (tid >> 4) + i * (kR192Threads / 16) < ntok);
  }

  constexpr float kNorm = HAD ? 0.07216878364870323f : 1.0f;  // 1/sqrt(192)
  if constexpr (HAD) {
    // this lane's Paley signs P[A + 4 k][col(A, u)], in the lane's order of outputs: col(A, u)
    // = A + 4 u for u < 3, (A ^ 1) + 4 (u - 3) for u < 6 (kept after the A ^ 2 exchange), and
    // col(A ^ 2, u - 6) for u >= 6 (the partial sums sent to lane A ^ 2)
    float sgn[3][12];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int u = 0; u < 12; ++u) {
        auto sign_for = [&](int a) {  // compile-time signs of lane group a
          const int aa = u < 6 ? a : a ^ 2, uu = u < 6 ? u : u - 6;
          const int col = uu < 3 ? aa + 4 * uu : (aa ^ 1) + 4 * (uu - 3);
          return paley12(a + 4 * k, col);
        };
        const int s0 = sign_for(0), s1 = sign_for(1), s2 = sign_for(2), s3 = sign_for(3);
        sgn[k][u] = (float)(A == 0 ? s0 : A == 1 ? s1 : A == 2 ? s2 : s3);
      }
    const float sc1 = (C & 1) ? -1.0f : 1.0f, sc2 = (C & 2) ? -1.0f : 1.0f;  // H_16 signs across lanes
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      // H_16 over b = 4 C + j: stages on j inside the thread, on C across lanes
#pragma unroll
      for (int k = 0; k < 3; ++k)
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
      for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][k][j] = fmaf(sc1, v[i][k][j], lane_xor<1>(v[i][k][j]));
#pragma unroll
      for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][k][j] = fmaf(sc2, v[i][k][j], lane_xor<2>(v[i][k][j]));
      // P_12 over a = A + 4 k, for each b
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float part[12];
#pragma unroll
        for (int u = 0; u < 12; ++u)
          part[u] = fmaf(v[i][0][j], sgn[0][u], fmaf(v[i][1][j], sgn[1][u], v[i][2][j] * sgn[2][u]));
        // lane A ^ 2 sends its positions 6..11: its partial sums of this lane's positions 0..5
#pragma unroll
        for (int u = 0; u < 6; ++u) part[u] += lane_xor<8>(part[6 + u]);
        // lane A ^ 1 sends its positions 3..5: its partial sums of this lane's 0..2
#pragma unroll
        for (int u = 0; u < 3; ++u) v[i][u][j] = part[u] + lane_xor_swizzle<4>(part[3 + u]);
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[i][k][j]));

  // block absmax and the power-of-two scale of the values times 1/sqrt(192) (rotated) or
  // of the values; the final product applies (1/sqrt(192)) 2^-ks at once, which rounds as
  // the two products would (2^-ks is an exact shift), and stays within +-448
  const int ks = block_scale_exponent<kR192Threads>(amax * kNorm, red);
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, ks);
  const float f = ldexpf(kNorm, -ks);

#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = (tid >> 4) + i * (kR192Threads / 16);
    if (ntok == BLOCK || row < ntok) {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int w = cvt_pk_fp8<true>(v[i][k][2] * f, v[i][k][3] * f,
                                       cvt_pk_fp8<false>(v[i][k][0] * f, v[i][k][1] * f, 0));
        __builtin_nontemporal_store((unsigned)w,
                                    (unsigned*)(codes + base + (size_t)row * D + 64 * k + 16 * A + 4 * C));
      }
    }
  }
}

template <int D, int BLOCK, bool BF16IN, bool HAD>
static hipError_t launch_q(const QuantArgs& a, hipStream_t stream) {
  const int nb = (a.S + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.B * a.H * nb;
  if constexpr (D == 192) {
    hipLaunchKernelGGL((quantize_d192_kernel<BLOCK, BF16IN, HAD>), dim3((unsigned)grid), dim3(kR192Threads), 0, stream,
                       a.x, a.codes, a.scales, a.S, nb);
  } else {
    hipLaunchKernelGGL((quantize_d128_kernel<BLOCK, BF16IN, HAD>), dim3((unsigned)grid), dim3(kR128Threads), 0, stream,
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
