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
// One workgroup per (batch, head, token block); in the plain passes and the rotation of
// order 128, 16 lanes per row, each lane holding chunks of 4 consecutive elements, so that
// a wave's load covers whole 64-byte runs of 4 rows (whole cache lines); loads and stores
// carry the nontemporal hint (x is read once, the codes are read by a later kernel). The
// block stays in registers between the absmax reduction and the conversion, so HBM sees one
// read of x and one write of the codes; full blocks load without per-row guards, and two or
// more workgroups share a CU so that one's loads overlap another's arithmetic. There are
// three kernels: quantize_d128_kernel (D = 128, the rotation a compile-time option),
// quantize_d192_kernel (D = 192, plain) and quantize_d192_rot_kernel (D = 192, rotated, with
// a lane layout of its own); their lane layouts put the transforms' cross-lane steps on
// cheap lane exchanges.
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

// Plain pass: one workgroup per (batch, head, token block); 16 lanes per row. Lane l = 4 A + C
// of a row holds the three 16-byte chunks at elements 64 k + 16 A + 4 C (k < 3), so that a
// row's 16 lanes load 256 contiguous bytes per k.
constexpr int kR192Threads = 512;  // 32 rows at a time: 4 (or 2) rows per thread; two workgroups fit a CU

template <int BLOCK, bool BF16IN>
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

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[i][k][j]));

  // block absmax and its power-of-two scale; the product with 2^-ks is an exact shift
  const int ks = block_scale_exponent<kR192Threads>(amax, red);
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, ks);
  const float f = ldexpf(1.0f, -ks);

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

// Rotated pass: four lanes per row. Lane C (< 4) of a row holds b = 4 C + j (j < 4) of all
// twelve a: the twelve 16-byte chunks at elements 16 a + 4 C. H_16 then has its stages on j
// inside the thread and its stages on C on DPP quad exchanges, and P_12 runs inside the
// thread with compile-time signs, in the short form that Paley's construction allows: with
// X[f] = x[f + 1] (f < 11, read as an element of GF(11)), T the sum of the X and U = x[0] - T,
//   y[0] = U,   y[f' + 1] = U + 2 (X[f'] + sum over the quadratic residues d of X[f' - d]),
// since the core's sum of chi(f' - f) X[f] is twice the residue sum minus (T - X[f']), and
// the diagonal and the first row add X[f'] and x[0]. With the residues {1, 3, 4, 5, 9} the
// six-term sums share the pairs p[f] = X[f] + X[f - 1] and the triples p[f] + X[f - 2]: 66
// additions for the twelve outputs where the sign-by-sign form takes 132. With float32
// input a lane's load covers 64 bytes of each of 16 rows, half of a 128-byte line, and the
// line's other half comes with the next chunk's load: these loads carry no nontemporal hint,
// with which the pass took about 5 % longer. Bfloat16 rows come in through LDS (below), and
// the codes go out through LDS in 64-byte row runs.
// Against the sign-by-sign form on the 16-lanes-a-row layout (36 multiply-adds with lane
// signs and 9 exchanges per column of a lane), the pass runs about 4 % slower at settled
// clocks and 10 % faster just after the GPU has been idle, when that form's arithmetic
// made it a fifth slower than the plain pass.
constexpr int kResidues[5] = {1, 3, 4, 5, 9};

// The short form on integer inputs, checked against P_12 on every unit vector at compile time.
constexpr bool paley12_short_form_holds() {
  for (int d : kResidues)
    if (gf11_chi(d) != 1) return false;
  for (int a = 0; a < 12; ++a) {
    int x[12] = {};
    x[a] = 1;
    int T = 0;
    for (int f = 0; f < 11; ++f) T += x[f + 1];
    const int U = x[0] - T;
    for (int o = 0; o < 12; ++o) {
      int y = U;
      if (o > 0) {
        const int fo = o - 1;
        const int p0 = x[1 + fo] + x[1 + (fo + 10) % 11];                                  // d = 0, 1
        const int t3 = x[1 + (fo + 8) % 11] + x[1 + (fo + 7) % 11] + x[1 + (fo + 6) % 11];  // d = 3, 4, 5
        y += 2 * (p0 + t3 + x[1 + (fo + 2) % 11]);                                          // d = 9
      }
      if (y != paley12(a, o)) return false;
    }
  }
  return true;
}
static_assert(paley12_short_form_holds(), "P_12 short form");

template <int BLOCK, bool BF16IN>
__global__ __launch_bounds__(4 * BLOCK) void quantize_d192_rot_kernel(const void* __restrict__ x,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ scales, int S, int nb) {
  constexpr int D = 192, kThreads = 4 * BLOCK;
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x, C = tid & 3, row = tid >> 2;
  const int bh = blockIdx.x / nb;
  const int blk = blockIdx.x - bh * nb;
  const int t0 = blk * BLOCK;
  const int ntok = min(BLOCK, S - t0);
  const bool live = ntok == BLOCK || row < ntok;
  const size_t off = ((size_t)bh * S + t0 + row) * D + 4 * C;  // this lane's first chunk
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  // The workgroup's rows in LDS, kRowWords words apart: the codes on their way out and,
  // with bfloat16 input, the input on its way in. A wave uses only its own 16 rows, so
  // ordering within the wave is all the staging needs.
  constexpr int kRowWords = BF16IN ? 104 : 52;
  __shared__ unsigned rows_lds[BLOCK * kRowWords];
  unsigned* const srow = rows_lds + row * kRowWords;

  float v[12][4];
  if constexpr (BF16IN) {
    // A bfloat16 chunk is 8 bytes, so loads in the lane layout would cover 32 bytes of each
    // of 16 rows. A wave's 16 rows are 6 KiB of contiguous input instead: six loads of 16
    // bytes a lane, each a contiguous KiB, go to the wave's LDS rows (104 words apart: 16-byte
    // aligned, and the 8-byte reads below take the four passes their 512 bytes need), and
    // each lane reads its chunks from there. Rows past the tensor's end hold zeros.
    const int wrow0 = (tid >> 6) * 16, l = tid & 63;
    const char* const src = (const char*)x + ((size_t)bh * S + t0 + wrow0) * (2 * D);
    char* const dst = (char*)(rows_lds + wrow0 * kRowWords);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int byte = 1024 * i + 16 * l;  // within the wave's 6 KiB
      const int rr = byte / (2 * D), cc = byte - rr * (2 * D);
      v4u w = v4u{0u, 0u, 0u, 0u};
      if (ntok == BLOCK || wrow0 + rr < ntok) w = *(const v4u*)(src + byte);
      *(v4u*)(dst + rr * (4 * kRowWords) + cc) = w;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int a = 0; a < 12; ++a) {
      const v2u w = *(const v2u*)((const char*)srow + 32 * a + 8 * C);
      v[a][0] = __builtin_bit_cast(float, w[0] << 16);
      v[a][1] = __builtin_bit_cast(float, w[0] & 0xFFFF0000u);
      v[a][2] = __builtin_bit_cast(float, w[1] << 16);
      v[a][3] = __builtin_bit_cast(float, w[1] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int a = 0; a < 12; ++a) {
      if (!live) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[a][j] = 0.0f;
      } else {
        const v4f w = *(const v4f*)((const float*)x + off + 16 * a);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[a][j] = w[j];
      }
    }
  }

  // H_16 over b = 4 C + j: stages on j inside the thread, on C across lanes
#pragma unroll
  for (int a = 0; a < 12; ++a)
#pragma unroll
    for (int s = 1; s < 4; s <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!(j & s)) {
          const float lo = v[a][j], hi = v[a][j + s];
          v[a][j] = lo + hi;
          v[a][j + s] = lo - hi;
        }
  const float sc1 = (C & 1) ? -1.0f : 1.0f, sc2 = (C & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int a = 0; a < 12; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) v[a][j] = fmaf(sc1, v[a][j], lane_xor<1>(v[a][j]));
#pragma unroll
  for (int a = 0; a < 12; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) v[a][j] = fmaf(sc2, v[a][j], lane_xor<2>(v[a][j]));

  // P_12 over a, for each b, in the short form
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float X[11], p[11], t[11];
#pragma unroll
    for (int f = 0; f < 11; ++f) X[f] = v[f + 1][j];
    const float T = ((X[0] + X[1]) + (X[2] + X[3])) + ((X[4] + X[5]) + (X[6] + X[7])) + ((X[8] + X[9]) + X[10]);
    const float U = v[0][j] - T;
#pragma unroll
    for (int f = 0; f < 11; ++f) p[f] = X[f] + X[(f + 10) % 11];
#pragma unroll
    for (int f = 0; f < 11; ++f) t[f] = p[f] + X[(f + 9) % 11];
    v[0][j] = U;
#pragma unroll
    for (int f = 0; f < 11; ++f) v[f + 1][j] = fmaf(2.0f, (p[f] + t[(f + 8) % 11]) + X[(f + 2) % 11], U);
  }

  float amax = 0.0f;
#pragma unroll
  for (int a = 0; a < 12; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[a][j]));

  // block absmax and the power-of-two scale of the values times 1/sqrt(192); the final
  // product applies (1/sqrt(192)) 2^-ks at once, which rounds as the two products would
  // (2^-ks is an exact shift), and stays within +-448
  constexpr float kNorm = 0.07216878364870323f;  // 1/sqrt(192)
  const int ks = block_scale_exponent<kThreads>(amax * kNorm, red);
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, ks);
  const float f = ldexpf(kNorm, -ks);
  // The codes go through the row's LDS words: lane C writes its 4 bytes of each a (bytes
  // 16 a + 4 C of the row), then reads bytes 64 m + 16 C (m < 3), so that a row's four lanes
  // store 64 contiguous bytes per instruction rather than four 4-byte pieces 16 bytes apart.
  // (52 words apart, the writes of a wave's 16 rows spread over all 32 banks.) A row is
  // written and read by its own four lanes only; with bfloat16 input its input words were
  // all read before: a wave's LDS operations complete in order.
#pragma unroll
  for (int a = 0; a < 12; ++a)
    srow[4 * a + C] = cvt_pk_fp8<true>(v[a][2] * f, v[a][3] * f, cvt_pk_fp8<false>(v[a][0] * f, v[a][1] * f, 0));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (live) {
    const size_t out = off - 4 * C;  // the row's first code
#pragma unroll
    for (int m = 0; m < 3; ++m)
      __builtin_nontemporal_store(*(const v4u*)(srow + 16 * m + 4 * C), (v4u*)(codes + out + 64 * m + 16 * C));
  }
}

template <int D, int BLOCK, bool BF16IN, bool HAD>
static hipError_t launch_q(const QuantArgs& a, hipStream_t stream) {
  const int nb = (a.S + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.B * a.H * nb;
  if constexpr (D == 192 && HAD) {
    hipLaunchKernelGGL((quantize_d192_rot_kernel<BLOCK, BF16IN>), dim3((unsigned)grid), dim3(4 * BLOCK), 0, stream,
                       a.x, a.codes, a.scales, a.S, nb);
  } else if constexpr (D == 192) {
    hipLaunchKernelGGL((quantize_d192_kernel<BLOCK, BF16IN>), dim3((unsigned)grid), dim3(kR192Threads), 0, stream,
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
