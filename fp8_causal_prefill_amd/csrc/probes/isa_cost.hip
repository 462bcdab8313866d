// Instruction costs on gfx950 behind the attention kernels' design (a stand-alone program;
// prints one JSON object). Every kernel runs one workgroup per CU with one or two waves per
// SIMD, loops over registers only (no memory access inside the timed loop) and writes one
// value per thread to a sink buffer; cycles come from clock64 around the loop, and a SIMD's
// time is the longest of its waves'.
//
//  * matrix instructions: cycles per v_mfma_scale_f32_32x32x64_f8f6f4 / 16x16x128 with e4m3
//    and e2m1 operands (four independent accumulators, one wave per SIMD);
//  * vector instructions: SIMD cycles per wave64 instruction at two waves per SIMD (sixteen
//    independent chains per wave);
//  * overlap: one wave per SIMD issuing 8 matrix instructions and 8 N vector instructions
//    per iteration, against either alone;
//  * LDS reads: bytes per clock per CU for ds_read_b128 and the two transposing 64-bit
//    reads the attention kernels use for V (8-bit and 16-bit elements), four waves per
//    SIMD, each wave reading a contiguous run of addresses.
//
// Built a second time as a shared library (-DISA_COST_LIB, no main), the same kernels serve
// energy measurements: isa_energy_launch() runs one case on every CU of the chip for a given
// number of iterations on a caller's stream, so that a caller sampling the board's power can
// attribute energy to each instruction class (see the isa_energy_* declarations below).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4bf lds_v4bf;

#define CK(x)                                                                  \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

constexpr int kBlocks = 256;
constexpr int kMaxThreads = 1024;

// ---- matrix instructions ----
// (ONES_A: operand A is e2m1 1.0 in every element, as in the FP8 kernel's row-sum product)
template <int FA, int FB, bool BIG, bool ONES_A = false>
__global__ void mfma_rate(const int* in, long long* cyc, float* sink, int iters) {
  const int l = threadIdx.x & 63;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = ONES_A ? 0x22222222 : in[l * 8 + i];
    b[i] = in[(l ^ 5) * 8 + i];
  }
  int s0 = 127, s1 = 127;
  asm volatile("" : "+v"(s0), "+v"(s1));
  v4f c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  v16f d0 = {0}, d1 = {0}, d2 = {0}, d3 = {0};
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    if constexpr (BIG) {
      d0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d0, FA, FB, 0, s0, 0, s1);
      d1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d1, FA, FB, 0, s0, 0, s1);
      d2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d2, FA, FB, 0, s0, 0, s1);
      d3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d3, FA, FB, 0, s0, 0, s1);
    } else {
      c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, FA, FB, 0, s0, 0, s1);
      c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, FA, FB, 0, s0, 0, s1);
      c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, FA, FB, 0, s0, 0, s1);
      c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, FA, FB, 0, s0, 0, s1);
    }
  }
  const long long t1 = clock64();
  if (l == 0) cyc[blockIdx.x * 16 + (threadIdx.x >> 6)] = t1 - t0;
  float s = 0;
  for (int r = 0; r < 4; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  for (int r = 0; r < 16; ++r) s += d0[r] + d1[r] + d2[r] + d3[r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// bf16 32x32x16 (four independent accumulators, one wave per SIMD). Each 16-bit half of an
// input word gives one element: its sign and mantissa bits, and an exponent in [2^-15, 2^0]
// from four more of its bits (magnitudes like the attention kernels' operands; zero words
// give zero elements).
__device__ inline __bf16 probe_bf16(unsigned v) {
  const unsigned h = v & 0xffffu;
  return __builtin_bit_cast(__bf16, (unsigned short)(h == 0 ? 0 : (h & 0x807fu) | ((112u + ((h >> 7) & 15u)) << 7)));
}
__global__ void mfma_bf16_rate(const int* in, long long* cyc, float* sink, int iters) {
  const int l = threadIdx.x & 63;
  v8bf a, b;
  for (int i = 0; i < 4; ++i) {
    const unsigned x = (unsigned)in[l * 4 + i], y = (unsigned)in[(l ^ 5) * 4 + i];
    a[2 * i] = probe_bf16(x);
    a[2 * i + 1] = probe_bf16(x >> 16);
    b[2 * i] = probe_bf16(y);
    b[2 * i + 1] = probe_bf16(y >> 16);
  }
  v16f d0 = {0}, d1 = {0}, d2 = {0}, d3 = {0};
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d1, 0, 0, 0);
    d2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d2, 0, 0, 0);
    d3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d3, 0, 0, 0);
  }
  const long long t1 = clock64();
  if (l == 0) cyc[blockIdx.x * 16 + (threadIdx.x >> 6)] = t1 - t0;
  float s = 0;
  for (int r = 0; r < 16; ++r) s += d0[r] + d1[r] + d2[r] + d3[r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// ---- vector instructions (and optionally 8 matrix instructions per iteration) ----
template <int OP, int NV, bool MF>
__global__ void valu_rate(const int* in, long long* cyc, float* sink, int iters) {
  const int l = threadIdx.x & 63;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = in[l * 8 + i];
    b[i] = in[(l ^ 7) * 8 + i];
  }
  v16f m0 = {0}, m1 = {0}, m2 = {0}, m3 = {0};
  float x[16];
  int u[16];
  for (int i = 0; i < 16; ++i) {
    x[i] = (float)in[l + i] * 1e-6f + 0.5f + (float)i * 1e-3f;
    u[i] = in[l + i + 64];
  }
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if constexpr (MF) {
        v16f& c = (m & 3) == 0 ? m0 : (m & 3) == 1 ? m1 : (m & 3) == 2 ? m2 : m3;
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int i = (m * NV + v) & 15;
        if constexpr (OP == 0) x[i] = fmaf(x[i], 0.999f, 0.25f);
        else if constexpr (OP == 1) x[i] = __builtin_amdgcn_exp2f(-x[i]);  // stays in (0.5, 1)
        else if constexpr (OP == 2) u[i] = __builtin_amdgcn_cvt_pk_fp8_f32(x[i], x[(i + 1) & 15], u[i], false);
        else if constexpr (OP == 3) u[i] = __builtin_amdgcn_cvt_pk_u8_f32(x[i], 1, u[i]);
        else if constexpr (OP == 4) x[i] = fmaxf(fmaxf(x[i], x[(i + 1) & 15]), x[(i + 2) & 15]);
        else if constexpr (OP == 5) u[i] = __builtin_amdgcn_perm(u[i], u[(i + 1) & 15], 0x03020100u + i);
        else if constexpr (OP == 6) u[i] = __builtin_amdgcn_mov_dpp(u[i], 0xB1, 0xF, 0xF, true);
        else if constexpr (OP == 7) x[i] = fmaf(x[i], x[i], -1.9f);  // chaotic in [-1.9, 1.97]: bits keep changing
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const long long t1 = clock64();
  if (l == 0) cyc[blockIdx.x * 16 + (threadIdx.x >> 6)] = t1 - t0;
  float s = 0;
  for (int i = 0; i < 16; ++i) s += x[i] + (float)u[i] + m0[i] + m1[i] + m2[i] + m3[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// ---- LDS reads: 0 ds_read_b128, 1 ds_read_b64_tr_b8, 2 ds_read_b64_tr_b16 ----
// Sixteen waves per CU (four per SIMD); each keeps up to 16 reads in flight: batches of
// eight reads alternate between two register sets, the next batch issued before the
// current one is consumed.
constexpr int kLdsBytes = 65536;
template <int KIND>
__global__ void __launch_bounds__(1024) lds_rate(const int* in, long long* cyc, float* sink, int iters) {
  __shared__ __attribute__((aligned(16))) int lds[kLdsBytes / 4];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += blockDim.x) lds[i] = in[i & 4095] + i;
  __syncthreads();
  const unsigned lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* base = reinterpret_cast<const char*>(lds);
  constexpr unsigned kLaneBytes = KIND == 0 ? 16 : 8;
  // read r of batch j: one contiguous run of 64 * kLaneBytes bytes per wave; the mask keeps
  // every access inside the 64 KiB array (offset + kLaneBytes <= 65536)
  auto at = [&](int j, int r) {
    return base + (((unsigned)(j * 8 + r) * 4096u + wave * 1024u + lane * kLaneBytes) & (65536u - kLaneBytes));
  };
  auto load = [&](int j, int r) -> v4i {
    if constexpr (KIND == 0) {
      return *reinterpret_cast<const v4i*>(at(j, r));
    } else if constexpr (KIND == 1) {
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)at(j, r));
      return v4i{x[0], x[1], 0, 0};
    } else {
      const v2i x = __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)at(j, r)));
      return v4i{x[0], x[1], 0, 0};
    }
  };
  unsigned acc0 = 0, acc1 = 0;
  auto use = [&](const v4i& x) {
    acc0 += (unsigned)x[0] + (unsigned)x[1];
    if constexpr (KIND == 0) acc1 += (unsigned)x[2] + (unsigned)x[3];
  };
  v4i a[8], b[8];
  const long long t0 = clock64();
  // the clock read is a scalar memory instruction: waiting for it here keeps it from
  // forcing a full drain of the LDS counter inside the loop
  asm volatile("; clock %0" ::"s"(t0));
#pragma unroll
  for (int r = 0; r < 8; ++r) a[r] = load(0, r);
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int r = 0; r < 8; ++r) b[r] = load(it + 1, r);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 8; ++r) use(a[r]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 8; ++r) a[r] = load(it + 2, r);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 8; ++r) use(b[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) use(a[r]);
  const long long t1 = clock64();
  if (lane == 0) cyc[blockIdx.x * 16 + wave] = t1 - t0;
  sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc0 ^ acc1);
}

// ---- the softmax's vector work per wave-step of the exact FP8 kernel, on changing data ----
// Per iteration and lane: 32 scores advanced by s = s^2 - 1.9 (one FMA each; the map keeps
// s in [-1.9, 1.97] and chaotic, so operand bits change like those of real scores), their
// exponentials, the running row maximum over them (16 three-input maxima), and their e4m3
// codes (16 packing conversions): 96 vector instructions, the kernel's per-step mix without
// its bookkeeping.
__global__ void softmax_mix_rate(const int* in, long long* cyc, float* sink, int iters) {
  const int l = threadIdx.x & 63;
  float sc[32];
  for (int j = 0; j < 32; ++j) sc[j] = (float)(in[(l * 32 + j) & 4095] & 0xffff) * (3.8f / 65536.0f) - 1.9f;
  float m0 = -INFINITY, m1 = -INFINITY;
  int pk[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 32; ++j) sc[j] = fmaf(sc[j], sc[j], -1.9f);
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      m0 = fmaxf(fmaxf(m0, sc[2 * j]), sc[2 * j + 1]);
      m1 = fmaxf(fmaxf(m1, sc[2 * j + 2]), sc[2 * j + 3]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p0 = __builtin_amdgcn_exp2f(sc[4 * j]), p1 = __builtin_amdgcn_exp2f(sc[4 * j + 1]);
      const float p2 = __builtin_amdgcn_exp2f(sc[4 * j + 2]), p3 = __builtin_amdgcn_exp2f(sc[4 * j + 3]);
      pk[j] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pk[j], false), true);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const long long t1 = clock64();
  if (l == 0) cyc[blockIdx.x * 16 + (threadIdx.x >> 6)] = t1 - t0;
  int acc = 0;
  for (int j = 0; j < 8; ++j) acc ^= pk[j];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = m0 + m1 + (float)acc;
}

// ---- idle and scalar baselines for the energy cases ----
__global__ void sleep_loop(const int* in, long long* cyc, float* sink, int iters) {
  for (int it = 0; it < iters; ++it) __builtin_amdgcn_s_sleep(8);  // about 512 clocks
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * 16 + (threadIdx.x >> 6)] = iters;
  sink[blockIdx.x * blockDim.x + threadIdx.x] = 0.0f;
}

__global__ void salu_rate(const int* in, long long* cyc, float* sink, int iters) {
  unsigned x = (unsigned)in[blockIdx.x & 4095], y = (unsigned)in[(blockIdx.x + 1) & 4095];
  x = __builtin_amdgcn_readfirstlane(x);
  y = __builtin_amdgcn_readfirstlane(y);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("s_add_u32 %0, %0, %1" : "+s"(x) : "s"(y) : "scc");
  }
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * 16 + (threadIdx.x >> 6)] = x;
  sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)x;
}

static int* g_in;
static int* g_zero;
static long long* g_cyc;
static float* g_sink;

// the kernels' buffers and inputs: random bytes (no e4m3 NaN codes) and zeros
static hipError_t alloc_buffers() {
  hipError_t e;
  if ((e = hipMalloc(&g_in, 4096 * sizeof(int))) != hipSuccess) return e;
  if ((e = hipMalloc(&g_zero, 4096 * sizeof(int))) != hipSuccess) return e;
  if ((e = hipMalloc(&g_cyc, kBlocks * 16 * sizeof(long long))) != hipSuccess) return e;
  if ((e = hipMalloc(&g_sink, kBlocks * kMaxThreads * sizeof(float))) != hipSuccess) return e;
  static int h[4096];
  srand(1);
  for (int i = 0; i < 4096; ++i) {
    // four random bytes, each an e4m3 or two e2m1 codes: signs and mantissas as random as in
    // real operands, with e4m3's NaN codes (S.1111.111) moved to the largest finite ones
    unsigned w = ((unsigned)rand() << 16) ^ (unsigned)rand();
    for (int k = 0; k < 4; ++k)
      if (((w >> (8 * k)) & 0x7fu) == 0x7fu) w ^= 1u << (8 * k);
    h[i] = (int)w;
  }
  if ((e = hipMemcpy(g_in, h, sizeof(h), hipMemcpyHostToDevice)) != hipSuccess) return e;
  return hipMemset(g_zero, 0, 4096 * sizeof(int));
}

// mean over CUs of the slowest wave's cycles
template <class K>
static double simd_cycles(K kernel, int waves_per_simd, int iters) {
  const int threads = 256 * waves_per_simd;
  for (int rep = 0; rep < 2; ++rep) {  // the first launch warms the clock and the code
    hipLaunchKernelGGL(kernel, dim3(kBlocks), dim3(threads), 0, 0, g_in, g_cyc, g_sink, iters);
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
  }
  static long long h[kBlocks * 16];
  CK(hipMemcpy(h, g_cyc, sizeof(h), hipMemcpyDeviceToHost));
  double s = 0;
  for (int b = 0; b < kBlocks; ++b) {
    long long m = 0;
    for (int w = 0; w < 4 * waves_per_simd; ++w) m = h[b * 16 + w] > m ? h[b * 16 + w] : m;
    s += (double)m;
  }
  return s / kBlocks;
}

// ---- energy cases: every case runs one workgroup per CU (256), with the waves per SIMD
// given, for `iters` iterations; instructions are counted per wave64 instruction ----
typedef void (*ProbeKernel)(const int*, long long*, float*, int);
struct EnergyCase {
  const char* name;
  ProbeKernel kernel;
  int waves_per_simd;
  bool zero_input;
  double per_iteration;  // instructions of the measured class per wave and iteration
};
static const EnergyCase kEnergyCases[] = {
    {"idle (s_sleep, 2 waves per SIMD)", sleep_loop, 2, false, 0.0},
    {"s_add_u32 (2 waves per SIMD)", salu_rate, 2, false, 16.0},
    {"mfma 32x32x64 e4m3, random operands (1 wave per SIMD)", mfma_rate<0, 0, true>, 1, false, 4.0},
    {"mfma 32x32x64 e4m3, zero operands (1 wave per SIMD)", mfma_rate<0, 0, true>, 1, true, 4.0},
    {"mfma 32x32x64 e2m1 x e4m3, random operands (1 wave per SIMD)", mfma_rate<4, 0, true>, 1, false, 4.0},
    {"mfma 32x32x64 e2m1 ones x e4m3 random (1 wave per SIMD)", mfma_rate<4, 0, true, true>, 1, false, 4.0},
    {"mfma 32x32x16 bf16, random operands (1 wave per SIMD)", mfma_bf16_rate, 1, false, 4.0},
    {"mfma 32x32x16 bf16, zero operands (1 wave per SIMD)", mfma_bf16_rate, 1, true, 4.0},
    {"v_fma_f32, converging operands (2 waves per SIMD)", valu_rate<0, 8, false>, 2, false, 64.0},
    {"v_fma_f32 on chaotic operands, x = x * x - 1.9 (2 waves per SIMD)", valu_rate<7, 8, false>, 2, false, 64.0},
    {"v_exp_f32 (2 waves per SIMD)", valu_rate<1, 8, false>, 2, false, 64.0},
    {"v_cvt_pk_fp8_f32 (2 waves per SIMD)", valu_rate<2, 8, false>, 2, false, 64.0},
    {"v_max3_f32 (2 waves per SIMD)", valu_rate<4, 8, false>, 2, false, 64.0},
    {"softmax mix: 32 fma, 32 exp, 16 max3, 16 cvt_pk_fp8 on chaotic scores (2 waves per SIMD)", softmax_mix_rate, 2,
     false, 96.0},
    {"ds_read_b128 (4 waves per SIMD)", lds_rate<0>, 4, false, 8.0},
    {"ds_read_b64_tr_b8 (4 waves per SIMD)", lds_rate<1>, 4, false, 8.0},
    {"ds_read_b64_tr_b16 (4 waves per SIMD)", lds_rate<2>, 4, false, 8.0},
};
constexpr int kEnergyCaseCount = sizeof(kEnergyCases) / sizeof(kEnergyCases[0]);

extern "C" {
// number of energy cases, and the name of case i (null when i is out of range)
int isa_energy_case_count() { return kEnergyCaseCount; }
const char* isa_energy_case_name(int i) { return i >= 0 && i < kEnergyCaseCount ? kEnergyCases[i].name : nullptr; }
// wave64 instructions of the case's class that one launch of `iters` iterations executes
// (the LDS cases' loops take iterations in pairs and read one batch ahead: iters + 1 batches)
double isa_energy_case_instructions(int i, int iters) {
  if (i < 0 || i >= kEnergyCaseCount) return -1.0;
  const EnergyCase& c = kEnergyCases[i];
  const double waves = (double)kBlocks * 4 * c.waves_per_simd;
  const bool lds = c.kernel == lds_rate<0> || c.kernel == lds_rate<1> || c.kernel == lds_rate<2>;
  const double its = lds ? (double)((iters + 1) / 2 * 2 + 1) : (double)iters;
  return waves * its * c.per_iteration;
}
// launches case i once on `stream` (a hipStream_t; null for the default stream) without
// waiting for it; buffers are allocated on the first call. Returns a hipError_t code: 0 on
// success, hipErrorInvalidValue for an unknown case or iters outside [2, 2^30].
int isa_energy_launch(int i, int iters, void* stream) {
  if (i < 0 || i >= kEnergyCaseCount || iters < 2 || iters > (1 << 30)) return (int)hipErrorInvalidValue;
  static hipError_t ready = alloc_buffers();
  if (ready != hipSuccess) return (int)ready;
  const EnergyCase& c = kEnergyCases[i];
  hipLaunchKernelGGL(c.kernel, dim3(kBlocks), dim3(256 * c.waves_per_simd), 0, (hipStream_t)stream,
                     c.zero_input ? g_zero : g_in, g_cyc, g_sink, iters);
  return (int)hipGetLastError();
}
}

#ifndef ISA_COST_LIB
int main() {
  CK(alloc_buffers());

  printf("{\"matrix_cycles_per_instruction\": {");
  const int mi = 256;
  const double per = 4.0 * mi;
  printf("\"32x32x64 e4m3 x e4m3\": %.1f, ", simd_cycles(mfma_rate<0, 0, true>, 1, mi) / per);
  printf("\"32x32x64 e2m1 x e4m3\": %.1f, ", simd_cycles(mfma_rate<4, 0, true>, 1, mi) / per);
  printf("\"32x32x64 e2m1 x e2m1\": %.1f, ", simd_cycles(mfma_rate<4, 4, true>, 1, mi) / per);
  printf("\"16x16x128 e4m3 x e4m3\": %.1f, ", simd_cycles(mfma_rate<0, 0, false>, 1, mi) / per);
  printf("\"16x16x128 e2m1 x e4m3\": %.1f, ", simd_cycles(mfma_rate<4, 0, false>, 1, mi) / per);
  printf("\"16x16x128 e2m1 x e2m1\": %.1f}, ", simd_cycles(mfma_rate<4, 4, false>, 1, mi) / per);

  // 2 waves per SIMD: SIMD cycles per wave64 instruction = slowest wave / (iters 64 * 2)
  const int vi = 256;
  auto vr = [&](auto k) { return simd_cycles(k, 2, vi) / (vi * 64.0 * 2); };
  printf("\"vector_simd_cycles_per_instruction\": {");
  printf("\"v_fma_f32\": %.2f, ", vr(valu_rate<0, 8, false>));
  printf("\"v_exp_f32\": %.2f, ", vr(valu_rate<1, 8, false>));
  printf("\"v_cvt_pk_fp8_f32\": %.2f, ", vr(valu_rate<2, 8, false>));
  printf("\"v_cvt_pk_u8_f32\": %.2f, ", vr(valu_rate<3, 8, false>));
  printf("\"v_max3_f32\": %.2f, ", vr(valu_rate<4, 8, false>));
  printf("\"v_perm_b32\": %.2f, ", vr(valu_rate<5, 8, false>));
  printf("\"v_mov_b32_dpp\": %.2f}, ", vr(valu_rate<6, 8, false>));

  // overlap in one wave per SIMD: cycles per iteration of 8 MFMA and 8 N vector instructions
  const int oi = 256;
  auto ov = [&](auto k) { return simd_cycles(k, 1, oi) / oi; };
  printf("\"one_wave_cycles_per_iteration\": {");
  printf("\"8 mfma\": %.1f, ", ov(valu_rate<0, 0, true>));
  printf("\"32 v_exp_f32\": %.1f, ", ov(valu_rate<1, 4, false>));
  printf("\"8 mfma + 32 v_exp_f32\": %.1f, ", ov(valu_rate<1, 4, true>));
  printf("\"64 v_fma_f32\": %.1f, ", ov(valu_rate<0, 8, false>));
  printf("\"8 mfma + 64 v_fma_f32\": %.1f, ", ov(valu_rate<0, 8, true>));
  printf("\"32 v_cvt_pk_fp8_f32\": %.1f, ", ov(valu_rate<2, 4, false>));
  printf("\"8 mfma + 32 v_cvt_pk_fp8_f32\": %.1f}, ", ov(valu_rate<2, 4, true>));

  // LDS: bytes read per clock per CU, sixteen waves (four per SIMD), eight reads per batch,
  // li + 1 batches per wave (li even)
  const int li = 512;
  auto lr = [&](auto k, double bytes_per_lane) {
    return 16.0 * (li + 1) * 8 * 64 * bytes_per_lane / simd_cycles(k, 4, li);
  };
  printf("\"lds_bytes_per_clock_per_cu\": {");
  printf("\"ds_read_b128\": %.0f, ", lr(lds_rate<0>, 16));
  printf("\"ds_read_b64_tr_b8\": %.0f, ", lr(lds_rate<1>, 8));
  printf("\"ds_read_b64_tr_b16\": %.0f}}\n", lr(lds_rate<2>, 8));
  return 0;
}
#endif
