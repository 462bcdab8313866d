// Merge of partial attention results over disjoint key sets.
//
// Zyphra "Inference Wave 2", section on CSA dual-scope decode: when the keys of one
// attention call are split into shards, each shard returns its partial output together
// with the log-sum-exp of its scores, and one merge step turns the parts into the
// result of a single pass over all keys. For parts p with (O_p, LSE_p) of one query row:
//
//     M = max_p LSE_p,  w_p = exp(LSE_p - M),  W = sum_p w_p
//     O = sum_p w_p O_p / W,  LSE = M + ln W
//
// A part whose row saw no key has LSE_p = -inf and weight zero; a row that no part saw
// gets O = 0, LSE = -inf.
//
// HBM-bound: each row reads n_parts * (2 Dv + 4) bytes and writes 2 Dv (+ 4) bytes. A
// group of Dv / 8 consecutive lanes owns a row, each lane 8 output values (16 bytes), so
// every load and store of a wave is one contiguous run. The parts are read once and the
// output is left for a later kernel, so loads and stores carry the nontemporal hint; with
// it, and one workgroup per block of rows rather than a capped grid that loops, the merge
// of 32 x 32K rows of two parts went from 151 to 128 us (5.4 to 6.4 TB/s).
#include <math.h>

#include "device.h"
#include "launch.h"

namespace zyfa {

constexpr int kMergeThreads = 256;
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Parts are taken in chunks of CHUNK: every load of a chunk (its log-sum-exps and its
// 16-byte pieces of O) is issued before any is used, so a decode merge (few rows, many
// parts) waits for one memory round trip per chunk instead of one per part. The launcher
// takes the least chunk of 2, 4, 8 or 16 that holds all parts (fewer registers, more
// waves, for the HBM-bound merges of many rows and few parts); then the maximum is final
// before any weight is formed. Beyond 16 parts the running maximum moves chunk by chunk
// and the sums are rescaled by exp(old - new).
template <int LANES, int CHUNK>  // lanes per row = Dv / 8
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const uint16_t* __restrict__ o_parts,
                                                                   const float* __restrict__ lse_parts,
                                                                   int n_parts, uint16_t* __restrict__ o,
                                                                   float* __restrict__ lse, long long rows) {
  constexpr int ROWS_PER_BLOCK = kMergeThreads / LANES;
  constexpr int DV = 8 * LANES;
  const int sub = threadIdx.x % LANES;
  const long long stride = (long long)gridDim.x * ROWS_PER_BLOCK;
  for (long long r = (long long)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / LANES; r < rows; r += stride) {
    float m = -INFINITY;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.0f;
    for (int p0 = 0; p0 < n_parts; p0 += CHUNK) {
      float l[CHUNK];
      uint4 x[CHUNK];
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) {
        const int p = p0 + i;
        if (p < n_parts) {
          l[i] = __builtin_nontemporal_load(lse_parts + (long long)p * rows + r);
          const v4u w = __builtin_nontemporal_load((const v4u*)(o_parts + ((long long)p * rows + r) * DV + 8 * sub));
          x[i] = uint4{w[0], w[1], w[2], w[3]};
        } else {
          l[i] = -INFINITY;
          x[i] = uint4{0u, 0u, 0u, 0u};
        }
      }
      float mc = m;
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) mc = fmaxf(mc, l[i]);
      if (mc == -INFINITY) continue;  // no part so far saw a key
      if (mc > m && m > -INFINITY) {  // (only from the second chunk on)
        const float a = expf(m - mc);
        wsum *= a;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= a;
      }
      m = mc;
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) {
        const float w = expf(l[i] - m);  // exp(-inf) = 0
        wsum += w;
        const uint32_t xw[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = fmaf(w, __uint_as_float(xw[j] << 16), acc[2 * j]);
          acc[2 * j + 1] = fmaf(w, __uint_as_float(xw[j] & 0xffff0000u), acc[2 * j + 1]);
        }
      }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    uint4 y;
    y.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    y.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    y.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
    y.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
    __builtin_nontemporal_store(v4u{y.x, y.y, y.z, y.w}, (v4u*)(o + r * DV + 8 * sub));
    if (lse != nullptr && sub == 0) lse[r] = wsum > 0.0f ? m + logf(wsum) : -INFINITY;
  }
}

template <int LANES>
static hipError_t launch_merge_t(const MergeArgs& a, hipStream_t stream) {
  constexpr int ROWS_PER_BLOCK = kMergeThreads / LANES;
  const long long blocks = (a.rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  // one workgroup per block of rows, each with a single round of loads; past 2^22
  // workgroups (2^30 work-items, within the 32-bit work-item count of a grid dimension)
  // the grid-stride loop takes the rest
  constexpr long long kMaxGrid = 1LL << 22;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kMergeThreads), 0, stream, a.o_parts, a.lse_parts, a.n_parts, a.o,
                       a.lse, a.rows);
  };
  if (a.n_parts <= 2) go(attn_merge_kernel<LANES, 2>);
  else if (a.n_parts <= 4) go(attn_merge_kernel<LANES, 4>);
  else if (a.n_parts <= 8) go(attn_merge_kernel<LANES, 8>);
  else go(attn_merge_kernel<LANES, 16>);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream) {
  switch (a.Dv) {
    case 64: return launch_merge_t<8>(a, stream);
    case 128: return launch_merge_t<16>(a, stream);
    case 256: return launch_merge_t<32>(a, stream);
    case 512: return launch_merge_t<64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace zyfa
