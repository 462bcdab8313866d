// Causal prefill attention forward on gfx950: FP8 (e4m3 with per-block scales) and BF16.
//
// "ZYFA: Fast and Accurate FP8 Attention on AMD MI355X":
//  * Introduction: FlashAttention-style tiling keeps the score matrix on chip, so
//    HBM traffic is linear in S and the kernel is bound by the matrix cores.
//  * "Precision and Underflow of FP8 Probabilities" and "Per-Block Scaling and
//    Normalization by the Rounded Row Sum": probabilities of each (query row,
//    64-key block) are multiplied by a power of two that puts the block maximum in
//    [1, 2) before rounding to e4m3; the scaled FP8 matrix instruction divides it
//    back out; each row is normalised by the sum of exactly the rounded values
//    that multiply V.
//  * "Lean P": probabilities are formed in base 2, p = 2^x with x the score minus
//    the row maximum in base-2 units (this kernel evaluates 2^x exactly with the
//    hardware exponential and rounds it to e4m3 - the page's "exact P").
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//  * Each wave owns 32 query rows and computes S^T = K Q^T on 32x32 MFMA tiles,
//    so every lane holds the scores of one query row (lane % 32) for half of the
//    keys of a tile; row maxima need one lane-half exchange (v_permlane32_swap).
//  * K and V tiles of 64 keys are staged through LDS (double buffered, padded rows)
//    with coalesced 16-byte global loads; K is read back in MFMA operand layout,
//    V with the LDS transpose read so that keys land along the reduction axis.
//  * O^T = V^T P^T accumulates on the MFMA with each lane owning one query row, so
//    rescaling O by a per-row factor is a per-lane multiply.
//  * The running maximum used as the exponent reference is updated lazily: O and
//    the row sum are rescaled only when a row's maximum grows by more than
//    kLazyThreshold binades (the per-block power of two keeps FP8 probabilities in
//    range regardless, and float32 accumulators have ample headroom).
//  * Causal-block skipping: a wave visits key tiles 0 .. (its last row) / 64 only;
//    the mask is evaluated on the tile that straddles the diagonal.
//  * Scheduling: workgroups are issued heaviest (last query tile) first; within a
//    round over heads, consecutive workgroup ids (which the hardware spreads over
//    the 8 XCDs) are mapped so that each XCD serves a contiguous range of heads,
//    and query heads sharing a key/value head hit the same L2.
#include <math.h>

#include "device.h"
#include "launch.h"

namespace zyfa {

constexpr float kLazyThreshold = 8.0f;

template <bool FP8, int DQK>
struct Cfg {
  static constexpr int DV = 128;
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;  // query rows per workgroup
  static constexpr int BN = 64;          // keys per tile
  static constexpr int ESZ = FP8 ? 1 : 2;
  static constexpr int KROW = DQK * ESZ;  // bytes of one K row
  static constexpr int VROW = DV * ESZ;
  static constexpr int KPITCH = KROW + 16;  // padded LDS row pitch: 16 consecutive rows hit distinct banks
  static constexpr int VPITCH = VROW + 16;
  static constexpr int KTILE = BN * KPITCH;
  static constexpr int VTILE = BN * VPITCH;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int KCHUNKS = BN * KROW / 16 / THREADS;  // 16-byte global loads per thread per tile
  static constexpr int VCHUNKS = BN * VROW / 16 / THREADS;
  static constexpr int KSTEP = FP8 ? 64 : 16;  // MFMA reduction depth
  static constexpr int NKS = DQK / KSTEP;
  static_assert(BN * KROW % (16 * THREADS) == 0 && BN * VROW % (16 * THREADS) == 0, "tile load split");
  static_assert(DQK % KSTEP == 0, "head dim must divide the MFMA depth");
};

struct AttnParams {
  const char* q;
  const char* k;
  const char* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, S, nb, scale_block, n_qtiles;
  float scale_log2;  // softmax_scale * log2(e)
};

template <bool FP8>
using QOp = typename std::conditional<FP8, v8i, v8bf>::type;

template <bool FP8, int DQK>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnParams p) {
  using C = Cfg<FP8, DQK>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int S = p.S;

  // ---- work item: (batch, query head, query tile), heaviest tile first ----
  const int NH = p.B * p.Hq;
  const int id = blockIdx.x;
  const int round = id / NH;
  const int in_round = id - round * NH;
  int head = in_round;
  if (NH % 8 == 0) head = (in_round & 7) * (NH >> 3) + (in_round >> 3);
  const int qt = p.n_qtiles - 1 - round;
  const int b = head / p.Hq;
  const int hq = head - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);

  const int q0_wg = qt * C::BM;
  const int q0 = q0_wg + wave * 32;
  const int n_tiles = (min(q0_wg + C::BM, S) - 1) / C::BN + 1;
  const bool wave_active = q0 < S;
  const int n_tiles_w = wave_active ? (min(q0 + 32, S) - 1) / C::BN + 1 : 0;
  const int my_q = q0 + l32;

  const size_t bh_q = (size_t)(b * p.Hq + hq);
  const size_t bh_kv = (size_t)(b * p.Hkv + hkv);
  const char* kbase = p.k + bh_kv * S * C::KROW;
  const char* vbase = p.v + bh_kv * S * C::VROW;

  // ---- Q operand (B of S^T = K Q^T): lane holds Q[my_q][c*KSTEP + h*KSTEP/2 ...] ----
  QOp<FP8> qreg[C::NKS];
  {
    const char* qrow = p.q + (bh_q * S + min(my_q, S - 1)) * C::KROW;
#pragma unroll
    for (int c = 0; c < C::NKS; ++c) {
      const char* src = qrow + (c * C::KSTEP + h * (C::KSTEP / 2)) * C::ESZ;
      if constexpr (FP8) {
        v4i lo = *(const v4i*)src;
        v4i hi = *(const v4i*)(src + 16);
        qreg[c] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        qreg[c] = *(const v8bf*)src;
      }
    }
  }

  float q_scale = 1.0f;
  if constexpr (FP8) q_scale = p.q_scale[bh_q * p.nb + min(q0, S - 1) / p.scale_block];

  // ---- global -> register -> LDS staging of K and V tiles ----
  v4i kst[C::KCHUNKS];
  v4i vst[C::VCHUNKS];
  auto gload = [&](int t) {
    const int kt = t * C::BN;
#pragma unroll
    for (int i = 0; i < C::KCHUNKS; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = c / (C::KROW / 16);
      const int col = c % (C::KROW / 16);
      const int gr = min(kt + row, S - 1);
      kst[i] = *(const v4i*)(kbase + (size_t)gr * C::KROW + col * 16);
    }
#pragma unroll
    for (int i = 0; i < C::VCHUNKS; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = c / (C::VROW / 16);
      const int col = c % (C::VROW / 16);
      const int gr = min(kt + row, S - 1);
      vst[i] = *(const v4i*)(vbase + (size_t)gr * C::VROW + col * 16);
    }
  };
  auto lstore = [&](int buf) {
    char* ks = smem + buf * C::STAGE;
    char* vs = ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::KCHUNKS; ++i) {
      const int c = tid + i * C::THREADS;
      *(v4i*)(ks + (c / (C::KROW / 16)) * C::KPITCH + (c % (C::KROW / 16)) * 16) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < C::VCHUNKS; ++i) {
      const int c = tid + i * C::THREADS;
      *(v4i*)(vs + (c / (C::VROW / 16)) * C::VPITCH + (c % (C::VROW / 16)) * 16) = vst[i];
    }
  };

  // ---- per-row state (each lane owns query row my_q) ----
  v16f oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc[d] = v16f{0};
  float m_ref = -INFINITY;  // exponent reference (base-2 units)
  float l_sum = 0.0f;       // row sum in units of 2^m_ref
  const int k127 = opaque(kE8M0One);
  const v8i ones_fp8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) gload(t + 1);

    if (t < n_tiles_w) {
      const char* ks = smem + (t & 1) * C::STAGE;
      const char* vs = ks + C::KTILE;
      const int kt = t * C::BN;

      // S^T[key][query] for keys kt + 32g + (8(r/4) + 4h + r%4)
      v16f sacc[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        sacc[g] = v16f{0};
        const char* krow = ks + (32 * g + l32) * C::KPITCH + h * (C::KSTEP / 2) * C::ESZ;
#pragma unroll
        for (int c = 0; c < C::NKS; ++c) {
          const char* src = krow + c * C::KSTEP * C::ESZ;
          if constexpr (FP8) {
            v4i lo = *(const v4i*)src;
            v4i hi = *(const v4i*)(src + 16);
            v8i a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            sacc[g] = mfma_fp8(a, qreg[c], sacc[g]);
          } else {
            v8bf a = *(const v8bf*)src;
            sacc[g] = mfma_bf16(a, qreg[c], sacc[g]);
          }
        }
      }

      // causal mask on the tile that reaches past the wave's first row
      if (kt + C::BN - 1 > q0) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * g + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > my_q) sacc[g][r] = -INFINITY;
          }
      }

      // row maximum over the 64 keys of the tile
      float bm = -INFINITY;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) bm = fmaxf(bm, sacc[g][r]);
      bm = max_across_halves(bm);

      float c_log2 = p.scale_log2;
      float k_scale = 1.0f, v_scale = 1.0f;
      if constexpr (FP8) {
        const size_t si = bh_kv * p.nb + kt / p.scale_block;
        k_scale = p.k_scale[si];
        v_scale = p.v_scale[si];
        c_log2 = p.scale_log2 * q_scale * k_scale;
      }
      const float xmax = bm * c_log2;  // every visited tile has an unmasked key per row: finite

      // lazy update of the exponent reference; a row's result depends on its own
      // scores only (rows that do not need a new reference keep theirs: alpha = 1)
      const bool grow = xmax > m_ref + kLazyThreshold;
      if (__any(grow)) {
        const float m_new = grow ? xmax : m_ref;
        const float alpha = fast_exp2(m_ref - m_new);  // 0 on the first tile
#pragma unroll
        for (int d = 0; d < 4; ++d) oacc[d] *= alpha;
        l_sum *= alpha;
        m_ref = m_new;
      }

      if constexpr (FP8) {
        // block power of two: 2^-eb puts the block maximum of this row in [1, 2)
        const int eb = max((int)floorf(xmax - m_ref), -126);
        // V scale = rv * 2^ev with rv in [1, 2): 2^ev goes to the V operand's E8M0
        // scale, rv is folded into the probabilities before rounding
        int ev;
        const float rv = 2.0f * frexpf(v_scale, &ev);
        ev -= 1;
        const float bias = m_ref + (float)eb - __builtin_amdgcn_logf(rv);
        int pw[8];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = fast_exp2(fmaf(sacc[g][4 * w + 0], c_log2, -bias));
            const float p1 = fast_exp2(fmaf(sacc[g][4 * w + 1], c_log2, -bias));
            const float p2 = fast_exp2(fmaf(sacc[g][4 * w + 2], c_log2, -bias));
            const float p3 = fast_exp2(fmaf(sacc[g][4 * w + 3], c_log2, -bias));
            int word = cvt_pk_fp8<false>(p0, p1, 0);
            pw[4 * g + w] = cvt_pk_fp8<true>(p2, p3, word);
          }
        const v8i pv = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
        const int scale_p = kE8M0One + eb;
        const int scale_v = opaque(kE8M0One + ev);

        // O^T[dv][query] += V^T P^T; V^T operand via LDS transpose reads:
        // byte j of a lane's operand is key 32(j/16) + 8((j%16)/4) + 4h + j%4,
        // the same key order as the probability bytes.
        const int r8 = (lane & 15) >> 1;
        const int colbase = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          int va[8];
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int key = 32 * (qd >> 1) + 16 * (qd & 1) + 8 * (r8 >> 2) + 4 * h + (r8 & 3);
            const char* src = vs + key * C::VPITCH + 32 * d + colbase;
            v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)src);
            va[2 * qd] = x[0];
            va[2 * qd + 1] = x[1];
          }
          const v8i a = {va[0], va[1], va[2], va[3], va[4], va[5], va[6], va[7]};
          oacc[d] = mfma_fp8_scaled(a, pv, oacc[d], scale_v, scale_p);
        }
        // rounded row sum: the same probability bytes and scales, against a ones matrix
        const v16f rs = mfma_fp8_scaled(ones_fp8, pv, v16f{0}, k127, scale_p);
        l_sum = fmaf(rs[0], 1.0f / rv, l_sum);
      } else {
        // BF16: p = 2^(x - m_ref) rounded to bf16 for P V; row sum in float32
        float part = 0.0f;
        v8bf pb[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int g = tt >> 1;
          const int r0 = 8 * (tt & 1);
          float pr[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pr[j] = fast_exp2(fmaf(sacc[g][r0 + j], c_log2, -m_ref));
            part += pr[j];
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[tt][j] = (__bf16)pr[j];
        }
        l_sum += part;
        const int r4 = (lane & 15) >> 2;
        const int colbase = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int key0 = 32 * (tt >> 1) + 16 * (tt & 1) + 4 * h + r4;
            const char* src0 = vs + key0 * C::VPITCH + (32 * d + colbase) * 2;
            const char* src1 = src0 + 8 * C::VPITCH;
            const v4bf x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)src0);
            const v4bf x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)src1);
            const v8bf a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[d] = mfma_bf16(a, pb[tt], oacc[d]);
          }
        }
      }
    }

    if (t + 1 < n_tiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
  if constexpr (!FP8) l_sum = sum_across_halves(l_sum);
  if (my_q >= S) return;

  const float inv_l = 1.0f / l_sum;
  uint16_t* orow = p.o + (bh_q * S + my_q) * C::DV;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dv = 32 * d + 8 * r4 + 4 * h;
      uint2 w;
      w.x = pack_bf16x2(oacc[d][4 * r4 + 0] * inv_l, oacc[d][4 * r4 + 1] * inv_l);
      w.y = pack_bf16x2(oacc[d][4 * r4 + 2] * inv_l, oacc[d][4 * r4 + 3] * inv_l);
      *(uint2*)(orow + dv) = w;
    }
  if (p.lse != nullptr && h == 0) p.lse[bh_q * S + my_q] = kLn2 * (m_ref + log2f(l_sum));
}

template <bool FP8, int DQK>
static hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  using C = Cfg<FP8, DQK>;
  AttnParams p;
  p.q = (const char*)a.q;
  p.k = (const char*)a.k;
  p.v = (const char*)a.v;
  p.q_scale = a.q_scale;
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.o = a.o;
  p.lse = a.lse;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.S = a.S;
  p.scale_block = FP8 ? a.scale_block : 1;
  p.nb = FP8 ? (a.S + a.scale_block - 1) / a.scale_block : 0;
  p.n_qtiles = (a.S + C::BM - 1) / C::BM;
  p.scale_log2 = a.softmax_scale * kLog2e;
  const long long grid = (long long)p.n_qtiles * a.B * a.Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<FP8, DQK>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_fp8(const AttnArgs& a, hipStream_t stream) {
  return a.Dqk == 192 ? launch<true, 192>(a, stream) : launch<true, 128>(a, stream);
}

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  return a.Dqk == 192 ? launch<false, 192>(a, stream) : launch<false, 128>(a, stream);
}

}  // namespace zyfa
