// Causal prefill attention forward on gfx950: FP8 (e4m3 with per-block scales) and BF16.
//
// "ZYFA: Fast and Accurate FP8 Attention on AMD MI355X":
//  * Introduction: FlashAttention-style tiling keeps the score matrix on chip, so
//    HBM traffic is linear in S and the kernel is bound by the matrix cores.
//  * "Vector-Pipe Cost of the Softmax" / "Software Ordering of Matrix
//    Instructions": in FP8 the softmax needs about as many vector cycles as the
//    matrix products need matrix cycles, and only the instruction order overlaps
//    the two, so the loop below is software-pipelined and its schedule is fixed
//    by hand.
//  * "Precision and Underflow of FP8 Probabilities" and "Per-Block Scaling and
//    Normalization by the Rounded Row Sum": probabilities of each (query row,
//    64-key block) are multiplied by a power of two that puts the block maximum near
//    1 (here in [128, 256), kPHeadroom binades above [1, 2), which keeps 7 more binades
//    of small weights out of e4m3's subnormal range) before rounding to e4m3; the scaled
//    FP8 matrix instruction divides it
//    back out; each row is normalised by the sum of exactly the rounded values
//    that multiply V, computed by one more matrix instruction.
//  * "Lean P": probabilities are formed in base 2, p = 2^x with x the score minus
//    the row maximum in base-2 units. The default mode evaluates 2^x with the hardware
//    exponential and rounds it to e4m3 (the page's "exact P"); the lean mode takes the
//    e4m3 code as a linear function of x (the page's lean P).
//
// Work decomposition (one workgroup = 32 query rows per wave of one head: 8 waves,
// one workgroup per CU, two waves per SIMD):
//  * Each wave owns 32 query rows and computes S^T = K Q^T on 32x32 MFMA tiles,
//    so every lane holds the scores of one query row (lane % 32) for half of the
//    keys of a tile; row maxima need one lane-half exchange (v_permlane32_swap).
//  * K and V tiles of 64 keys are staged through LDS rings of two buffers each,
//    with coalesced 16-byte global loads issued two tiles ahead. K is read back in
//    MFMA operand layout; V with the LDS transpose read so that keys land along the
//    reduction axis. Row pitches (and, for FP8, a swap of key bits 2 and 3 in the
//    V row order) make every LDS read of a half-wave hit 64 distinct banks.
//  * O^T = V^T P^T accumulates on the MFMA with each lane owning one query row, so
//    rescaling O by a per-row factor is a per-lane multiply.
//  * Pipeline per 64-key tile t, in both precisions: the iteration that forms the
//    probabilities of tile t also issues the QK products of tile t+1 and the PV
//    products of tile t-1 (P_{t-1} V_{t-1}, one stage late), so that its matrix work
//    (FP8: 4 QK, 4 PV and 1 row-sum instructions; BF16: 16 QK and 16 PV) overlaps all
//    of its vector work. The steady iterations issue one matrix instruction per
//    slot, with the vector work spread over the slots and sched_barrier fencing
//    them.
//  * The exponent reference m_ref is an integer that is raised lazily: only when a
//    row's maximum exceeds it by more than kLazyThreshold binades are O and the row
//    sum rescaled (by a power of two; the in-flight probabilities of the previous
//    tile are re-scaled exactly, for FP8 through their E8M0 scale).
//  * Causal-block skipping: a workgroup visits key tiles 0 .. (its last row) / 64;
//    the mask is evaluated only on tiles that reach past a wave's first row.
//  * Scheduling: workgroups are issued heaviest (last query tile) first; within a
//    round over heads, consecutive workgroup ids (which the hardware spreads over
//    the 8 XCDs) are mapped so that each XCD serves the same range of query heads of
//    every batch entry: query heads sharing a key/value head hit the same L2, and
//    batch entries of different lengths (a packed batch) spread over all XCDs.
#include <math.h>

#include <type_traits>

#include "device.h"
#include "launch.h"
#ifdef ZYFA_TIMELINE
#include "../../include/zyfa_timeline.h"
#endif

namespace zyfa {

#ifdef ZYFA_TIMELINE
// Timeline build only (libzyfa_timeline.so): one record per workgroup of the eight-wave
// prefill kernels, written by its first thread (fields as include/zyfa_timeline.h lists).
// In the library proper the two hooks below expand to nothing.
__device__ unsigned long long timeline[ZYFA_TIMELINE_WORKGROUPS * ZYFA_TIMELINE_FIELDS];
#define ZYFA_TL_CLOCK(field) tl_put(field, __builtin_amdgcn_s_memrealtime())
#define ZYFA_TL_PUT(field, x) tl_put(field, x)
#else
#define ZYFA_TL_CLOCK(field) ((void)0)
#define ZYFA_TL_PUT(field, x) ((void)0)
#endif

// The reference moves only when a row's maximum exceeds it by more than kLazyThreshold
// binades. The probabilities' block scaling does not depend on it (every block maximum lands
// in [128, 256) whatever the reference); it bounds O and the row sum, which stay in units of
// 2^reference: each key adds at most 2^(kLazyThreshold + 1) |v|, so with at most 2^30 keys
// O stays finite in float32 for |v| < 2^(97 - kLazyThreshold) = 2^73. A larger threshold
// moves the reference less often on concentrated attention (activation-like inputs: 23 % of
// a wave's tiles at 8 binades, 15 % at 24; 2 % faster).
constexpr float kLazyThreshold = 24.0f;
// Exponent reference of a row that has seen no key yet: finite, so that masked scores give
// probabilities of exactly zero, and far below any score, so the first visible key moves it.
constexpr float kRefEmpty = -1e30f;
// FP8 probabilities of a (query row, 64-key block) are scaled by a power of two that puts
// the block maximum in [2^kPHeadroom, 2^(kPHeadroom + 1)): every e4m3 binade above the
// subnormal range carries the same relative precision, and the headroom keeps weights down
// to 2^-(6 + kPHeadroom) of their block maximum out of it (down to 2^-6 without headroom),
// while the block maximum stays below 256 and e4m3's largest value, 448.
constexpr int kPHeadroom = 7;
// Lean probabilities: the e4m3 code of p = 2^y is close to 8 y + 56 (eight codes per binade,
// 56 the code of 1.0), but inside each binade 2^y lies below the straight line, by up to 0.69
// codes. The code is therefore taken on a grid twice as fine, c16 = round(16 y + kLean16Bias),
// then halved, with the odd half-steps rounded up where the halved code's 3 mantissa bits are
// 0, 6 or 7 (bit m of kLeanUp), down elsewhere: the thresholds between codes then follow the
// exponential's curvature. The offset and the table were fitted to the error of the output
// after normalisation by the rounded row sum, which cancels any common factor of the weights.
constexpr float kLean16Bias = 110.25f;
constexpr unsigned kLeanUpLo = 0x00000001u;  // table bytes 0-3 (mantissas 0..3): round up at 0
constexpr unsigned kLeanUpHi = 0x01010000u;  // table bytes 4-7 (mantissas 4..7): round up at 6, 7
// The lean codes' values average 0.95917 of the probabilities they code (weighted by the
// probabilities, over a binade): the row sum that enters the log-sum-exp is divided by it,
// leaving each code off by at most 0.068 in log (the output, normalised by the same codes'
// sum, does not depend on a common factor).
constexpr float kLeanSumScale = 1.0425686f;

template <bool FP8, int DQK, int NWAVES = 8>
struct Cfg {
  static constexpr int DV = 128;
  // Eight waves: 256 query rows share each K/V tile copy, halving the copy traffic per
  // FLOP against four. FP8 decode of up to 32 query heads per key/value head takes one
  // wave: small workgroups, several per compute unit, keep more tile copies in flight.
  static constexpr int WAVES = NWAVES;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;  // query rows per workgroup
  static constexpr int BN = 64;          // keys per tile
  static constexpr int ESZ = FP8 ? 1 : 2;
  static constexpr int KROW = DQK * ESZ;  // bytes of one K row
  static constexpr int VROW = DV * ESZ;
  // LDS tiles are stored as column blocks of 64 bytes: block c holds bytes [64c, 64c+64)
  // of every row, 16-byte chunk j of row r at chunk j ^ x(r) within the row's 64 bytes.
  // K (x = (r >> 2) & 3): the 16-byte operand reads of 16 consecutive rows hit 16
  // distinct 4-bank groups. V: FP8 rows are stored in key order with bits 2 and 3
  // swapped and x = 2 ((r >> 2) & 1), so each half-wave transpose read (8 consecutive
  // rows x 2 chunks) hits distinct banks; BF16 transpose reads (4 consecutive rows x
  // 4 chunks) need no swizzle. No padding, so tiles can be filled by direct
  // global-to-LDS loads, one contiguous 1 KiB run per wave instruction.
  static constexpr int KBLK = BN * 64;  // bytes of one column block
  static constexpr int KBUF = BN * KROW;
  static constexpr int VBUF = BN * VROW;
  // LDS ring depth per tensor: two buffers, one barrier per iteration
  static constexpr int NBUF = 2;
  static constexpr int LDS_BYTES = NBUF * (KBUF + VBUF);
  // 16-byte copies per tile, and per thread (rounded up: a tile that does not split
  // evenly over the threads leaves whole waves idle in its last round)
  static constexpr int KSLOTS = BN * KROW / 16;
  static constexpr int VSLOTS = BN * VROW / 16;
  static constexpr int KCHUNKS = (KSLOTS + THREADS - 1) / THREADS;
  static constexpr int VCHUNKS = (VSLOTS + THREADS - 1) / THREADS;
  static constexpr int KSTEP = FP8 ? 64 : 16;  // MFMA reduction depth
  static constexpr int NKS = DQK / KSTEP;
  static_assert(KSLOTS % 64 == 0 && VSLOTS % 64 == 0, "tile copies split into whole waves");
  static_assert(DQK % KSTEP == 0, "head dim must divide the MFMA depth");
  static_assert(WAVES == 1 || BM % (2 * BN) == 0,
                "causal prefill relies on an even number of key tiles per query tile (one-wave workgroups "
                "serve decode only, whose rows see every key)");
};

// Key positions inside the kernel are relative to the window's first key k_begin: the
// window holds keys 0 .. Sk - 1, and query row i (of the Q tensor) sits at position
// d + i, so it sees keys j <= min(d + i, Sk - 1). A row with d + i < 0 sees no key.
struct AttnParams {
  const char* q;
  const char* k;
  const char* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv;
  int Sq;       // rows per head of Q, O and LSE
  int Skv;      // rows per head of K and V
  int k_begin;  // first key of the window (a multiple of the key tile)
  int Sk;       // keys in the window
  int d;        // position of query row 0 relative to k_begin
  int nbq, nbk, scale_shift, n_qtiles;  // scale blocks of Q and of K/V (1 << scale_shift tokens)
  float scale_log2;  // softmax_scale * log2(e)
  // packed batch of sequences of different lengths (null otherwise): B sequences, sequence
  // b being tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1 of every head of [H, Sq = Skv, D]
  // tensors, causal within itself; no sequence longer than max_seqlen
  const int* cu_seqlens;
  int max_seqlen;
  // paged key/value cache (PAGED kernels): K and V are [num_pages, Hkv, 1 << page_shift, D]
  // and their FP8 scales [num_pages, Hkv, pages' scale blocks]; sequence b's logical page j
  // is block_table[b * max_pages + j]; its kv_lens[b] tokens end with the chunk of new
  // tokens that cu_seqlens gives (rows of Q, O, LSE, packed as in a varlen batch)
  const int* block_table;
  const int* kv_lens;
  int max_pages, num_pages, page_shift;
  // decode (PAGED kernels with split_keys > 0): the Sq rows of each (b, head) of Q are the
  // query heads of one KV group, one token each at position kv_lens[b] - 1; query tile qt
  // of the grid is the key split [qt * split_keys, (qt + 1) * split_keys), whose partial
  // O and LSE go to rows qt * part_rows + (row of Q)
  int split_keys;
  size_t part_rows;
  // debug (environment variable ZYFA_LDS_POISON): LDS starts as all-ones bytes, a NaN in
  // both e4m3 and bf16, so that a read of any byte no tile copy wrote reaches the output
  int poison_lds;
};

template <bool FP8>
using QOp = typename std::conditional<FP8, v8i, v8bf>::type;

// LDS row of key k within an FP8 V tile: key bits 2 and 3 swapped, so that the 8 keys
// one 16-lane group reads with a transpose load ({0-3, 8-11} or {4-7, 12-15} within a
// 16-key run) occupy 8 consecutive rows.
__device__ __forceinline__ int fp8_vrow(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// (one-wave workgroups may take all 512 registers of a lane: four per compute unit, each a
// wave of its own SIMD)
template <bool FP8, int DQK, bool LEAN, bool PAGED, int WAVES = 8>
__global__ __launch_bounds__((Cfg<FP8, DQK, WAVES>::THREADS), (WAVES == 1 ? 1 : 2)) void attn_fwd_kernel(AttnParams p) {
  static_assert(FP8 || !LEAN, "lean probabilities are an FP8 mode");
  static_assert(WAVES == 8 || (PAGED && FP8), "one-wave workgroups serve FP8 decode only");
  using C = Cfg<FP8, DQK, WAVES>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  char* const kring = smem;                // [2 buffers][column blocks][BN rows][64 bytes]
  char* const vring = smem + C::NBUF * C::KBUF;  // same layout for V

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
#ifdef ZYFA_TIMELINE
  const bool tl_on = blockIdx.x < ZYFA_TIMELINE_WORKGROUPS && tid == 0;
  unsigned long long* const tl = timeline + (size_t)blockIdx.x * ZYFA_TIMELINE_FIELDS;
  auto tl_put = [&](int field, unsigned long long x) {
    if constexpr (!PAGED && WAVES == 8) {
      if (tl_on) tl[field] = x;
    }
  };
  ZYFA_TL_CLOCK(0);
  ZYFA_TL_PUT(4, __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11)));   // HW_ID
  ZYFA_TL_PUT(5, __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11)));  // XCC_ID
#endif

  // ---- work item: (batch, query head, query tile), heaviest tile first ----
  const int NH = p.B * p.Hq;
  const int id = blockIdx.x;
  const int round = id / NH;
  const int in_round = id - round * NH;
  // consecutive workgroup ids go to the 8 XCDs in turn: XCD x (id mod 8) serves query heads
  // x Hq/8 .. (x + 1) Hq/8 - 1 of every batch entry, so that the query heads of a GQA group
  // share one L2 and every batch entry (a sequence of its own length, in a packed batch) is
  // spread over all XCDs
  int head = in_round;
  if (p.Hq % 8 == 0) {
    const int per = p.Hq >> 3, j = in_round >> 3, bb = j / per;
    head = bb * p.Hq + (in_round & 7) * per + (j - bb * per);
  } else if (NH % 8 == 0) {
    head = (in_round & 7) * (NH >> 3) + (in_round >> 3);
  }
  const int qt = p.n_qtiles - 1 - round;
  const int b = head / p.Hq;
  const int hq = head - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);

  // ---- the work item's geometry (wave-uniform) ----
  int Sq = p.Sq, Sk = p.Sk, dpos = p.d, k_begin = p.k_begin;
  size_t q_row0 = (size_t)(b * p.Hq + hq) * p.Sq;      // row of Q, O and LSE holding this head's query 0
  size_t kv_row0 = (size_t)(b * p.Hkv + hkv) * p.Skv;  // row of K and V holding this head's key 0
  int q_pos0 = 0;                                        // token position of query 0 (for Q scale blocks)
  size_t q_sc0 = (size_t)(b * p.Hq + hq) * p.nbq;
  size_t kv_sc0 = (size_t)(b * p.Hkv + hkv) * p.nbk;
  size_t o_split = 0;  // decode: first row of this split's partial results in O and LSE
  if constexpr (PAGED) {
   if (p.split_keys > 0) {
    // decode: every row sees every key of the sequence; this workgroup takes its split of
    // them (an empty split, or a malformed kv_lens entry, gives O = 0 and LSE = -inf,
    // which the merge of the splits ignores)
    const int kvl = p.kv_lens[b];
    const int lo = qt * p.split_keys;
    const bool ok = kvl >= 1 && kvl <= (p.max_pages << p.page_shift) && kvl <= p.n_qtiles * p.split_keys;
    k_begin = lo;
    Sk = ok ? max(0, min(p.split_keys, kvl - lo)) : 0;
    dpos = kvl - 1 - lo;
    o_split = (size_t)qt * p.part_rows;
   } else {
    // a chunk of new tokens (rows s0 .. s1 - 1 of the packed Q) that ends sequence b's
    // kv_lens[b] cached tokens: row i sits at position kvl - L + i and sees keys up to it.
    // Malformed entries leave the chunk unwritten, as for a packed batch.
    const int s0 = p.cu_seqlens[b], s1 = p.cu_seqlens[b + 1], kvl = p.kv_lens[b];
    if (s0 < 0 || (s0 & (C::BN - 1)) != 0 || s1 <= s0 || s1 > p.Sq || s1 - s0 > p.max_seqlen || kvl < s1 - s0 ||
        kvl > (p.max_pages << p.page_shift))
      return;
    Sq = s1 - s0;
    Sk = kvl;
    dpos = kvl - Sq;
    k_begin = 0;
    q_row0 = (size_t)hq * p.Sq + s0;
    q_pos0 = s0;
    q_sc0 = (size_t)hq * p.nbq;
    if (qt * C::BM >= Sq) return;
   }
  } else if (p.cu_seqlens != nullptr) {
    // packed batch: sequence b is tokens s0 .. s1 - 1 of every head, causal within itself.
    // A malformed entry (a start off the key tile, decreasing, past the tensor, longer
    // than max_seqlen) leaves the sequence unwritten, as do workgroups past its end.
    const int s0 = p.cu_seqlens[b], s1 = p.cu_seqlens[b + 1];
    if (s0 < 0 || (s0 & (C::BN - 1)) != 0 || s1 < s0 || s1 > p.Skv || s1 - s0 > p.max_seqlen) return;
    Sq = Sk = s1 - s0;
    dpos = 0;
    k_begin = s0;
    q_row0 = (size_t)hq * p.Sq + s0;
    kv_row0 = (size_t)hkv * p.Skv;
    q_pos0 = s0;
    q_sc0 = (size_t)hq * p.nbq;
    kv_sc0 = (size_t)hkv * p.nbk;
    if (qt * C::BM >= Sq) return;
  }

  const size_t o_row0 = q_row0 + o_split;  // row of O and LSE holding query 0
  const int q0_wg = PAGED && p.split_keys > 0 ? 0 : qt * C::BM;
  const int q0 = q0_wg + __builtin_amdgcn_readfirstlane(wave) * 32;  // (wave-uniform)
  // this lane's query row, recomputed from the lane id where needed (not kept in a register)
  auto row_of_lane = [&] { return q0 + (int)(__lane_id() & 31); };
  const int my_q = row_of_lane();
  // last key of the window visible to this lane's row, and to the wave's first row
  const int lim_q = min(dpos + my_q, Sk - 1);
  const int lim_w = min(dpos + q0, Sk - 1);
  // every wave runs the workgroup's trip count (key tiles up to the last one its last row
  // sees); tiles past a wave's rows are fully masked
  const int last_key = min(dpos + min(q0_wg + C::BM, Sq) - 1, Sk - 1);
  const int n = last_key < 0 ? 0 : last_key / C::BN + 1;

  if (n == 0) {
    // no row of the workgroup sees a key of the window: O = 0, LSE = -inf
    if (my_q < Sq) {
      uint16_t* orow = p.o + (o_row0 + my_q) * C::DV;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) *(uint2*)(orow + 32 * d + 8 * r4 + 4 * h) = uint2{0u, 0u};
      if (p.lse != nullptr && h == 0) p.lse[o_row0 + my_q] = -INFINITY;
    }
    return;
  }

  const char* kbase = p.k + (kv_row0 + k_begin) * C::KROW;
  const char* vbase = p.v + (kv_row0 + k_begin) * C::VROW;
  const float* kscale = p.k_scale + kv_sc0;
  const float* vscale = p.v_scale + kv_sc0;
  // PAGED: the cache page holding key tile t (a tile never straddles pages: a page holds
  // whole tiles), and the row of the cache ([pages x Hkv x page rows] rows of D) holding
  // the tile's first key. Page indices are clamped to the table and the cache, so a
  // malformed table reads wrong rows, never past the tensors.
  // (the table is read through the constant address space: nothing writes it while the
  // kernel runs, so the entry comes in by a scalar load. A vector load of the one address
  // made every wave wait, at each iteration, for its earlier tile copies as well: the
  // vector memory counter drains in order, and the entry is needed in a scalar register.)
  auto page_of = [&](int t) -> int {
    const int j = min((k_begin + t * C::BN) >> p.page_shift, p.max_pages - 1);
    const auto table = (const __attribute__((address_space(4))) int*)p.block_table;
    return min(max(table[(size_t)b * p.max_pages + j], 0), p.num_pages - 1);
  };
  auto page_row = [&](int pg, int t) -> size_t {
    return (((size_t)pg * p.Hkv + hkv) << p.page_shift) + ((k_begin + t * C::BN) & ((1 << p.page_shift) - 1));
  };
  // the pages of tiles t+1 and t+2 while iteration t runs: the page of tile t+3 is read
  // during iteration t (like the FP8 scales), so that no copy waits for the table
  int pg1 = 0, pg2 = 0;
  const int pg0 = PAGED ? page_of(0) : 0;
  if constexpr (PAGED) {
    pg1 = page_of(1);
    pg2 = page_of(2);
  }
  auto next_pages = [&](int pg3) {
    if constexpr (PAGED) {
      pg1 = pg2;
      pg2 = pg3;
    }
  };

  // ---- Q operand (B of S^T = K Q^T): lane holds Q[my_q][c*KSTEP + h*KSTEP/2 ...] ----
  QOp<FP8> qreg[C::NKS];
  {
    const char* qrow = p.q + (q_row0 + min(my_q, Sq - 1)) * C::KROW;
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
  float c_q = p.scale_log2;  // multiplies raw scores into base-2 units (times the tile's k scale for FP8)
  if constexpr (FP8) c_q *= p.q_scale[q_sc0 + ((q_pos0 + min(q0, Sq - 1)) >> p.scale_shift)];

  // ---- direct global -> LDS staging ----
  // 16-byte position pos of a buffer is (column block, row r, stored chunk); the lane
  // that fills it fetches the global chunk stored there. Each wave instruction fills 64
  // consecutive positions (1 KiB), lane l at position base + l. A lane's source offset
  // within a tile does not depend on the tile; only the last tile of a window whose
  // length is not a multiple of BN clamps its rows to the window's last key.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // does this wave copy chunk i of a tile (always, unless the tile's last round of
  // copies does not reach every wave)?
  auto k_live = [&](int i) { return (i + 1) * C::THREADS <= C::KSLOTS || wave_u * 64 + i * C::THREADS < C::KSLOTS; };
  auto v_live = [&](int i) { return (i + 1) * C::THREADS <= C::VSLOTS || wave_u * 64 + i * C::THREADS < C::VSLOTS; };
  auto k_pos_row = [&](int i) { return ((tid + i * C::THREADS) >> 2) % C::BN; };
  auto k_pos_off = [&](int i) {  // bytes within the K row
    const int pos = tid + i * C::THREADS;
    const int r = (pos >> 2) % C::BN;
    return (pos / (4 * C::BN)) * 64 + ((pos & 3) ^ ((r >> 2) & 3)) * 16;
  };
  auto v_pos_row = [&](int i) {  // key (row of the global tile) stored at this position
    const int r = ((tid + i * C::THREADS) >> 2) % C::BN;
    return FP8 ? fp8_vrow(r) : r;
  };
  auto v_pos_off = [&](int i) {
    const int pos = tid + i * C::THREADS;
    const int r = (pos >> 2) % C::BN;
    return (pos / (4 * C::BN)) * 64 + (FP8 ? ((pos & 3) ^ (2 * ((r >> 2) & 1))) : (pos & 3)) * 16;
  };
  // With one wave, copy i of a tile is copy 0 moved by 16 (i mod 4) rows and i / 4 column
  // blocks (the swizzle depends on row bits 2 and 3 only): one offset register per tensor
  // and a constant per copy, instead of a register per copy.
  constexpr bool ONE_WAVE = C::THREADS == 64;
  constexpr int NKSRC = ONE_WAVE ? 1 : C::KCHUNKS, NVSRC = ONE_WAVE ? 1 : C::VCHUNKS;
  uint32_t k_src[NKSRC], v_src[NVSRC];
#pragma unroll
  for (int i = 0; i < NKSRC; ++i) k_src[i] = k_pos_row(i) * C::KROW + k_pos_off(i);
#pragma unroll
  for (int i = 0; i < NVSRC; ++i) v_src[i] = v_pos_row(i) * C::VROW + v_pos_off(i);
  // (tile base, per-lane offset) of copy i
  auto k_copy = [&](const char* tile, int i, uint32_t& off) -> const char* {
    if constexpr (ONE_WAVE) {
      off = k_src[0];
      return tile + 16 * (i & 3) * C::KROW + (i >> 2) * 64;
    } else {
      off = k_src[i];
      return tile;
    }
  };
  auto v_copy = [&](const char* tile, int i, uint32_t& off) -> const char* {
    if constexpr (ONE_WAVE) {
      off = v_src[0];
      return tile + 16 * (i & 3) * C::VROW + (i >> 2) * 64;
    } else {
      off = v_src[i];
      return tile;
    }
  };
  const uint32_t k_lds = lds_address(kring), v_lds = lds_address(vring);
  // One-wave workgroups serve decode, where every cached key and value tile is read by one
  // workgroup only: their copies carry the nontemporal hint (8 x 32K keys: 95.5 against
  // 100.7 us). Prefill tiles are read by every query tile of their head, through L2.
  constexpr bool kStreamKV = WAVES == 1;

  // first K / V byte of key tile t (t0 = t * BN; PAGED: in cache page pg)
  auto k_tile = [&](int t, int pg) -> const char* {
    if constexpr (PAGED) return p.k + page_row(pg, t) * C::KROW;
    else return kbase + (size_t)(t * C::BN) * C::KROW;
  };
  auto v_tile = [&](int t, int pg) -> const char* {
    if constexpr (PAGED) return p.v + page_row(pg, t) * C::VROW;
    else return vbase + (size_t)(t * C::BN) * C::VROW;
  };
  auto fill_k = [&](int t, int buf, int pg) {
    const int t0 = t * C::BN;
    const uint32_t dst = k_lds + buf * C::KBUF + wave_u * 64 * 16;
    if (t0 + C::BN <= Sk) {
      const char* tile = k_tile(t, pg);
#pragma unroll
      for (int i = 0; i < C::KCHUNKS; ++i) {
        uint32_t off;
        const char* base = k_copy(tile, i, off);
        if (k_live(i)) lds_copy16<kStreamKV>(base, off, dst + i * C::THREADS * 16);
      }
    } else {
      // rows past the window's last key repeat it (>= t0: the same tile, and page)
      const char* tile = PAGED ? k_tile(t, pg) : kbase;
      const int r0 = PAGED ? t0 : 0;
#pragma unroll
      for (int i = 0; i < C::KCHUNKS; ++i) {
        const int gr = min(t0 + k_pos_row(i), Sk - 1);
        if (k_live(i)) lds_copy16(tile + (size_t)(gr - r0) * C::KROW + k_pos_off(i), dst + i * C::THREADS * 16);
      }
    }
  };
  auto fill_v = [&](int t, int buf, int pg) {
    const int t0 = t * C::BN;
    const uint32_t dst = v_lds + buf * C::VBUF + wave_u * 64 * 16;
    if (t0 + C::BN <= Sk) {
      const char* tile = v_tile(t, pg);
#pragma unroll
      for (int i = 0; i < C::VCHUNKS; ++i) {
        uint32_t off;
        const char* base = v_copy(tile, i, off);
        if (v_live(i)) lds_copy16<kStreamKV>(base, off, dst + i * C::THREADS * 16);
      }
    } else {
      const char* tile = PAGED ? v_tile(t, pg) : vbase;
      const int r0 = PAGED ? t0 : 0;
#pragma unroll
      for (int i = 0; i < C::VCHUNKS; ++i) {
        const int gr = min(t0 + v_pos_row(i), Sk - 1);
        if (v_live(i)) lds_copy16(tile + (size_t)(gr - r0) * C::VROW + v_pos_off(i), dst + i * C::THREADS * 16);
      }
    }
  };
  // the copies of full tiles, for iterations that only see full tiles (no branch)
  auto fill_k_full = [&](int t, int buf, int pg) {
    const char* tile = k_tile(t, pg);
    const uint32_t dst = k_lds + buf * C::KBUF + wave_u * 64 * 16;
#pragma unroll
    for (int i = 0; i < C::KCHUNKS; ++i) {
      uint32_t off;
      const char* base = k_copy(tile, i, off);
      if (k_live(i)) lds_copy16<kStreamKV>(base, off, dst + i * C::THREADS * 16);
    }
  };
  auto fill_v_full = [&](int t, int buf, int pg) {
    const char* tile = v_tile(t, pg);
    const uint32_t dst = v_lds + buf * C::VBUF + wave_u * 64 * 16;
#pragma unroll
    for (int i = 0; i < C::VCHUNKS; ++i) {
      uint32_t off;
      const char* base = v_copy(tile, i, off);
      if (v_live(i)) lds_copy16<kStreamKV>(base, off, dst + i * C::THREADS * 16);
    }
  };
  // make this wave's copies complete before the barrier that publishes them
  auto wait_fills = [] { wait_vmem(); };

  // ---- per-lane LDS read offsets (the rest of each address is an immediate) ----
  const int xk = (l32 >> 2) & 3;
  int k_off0, k_off1;  // FP8: chunks 2h, 2h+1 of block c; BF16: chunk h (c even), 2+h (c odd) of block c/2
  if constexpr (FP8) {
    k_off0 = l32 * 64 + 16 * ((2 * h) ^ xk);
    k_off1 = l32 * 64 + 16 * ((2 * h + 1) ^ xk);
  } else {
    k_off0 = l32 * 64 + 16 * (h ^ xk);
    k_off1 = l32 * 64 + 16 * ((2 + h) ^ xk);
  }
  const int g1 = (lane >> 4) & 1;
  int v_off0, v_off1;  // FP8: dv block halves 0 / 1 of a 64-byte column block
  if constexpr (FP8) {
    const int r8 = (lane & 15) >> 1;
    const int xv = 2 * ((r8 >> 2) & 1);
    v_off0 = (8 * h + r8) * 64 + 16 * (g1 ^ xv) + 8 * (lane & 1);
    v_off1 = (8 * h + r8) * 64 + 16 * ((2 + g1) ^ xv) + 8 * (lane & 1);
  } else {
    v_off0 = (4 * h + ((lane & 15) >> 2)) * 64 + 32 * g1 + 8 * (lane & 3);
    v_off1 = v_off0;
  }

  // S^T[key][query] of a tile, keys 32g + 8(r/4) + 4h + r%4 (registers r of sacc[g])
  auto qk = [&](int buf, v16f (&s)[2]) {
    const char* kb = kring + buf * C::KBUF;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      s[g] = v16f{0};
#pragma unroll
      for (int c = 0; c < C::NKS; ++c) {
        if constexpr (FP8) {
          const char* blk = kb + c * C::KBLK + 32 * g * 64;
          const v4i lo = *(const v4i*)(blk + k_off0);
          const v4i hi = *(const v4i*)(blk + k_off1);
          const v8i a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          s[g] = mfma_fp8(a, qreg[c], s[g]);
        } else {
          const char* blk = kb + (c >> 1) * C::KBLK + 32 * g * 64;
          s[g] = mfma_bf16(*(const v8bf*)(blk + ((c & 1) ? k_off1 : k_off0)), qreg[c], s[g]);
        }
      }
    }
  };
  auto mask = [&](v16f (&s)[2], int t) {
    const int kt = t * C::BN;
    if (kt + C::BN - 1 > lim_w) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt + 32 * g + 8 * (r >> 2) + 4 * h + (r & 3) > lim_q) s[g][r] = -INFINITY;
    }
  };
  // the same mask, branch-free (one compare and one select per score): for steady
  // iterations over the diagonal tiles, where a branch would split the slot schedule
  auto mask_nb = [&](v16f (&s)[2], int t) {
    const int lim = lim_q - t * C::BN - 4 * h;  // key offsets within the tile up to lim stay
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[g][r] = (32 * g + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[g][r];
  };
  auto rowmax = [&](const v16f (&s)[2]) {
    float m0 = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) m0 = fmaxf(fmaxf(m0, s[0][r]), s[1][r]);
    return max_across_halves(m0);
  };

  v16f oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc[d] = v16f{0};

  // ---- prologue: K0, V0, K1 resident; scores and maxima of tile 0 ----
  if (p.poison_lds) {
    for (int i = tid; i < C::LDS_BYTES / 16; i += C::THREADS) *(v4i*)(smem + 16 * i) = v4i{-1, -1, -1, -1};
    __syncthreads();
  }
  fill_k(0, 0, pg0);
  fill_v(0, 0, pg0);
  if (n > 1) fill_k(1, 1, pg1);
  {
    // the PV stage of the first iteration multiplies an all-zero P with the buffer of
    // "V_-1": make that buffer finite
#pragma unroll
    for (int i = 0; i < C::VCHUNKS; ++i)
      if (tid + i * C::THREADS < C::VSLOTS)
        *(v4i*)(vring + (C::NBUF - 1) * C::VBUF + (tid + i * C::THREADS) * 16) = v4i{0, 0, 0, 0};
  }
  wait_fills();
  __syncthreads();

  // Decode: a wave whose rows all lie past the workgroup's Sq query heads has no work but
  // its share of the tile copies; it runs only those, with the same barriers (one per
  // iteration: copy K_{t+2}; wait for the copies and publish them; copy V_{t+1}, as every
  // iteration of the pipelines below does, on the same buffers)
  // (BF16 only: in the FP8 instantiations the extra path cost the paged kernels at the MLA
  // shape five more spilled registers, and an FP8 group of more than 32 query heads, the
  // only FP8 decode on eight waves, is rare; its surplus waves compute clamped rows)
  const bool idle = PAGED && !FP8 && p.split_keys > 0 && q0 >= Sq;
  auto idle_loop = [&] {
    for (int t = 0; t < n; ++t) {
      const int pg3 = PAGED ? page_of(t + 3) : 0;
      if (t + 2 < n) fill_k(t + 2, (t + 2) % C::NBUF, pg2);
      wait_fills();
      __syncthreads();
      if (t + 1 < n) fill_v(t + 1, (t + 1) % C::NBUF, pg1);
      next_pages(pg3);
    }
  };

  // key tiles that every row of the workgroup sees whole (full tiles inside the window)
  const int n_full = max(0, (min(dpos + q0_wg, Sk - 1) + 1) / C::BN);
  // iterations t < n_steady need no causal mask on tile t+1 in any wave and prefetch
  // K_{t+2}: their bodies are branch-free and carry a fixed instruction schedule. The even
  // n_steady is at most n_full - 2, so every tile they fetch (t + 2 <= n_full - 1) is a
  // full tile inside the window: no clamping.
  const int n_steady = max(0, min(n - 2, n_full - 2)) & ~1;

  v16f sa[2], sb[2];
  qk(0, sa);
  // every wave has read K_0 before any wave's first iteration copies a tile into its buffer
  __syncthreads();
  mask(sa, 0);
  float c_cur = c_q;
  if constexpr (FP8) {
    if constexpr (PAGED) c_cur *= p.k_scale[page_row(pg0, 0) >> p.scale_shift];
    else c_cur *= kscale[min(k_begin >> p.scale_shift, p.nbk - 1)];
  }
  // tile 0 holds the window's key 0, which every row at a position >= 0 sees: finite there
  float xmax0 = rowmax(sa) * c_cur;
  float m_ref = xmax0 > -INFINITY ? ceilf(xmax0) : kRefEmpty;
  bool rescale = false;

  // epilogue: O / o_div as bfloat16, and the log-sum-exp of the row sum l_sum (o_div is
  // l_sum in the units O is accumulated in: they differ when the FP8 V scale is not a power
  // of two, and the log-sum-exp must not depend on V).
  // A lane holds half of its row's 128 values, in 8-byte pieces that alternate with the
  // other half's lane. Stored from there, each store instruction would write 32 rows in
  // 16-byte pieces, and a workgroup's 64 KiB of O would drain slowly, holding its compute
  // unit. So the eight-wave prefill kernels stage each wave's rows through LDS, 64 values of
  // each row per pass in the wave's 4 KiB (128-byte rows, 16-byte chunk c of row r at chunk
  // c ^ (r & 7), so that the writes and the reads below hit distinct banks), and store whole
  // 128-byte lines: 8 rows per instruction. (Decode keeps the direct stores: its rows are a
  // few query heads, and BF16 decode has waves that leave before the epilogue.)
  auto store_out = [&](float o_div, float l_sum) {
    const int my_q = row_of_lane();
    const float inv_l = l_sum > 0.0f ? 1.0f / o_div : 0.0f;  // a row with no key: O = 0, LSE = -inf
    auto piece = [&](int d, int r4) {  // values 32 d + 8 r4 + 4 h .. + 3 of this lane's row
      uint2 w;
      w.x = pack_bf16x2(oacc[d][4 * r4 + 0] * inv_l, oacc[d][4 * r4 + 1] * inv_l);
      w.y = pack_bf16x2(oacc[d][4 * r4 + 2] * inv_l, oacc[d][4 * r4 + 3] * inv_l);
      return w;
    };
    bool staged = C::WAVES == 8;
    if constexpr (PAGED) staged = staged && p.split_keys == 0;
    if (staged) {
      static_assert(C::WAVES != 8 || C::LDS_BYTES >= 8 * 4096, "staging needs 4 KiB of LDS per wave");
      // (uniform over the workgroup: every wave gets here) no wave still reads the K / V
      // ring that the staging reuses
      __syncthreads();
      if (q0 < Sq) {
        char* const area = smem + wave_u * 4096;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
          for (int dd = 0; dd < 2; ++dd)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int c = 4 * dd + r4;  // 16-byte chunk of the pass's 128 bytes of the row
              *(uint2*)(area + l32 * 128 + ((c ^ (l32 & 7)) << 4) + 8 * h) = piece(2 * pass + dd, r4);
            }
          // the wave's own writes, read back by other lanes of the wave
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int c = lane & 7;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int r = 8 * k + (lane >> 3);
            const uint4 x = *(const uint4*)(area + r * 128 + ((c ^ (r & 7)) << 4));
            if (q0 + r < Sq) *(uint4*)(p.o + (o_row0 + q0 + r) * C::DV + 64 * pass + 8 * c) = x;
          }
          // the next pass overwrites the area only after every lane has read it
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
    } else if (q0 < Sq && my_q < Sq) {
      uint16_t* orow = p.o + (o_row0 + my_q) * C::DV;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) *(uint2*)(orow + 32 * d + 8 * r4 + 4 * h) = piece(d, r4);
    }
    if (p.lse != nullptr && h == 0 && q0 < Sq && my_q < Sq) p.lse[o_row0 + my_q] = kLn2 * (m_ref + log2f(l_sum));
  };

  if constexpr (FP8) {
    // ===================== FP8: three-stage pipeline =====================
    const int k127 = opaque(kE8M0One);

    // V scale = rv * 2^ev, rv in [1, 2): 2^ev is the V operand's E8M0 scale (exact);
    // rv is 1 for power-of-two scales (as zyfa_quantize_fp8 writes them). O is kept in
    // units of 1 / rv of the last tile added, and rescaled by the ratio when rv changes.
    v16f rs_acc = v16f{0};  // rounded row sum, accumulated on the MFMA (any register holds it)
    float rv_o = 1.0f;      // O holds sum(w v) / rv_o

    // (the scale is the same in every lane: integer fields of its bits, on the scalar
    // unit; for a normal float, sv is its biased exponent and rv keeps sign and mantissa.
    // A subnormal scale m 2^-149 (0 < m < 2^23) takes E8M0 code 0, 2^-127, and rv = m 2^-22
    // in (0, 2), normalised here with integer operations: exact, and branch-free)
    auto vsplit = [&](float vsc, float& rv, int& sv) {
      const int b = __builtin_amdgcn_readfirstlane(__float_as_int(vsc));
      sv = (b >> 23) & 0xff;
      const int mant = b & 0x7fffff;
      const int top = 31 - __builtin_clz(mant | 1);  // leading bit of a subnormal's mantissa
      const int sub = (b & (int)0x80000000) | ((top + 105) << 23) | ((mant << (23 - top)) & 0x7fffff);
      rv = __int_as_float(sv != 0 ? ((b & (int)0x807fffff) | 0x3f800000) : sub);
    };
    // K and V scales of tile t+1 while iteration t runs; the loads for tile t+2 are
    // issued at the top of iteration t, ahead of the tile fills whose wait covers them
    // K and V scales of a tile (PAGED: page scale blocks, indexed by the tile's cache row; a
    // page holds whole scale blocks)
    auto sidx = [&](int tile) { return min((k_begin + tile * C::BN) >> p.scale_shift, p.nbk - 1); };
    auto ksc = [&](int tile, int pg) {
      if constexpr (PAGED) return p.k_scale[page_row(pg, tile) >> p.scale_shift];
      else return kscale[sidx(tile)];
    };
    auto vsc = [&](int tile, int pg) {
      if constexpr (PAGED) return p.v_scale[page_row(pg, tile) >> p.scale_shift];
      else return vscale[sidx(tile)];
    };
    float ks_next = ksc(1, pg1);
    float vs_next = vsc(1, pg1);
    // scale exponent e of a block whose row maximum is xmax (base 2): p = 2^(s c - m_ref - e)
    // puts the maximum in [2^kPHeadroom, 2^(kPHeadroom + 1)); 2^-e is the E8M0 scale code
    // 127 + e, kept >= 1 (a block more than 119 binades below the reference holds weights
    // that round to zero either way)
    auto block_exp = [&](float xmax) {
      return (int)fmaxf(floorf(xmax - m_ref) - (float)kPHeadroom, -126.0f);
    };

    float rv_cur;
    int sv_cur;
    vsplit(vsc(0, pg0), rv_cur, sv_cur);
    int eb_cur = block_exp(xmax0);

    v8i pa = v8i{0}, pb = v8i{0};
    int sp_prev = kE8M0One, sv_prev = kE8M0One;
    float rv_prev = 1.0f;
    // Lazy reference: m_ref moves (to the ceiling of a row's new maximum) only for rows
    // whose maximum exceeds it by more than kLazyThreshold. The iteration that sees tile
    // t+1's maxima takes the decision (grow; rescale = some row grows) and the block
    // exponent against the current m_ref; fix_units at the top of the next iteration
    // moves m_ref, recomputes that exponent and rescales O (rare, wave-uniform branch).
    float xmax_pend = 0.0f;  // tile t+1's row maxima in base-2 units
    bool grow = false;

    // e4m3 codes of four probabilities p = 2^(s c - bias) of one query row (s: raw
    // scores j0..j0+3 of a 32-key group), packed low byte first. Exact mode: hardware
    // exponential, then round-to-nearest-even conversion. Lean mode ("Lean P: Linear
    // Approximation of the FP8 Code"): the code as a linear function of y = s c - bias on
    // the grid of sixteen steps per binade, round-half-even(16 y + kLean16Bias) clamped to
    // [0, 255], then halved to e4m3's eight with the mantissa-dependent rounding of the odd
    // half-steps (a byte lookup of the four codes at once). y < kPHeadroom + 1 keeps the
    // code at most 119, below e4m3's NaN code 127. Per score: one FMA and one conversion,
    // plus six integer operations per four scores, instead of an exponential and half a
    // conversion.
    auto p_codes = [&](const v16f& sv, int j0, float c, float bias) -> int {
      if constexpr (LEAN) {
        const float c16 = 16.0f * c, b16 = fmaf(-16.0f, bias, kLean16Bias);
        unsigned r = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sv[j0 + 0], c16, b16), 0, 0u);
        r = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sv[j0 + 1], c16, b16), 1, r);
        r = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sv[j0 + 2], c16, b16), 2, r);
        r = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sv[j0 + 3], c16, b16), 3, r);
        // per byte: (c16 + up[(c16 >> 1) & 7]) >> 1, no carry between bytes (c16 <= 239)
        const unsigned up = __builtin_amdgcn_perm(kLeanUpHi, kLeanUpLo, (r >> 1) & 0x07070707u);
        return (int)(((r + up) >> 1) & 0x7F7F7F7Fu);
      } else {
        const float p0 = fast_exp2(fmaf(sv[j0 + 0], c, -bias));
        const float p1 = fast_exp2(fmaf(sv[j0 + 1], c, -bias));
        const float p2 = fast_exp2(fmaf(sv[j0 + 2], c, -bias));
        const float p3 = fast_exp2(fmaf(sv[j0 + 3], c, -bias));
        // (the low-half conversion keeps the high half of its destination, which the
        // second conversion overwrites: passing p0's bits there, a register that dies in
        // this instruction, spares clearing one)
        return cvt_pk_fp8<true>(p2, p3, cvt_pk_fp8<false>(p0, p1, __float_as_int(p0)));
      }
    };

    // bring O and the row sum to the units of the P about to be added: the pending
    // reference move (a power of two, 2^(m_ref - m_new); the in-flight P gets it through
    // its E8M0 scale) and the V-scale mantissa ratio. Both are rare: the branch is
    // uniform per wave.
    auto fix_units = [&]() {
      if (rescale || __float_as_int(rv_prev) != __float_as_int(rv_o)) {
        rare_branch();
        int la = 0;
        float a = 1.0f;
        if (rescale) {
          const float m_new = grow ? ceilf(xmax_pend) : m_ref;
          la = (int)fmaxf(m_ref - m_new, -256.0f);  // (from an empty row's reference: any factor below 2^-149 is 0)
          a = fast_exp2((float)la);
          m_ref = m_new;
          eb_cur = block_exp(xmax_pend);
        }
        const float f = a * (rv_o / rv_prev);
#pragma unroll
        for (int d = 0; d < 4; ++d) oacc[d] *= f;
        if (rescale) {
          rs_acc[0] *= a;
          sp_prev = max(sp_prev + la, 0);
        }
        rv_o = rv_prev;
        rescale = false;
      }
    };

    // O^T += V^T P^T and the rounded row sum, for the tile whose P is pp
    auto pv = [&](const v8i& pp, int sp, int sv, int vbuf) {
      const char* vb = vring + vbuf * C::VBUF;
      const int svr = opaque(sv);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        int va[8];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const char* src = vb + (d >> 1) * C::KBLK + 16 * qd * 64 + ((d & 1) ? v_off1 : v_off0);
          v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)src);
          va[2 * qd] = x[0];
          va[2 * qd + 1] = x[1];
        }
        const v8i a = {va[0], va[1], va[2], va[3], va[4], va[5], va[6], va[7]};
        oacc[d] = mfma_fp8_scaled(a, pp, oacc[d], svr, sp);
      }
      rs_acc = mfma_ones_fp4_by_fp8(pp, rs_acc, k127, sp);
    };

    // Generic iteration t (the diagonal tiles and the tail), in program order: copy
    // K_{t+2}; QK of tile t+1; PV of tile t-1; P of tile t; maxima of tile t+1 (masked)
    // and the lazy decision; barrier; copy V_{t+1}.
    auto step = [&](int t, v16f (&s_cur)[2], v16f (&s_next)[2], v8i& p_prev, v8i& p_cur) {
      const bool has_next = t + 1 < n;
      fix_units();
      const int pg3 = PAGED ? page_of(t + 3) : 0;
      const float ks_pf = ksc(t + 2, pg2);
      const float vs_pf = vsc(t + 2, pg2);
      if (t + 2 < n) fill_k(t + 2, (t + 2) % C::NBUF, pg2);
      if (has_next) qk((t + 1) % C::NBUF, s_next);
      pv(p_prev, sp_prev, sv_prev, (t + C::NBUF - 1) % C::NBUF);

      // p = 2^(s*c - m_ref - eb): the block maximum lands in [2^kPHeadroom, 2^(kPHeadroom+1)),
      // rounded to e4m3
      const float bias = m_ref + (float)eb_cur;
      int pw[8];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pw[4 * g + w] = p_codes(s_cur[g], 4 * w, c_cur, bias);
        }
      p_cur = v8i{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
      sp_prev = kE8M0One + eb_cur;
      sv_prev = sv_cur;
      rv_prev = rv_cur;

      float xmax = 0.0f, c_next = c_cur;
      if (has_next) {
        mask(s_next, t + 1);
        c_next = c_q * ks_next;
        xmax = rowmax(s_next) * c_next;
      }
      if (has_next) {
        // lazy reference decision (carried out by the next fix_units)
        grow = xmax > m_ref + kLazyThreshold;
        rescale = __any(grow);
        xmax_pend = xmax;
        vsplit(vs_next, rv_cur, sv_cur);
        eb_cur = block_exp(xmax);
        c_cur = c_next;
      }
      wait_fills();
      ks_next = ks_pf;
      vs_next = vs_pf;
      __syncthreads();
      if (has_next) fill_v(t + 1, (t + 1) % C::NBUF, pg1);
      next_pages(pg3);
    };

    // Steady iteration, hand-ordered: slot i issues matrix instruction i (QK of tile t+1,
    // then PV and the row sum of tile t-1), fetches the LDS operands of instruction i+2,
    // and runs one 64-cycle share of the vector work (4 exponentials and 2 conversions of
    // tile t's probabilities, or the maxima of tile t+1 once its scores are complete).
    // sched_barrier keeps each slot's instructions in place.
    // MASKED: the same schedule over the diagonal tiles (any iteration with a next tile):
    // tile t+1's scores are masked before its maxima, and the copies clamp to the
    // sequence (K_{t+2} only if it exists).
    auto steady_step = [&](auto masked_tag, int t, v16f (&s_cur)[2], v16f (&s_next)[2], v8i& p_prev, v8i& p_cur) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      constexpr int NQK = 2 * C::NKS;
      constexpr int NSLOT = NQK + 5;
      fix_units();
      const char* kb = kring + ((t + 1) % C::NBUF) * C::KBUF;
      const char* vb = vring + ((t + C::NBUF - 1) % C::NBUF) * C::VBUF;  // V of tile t-1
      const float bias = m_ref + (float)eb_cur;
      const int svr = opaque(sv_prev);
      const int sp = sp_prev;
      v8i op[3];
      auto read_op = [&](int i, v8i& dst) {
        if (i < NQK) {
          const char* blk = kb + (i >> 1) * C::KBLK + 32 * (i & 1) * 64;
          const v4i lo = *(const v4i*)(blk + k_off0);
          const v4i hi = *(const v4i*)(blk + k_off1);
          dst = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else if (i < NQK + 4) {
          const int d = i - NQK;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const char* src = vb + (d >> 1) * C::KBLK + 16 * qd * 64 + ((d & 1) ? v_off1 : v_off0);
            const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)src);
            dst[2 * qd] = x[0];
            dst[2 * qd + 1] = x[1];
          }
        }
      };
      const int pg3 = PAGED ? page_of(t + 3) : 0;
      const float ks_pf = ksc(t + 2, pg2);
      const float vs_pf = vsc(t + 2, pg2);
      read_op(0, op[0]);
      read_op(1, op[1]);
      if constexpr (MASKED) {
        if (t + 2 < n) fill_k(t + 2, (t + 2) % C::NBUF, pg2);
      } else {
        fill_k_full(t + 2, (t + 2) % C::NBUF, pg2);
      }
      s_next[0] = v16f{0};
      s_next[1] = v16f{0};
      // tile t's values, before the update for tile t+1 inside the slots replaces them
      const float c_t = c_cur;
      const int eb_t = eb_cur, sv_t = sv_cur;
      const float rv_t = rv_cur;
      float mx = -INFINITY, xmax = 0.0f, c_next = 0.0f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NSLOT; ++i) {
        // operand reads first, then the vector share, then the matrix instruction: the
        // wait for the operands of instruction i (read two slots earlier) comes after
        // this slot's vector work has issued
        if (i + 2 < NSLOT) read_op(i + 2, op[(i + 2) % 3]);
        if (i < 8) {
          const int g = i >> 2, w = i & 3;
          p_cur[i] = p_codes(s_cur[g], 4 * w, c_t, bias);
          keep_here(p_cur[i]);
        }
        // the scores of tile t+1 are complete one slot after the last QK instruction:
        // row maxima in slots NSLOT-4 and NSLOT-3, then the lazy reference update for
        // tile t+1 in the last two slots, beside the PV and row-sum instructions
        if constexpr (MASKED) {
          if (i == NSLOT - 4) mask_nb(s_next, t + 1);
        }
        if (i == NSLOT - 4 || i == NSLOT - 3) {
          const int r0 = i == NSLOT - 4 ? 0 : 8;
#pragma unroll
          for (int r = r0; r < r0 + 8; ++r) mx = fmaxf(fmaxf(mx, s_next[0][r]), s_next[1][r]);
        }
        if (i == NSLOT - 2) {
          // (the scales were loaded an iteration earlier; opaque keeps their use, and the
          // wait for their loads, in this slot)
          c_next = c_q * opaque_f(ks_next);
          xmax = max_across_halves(mx) * c_next;
          grow = xmax > m_ref + kLazyThreshold;
          rescale = __any(grow);
        }
        if (i == NSLOT - 1) {
          xmax_pend = xmax;
          vsplit(opaque_f(vs_next), rv_cur, sv_cur);
          eb_cur = block_exp(xmax);
          c_cur = c_next;
        }
        if (i < NQK)
          s_next[i & 1] = mfma_fp8(op[i % 3], qreg[i >> 1], s_next[i & 1]);
        else if (i < NQK + 4)
          oacc[i - NQK] = mfma_fp8_scaled(op[i % 3], p_prev, oacc[i - NQK], svr, sp);
        else
          rs_acc = mfma_ones_fp4_by_fp8(p_prev, rs_acc, k127, sp);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the products of this iteration stay in its slots (the next iteration's unit fix
      // is a branch, and the compiler would otherwise sink them past it)
#pragma unroll
      for (int d = 0; d < 4; ++d) keep_here(oacc[d]);
      keep_here(rs_acc);
      sp_prev = kE8M0One + eb_t;
      sv_prev = sv_t;
      rv_prev = rv_t;
      ks_next = ks_pf;
      vs_next = vs_pf;
      wait_fills();
      __syncthreads();
      // V_{t+1} replaces V_{t-1}, last read by this iteration's PV products
      if constexpr (MASKED) {
        fill_v(t + 1, (t + 1) % C::NBUF, pg1);
      } else {
        fill_v_full(t + 1, (t + 1) % C::NBUF, pg1);
      }
      next_pages(pg3);
    };

    ZYFA_TL_PUT(6, (unsigned long long)n);
    ZYFA_TL_CLOCK(1);
    int t = 0;
    for (; t < n_steady; t += 2) {
      steady_step(std::false_type{}, t, sa, sb, pa, pb);
      steady_step(std::false_type{}, t + 1, sb, sa, pb, pa);
    }
    // the diagonal tiles, in pairs while both iterations of a pair have a next tile
    for (; t + 2 < n; t += 2) {
      steady_step(std::true_type{}, t, sa, sb, pa, pb);
      steady_step(std::true_type{}, t + 1, sb, sa, pb, pa);
    }
    for (; t < n; t += 2) {
      step(t, sa, sb, pa, pb);
      if (t + 1 < n) step(t + 1, sb, sa, pb, pa);
    }
    // drain: PV of the last tile (its P is pb if n - 1 is even, else pa)
    ZYFA_TL_CLOCK(2);
    fix_units();
    pv(((n - 1) & 1) ? pa : pb, sp_prev, sv_prev, (n - 1) % C::NBUF);
#pragma unroll
    for (int d = 0; d < 4; ++d) pin_acc(oacc[d]);
    pin_acc(rs_acc);
    // O = oacc * rv_o / l; the log-sum-exp from l alone
    store_out(rs_acc[0] / rv_o, LEAN ? rs_acc[0] * kLeanSumScale : rs_acc[0]);
    ZYFA_TL_CLOCK(3);
  } else {
    // ===================== BF16: three-stage pipeline =====================
    // Iteration t: PV of tile t-1 (its P formed in iteration t-1), then the maxima of
    // tile t with the lazy reference decision, P of tile t (bf16; float32 row sum of the
    // unrounded values), and QK of tile t+1. P and S each live in one set of registers:
    // P's operand tt is rewritten only after the PV products that read it, and a key
    // group's scores only after its probabilities are formed. A reference move (rare,
    // before any probability of tile t) scales the row sum at once and O at the top of
    // the next iteration, once the PV of the old-unit P has been added; the factor is a
    // power of two, exact in float32.
    float l_part = 0.0f;   // this lane's half of the row sum
    float o_fix = 1.0f;    // pending factor for O
    bool o_pending = false;
    // P of a tile: dword k packs scores 2k, 2k+1 (score i is s[i / 16][i % 16]), so the
    // operand of PV instruction tt (keys 16 tt .. 16 tt + 15) is dwords 4 tt .. 4 tt + 3
    v4i pw[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) pw[tt] = v4i{0, 0, 0, 0};
    v16f (&sc)[2] = sa;  // scores of the current tile, then of the next

    auto fix_o = [&]() {
      if (o_pending) {
        rare_branch();
#pragma unroll
        for (int d = 0; d < 4; ++d) oacc[d] *= o_fix;
        o_fix = 1.0f;
        o_pending = false;
      }
    };
    // lazy reference decision for the tile whose row maxima (base-2 units) are xmax:
    // m_ref moves to ceil(xmax) in rows that exceed it by more than kLazyThreshold
    auto lazy_ref = [&](float xmax) {
      const bool grow = xmax > m_ref + kLazyThreshold;
      if (__any(grow)) {
        rare_branch();
        const float m_new = grow ? ceilf(xmax) : m_ref;
        const float a = fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_part *= a;
        o_fix *= a;
        o_pending = true;
      }
    };
    auto v_operand = [&](const char* vb, int d, int tt) {
      const char* src = vb + d * C::KBLK + (32 * (tt >> 1) + 16 * (tt & 1)) * 64;
      const v4bf x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)src);
      const v4bf x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(src + 8 * 64));
      return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // probability of score i of the current tile
    auto prob = [&](int i) {
      const float pr = fast_exp2(fmaf(sc[i >> 4][i & 15], c_cur, -m_ref));
      l_part += pr;
      return pr;
    };

    // Generic iteration (the diagonal tiles and the tail), in program order.
    auto step = [&](int t) {
      fix_o();
      const int pg3 = PAGED ? page_of(t + 3) : 0;
      if (t + 2 < n) fill_k(t + 2, t & 1, pg2);
      {
        const char* vb = vring + ((t + 1) & 1) * C::VBUF + v_off0;  // V of tile t-1
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            oacc[d] = mfma_bf16(v_operand(vb, d, tt), __builtin_bit_cast(v8bf, pw[tt]), oacc[d]);
      }
      mask(sc, t);
      lazy_ref(rowmax(sc) * c_cur);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float p0 = prob(2 * k);
        pw[k >> 2][k & 3] = (int)pack_bf16x2(p0, prob(2 * k + 1));
      }
      if (t + 1 < n) qk((t + 1) & 1, sc);
      wait_fills();
      __syncthreads();
      if (t + 1 < n) fill_v(t + 1, (t + 1) & 1, pg1);
      next_pages(pg3);
    };

    // Steady iteration, hand-ordered: slot i issues matrix instruction i (PV of tile t-1:
    // dv block j % 4, key chunk j / 4 for j = i; then QK of tile t+1: key group j / NKS,
    // head-dim chunk j % NKS for j = i - 16), fetches the LDS operand of instruction
    // i+2, and runs one share of the vector work: the maxima of key group 1 (slots 0-1;
    // group 0 was done at the end of the previous iteration), the lazy decision (slots
    // 2-3), the 32 probabilities (score i in slot 4 + 5i/8: slots 4-23), and the maxima
    // of the next tile's key group 0 (four slots from MX0_SLOT, two after its last
    // product).
    constexpr int NQKB = 2 * C::NKS;
    constexpr int NSLOTB = 16 + NQKB;
    constexpr int MX0_SLOT = 16 + C::NKS + 1;
    static_assert(C::NKS == 8 || C::NKS == 12, "BF16 slot plan");
    // steady iterations: tile t unmasked in every row of the workgroup, K_{t+2} a full
    // tile inside the window, and a next tile
    const int n_steady_b = max(0, min(n_full, min(Sk / C::BN - 2, n - 1)));
    float mx0 = -INFINITY;  // row maxima of the current tile's key group 0 (this lane's half)
    // MASKED: the same schedule over the diagonal tiles (any iteration with a next tile):
    // tile t's scores are masked in slot 0 and its maxima taken over both key groups
    // there (the group-0 maxima carried from the previous iteration were unmasked); the
    // copies clamp to the sequence (K_{t+2} only if it exists).
    auto steady_step = [&](auto masked_tag, int t) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      fix_o();
      const int pg3 = PAGED ? page_of(t + 3) : 0;
      if constexpr (MASKED) {
        if (t + 2 < n) fill_k(t + 2, t & 1, pg2);
      } else {
        fill_k_full(t + 2, t & 1, pg2);
      }
      const char* kb = kring + ((t + 1) & 1) * C::KBUF;           // K of tile t+1
      const char* vb = vring + ((t + 1) & 1) * C::VBUF + v_off0;  // V of tile t-1
      auto read_op = [&](int i) -> v8bf {
        if (i < 16) return v_operand(vb, i & 3, i >> 2);
        const int j = i - 16, g = j / C::NKS, c = j % C::NKS;
        return *(const v8bf*)(kb + (c >> 1) * C::KBLK + 32 * g * 64 + ((c & 1) ? k_off1 : k_off0));
      };
      v8bf op[3];
      op[0] = read_op(0);
      op[1] = read_op(1);
      float mx = MASKED ? -INFINITY : mx0, xmax = 0.0f, p_even = 0.0f;
      // Waves w and w + 4 share a SIMD and leave each barrier together; the arbiter favours
      // the older one, which then waits at the next barrier while the younger finishes its
      // slots alone (measured in cycle stamps: about a fifth of the iteration). The younger
      // wave takes precedence for the first three quarters of the slots (1.3-1.6 % faster,
      // A/B on one box).
      if (wave_u >= 4) __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
      for (int i = 0; i < NSLOTB; ++i) {
        if (i == 3 * NSLOTB / 4) __builtin_amdgcn_s_setprio(0);
        if (i + 2 < NSLOTB) op[(i + 2) % 3] = read_op(i + 2);
        if constexpr (MASKED) {
          if (i == 0) mask_nb(sc, t);
        }
        if (i < 2) {
#pragma unroll
          for (int r = 8 * i; r < 8 * i + 8; ++r) {
            mx = fmaxf(mx, sc[1][r]);
            if constexpr (MASKED) mx = fmaxf(mx, sc[0][r]);
          }
        }
        if (i == 2) xmax = max_across_halves(mx) * c_cur;
#pragma clang loop unroll(full)
        for (int k = 0; k < 32; ++k) {
          if (4 + ((5 * k) >> 3) == i) {
            const float pr = prob(k);
            if (k & 1) {
              pw[k >> 3][(k >> 1) & 3] = (int)pack_bf16x2(p_even, pr);
              keep_here(pw[k >> 3]);
            } else {
              p_even = pr;
            }
          }
        }
        if (i >= MX0_SLOT && i < MX0_SLOT + 4) {
          if (i == MX0_SLOT) mx0 = -INFINITY;
#pragma unroll
          for (int r = 4 * (i - MX0_SLOT); r < 4 * (i - MX0_SLOT) + 4; ++r) mx0 = fmaxf(mx0, sc[0][r]);
        }
        if (i < 16) {
          oacc[i & 3] = mfma_bf16(op[i % 3], __builtin_bit_cast(v8bf, pw[i >> 2]), oacc[i & 3]);
        } else {
          const int j = i - 16, g = j / C::NKS, c = j % C::NKS;
          // (a group's first product starts from zero: no register clearing)
          sc[g] = mfma_bf16(op[i % 3], qreg[c], c == 0 ? v16f{0} : sc[g]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (i == 3) {
          lazy_ref(xmax);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the products of this iteration stay in its slots (the next iteration's O fix is a
      // branch, and the compiler would otherwise sink them past it)
#pragma unroll
      for (int d = 0; d < 4; ++d) keep_here(oacc[d]);
      wait_fills();
      __syncthreads();
      // V_{t+1} replaces V_{t-1}, last read by this iteration's PV products
      if constexpr (MASKED) {
        fill_v(t + 1, (t + 1) & 1, pg1);
      } else {
        fill_v_full(t + 1, (t + 1) & 1, pg1);
      }
      next_pages(pg3);
    };

    // the tile-0 scores are in sc (masked); the steady iterations need the maxima of
    // their tile's key group 0 on entry
    {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx0 = fmaxf(mx0, sc[0][r]);
    }
    if (idle) {
      idle_loop();
      return;
    }
    ZYFA_TL_PUT(6, (unsigned long long)n);
    ZYFA_TL_CLOCK(1);
    int t = 0;
    for (; t < n_steady_b; ++t) steady_step(std::false_type{}, t);
    for (; t + 1 < n; ++t) steady_step(std::true_type{}, t);  // the diagonal tiles
    for (; t < n; ++t) step(t);
    // drain: PV of the last tile
    ZYFA_TL_CLOCK(2);
    fix_o();
    {
      const char* vb = vring + ((n - 1) & 1) * C::VBUF + v_off0;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          oacc[d] = mfma_bf16(v_operand(vb, d, tt), __builtin_bit_cast(v8bf, pw[tt]), oacc[d]);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) pin_acc(oacc[d]);
    const float l_sum = sum_across_halves(l_part);
    store_out(l_sum, l_sum);
    ZYFA_TL_CLOCK(3);
  }
}

template <bool FP8, int DQK, bool LEAN = false, bool PAGED = false, int WAVES = 8>
static hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  using C = Cfg<FP8, DQK, WAVES>;
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
  p.Sq = a.Sq;
  p.Skv = a.Skv;
  p.k_begin = a.k_begin;
  p.Sk = a.k_end - a.k_begin;
  p.d = a.q_offset - a.k_begin;
  p.scale_shift = FP8 ? (a.scale_block == 64 ? 6 : 7) : 0;
  p.nbq = FP8 ? (a.Sq + a.scale_block - 1) / a.scale_block : 0;
  p.nbk = FP8 ? (a.Skv + a.scale_block - 1) / a.scale_block : 0;
  p.cu_seqlens = a.cu_seqlens;
  p.max_seqlen = a.max_seqlen;
  p.block_table = a.block_table;
  p.kv_lens = a.kv_lens;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.page_shift = a.page_size == 64 ? 6 : a.page_size == 128 ? 7 : 8;
  p.split_keys = a.split_keys;
  p.part_rows = (size_t)a.part_rows;
  p.poison_lds = lds_poison_requested() ? 1 : 0;
  p.n_qtiles = a.split_keys > 0 ? a.n_splits
                                : ((a.cu_seqlens != nullptr ? a.max_seqlen : a.Sq) + C::BM - 1) / C::BM;
  p.scale_log2 = a.softmax_scale * kLog2e;
  const long long grid = (long long)p.n_qtiles * a.B * a.Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<FP8, DQK, LEAN, PAGED, WAVES>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream,
                     p);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_fp8(const AttnArgs& a, bool lean, hipStream_t stream) {
  if (a.block_table != nullptr && a.split_keys > 0 && a.Sq <= 32) {  // decode, one wave per workgroup
    if (lean)
      return a.Dqk == 192 ? launch<true, 192, true, true, 1>(a, stream) : launch<true, 128, true, true, 1>(a, stream);
    return a.Dqk == 192 ? launch<true, 192, false, true, 1>(a, stream) : launch<true, 128, false, true, 1>(a, stream);
  }
  if (a.block_table != nullptr) {
    if (lean) return a.Dqk == 192 ? launch<true, 192, true, true>(a, stream) : launch<true, 128, true, true>(a, stream);
    return a.Dqk == 192 ? launch<true, 192, false, true>(a, stream) : launch<true, 128, false, true>(a, stream);
  }
  if (lean) return a.Dqk == 192 ? launch<true, 192, true>(a, stream) : launch<true, 128, true>(a, stream);
  return a.Dqk == 192 ? launch<true, 192>(a, stream) : launch<true, 128>(a, stream);
}

#ifdef ZYFA_TIMELINE
}  // namespace zyfa

extern "C" int zyfa_timeline_clear(void* stream) {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(zyfa::timeline));
  if (e == hipSuccess) e = hipMemsetAsync(p, 0, sizeof(zyfa::timeline), (hipStream_t)stream);
  return (int)e;
}

extern "C" int zyfa_timeline_read(unsigned long long* host, long long n_workgroups) {
  if (host == nullptr || n_workgroups < 0 || n_workgroups > ZYFA_TIMELINE_WORKGROUPS) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(zyfa::timeline),
                                  (size_t)n_workgroups * ZYFA_TIMELINE_FIELDS * sizeof(unsigned long long), 0,
                                  hipMemcpyDeviceToHost);
}

namespace zyfa {
#endif

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  // (BF16 decode stays on the eight-wave workgroup: a one-wave BF16 workgroup measured
  // four times slower)
  if (a.block_table != nullptr)
    return a.Dqk == 192 ? launch<false, 192, false, true>(a, stream) : launch<false, 128, false, true>(a, stream);
  return a.Dqk == 192 ? launch<false, 192>(a, stream) : launch<false, 128>(a, stream);
}

}  // namespace zyfa
