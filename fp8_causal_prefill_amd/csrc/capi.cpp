// The C ABI declared in include/zyfa.h: argument validation, dispatch, status codes.
// Every check runs on the host before any HIP call, so an invalid request enqueues
// no device work and touches no device state.
#include <math.h>
#include <stdarg.h>

#include <initializer_list>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/zyfa.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

// a nonempty environment variable other than "0"
bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

zyfa_status fail(zyfa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  // ZYFA_DEBUG: every failed call also reports its message on stderr
  if (env_flag("ZYFA_DEBUG")) fprintf(stderr, "zyfa: %s: %s\n", zyfa_status_string(st), g_last_error);
  return st;
}

zyfa_status ok() {
  g_last_error[0] = '\0';
  return ZYFA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Whether the product of positive factors exceeds limit (>= 0), decided without forming
// any product larger than limit: the running product p times the next factor f exceeds
// limit exactly when p > floor(limit / f).
bool product_exceeds(long long limit, std::initializer_list<long long> factors) {
  long long p = 1;
  for (const long long f : factors) {
    if (p > limit / f) return true;
    p *= f;
  }
  return false;
}

// Largest element count any tensor may have (keeps every 64-bit offset far from overflow
// and every per-head row count within int range).
constexpr long long kMaxElems = 1LL << 40;
// Largest sequence position a query row may have (keeps position arithmetic in int range).
constexpr long long kMaxPosition = 1LL << 30;

zyfa_status check_attn_common(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
                              int Hq, int Hkv, int Sq, int Skv, int q_offset, int k_begin, int k_end, int Dqk, int Dv,
                              float softmax_scale) {
  if (!q || !k || !v || !o) return fail(ZYFA_ERR_INVALID_ARGUMENT, "q, k, v and o must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "B, Hq, Hkv and the sequence lengths must be positive (got %d, %d, %d, %d, %d)",
                B, Hq, Hkv, Sq, Skv);
  if (Hq % Hkv != 0) return fail(ZYFA_ERR_INVALID_ARGUMENT, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and positive");
  if (Dqk <= 0 || Dv <= 0) return fail(ZYFA_ERR_INVALID_ARGUMENT, "head dims must be positive");
  if (q_offset < 0 || (long long)q_offset + Sq > kMaxPosition)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "q_offset (%d) must be >= 0 and q_offset + Sq at most 2^30", q_offset);
  if (k_begin < 0 || k_begin >= k_end || k_end > Skv)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "the key window [%d, %d) must be non-empty and inside [0, Skv = %d)",
                k_begin, k_end, Skv);
  if (k_begin % zyfa::kKeyTile != 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "k_begin (%d) must be a multiple of %d", k_begin, zyfa::kKeyTile);
  const long long dmax = Dqk > Dv ? Dqk : Dv;
  if (product_exceeds(kMaxElems, {B, Hq, Sq, dmax}) || product_exceeds(kMaxElems, {B, Hkv, Skv, dmax}))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "tensor too large");
  if (!((Dqk == 128 && Dv == 128) || (Dqk == 192 && Dv == 128)))
    return fail(ZYFA_ERR_UNSUPPORTED, "(Dqk, Dv) = (%d, %d) is not supported; use (128, 128) or (192, 128)", Dqk, Dv);
  const long long n_qtiles = (Sq + 127) / 128;
  if (product_exceeds(0x7FFFFFFFLL, {n_qtiles, B, Hq})) return fail(ZYFA_ERR_UNSUPPORTED, "grid too large");
  if ((o == q || o == k || o == v) || (lse && (lse == q || lse == k || lse == v || lse == o)))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
  return ZYFA_OK;
}

}  // namespace

bool zyfa::lds_poison_requested() { return env_flag("ZYFA_LDS_POISON"); }

extern "C" {

int zyfa_abi_version(void) { return ZYFA_ABI_VERSION; }

const char* zyfa_status_string(int status) {
  switch (status) {
    case ZYFA_OK: return "ZYFA_OK";
    case ZYFA_ERR_INVALID_ARGUMENT: return "ZYFA_ERR_INVALID_ARGUMENT";
    case ZYFA_ERR_UNSUPPORTED: return "ZYFA_ERR_UNSUPPORTED";
    case ZYFA_ERR_LAUNCH: return "ZYFA_ERR_LAUNCH";
    default: return "ZYFA_UNKNOWN_STATUS";
  }
}

const char* zyfa_last_error(void) { return g_last_error; }

zyfa_status zyfa_quantize_fp8(const void* x, int x_is_bf16, uint8_t* codes, float* scales, int B, int H, int S,
                              int D, int scale_block, int hadamard, void* stream) {
  if (!x || !codes || !scales) return fail(ZYFA_ERR_INVALID_ARGUMENT, "x, codes and scales must be non-null");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (x_is_bf16 != 0 && x_is_bf16 != 1) return fail(ZYFA_ERR_INVALID_ARGUMENT, "x_is_bf16 must be 0 or 1");
  if (hadamard != 0 && hadamard != 1) return fail(ZYFA_ERR_INVALID_ARGUMENT, "hadamard must be 0 or 1");
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "B, H, S and D must be positive (got %d, %d, %d, %d)", B, H, S, D);
  if (scale_block != 64 && scale_block != 128)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale_block must be 64 or 128 (got %d)", scale_block);
  if (product_exceeds(kMaxElems, {B, H, S, D})) return fail(ZYFA_ERR_INVALID_ARGUMENT, "tensor too large");
  if (D != 128 && D != 192) return fail(ZYFA_ERR_UNSUPPORTED, "D = %d is not supported; use 128 or 192", D);

  const long long nb = (S + scale_block - 1) / scale_block;
  if (product_exceeds(0x7FFFFFFFLL, {nb, B, H})) return fail(ZYFA_ERR_UNSUPPORTED, "grid too large");
  if ((const void*)codes == x || (const void*)scales == x || (const void*)scales == (const void*)codes)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");

  zyfa::QuantArgs a{x, x_is_bf16, codes, scales, B, H, S, D, scale_block, hadamard};
  hipError_t e = zyfa::launch_quantize_fp8(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "quantize launch failed: %s", hipGetErrorString(e));
  return ok();
}

static zyfa_status attn_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                            const float* k_scale, const float* v_scale, int scale_block, uint16_t* o, float* lse,
                            int B, int Hq, int Hkv, int Sq, int Skv, int q_offset, int k_begin, int k_end, int Dqk,
                            int Dv, float softmax_scale, void* stream, bool lean) {
  zyfa_status st = check_attn_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, q_offset, k_begin, k_end, Dqk, Dv,
                                     softmax_scale);
  if (st != ZYFA_OK) return st;
  if (!q_scale || !k_scale || !v_scale) return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale pointers must be non-null");
  if (!aligned16(q_scale) || !aligned16(k_scale) || !aligned16(v_scale))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (scale_block != 64 && scale_block != 128)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale_block must be 64 or 128 (got %d)", scale_block);

  zyfa::AttnArgs a{q,   k,        v,       q_scale, k_scale, v_scale, o,           lse,          B, Hq, Hkv,
                   Sq,  Skv,      q_offset, k_begin, k_end,  Dqk,     Dv,          scale_block, softmax_scale};
  hipError_t e = zyfa::launch_attn_fwd_fp8(a, lean, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

static zyfa_status attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int B,
                             int Hq, int Hkv, int Sq, int Skv, int q_offset, int k_begin, int k_end, int Dqk, int Dv,
                             float softmax_scale, void* stream) {
  zyfa_status st = check_attn_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, q_offset, k_begin, k_end, Dqk, Dv,
                                     softmax_scale);
  if (st != ZYFA_OK) return st;
  zyfa::AttnArgs a{q,   k,        v,       nullptr, nullptr, nullptr, o,  lse, B, Hq, Hkv,
                   Sq,  Skv,      q_offset, k_begin, k_end,  Dqk,     Dv, 0,   softmax_scale};
  hipError_t e = zyfa::launch_attn_fwd_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

zyfa_status zyfa_attn_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                              const float* k_scale, const float* v_scale, int scale_block, uint16_t* o, float* lse,
                              int B, int Hq, int Hkv, int S, int Dqk, int Dv, float softmax_scale, void* stream) {
  return attn_fp8(q, k, v, q_scale, k_scale, v_scale, scale_block, o, lse, B, Hq, Hkv, S, S, 0, 0, S, Dqk, Dv,
                  softmax_scale, stream, false);
}

zyfa_status zyfa_attn_fwd_fp8_lean(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                                   const float* k_scale, const float* v_scale, int scale_block, uint16_t* o,
                                   float* lse, int B, int Hq, int Hkv, int S, int Dqk, int Dv, float softmax_scale,
                                   void* stream) {
  return attn_fp8(q, k, v, q_scale, k_scale, v_scale, scale_block, o, lse, B, Hq, Hkv, S, S, 0, 0, S, Dqk, Dv,
                  softmax_scale, stream, true);
}

zyfa_status zyfa_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                               int B, int Hq, int Hkv, int S, int Dqk, int Dv, float softmax_scale, void* stream) {
  return attn_bf16(q, k, v, o, lse, B, Hq, Hkv, S, S, 0, 0, S, Dqk, Dv, softmax_scale, stream);
}

zyfa_status zyfa_attn_fwd_fp8_range(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, int scale_block, uint16_t* o,
                                    float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int q_offset, int k_begin,
                                    int k_end, int Dqk, int Dv, float softmax_scale, int lean, void* stream) {
  if (lean != 0 && lean != 1) return fail(ZYFA_ERR_INVALID_ARGUMENT, "lean must be 0 or 1");
  return attn_fp8(q, k, v, q_scale, k_scale, v_scale, scale_block, o, lse, B, Hq, Hkv, Sq, Skv, q_offset, k_begin,
                  k_end, Dqk, Dv, softmax_scale, stream, lean == 1);
}

zyfa_status zyfa_attn_fwd_bf16_range(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                     float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int q_offset, int k_begin,
                                     int k_end, int Dqk, int Dv, float softmax_scale, void* stream) {
  return attn_bf16(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, q_offset, k_begin, k_end, Dqk, Dv, softmax_scale, stream);
}

static zyfa_status check_varlen(const int* cu_seqlens, int n_seqs, int max_seqlen, int Hq, int T) {
  if (!cu_seqlens) return fail(ZYFA_ERR_INVALID_ARGUMENT, "cu_seqlens must be non-null");
  if (((uintptr_t)cu_seqlens & 3u) != 0) return fail(ZYFA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  if (n_seqs <= 0 || max_seqlen <= 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "n_seqs and max_seqlen must be positive (got %d, %d)", n_seqs, max_seqlen);
  if (max_seqlen > T) return fail(ZYFA_ERR_INVALID_ARGUMENT, "max_seqlen (%d) exceeds T (%d)", max_seqlen, T);
  const long long n_qtiles = (max_seqlen + 127) / 128;
  if (product_exceeds(0x7FFFFFFFLL, {n_qtiles, n_seqs, Hq})) return fail(ZYFA_ERR_UNSUPPORTED, "grid too large");
  return ZYFA_OK;
}

zyfa_status zyfa_attn_fwd_fp8_varlen(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                                     const float* k_scale, const float* v_scale, int scale_block, uint16_t* o,
                                     float* lse, const int* cu_seqlens, int n_seqs, int max_seqlen, int Hq, int Hkv,
                                     int T, int Dqk, int Dv, float softmax_scale, int lean, void* stream) {
  if (lean != 0 && lean != 1) return fail(ZYFA_ERR_INVALID_ARGUMENT, "lean must be 0 or 1");
  zyfa_status st = check_attn_common(q, k, v, o, lse, 1, Hq, Hkv, T, T, 0, 0, T, Dqk, Dv, softmax_scale);
  if (st != ZYFA_OK) return st;
  st = check_varlen(cu_seqlens, n_seqs, max_seqlen, Hq, T);
  if (st != ZYFA_OK) return st;
  if (!q_scale || !k_scale || !v_scale) return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale pointers must be non-null");
  if (!aligned16(q_scale) || !aligned16(k_scale) || !aligned16(v_scale))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (scale_block != 64 && scale_block != 128)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale_block must be 64 or 128 (got %d)", scale_block);
  zyfa::AttnArgs a{q,  k, v,  q_scale, k_scale, v_scale, o,  lse,         n_seqs, Hq, Hkv,
                   T,  T, 0,  0,       T,       Dqk,     Dv, scale_block, softmax_scale};
  a.cu_seqlens = cu_seqlens;
  a.max_seqlen = max_seqlen;
  hipError_t e = zyfa::launch_attn_fwd_fp8(a, lean == 1, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

zyfa_status zyfa_attn_fwd_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                      float* lse, const int* cu_seqlens, int n_seqs, int max_seqlen, int Hq, int Hkv,
                                      int T, int Dqk, int Dv, float softmax_scale, void* stream) {
  zyfa_status st = check_attn_common(q, k, v, o, lse, 1, Hq, Hkv, T, T, 0, 0, T, Dqk, Dv, softmax_scale);
  if (st != ZYFA_OK) return st;
  st = check_varlen(cu_seqlens, n_seqs, max_seqlen, Hq, T);
  if (st != ZYFA_OK) return st;
  zyfa::AttnArgs a{q, k, v, nullptr, nullptr, nullptr, o,  lse, n_seqs, Hq, Hkv,
                   T, T, 0, 0,       T,       Dqk,     Dv, 0,   softmax_scale};
  a.cu_seqlens = cu_seqlens;
  a.max_seqlen = max_seqlen;
  hipError_t e = zyfa::launch_attn_fwd_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

static zyfa_status check_paged(const void* k_cache, const void* v_cache, const int* kv_lens,
                               const int* block_table, int n_seqs, int max_pages, int num_pages, int page_size, int Hkv,
                               int Dqk, int Dv) {
  if (!kv_lens || !block_table) return fail(ZYFA_ERR_INVALID_ARGUMENT, "kv_lens and block_table must be non-null");
  if (((uintptr_t)kv_lens & 3u) != 0 || ((uintptr_t)block_table & 3u) != 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "kv_lens and block_table must be 4-byte aligned");
  if (page_size != 64 && page_size != 128 && page_size != 256)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "page_size must be 64, 128 or 256 (got %d)", page_size);
  if (max_pages <= 0 || num_pages <= 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "max_pages and num_pages must be positive (got %d, %d)", max_pages,
                num_pages);
  if ((long long)max_pages * page_size > kMaxPosition)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "max_pages * page_size must be at most 2^30");
  const long long dmax = Dqk > Dv ? Dqk : Dv;
  if (product_exceeds(kMaxElems, {num_pages, Hkv, page_size, dmax}) ||
      product_exceeds(0x7FFFFFFFLL, {n_seqs, max_pages}))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "tensor too large");
  if (k_cache == v_cache) return fail(ZYFA_ERR_INVALID_ARGUMENT, "k_cache and v_cache must be distinct");
  return ZYFA_OK;
}

zyfa_status zyfa_attn_fwd_fp8_paged(const uint8_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                    const float* q_scale, const float* k_cache_scale, const float* v_cache_scale,
                                    int scale_block, uint16_t* o, float* lse, const int* cu_seqlens,
                                    const int* kv_lens, const int* block_table, int n_seqs, int max_seqlen,
                                    int max_pages, int num_pages, int page_size, int Hq, int Hkv, int T, int Dqk,
                                    int Dv, float softmax_scale, int lean, void* stream) {
  if (lean != 0 && lean != 1) return fail(ZYFA_ERR_INVALID_ARGUMENT, "lean must be 0 or 1");
  zyfa_status st = check_attn_common(q, k_cache, v_cache, o, lse, 1, Hq, Hkv, T, T, 0, 0, T, Dqk, Dv, softmax_scale);
  if (st != ZYFA_OK) return st;
  st = check_varlen(cu_seqlens, n_seqs, max_seqlen, Hq, T);
  if (st != ZYFA_OK) return st;
  st = check_paged(k_cache, v_cache, kv_lens, block_table, n_seqs, max_pages, num_pages, page_size, Hkv, Dqk, Dv);
  if (st != ZYFA_OK) return st;
  if (!q_scale || !k_cache_scale || !v_cache_scale)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale pointers must be non-null");
  if (!aligned16(q_scale) || !aligned16(k_cache_scale) || !aligned16(v_cache_scale))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (scale_block != 64 && scale_block != 128)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale_block must be 64 or 128 (got %d)", scale_block);
  if (page_size % scale_block != 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "page_size (%d) must be a multiple of scale_block (%d)", page_size,
                scale_block);
  zyfa::AttnArgs a{q,  k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, o, lse, n_seqs, Hq, Hkv,
                   T,  T,       0,       0,       T,             Dqk,                       Dv, scale_block, softmax_scale};
  a.cu_seqlens = cu_seqlens;
  a.max_seqlen = max_seqlen;
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.page_size = page_size;
  hipError_t e = zyfa::launch_attn_fwd_fp8(a, lean == 1, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

zyfa_status zyfa_attn_fwd_bf16_paged(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                     uint16_t* o, float* lse, const int* cu_seqlens, const int* kv_lens,
                                     const int* block_table, int n_seqs, int max_seqlen, int max_pages,
                                     int num_pages, int page_size, int Hq, int Hkv, int T, int Dqk, int Dv,
                                     float softmax_scale, void* stream) {
  zyfa_status st = check_attn_common(q, k_cache, v_cache, o, lse, 1, Hq, Hkv, T, T, 0, 0, T, Dqk, Dv, softmax_scale);
  if (st != ZYFA_OK) return st;
  st = check_varlen(cu_seqlens, n_seqs, max_seqlen, Hq, T);
  if (st != ZYFA_OK) return st;
  st = check_paged(k_cache, v_cache, kv_lens, block_table, n_seqs, max_pages, num_pages, page_size, Hkv, Dqk, Dv);
  if (st != ZYFA_OK) return st;
  zyfa::AttnArgs a{q, k_cache, v_cache, nullptr, nullptr, nullptr, o,  lse, n_seqs, Hq, Hkv,
                   T, T,       0,       0,       T,       Dqk,     Dv, 0,   softmax_scale};
  a.cu_seqlens = cu_seqlens;
  a.max_seqlen = max_seqlen;
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.page_size = page_size;
  hipError_t e = zyfa::launch_attn_fwd_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

static long long decode_splits(int max_kv_len, int split_keys) { return (max_kv_len + (long long)split_keys - 1) / split_keys; }

long long zyfa_attn_decode_workspace_bytes(int B, int Hq, int Dv, int max_kv_len, int split_keys) {
  if (B <= 0 || Hq <= 0 || Dv <= 0 || max_kv_len <= 0 || split_keys <= 0) return -1;
  const long long parts = decode_splits(max_kv_len, split_keys);
  if (parts <= 1) return 0;
  const long long rows = (long long)B * Hq;
  // rows * (2 Dv + 4) * parts <= 2^60, compared in division form so that no product
  // can overflow (then none below does either)
  if (rows > ((1LL << 60) / parts) / (2LL * Dv + 4)) return -1;
  const long long o_bytes = (parts * rows * Dv * 2 + 255) / 256 * 256;
  return o_bytes + parts * rows * 4;
}

// Checks and launches shared by the two decode entry points: the attention kernel on
// each key split (partial results in the workspace, or straight into o / lse when there
// is one split), then the merge of the splits.
static zyfa_status decode_paged(const void* q, const void* k_cache, const void* v_cache, const float* q_scale,
                                const float* k_cache_scale, const float* v_cache_scale, int scale_block, uint16_t* o,
                                float* lse, const int* kv_lens, const int* block_table, int B, int max_kv_len,
                                int max_pages, int num_pages, int page_size, int Hq, int Hkv, int Dqk, int Dv,
                                float softmax_scale, int split_keys, void* workspace, long long workspace_bytes,
                                bool fp8, bool lean, void* stream, bool use_scratch = false) {
  zyfa_status st = check_attn_common(q, k_cache, v_cache, o, lse, B, Hq, Hkv, 1, 1, 0, 0, 1, Dqk, Dv, softmax_scale);
  if (st != ZYFA_OK) return st;
  st = check_paged(k_cache, v_cache, kv_lens, block_table, B, max_pages, num_pages, page_size, Hkv, Dqk, Dv);
  if (st != ZYFA_OK) return st;
  const int g = Hq / Hkv;
  if (g > 256) return fail(ZYFA_ERR_UNSUPPORTED, "at most 256 query heads per key/value head (got %d)", g);
  if (max_kv_len <= 0 || (long long)max_kv_len > (long long)max_pages * page_size)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "max_kv_len (%d) must be in 1 .. max_pages * page_size", max_kv_len);
  if (split_keys <= 0 || split_keys % zyfa::kKeyTile != 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "split_keys (%d) must be a positive multiple of %d", split_keys,
                zyfa::kKeyTile);
  const long long parts = decode_splits(max_kv_len, split_keys);
  if (product_exceeds(0x7FFFFFFFLL, {parts, B, Hkv})) return fail(ZYFA_ERR_UNSUPPORTED, "grid too large");
  const long long need = zyfa_attn_decode_workspace_bytes(B, Hq, Dv, max_kv_len, split_keys);
  if (need < 0) return fail(ZYFA_ERR_UNSUPPORTED, "the splits' partial results would exceed 2^60 bytes");
  if (use_scratch) {
    // the allocation-free entry point: the partial results go to the library's per-GPU
    // scratch array (none is needed with one split)
    if (need > (long long)zyfa::kScratchBytes)
      return fail(ZYFA_ERR_UNSUPPORTED,
                  "the splits' partial results need %lld bytes; the allocation-free decode holds %lld (use larger "
                  "split_keys, or zyfa_attn_decode_fp8_paged with a workspace)",
                  need, (long long)zyfa::kScratchBytes);
    workspace = nullptr;  // (looked up once every argument has passed its checks)
  } else if (parts > 1) {
    if (!workspace || ((uintptr_t)workspace & 255u) != 0)
      return fail(ZYFA_ERR_INVALID_ARGUMENT, "workspace must be non-null and 256-byte aligned");
    if (workspace == (const void*)o || workspace == (const void*)lse || workspace == q || workspace == k_cache ||
        workspace == v_cache)
      return fail(ZYFA_ERR_INVALID_ARGUMENT, "workspace must not alias the inputs or outputs");
    if (workspace_bytes < need)
      return fail(ZYFA_ERR_INVALID_ARGUMENT, "workspace holds %lld bytes; %lld needed", workspace_bytes, need);
  }
  if (fp8) {
    if (!q_scale || !k_cache_scale || !v_cache_scale)
      return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale pointers must be non-null");
    if (!aligned16(q_scale) || !aligned16(k_cache_scale) || !aligned16(v_cache_scale))
      return fail(ZYFA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    if (scale_block != 64 && scale_block != 128)
      return fail(ZYFA_ERR_INVALID_ARGUMENT, "scale_block must be 64 or 128 (got %d)", scale_block);
    if (page_size % scale_block != 0)
      return fail(ZYFA_ERR_INVALID_ARGUMENT, "page_size (%d) must be a multiple of scale_block (%d)", page_size,
                  scale_block);
  }
  if (use_scratch && parts > 1) {
    const hipError_t e = zyfa::scratch_of_stream_device((hipStream_t)stream, &workspace);
    if (e != hipSuccess || workspace == nullptr)
      return fail(ZYFA_ERR_LAUNCH, "device scratch lookup failed: %s", hipGetErrorString(e));
  }
  const long long rows = (long long)B * Hq;
  uint16_t* o_parts = parts > 1 ? (uint16_t*)workspace : o;
  float* lse_parts = parts > 1 ? (float*)((char*)workspace + (parts * rows * Dv * 2 + 255) / 256 * 256) : lse;
  // the kernels see each KV group as one "head" whose g rows are its query heads
  zyfa::AttnArgs a{q,        k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, o_parts, lse_parts, B, Hkv,
                   Hkv,      g,       page_size, 0,     0,             1,             Dqk,     Dv,
                   fp8 ? scale_block : 0, softmax_scale};
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.split_keys = split_keys;
  a.n_splits = (int)parts;
  a.part_rows = rows;
  hipError_t e = fp8 ? zyfa::launch_attn_fwd_fp8(a, lean, (hipStream_t)stream)
                     : zyfa::launch_attn_fwd_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  if (parts > 1) {
    zyfa::MergeArgs m{o_parts, lse_parts, (int)parts, o, lse, rows, Dv};
    e = zyfa::launch_attn_merge(m, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

zyfa_status zyfa_attn_decode_fp8_paged(const uint8_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                       const float* q_scale, const float* k_cache_scale, const float* v_cache_scale,
                                       int scale_block, uint16_t* o, float* lse, const int* kv_lens,
                                       const int* block_table, int B, int max_kv_len, int max_pages, int num_pages,
                                       int page_size, int Hq, int Hkv, int Dqk, int Dv, float softmax_scale,
                                       int split_keys, void* workspace, long long workspace_bytes, int lean,
                                       void* stream) {
  if (lean != 0 && lean != 1) return fail(ZYFA_ERR_INVALID_ARGUMENT, "lean must be 0 or 1");
  return decode_paged(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, scale_block, o, lse, kv_lens,
                      block_table, B, max_kv_len, max_pages, num_pages, page_size, Hq, Hkv, Dqk, Dv, softmax_scale,
                      split_keys, workspace, workspace_bytes, true, lean == 1, stream);
}

zyfa_status zyfa_attn_decode_fp8_paged_noalloc(const uint8_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                               const float* q_scale, const float* k_cache_scale,
                                               const float* v_cache_scale, int scale_block, uint16_t* o, float* lse,
                                               const int* kv_lens, const int* block_table, int B, int max_kv_len,
                                               int max_pages, int num_pages, int page_size, int Hq, int Hkv, int Dqk,
                                               int Dv, float softmax_scale, int split_keys, int lean, void* stream) {
  if (lean != 0 && lean != 1) return fail(ZYFA_ERR_INVALID_ARGUMENT, "lean must be 0 or 1");
  return decode_paged(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, scale_block, o, lse, kv_lens,
                      block_table, B, max_kv_len, max_pages, num_pages, page_size, Hq, Hkv, Dqk, Dv, softmax_scale,
                      split_keys, nullptr, 0, true, lean == 1, stream, /*use_scratch=*/true);
}

zyfa_status zyfa_attn_decode_bf16_paged(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                        uint16_t* o, float* lse, const int* kv_lens, const int* block_table, int B,
                                        int max_kv_len, int max_pages, int num_pages, int page_size, int Hq, int Hkv,
                                        int Dqk, int Dv, float softmax_scale, int split_keys, void* workspace,
                                        long long workspace_bytes, void* stream) {
  return decode_paged(q, k_cache, v_cache, nullptr, nullptr, nullptr, 0, o, lse, kv_lens, block_table, B,
                      max_kv_len, max_pages, num_pages, page_size, Hq, Hkv, Dqk, Dv, softmax_scale, split_keys,
                      workspace, workspace_bytes, false, false, stream);
}

zyfa_status zyfa_attn_merge(const uint16_t* o_parts, const float* lse_parts, int n_parts, uint16_t* o, float* lse,
                            long long rows, int Dv, void* stream) {
  if (!o_parts || !lse_parts || !o) return fail(ZYFA_ERR_INVALID_ARGUMENT, "o_parts, lse_parts and o must be non-null");
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (n_parts <= 0 || rows <= 0)
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "n_parts and rows must be positive (got %d, %lld)", n_parts, rows);
  if (Dv != 64 && Dv != 128 && Dv != 256 && Dv != 512)
    return fail(ZYFA_ERR_UNSUPPORTED, "Dv = %d is not supported; use 64, 128, 256 or 512", Dv);
  if (product_exceeds(kMaxElems, {n_parts, rows, Dv})) return fail(ZYFA_ERR_INVALID_ARGUMENT, "tensor too large");
  if ((const void*)o == (const void*)o_parts || (const void*)o == (const void*)lse_parts ||
      (lse && ((const void*)lse == (const void*)o_parts || (const void*)lse == (const void*)lse_parts ||
               (const void*)lse == (const void*)o)))
    return fail(ZYFA_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
  zyfa::MergeArgs a{o_parts, lse_parts, n_parts, o, lse, rows, Dv};
  hipError_t e = zyfa::launch_attn_merge(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ZYFA_ERR_LAUNCH, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
