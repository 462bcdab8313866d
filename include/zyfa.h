/*
 * zyfa.h - C ABI of the MI355X (gfx950) causal prefill attention library.
 *
 * The library computes causal forward ("prefill") attention
 *
 *     O = softmax(Q K^T * softmax_scale + causal mask) V
 *
 * for equal query and key lengths (and, through the entry points further down, for a
 * chunk of query rows against a key window, packed batches of sequences, chunks and
 * single decode tokens against a paged key/value cache, and the merge of partial
 * results), in two precisions:
 *
 *   - FP8: Q, K, V as OCP e4m3 (E4M3FN) codes with one float32 scale per
 *     (batch, head, block of scale_block tokens);
 *   - BF16: Q, K, V as bfloat16.
 *
 * Head shapes: Dqk = Dv = 128 (query heads may share key/value heads: GQA), and
 * the MLA shape Dqk = 192, Dv = 128.
 *
 * Source: "ZYFA: Fast and Accurate FP8 Attention on AMD MI355X" -- Introduction
 * (the operation and the two head shapes, footnote 4 for MLA), "Methodology and
 * Limitations" (causal, equal query and key lengths, no decode / paged KV /
 * variable-length batches), "Per-Block Scaling and Normalization by the Rounded
 * Row Sum" (the FP8 probability scaling and normalisation), footnote 2 (inputs
 * are quantized in separate passes, with an optional Hadamard rotation of Q
 * and K fused into the quantization).
 *
 * Conventions shared by every entry point:
 *
 *   Layout     Every tensor is dense row-major [B, H, S, D] (D fastest), the
 *              order of PyTorch's scaled_dot_product_attention, unless an entry
 *              point states otherwise (packed batches, paged caches, decode).
 *              Scales are dense [B, H, nb] with nb = ceil(S / scale_block). Query
 *              head h reads key/value head h / (Hq / Hkv).
 *   Memory     All pointers are device pointers owned by the caller and must be
 *              16-byte aligned. Outputs must not alias inputs. The library never
 *              allocates, frees or synchronises (decode takes its scratch space
 *              from a caller's workspace).
 *   Streams    `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *              all work is enqueued on it and the call returns without waiting.
 *              Every pointer must be memory of the stream's device (for the null
 *              stream, the current device).
 *   Errors     Argument checks happen on the host before any device work; a
 *              failing call enqueues nothing. ZYFA_ERR_LAUNCH reports a failed
 *              kernel launch. Faults inside a kernel surface at the caller's next
 *              synchronisation. Inputs are not scanned for NaN / Inf; e4m3 NaN
 *              codes (0x7F, 0xFF) give undefined output.
 *   Threads    The library keeps no state between calls; calls are thread-safe.
 *              zyfa_last_error() reads a thread-local message.
 *   Debugging  Two environment variables, read at every call: ZYFA_DEBUG (any value
 *              but "" and "0") also prints each failed call's status and message on
 *              stderr; ZYFA_LDS_POISON fills the attention kernels' LDS with all-ones
 *              bytes (NaN in e4m3 and bfloat16) before their first tile copy, so that a
 *              read of a byte no copy wrote would show in the output (results are
 *              otherwise unchanged; the fill costs a few microseconds per launch).
 */
#ifndef ZYFA_H
#define ZYFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZYFA_ABI_VERSION 6

typedef enum zyfa_status {
  ZYFA_OK = 0,
  ZYFA_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad size, bad scale */
  ZYFA_ERR_UNSUPPORTED = 2,      /* a valid request the library has no kernel for */
  ZYFA_ERR_LAUNCH = 3            /* the HIP runtime rejected the kernel launch */
} zyfa_status;

/* ABI version of the loaded library (ZYFA_ABI_VERSION of its build). */
int zyfa_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* zyfa_status_string(int status);

/* Message describing why the calling thread's most recent failing call failed
 * (empty string if none). Valid until the thread's next library call. */
const char* zyfa_last_error(void);

/*
 * zyfa_quantize_fp8 -- quantize a tensor to e4m3 codes with per-block scales.
 *
 * Source: footnote 2 and section "FP8 Error in Full-Model Inference" of the ZYFA
 * page (a separate quantization pass; an optional Hadamard rotation of Q and K
 * over the head dimension, fused into that pass); FP8 GEMM on CDNA4 blog,
 * sections 2.2-2.3 (absmax scaling with a zero guard, round-to-nearest-even).
 *
 *   x            [B, H, S, D] float32 (x_is_bf16 = 0) or bfloat16 (x_is_bf16 = 1).
 *   codes        out: [B, H, S, D] e4m3 codes.
 *   scales       out: [B, H, nb] float32, nb = ceil(S / scale_block).
 *   scale_block  tokens per scale: 64 or 128.
 *   hadamard     0: none. 1: first rotate every row of D values by the orthonormal
 *                Hadamard matrix H_D / sqrt(D), as the row vector times the matrix:
 *                Sylvester's matrix for D = 128; for D = 192 (the MLA shape) the
 *                Kronecker product of Paley's order-12 matrix (first construction over
 *                GF(11)) and Sylvester's of order 16.
 *
 * For each (b, h, token block): amax = max |y| over the block's tokens and all D
 * channels (y = x, or the rotated row); s = the least power of two with
 * amax / s <= 448 (s >= 2^-126; s = 1 if amax == 0), the E8M0 form that the
 * scaled FP8 matrix instruction applies exactly; code = round-to-nearest-even
 * e4m3 of the exact quotient y / s, saturated to +-448. Without rotation the
 * result is bit-exact to that definition; with rotation y is computed in float32
 * (a fast Walsh-Hadamard transform; for D = 192 also the order-12 factor as sums).
 * The dequantized value of an element is decode(code) * s.
 */
zyfa_status zyfa_quantize_fp8(const void* x, int x_is_bf16, uint8_t* codes, float* scales, int B, int H,
                              int S, int D, int scale_block, int hadamard, void* stream);

/*
 * zyfa_attn_fwd_fp8 -- causal attention on e4m3 inputs.
 *
 * Source: ZYFA page, sections "Precision and Underflow of FP8 Probabilities" and
 * "Per-Block Scaling and Normalization by the Rounded Row Sum".
 *
 *   q, k, v      e4m3 codes: q [B, Hq, S, Dqk], k [B, Hkv, S, Dqk], v [B, Hkv, S, Dv].
 *   q_scale      [B, Hq, nb] float32; k_scale, v_scale [B, Hkv, nb] float32; each
 *                finite and > 0 (subnormal floats included). Dequantized input =
 *                decode(code) * scale. A V scale is split into a power of two, which
 *                the matrix instruction applies exactly as the V operand's E8M0 scale
 *                (2^-127 for a subnormal scale), and a factor rv in (0, 2) (1 for the
 *                power-of-two scales zyfa_quantize_fp8 writes): O is accumulated in
 *                units of 1 / rv of the latest key tile and multiplied by the ratio
 *                when rv changes, so the probabilities and their rounding do not
 *                depend on V. A zero, negative or non-finite scale gives undefined
 *                output, and so do dequantized V values of magnitude 2^73 or more (the
 *                unnormalised output, accumulated in float32, could overflow).
 *   scale_block  tokens per scale: 64 or 128.
 *   o            out: [B, Hq, S, Dv] bfloat16 (round-to-nearest-even).
 *   lse          out, may be NULL: [B, Hq, S] float32, natural-log log-sum-exp of
 *                the scaled scores of each query row.
 *   softmax_scale  multiplies Q K^T; finite and > 0 (usually 1/sqrt(Dqk)).
 *
 * Supported: (Dqk, Dv) in {(128, 128), (192, 128)}, Hq % Hkv == 0, any S >= 1.
 * Method: scores on the FP8 matrix cores; probabilities are formed with a
 * base-2 exponential, and every (query row, 64-key block) of probabilities is
 * multiplied by a power of two that puts its largest value in [128, 256) (the block
 * maximum "close to 1" of the source, moved 7 binades up so that weights down to 2^-13
 * of it stay out of e4m3's subnormal range) before the
 * round-to-nearest-even conversion to e4m3; the power of two is divided back out
 * by the scaled FP8 matrix instruction. Each row is normalised by the sum of the
 * rounded probabilities that multiply V, so the output is a weighted average
 * whose weights sum to one.
 */
zyfa_status zyfa_attn_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                              const float* k_scale, const float* v_scale, int scale_block, uint16_t* o,
                              float* lse, int B, int Hq, int Hkv, int S, int Dqk, int Dv, float softmax_scale,
                              void* stream);

/*
 * zyfa_attn_fwd_fp8_lean -- zyfa_attn_fwd_fp8 with linear probability codes.
 *
 * Source: ZYFA page, section "Lean P: Linear Approximation of the FP8 Code" (the
 * e4m3 code of 2^y is nearly linear in y, about 8 y plus a constant), and "Numerical
 * Accuracy" (its error is 1.22-1.36 times that of exactly rounded probabilities).
 *
 * Same arguments, layouts, scales, errors and output as zyfa_attn_fwd_fp8. Only the
 * probabilities differ: with y = s*c - bias the base-2 exponent of a probability after
 * its block scaling (y < 8), its code is taken from a straight line on a grid of sixteen
 * steps per binade, c16 = round-half-even(16 y + 110.25) clamped to [0, 255], then halved
 * to e4m3's eight steps per binade: (c16 + u) >> 1, where u = 1 if the halved code's three
 * mantissa bits are 0, 6 or 7 and u = 0 otherwise. The rounding up near the binade edges
 * follows the curvature of 2^y that a straight line of eight steps misses. One fused
 * multiply-add and one conversion per score plus six integer operations per four scores,
 * no exponential. The normalisation still uses the sum of exactly these codes' values, so
 * outputs remain weighted averages and their error is within a few percent of
 * zyfa_attn_fwd_fp8's (host emulation at 32K Gaussian tokens, late rows: 2.74e-2 against
 * 2.66e-2; a straight line of eight steps gives 3.08e-2). The codes' values average 0.959
 * of the probabilities; the log-sum-exp divides that factor out of the row sum.
 */
zyfa_status zyfa_attn_fwd_fp8_lean(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                                   const float* k_scale, const float* v_scale, int scale_block, uint16_t* o,
                                   float* lse, int B, int Hq, int Hkv, int S, int Dqk, int Dv, float softmax_scale,
                                   void* stream);

/*
 * zyfa_attn_fwd_bf16 -- causal attention on bfloat16 inputs.
 *
 * Source: ZYFA page, Introduction and section "Throughput on Gaussian Inputs"
 * (the BF16 kernels next to the FP8 ones).
 *
 *   q [B, Hq, S, Dqk], k [B, Hkv, S, Dqk], v [B, Hkv, S, Dv]: bfloat16 bit patterns.
 *   o out [B, Hq, S, Dv] bfloat16; lse out (may be NULL) [B, Hq, S] float32.
 *
 * Same shapes, scale and error rules as zyfa_attn_fwd_fp8. Probabilities are
 * rounded to bfloat16 for the P V product; the row sum is accumulated in float32.
 */
zyfa_status zyfa_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                               int B, int Hq, int Hkv, int S, int Dqk, int Dv, float softmax_scale, void* stream);

/*
 * zyfa_attn_fwd_fp8_range / zyfa_attn_fwd_bf16_range -- causal attention of a chunk of
 * query rows against a window of keys.
 *
 * Source: ZYFA page, Introduction and "Methodology and Limitations" (the causal forward
 * pass: a query attends to keys at positions up to its own); Zyphra "Inference Wave 2",
 * section on CSA dual-scope decode (keys split into shards, each returning a partial
 * output and its log-sum-exp, merged by zyfa_attn_merge). The same kernels as
 * zyfa_attn_fwd_fp8 / _bf16, which are the case Sq = Skv = S, q_offset = 0,
 * [k_begin, k_end) = [0, S).
 *
 *   q            [B, Hq, Sq, Dqk]: query row i is the token at sequence position
 *                q_offset + i.
 *   k, v         [B, Hkv, Skv, Dqk] and [B, Hkv, Skv, Dv]: key j is the token at
 *                position j.
 *   q_scale      FP8: [B, Hq, ceil(Sq / scale_block)], blocks of the rows of q;
 *   k_scale, v_scale  FP8: [B, Hkv, ceil(Skv / scale_block)], blocks of positions.
 *   o, lse       out: [B, Hq, Sq, Dv] bfloat16 and (may be NULL) [B, Hq, Sq] float32.
 *   k_begin, k_end  the key window: key j is visible to query row i iff
 *                k_begin <= j < k_end and j <= q_offset + i. 0 <= k_begin < k_end <= Skv
 *                and k_begin is a multiple of 64.
 *   q_offset     >= 0, with q_offset + Sq <= 2^30.
 *   lean         FP8 only: 0 = probabilities as in zyfa_attn_fwd_fp8, 1 = as in
 *                zyfa_attn_fwd_fp8_lean.
 *
 * A row that sees no key of the window (q_offset + i < k_begin) gets O = 0 and
 * LSE = -inf, the form zyfa_attn_merge expects of a part that holds none of the row's
 * keys. Chunked prefill over a cached prefix is q_offset = prefix length with the window
 * [0, q_offset + Sq); a split of the keys into windows gives parts that zyfa_attn_merge
 * combines. Other rules (pointers, alignment, streams, errors) as zyfa_attn_fwd_fp8;
 * invalid windows or offsets are ZYFA_ERR_INVALID_ARGUMENT.
 */
zyfa_status zyfa_attn_fwd_fp8_range(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, int scale_block, uint16_t* o,
                                    float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int q_offset, int k_begin,
                                    int k_end, int Dqk, int Dv, float softmax_scale, int lean, void* stream);

zyfa_status zyfa_attn_fwd_bf16_range(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                     float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int q_offset, int k_begin,
                                     int k_end, int Dqk, int Dv, float softmax_scale, void* stream);

/*
 * zyfa_attn_fwd_fp8_varlen / zyfa_attn_fwd_bf16_varlen -- causal attention over a batch
 * of sequences of different lengths, packed along the token axis.
 *
 * Source: ZYFA page, "Future Work" (batches of variable length) and Introduction (each
 * sequence is a causal prefill of its own). The same kernels as zyfa_attn_fwd_fp8 /
 * _bf16, with the batch index picking a sequence.
 *
 *   q            [Hq, T, Dqk]; k [Hkv, T, Dqk]; v [Hkv, T, Dv]: sequence i is tokens
 *                cu_seqlens[i] .. cu_seqlens[i+1] - 1 of every head.
 *   q_scale, k_scale, v_scale  FP8: [Hq, ceil(T / scale_block)] and
 *                [Hkv, ceil(T / scale_block)], blocks of the packed token axis (the
 *                layout zyfa_quantize_fp8 writes for a [1, H, T, D] tensor).
 *   o, lse       out: [Hq, T, Dv] bfloat16 and (may be NULL) [Hq, T] float32. Tokens
 *                after the last sequence (cu_seqlens[n_seqs] .. T - 1) are not written.
 *   cu_seqlens   device array of n_seqs + 1 ints, non-decreasing, every entry but the
 *                last a multiple of 64 (sequences start on a key tile), the last at most
 *                T; no sequence longer than max_seqlen. To pack sequences of any length,
 *                pad each but the last at its end to a multiple of 64 tokens (zeros keep
 *                the FP8 block scales unaffected): under the causal rule a sequence's
 *                real tokens never see the padding after them, so their outputs are
 *                those of the unpadded sequence; the padding rows' outputs are computed
 *                and meaningless. The array is read on the device: a sequence whose
 *                entries break these rules is left unwritten (no error is reported).
 *   max_seqlen   1 .. T; sizes the grid.
 *   lean         FP8 only: 0 or 1, as in zyfa_attn_fwd_fp8_range.
 *
 * Other rules (pointers, alignment, streams, errors, supported head shapes) as
 * zyfa_attn_fwd_fp8.
 */
zyfa_status zyfa_attn_fwd_fp8_varlen(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_scale,
                                     const float* k_scale, const float* v_scale, int scale_block, uint16_t* o,
                                     float* lse, const int* cu_seqlens, int n_seqs, int max_seqlen, int Hq, int Hkv,
                                     int T, int Dqk, int Dv, float softmax_scale, int lean, void* stream);

zyfa_status zyfa_attn_fwd_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                      float* lse, const int* cu_seqlens, int n_seqs, int max_seqlen, int Hq, int Hkv,
                                      int T, int Dqk, int Dv, float softmax_scale, void* stream);

/*
 * zyfa_attn_fwd_fp8_paged / zyfa_attn_fwd_bf16_paged -- prefill of chunks of new tokens
 * against a paged key/value cache.
 *
 * Source: ZYFA page, "Future Work" (paged KV caches, variable-length batches). Sequence i
 * holds kv_lens[i] tokens whose keys and values sit in pages of a shared cache; its
 * chunk of L_i = cu_seqlens[i+1] - cu_seqlens[i] new tokens is the last L_i of them (their
 * keys and values already written into the cache). Row r of the chunk is the token at
 * position kv_lens[i] - L_i + r and sees the sequence's keys 0 .. kv_lens[i] - L_i + r:
 * zyfa_attn_fwd_fp8_range on the gathered keys with q_offset = kv_lens[i] - L_i.
 *
 *   q            [Hq, T, Dqk]: the chunks packed along the token axis as in
 *                zyfa_attn_fwd_fp8_varlen (cu_seqlens: starts on multiples of 64;
 *                max_seqlen). A chunk padded at its end to a multiple of 64 rows counts
 *                its padding as the sequence's last tokens (in kv_lens[i], with keys and
 *                values in the cache after the sequence's own): the causal rule keeps them
 *                out of the real rows' results.
 *   k_cache      [num_pages, Hkv, page_size, Dqk]; v_cache [num_pages, Hkv, page_size, Dv]:
 *                page p holds page_size consecutive tokens of every key/value head.
 *   k_cache_scale, v_cache_scale  FP8: [num_pages, Hkv, page_size / scale_block], the
 *                layout zyfa_quantize_fp8 writes for the cache viewed as
 *                B = num_pages, H = Hkv, S = page_size. page_size must be a multiple of
 *                scale_block.
 *   q_scale      FP8: [Hq, ceil(T / scale_block)], as in zyfa_attn_fwd_fp8_varlen.
 *   block_table  device int32 [n_seqs, max_pages]: logical page j of sequence i (its tokens
 *                j * page_size ..) is cache page block_table[i * max_pages + j]. Pages may
 *                be shared between sequences and appear in any order.
 *   kv_lens      device int32 [n_seqs]: L_i <= kv_lens[i] <= max_pages * page_size.
 *   page_size    64, 128 or 256.
 *   o, lse       out: [Hq, T, Dv] bfloat16 and (may be NULL) [Hq, T] float32; rows outside
 *                every chunk are not written.
 *
 * The device arrays are read on the device: a sequence whose cu_seqlens or kv_lens entries
 * break the rules is left unwritten (no error is reported); a block_table entry outside
 * [0, num_pages) is clamped into it (the sequence's result is then meaningless, but no
 * read leaves the cache). Other rules (pointers, alignment, streams, errors, head shapes,
 * lean) as zyfa_attn_fwd_fp8_varlen.
 */
zyfa_status zyfa_attn_fwd_fp8_paged(const uint8_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                    const float* q_scale, const float* k_cache_scale, const float* v_cache_scale,
                                    int scale_block, uint16_t* o, float* lse, const int* cu_seqlens,
                                    const int* kv_lens, const int* block_table, int n_seqs, int max_seqlen,
                                    int max_pages, int num_pages, int page_size, int Hq, int Hkv, int T, int Dqk,
                                    int Dv, float softmax_scale, int lean, void* stream);

zyfa_status zyfa_attn_fwd_bf16_paged(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                     uint16_t* o, float* lse, const int* cu_seqlens, const int* kv_lens,
                                     const int* block_table, int n_seqs, int max_seqlen, int max_pages,
                                     int num_pages, int page_size, int Hq, int Hkv, int T, int Dqk, int Dv,
                                     float softmax_scale, void* stream);

/*
 * zyfa_attn_decode_fp8_paged / zyfa_attn_decode_bf16_paged -- one new token per sequence
 * against its paged key/value cache (decode).
 *
 * Source: ZYFA page, "Future Work" (decode support, paged KV caches); the split of the
 * keys and the log-sum-exp merge follow Zyphra "Inference Wave 2", section on CSA
 * dual-scope decode. Sequence b's new token is its last, at position kv_lens[b] - 1, and
 * sees all kv_lens[b] keys (its own key and value already in the cache). The keys are
 * cut into splits of split_keys keys; the attention kernel runs once per (sequence, KV
 * head, split) with the KV group's Hq / Hkv query heads as its rows, writes each split's
 * partial result to the workspace, and zyfa_attn_merge's kernel combines the splits.
 *
 *   q            [B, Hq, Dqk]: the new tokens' queries (FP8: e4m3 codes).
 *   q_scale      FP8: [B, Hkv, ceil((Hq / Hkv) / scale_block)]: one scale per block of
 *                the query heads of a KV group, the layout zyfa_quantize_fp8 writes for q
 *                viewed as [B, Hkv, Hq / Hkv, Dqk].
 *   k_cache, v_cache, k_cache_scale, v_cache_scale, block_table, page_size, num_pages,
 *                max_pages  as in zyfa_attn_fwd_fp8_paged (block_table [B, max_pages]).
 *   kv_lens      device int32 [B]: 1 <= kv_lens[b] <= max_kv_len.
 *   max_kv_len   host bound on kv_lens, 1 .. max_pages * page_size; sizes the grid.
 *   split_keys   keys per split: a positive multiple of 64. There are
 *                ceil(max_kv_len / split_keys) splits.
 *   workspace    device memory of zyfa_attn_decode_workspace_bytes(B, Hq, Dv, max_kv_len,
 *                split_keys) bytes, 256-byte aligned (none is needed, and NULL is
 *                accepted, with one split); its contents on entry do not matter.
 *   o, lse       out: [B, Hq, Dv] bfloat16 and (may be NULL) [B, Hq] float32.
 *   Hq / Hkv     at most 256.
 *
 * The splits' partial outputs are rounded to bfloat16 before the merge. A sequence whose
 * kv_lens entry breaks the rules gets O = 0 and LSE = -inf (no error is reported).
 * Other rules (pointers, alignment, streams, errors, head shapes, lean, block_table
 * clamping) as zyfa_attn_fwd_fp8_paged. Two kernels are enqueued on the stream.
 */
/* Workspace bytes a decode call with these sizes needs (0 with one split), or -1 for
 * non-positive sizes or a workspace beyond 2^60 bytes. */
long long zyfa_attn_decode_workspace_bytes(int B, int Hq, int Dv, int max_kv_len, int split_keys);

zyfa_status zyfa_attn_decode_fp8_paged(const uint8_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                       const float* q_scale, const float* k_cache_scale, const float* v_cache_scale,
                                       int scale_block, uint16_t* o, float* lse, const int* kv_lens,
                                       const int* block_table, int B, int max_kv_len, int max_pages, int num_pages,
                                       int page_size, int Hq, int Hkv, int Dqk, int Dv, float softmax_scale,
                                       int split_keys, void* workspace, long long workspace_bytes, int lean,
                                       void* stream);

/*
 * zyfa_attn_decode_fp8_paged_noalloc -- zyfa_attn_decode_fp8_paged for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, and harnesses that forbid
 * device allocations. It takes no workspace: the splits' partial results go to a device
 * array of 8 MiB (ZYFA_NOALLOC_SCRATCH_BYTES) that the library holds on every GPU it runs
 * on, from the first such call on that GPU until the process ends; a call uses the array
 * of its stream's device. The call allocates and
 * frees nothing (no hipMalloc, hipFree or allocating library routine); the caller still
 * passes the inputs and outputs.
 *
 * Arguments, layouts, results and errors as zyfa_attn_decode_fp8_paged without workspace
 * and workspace_bytes. A call whose partial results would need more than
 * ZYFA_NOALLOC_SCRATCH_BYTES (zyfa_attn_decode_workspace_bytes) fails with
 * ZYFA_ERR_UNSUPPORTED before any device work; larger split_keys need less. Every call on
 * one GPU shares that GPU's array, and nothing in it needs to start at zero (each split
 * writes all of its partial results before the merge reads them): calls that overlap on
 * one GPU (on different streams, or from different threads without ordering) race and give
 * undefined output; calls ordered on one stream are safe.
 */
#define ZYFA_NOALLOC_SCRATCH_BYTES (8LL << 20)

zyfa_status zyfa_attn_decode_fp8_paged_noalloc(const uint8_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                               const float* q_scale, const float* k_cache_scale,
                                               const float* v_cache_scale, int scale_block, uint16_t* o, float* lse,
                                               const int* kv_lens, const int* block_table, int B, int max_kv_len,
                                               int max_pages, int num_pages, int page_size, int Hq, int Hkv, int Dqk,
                                               int Dv, float softmax_scale, int split_keys, int lean, void* stream);

zyfa_status zyfa_attn_decode_bf16_paged(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                        uint16_t* o, float* lse, const int* kv_lens, const int* block_table, int B,
                                        int max_kv_len, int max_pages, int num_pages, int page_size, int Hq, int Hkv,
                                        int Dqk, int Dv, float softmax_scale, int split_keys, void* workspace,
                                        long long workspace_bytes, void* stream);

/*
 * zyfa_attn_merge -- combine partial attention results over disjoint key sets.
 *
 * Source: Zyphra "Inference Wave 2", section on CSA dual-scope decode: each key shard
 * produces a partial output and a log-sum-exp statistic, and a merge step combines them
 * into the answer of one pass over all keys.
 *
 *   o_parts      [n_parts, rows, Dv] bfloat16: the parts' outputs (e.g. n_parts stacked
 *                [B, H, S, Dv] tensors, rows = B * H * S).
 *   lse_parts    [n_parts, rows] float32, natural log; -inf marks a row for which the
 *                part saw no key (its output is then ignored).
 *   o            out: [rows, Dv] bfloat16 (round-to-nearest-even).
 *   lse          out, may be NULL: [rows] float32.
 *   Dv           64, 128, 256 or 512; n_parts >= 1; rows >= 1.
 *
 * Per row: M = max_p LSE_p, w_p = exp(LSE_p - M), O = sum_p w_p O_p / sum_p w_p,
 * LSE = M + ln sum_p w_p, in float32; a row no part saw gets O = 0, LSE = -inf.
 * Pointers: device, 16-byte aligned, outputs not aliasing inputs. Errors as above.
 */
zyfa_status zyfa_attn_merge(const uint16_t* o_parts, const float* lse_parts, int n_parts, uint16_t* o, float* lse,
                            long long rows, int Dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZYFA_H */
