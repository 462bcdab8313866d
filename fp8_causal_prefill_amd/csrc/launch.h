// Host-side launchers of the device kernels, called by the C ABI after it has
// validated every argument. Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zyfa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;  // FP8 only
  const float* k_scale;
  const float* v_scale;
  uint16_t* o;
  float* lse;            // may be null
  int B, Hq, Hkv;
  int Sq, Skv;           // rows per head of Q / O / LSE, and of K / V
  int q_offset;          // sequence position of query row 0
  int k_begin, k_end;    // key window [k_begin, k_end); k_begin a multiple of kKeyTile
  int Dqk, Dv;
  int scale_block;       // FP8 only
  float softmax_scale;
  // packed batch (null otherwise): B sequences in [H, Sq = Skv, D] tensors, sequence b
  // being tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1 (device array of B + 1 ints)
  const int* cu_seqlens = nullptr;
  int max_seqlen = 0;
  // paged key/value cache (non-null block_table): K, V [num_pages, Hkv, page_size, D];
  // sequence b's pages block_table[b * max_pages ...], its token count kv_lens[b]
  const int* block_table = nullptr;
  const int* kv_lens = nullptr;
  int max_pages = 0, num_pages = 0, page_size = 0;
  // decode over a paged cache (split_keys > 0, with block_table): Sq query heads per KV
  // head in each row group of Q; n_splits key splits of split_keys keys, partial results in
  // o / lse at rows split * part_rows + row
  int split_keys = 0, n_splits = 0;
  long long part_rows = 0;
};

// keys per tile of the attention kernels: a key window must start on a tile boundary
constexpr int kKeyTile = 64;

// Debug switch, read at every launch: a nonempty ZYFA_LDS_POISON other than "0" fills the
// attention kernels' LDS with NaN bytes before their first tile copy.
bool lds_poison_requested();

// lean: probabilities as linear e4m3 codes instead of rounded exponentials
hipError_t launch_attn_fwd_fp8(const AttnArgs& a, bool lean, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream);

struct QuantArgs {
  const void* x;
  int x_is_bf16;
  uint8_t* codes;
  float* scales;
  int B, H, S, D, scale_block, hadamard;
};

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream);

// Bytes of the file-scope device scratch array of scratch.hip (per GPU), and its device
// address on the device that `stream` belongs to (the current device for the null stream;
// looked up once per device; the error of that lookup).
constexpr size_t kScratchBytes = size_t(8) << 20;
hipError_t scratch_of_stream_device(hipStream_t stream, void** ptr);

struct MergeArgs {
  const uint16_t* o_parts;  // [n_parts, rows, Dv] bf16
  const float* lse_parts;   // [n_parts, rows]
  int n_parts;
  uint16_t* o;              // [rows, Dv] bf16
  float* lse;               // [rows], may be null
  long long rows;
  int Dv;                   // 64, 128, 256 or 512
};

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace zyfa
