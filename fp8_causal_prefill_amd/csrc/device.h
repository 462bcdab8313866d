// Device-side types and gfx950 instruction wrappers shared by the kernels.
//
// Operand layouts of the CDNA4 matrix instructions used here (wave of 64 lanes,
// lane l, h = l / 32):
//
//  * v_mfma_*_32x32x64_f8f6f4 (e4m3): each lane holds 32 bytes of A (row l % 32)
//    and 32 bytes of B (column l % 32) along K. An unscaled product only needs
//    A and B to agree on which K position each byte is. With scales, the two
//    32-wide scale blocks of K are {bytes 0-15 of lanes i and i+32} (scale from
//    lane i) and {bytes 16-31 of lanes i and i+32} (scale from lane i+32), for
//    A row / B column i; the scale is an E8M0 exponent in byte 0 of a VGPR.
//  * v_mfma_f32_32x32x16_bf16: 8 bf16 of A (row l % 32) and of B (column l % 32).
//  * 32x32 f32 accumulator: register r of lane l holds row 8(r/4) + 4h + r%4,
//    column l % 32.
//  * ds_read_b64_tr_b8: in each group of 16 lanes, lane 2r+c addresses 8 bytes
//    (half c of row r of an 8-row x 16-byte block); lane i receives byte i of
//    rows 0..7. ds_read_b64_tr_b16: lane 4r+c addresses 4 bf16 (quarter c of row
//    r of a 4-row x 16-element block); lane i receives element i of rows 0..3.
//  * v_permlane32_swap: exchanges a VGPR between lane i and lane i+32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zyfa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) v4bf lds_v4bf;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kE8M0One = 127;  // E8M0 exponent code of 1.0

// D += A * B on e4m3 with per-lane E8M0 scales (see the layout note above).
__device__ __forceinline__ v16f mfma_fp8_scaled(const v8i& a, const v8i& b, const v16f& c, int scale_a,
                                                int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// D += 1 * B per row of A: A is all ones in fp4 (e2m1, format 4 of the instruction's A
// operand: 1.0 is the nibble 0b0010, so every byte is 0x22 and the 64 reduction values of
// a lane take four registers), B e4m3 with E8M0 scale scale_b; scale_a is the E8M0 code
// 127 (1.0), passed in a register. Every output row is the column sums of B times
// 2^(scale_b - 127), exactly (products of 1.0 and e4m3 values).
__device__ __forceinline__ v16f mfma_ones_fp4_by_fp8(const v8i& b, const v16f& c, int scale_a, int scale_b) {
  const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};  // upper half unread
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, b, c, 4, 0, 0, scale_a, 0, scale_b);
}

// D += A * B on e4m3, no scaling.
__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keep a value in a VGPR so the compiler cannot fold it into an instruction constant
// (scale operands of the scaled MFMA must come from registers).
__device__ __forceinline__ int opaque(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
  return x;
}

// The same for a float: the value is only available from this point of the program on,
// so work depending on it cannot be hoisted above (e.g. out of a pipeline slot).
__device__ __forceinline__ float opaque_f(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
  return x;
}

// Materialise a matrix accumulator here, in the current (uniform) control flow. A
// matrix instruction reads its operands from all 64 lanes whatever EXEC holds, so it
// must not be moved into a lane-divergent region (such as a guarded output store),
// where operands built inside that region exist only in the active lanes.
//
// The asm helpers below are compiled in the device pass only: the host pass does not
// know VGPR constraints and would reject the kernels that use them.
__device__ __forceinline__ void pin_acc(v16f& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
}

// An empty use of x at this point of the program. The instruction producing x can
// then not be sunk below it (e.g. out of a software-pipeline slot into a later basic
// block where x is consumed), which the compiler otherwise does to shorten live ranges.
template <class T>
__device__ __forceinline__ void keep_here(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

// A side effect that stops the compiler from if-converting the rare branch it sits in
// (speculating its body into unconditional vector work).
__device__ __forceinline__ void rare_branch() { asm volatile(""); }

// ---- direct global -> LDS copies (16 bytes per lane) ----
// Lane l's 16 bytes land at LDS byte address lds + 16 l (lds is wave-uniform; the
// instruction takes it from M0). The copies are issued as inline assembly on purpose:
// the compiler then does not track them, and in particular does not make every later
// LDS read wait for all copies in flight (it cannot tell which buffer a copy writes).
// Completion is the caller's job: s_waitcnt vmcnt(0) in each wave, then a workgroup
// barrier, before any wave reads the buffer; and no copy may target a buffer that a wave
// can still be reading. M0 is written here; the compiler sets M0 right before each of
// its own uses, and this code has no other M0 user.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// source = base (wave-uniform) + off (per lane, bytes)
template <bool NT = false>  // NT: the nontemporal hint, for data read once (decode's cache)
__device__ __forceinline__ void lds_copy16(const void* base, uint32_t off, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(bu),
                 "s"(__builtin_amdgcn_readfirstlane((int)lds))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(bu),
                 "s"(__builtin_amdgcn_readfirstlane((int)lds))
                 : "memory", "m0");
#endif
}
// source = src (per lane)
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane((int)lds))
               : "memory", "m0");
#endif
}
#pragma clang diagnostic pop
// Wait for this wave's outstanding vector memory operations (the copies above included).
// The wait goes through the builtin, not inline assembly, so that the compiler's own
// counter tracking knows that every earlier load has completed and does not wait again
// for them later (such a wait, counted without the copies, would also hold the wave for
// loads issued after this point). Encoding: vmcnt 0, expcnt and lgkmcnt at their maxima.
__device__ __forceinline__ void wait_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
#endif
}

// The value of lane l ^ M, for M in {1, 2, 4, 8, 16}, without a trip through the LDS
// crossbar (which __shfl_xor takes): M = 1, 2 are DPP quad permutations; M = 8 is a DPP
// rotation of each 16-lane row by 8 lanes (which is l ^ 8 within the row); M = 4 picks a
// DPP row shift down or up by 4 by the lane's bit 2 (two moves and a select); M = 16 swaps
// the odd 16-lane rows of one copy with the even rows of another (v_permlane16_swap) and
// takes, per row, the copy that holds the partner row.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __builtin_bit_cast(int, v);
  // (every lane's source lane exists for these patterns, so the bound-control form, which
  // needs no copy of the old value in the destination, gives the same result)
  if constexpr (M == 1) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  } else if constexpr (M == 8) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));  // row_ror:8
  } else if constexpr (M == 4) {
    const int up = __builtin_amdgcn_update_dpp(x, x, 0x100 + M, 0xF, 0xF, false);    // row_shl: lane l + M
    const int down = __builtin_amdgcn_update_dpp(x, x, 0x110 + M, 0xF, 0xF, false);  // row_shr: lane l - M
    return __builtin_bit_cast(float, (__lane_id() & M) ? down : up);
  } else {
    static_assert(M == 16, "lane_xor: M must be 1, 2, 4, 8 or 16");
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    // r[0]: rows (0, 0, 2, 2) of x; r[1]: rows (1, 1, 3, 3)
    return __builtin_bit_cast(float, (__lane_id() & 16) ? r[0] : r[1]);
  }
}

// The value of lane l ^ M for M < 32 through ds_swizzle_b32 (bit mode: and-mask 31, xor-mask
// M, within each group of 32 lanes): the LDS crossbar moves it, no vector ALU instruction
// and no LDS memory access; the result comes back through the LDS queue (lgkmcnt).
template <int M>
__device__ __forceinline__ float lane_xor_swizzle(float v) {
  static_assert(M > 0 && M < 32, "swizzle xor stays within 32 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (M << 10)));
}

// max of a value across lanes i and i+32.
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// sum of a value across lanes i and i+32.
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Two floats -> two e4m3 codes (round-to-nearest-even; values must lie within +-448:
// the hardware conversion does not saturate), written to the low (HIGH = false) or
// high (HIGH = true) 16 bits of `old`.
template <bool HIGH>
__device__ __forceinline__ int cvt_pk_fp8(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HIGH);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  // one v_cvt_pk_bf16_f32 (round-to-nearest-even): a in the low half, b in the high half
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t){a, b}, v2bf_t));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace zyfa
