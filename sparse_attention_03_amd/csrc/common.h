// Shared device helpers for the gfx950 DSA kernels: MFMA wrappers, in-register
// dequantisation of the cache formats, and paged-cache addressing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

constexpr int kWave = 64;
constexpr int kIdxHeads = DSA_INDEX_HEADS;  // 32
constexpr int kIdxDim = DSA_INDEX_DIM;      // 128
constexpr int kLatDim = DSA_LATENT_DIM;     // 576
constexpr int kValDim = DSA_VALUE_DIM;      // 512

// ---------------------------------------------------------------- MFMA
// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.  Lane l
// supplies A[l%16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l%16]; it receives
// D[4*(l/16) + i][l%16], i < 4.  The order in which the 32 k-values are
// assigned to (lane group, slot) is free as long as A and B agree.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x16) * B(16x16), bf16: lane l supplies A[l%16][4*(l/16) ..
// +4) and B[4*(l/16) .. +4)[l%16]; D layout as above.
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x128) * B(128x16) with FP8 E4M3 inputs (unit block scales).
// Lane l supplies 32 k-values of row l%16 of A and of column l%16 of B; the
// instruction takes bytes 0-15 as k = 16*(l/16) .. +15 and bytes 16-31 as
// k = 64 + 16*(l/16) .. +15.  Under unit scales any k order that A and B
// share gives the same product, so callers place k as they like (e.g. 32
// consecutive values per lane).  D layout as above.
__device__ __forceinline__ f32x4 mfma16x16x128_fp8(i32x8 a, i32x8 b, f32x4 c) {
  // cbsz = blgp = 0 selects FP8 E4M3 for both operands; E8M0 scale 127 = 1.0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// D(16x16) += A(16x128) * B(128x16) with E2M1 (FP4) inputs and one E8M0 scale
// per lane: lane l supplies 32 consecutive k-values of row l%16 of A (16
// bytes of packed codes) and of column l%16 of B, each with the E8M0 code of
// its 32-value block (the MX block); products and scales are exact and the
// results accumulate in fp32.  D layout as above.
__device__ __forceinline__ f32x4 mfma16x16x128_fp4(i32x4 a, uint32_t scale_a, i32x4 b, uint32_t scale_b, f32x4 c) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  // cbsz = blgp = 4 selects FP4 E2M1 for both operands; opsel 0 takes byte 0
  // of each scale register
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, (int)scale_a, 0, (int)scale_b);
}

// ---------------------------------------------------------------- dequant
// Two E4M3 values (bytes 0,1 or 2,3 of `w`) -> two bf16.  E4M3 has a 3-bit
// mantissa and exponents 2^-9 .. 2^8, so the conversion is exact.
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
}

// Four E4M3 bytes of `w` -> four bf16 packed in two dwords.
__device__ __forceinline__ i32x2 e4m3x4_to_bf16(uint32_t w) {
  bf16x2 lo = e4m3x2_to_bf16(w, false);
  bf16x2 hi = e4m3x2_to_bf16(w, true);
  i32x2 r;
  r[0] = __builtin_bit_cast(int, lo);
  r[1] = __builtin_bit_cast(int, hi);
  return r;
}

// Eight E4M3 bytes -> one bf16x8 MFMA fragment.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  i32x2 a = e4m3x4_to_bf16(w0), b = e4m3x4_to_bf16(w1);
  i32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// Eight E2M1 codes (one dword, low nibble first) x a power-of-two scale ->
// bf16x8.  The scaled convert applies only the exponent of its scale operand,
// which is exact for E8M0 (MXFP4) scales.
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16x8(uint32_t w, float pow2_scale) {
  i32x4 r;
  r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, pow2_scale, 0));
  r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, pow2_scale, 1));
  r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, pow2_scale, 2));
  r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, pow2_scale, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// 2^x on the transcendental unit (v_exp_f32, about 1 ulp): 0 for -inf, and
// results below the normal range flush to 0, which a softmax weight (at most
// 2^8 against its running max) can lose without effect.  exp2f adds a range
// reduction for those results: four more instructions per weight.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 pair -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Eight E2M1 codes x an arbitrary (E4M3-valued) block scale -> bf16x8.  The
// product of a 2-significant-bit E2M1 value and a 4-significant-bit E4M3 value
// has at most 6 significant bits, so the fp32 product rounds to bf16 exactly.
__device__ __forceinline__ bf16x8 e2m1x8_times(uint32_t w, float scale) {
  i32x4 r;
#define DSA_E2M1_PAIR(b)                                                          \
  {                                                                               \
    const bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, 1.0f, b); \
    r[b] = (int)pack_bf16x2((float)v[0] * scale, (float)v[1] * scale);            \
  }
  DSA_E2M1_PAIR(0) DSA_E2M1_PAIR(1) DSA_E2M1_PAIR(2) DSA_E2M1_PAIR(3)
#undef DSA_E2M1_PAIR
  return __builtin_bit_cast(bf16x8, r);
}

// E8M0 code -> fp32 power of two 2^(code-127) (code 0 -> 2^-127, subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  return code == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(code << 23);
}

// E4M3 code -> fp32 (exact); used for NVFP4 block scales.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  bf16x2 v = e4m3x2_to_bf16(code & 0xFFu, false);
  return (float)v[0];
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- loads
__device__ __forceinline__ i32x4 ld16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ i32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

// ---------------------------------------------------------------- debug notes
// Debug builds (DSA_DEBUG=1) record, per translation unit, which kinds of
// device-resident metadata the kernels had to clamp or skip; the host reads
// and clears the words with dsa_check_debug_flag().  Release builds compile
// the notes away.
#ifndef DSA_DEBUG
#define DSA_DEBUG 0
#endif
#if DSA_DEBUG
static __device__ uint32_t dsa_debug_word;
#define DSA_DEBUG_NOTE(cond, bit)                         \
  do {                                                    \
    if (cond) atomicOr(&dsa_debug_word, (uint32_t)(bit)); \
  } while (0)
// Host side of one translation unit's word: its value, cleared (0 when the
// address cannot be resolved).
#define DSA_DEBUG_TAKE(name)                                                          \
  uint32_t debug_take_##name() {                                                      \
    void* a = nullptr;                                                                \
    uint32_t v = 0;                                                                   \
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(dsa_debug_word)) != hipSuccess || !a) return 0; \
    if (hipMemcpy(&v, a, 4, hipMemcpyDeviceToHost) != hipSuccess) return 0;           \
    if (hipMemset(a, 0, 4) != hipSuccess) return v;                                   \
    return v;                                                                         \
  }
#else
#define DSA_DEBUG_NOTE(cond, bit) \
  do {                            \
  } while (0)
#define DSA_DEBUG_TAKE(name) \
  uint32_t debug_take_##name() { return 0; }
#endif

// ---------------------------------------------------------------- paging
// Physical page of logical page `lp` of request `r`, or -1 when the
// block-table entry is outside the pool.
__device__ __forceinline__ int phys_page(const int32_t* __restrict__ bt, int bt_stride, int r, int lp,
                                         int num_pages) {
  int pg = bt ? bt[(int64_t)r * bt_stride + lp] : r;
  DSA_DEBUG_NOTE(pg < 0 || pg >= num_pages, DSA_DEBUG_ABSENT_PAGE);
  return (pg >= 0 && pg < num_pages) ? pg : -1;
}

// A visible count clamped to [0, max_vis].
__device__ __forceinline__ int clamp_vis(int v, int max_vis) {
  DSA_DEBUG_NOTE(v < 0 || v > max_vis, DSA_DEBUG_VIS_CLAMPED);
  return min(max(v, 0), max_vis);
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0.0 is
// mapped as +0.0.
// max(x, 0) on the bit pattern: non-negative floats are the non-negative
// int32 patterns, so one integer max is the ReLU (no NaN canonicalisation).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Lane-group exchanges (a row = 16 lanes).  permlane16_swap(x, y) swaps the odd
// rows of x with the even rows of y; permlane32_swap(x, y) swaps the upper 32
// lanes of x with the lower 32 lanes of y.  Both return (x', y').
struct f32pair {
  float x, y;
};
__device__ __forceinline__ f32pair swap_rows16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32pair swap_halves32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// The value of lane l ^ 16 (xor16) or l ^ 32 (xor32), by lane swaps instead
// of an LDS permute (g = l >> 4).
__device__ __forceinline__ float xor16(float x, int g) {
  const f32pair r = swap_rows16(x, x);  // odd rows get their even neighbour, and back
  return (g & 1) ? r.x : r.y;
}
__device__ __forceinline__ float xor32(float x, int g) {
  const f32pair r = swap_halves32(x, x);  // r.x: lower half twice, r.y: upper half twice
  return (g >> 1) ? r.x : r.y;
}

// Reduce-scatter over the four 16-lane rows: lane (g, c) holds v[0..3]; on
// return it holds sum over g' of v_{g'}[g] (its own row's share of the sum).
// After a swap every lane holds the two addends of its own share: a row swap
// of (v0, v1) leaves an even row with (its v0, its odd neighbour's v0) and an
// odd row with (its even neighbour's v1, its v1); the half swap of the pair
// sums does the same across the two 32-lane halves.  So each level is one
// swap and one add, with no select and no copy of the swapped operands.
__device__ __forceinline__ float rows_reduce_scatter4(const float (&v)[4]) {
  const f32pair a = swap_rows16(v[0], v[1]);
  const float s01 = a.x + a.y;  // even rows: v[0] of the row pair, odd rows: v[1]
  const f32pair b = swap_rows16(v[2], v[3]);
  const float s23 = b.x + b.y;
  const f32pair h = swap_halves32(s01, s23);
  return h.x + h.y;             // rows 0, 1: s01 of both halves; rows 2, 3: s23
}

__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace dsa
