// Device helpers shared by the BitLinear kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bit pattern, round to nearest even, by the conversion
// instruction (v_cvt_pk_bf16_f32; checked equal to the integer rounding
// (b + 0x7FFF + ((b >> 16) & 1)) >> 16 on 2^24 finite values including
// exact ties).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// two fp32 -> two bf16 in one dword (lo in bits 0..15)
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Squared-ReLU gating of one output from the exact integer products of its
// gate and up rows: relu(g)^2 * u with g = acc_g * scale, u = acc_u * scale
// (scale = gamma * alpha / 127), in fp32 without contraction.
__device__ __forceinline__ float glu_value(int acc_g, int acc_u, float scale) {
  const float g = (float)acc_g * scale;
  const float r = g > 0.0f ? g : 0.0f;
  return (r * r) * ((float)acc_u * scale);
}

// Signed trits of one 2-bit field of four packed bytes.  The field's codes
// (0, 1, 2 = trit + 1) select bytes 0xFF, 0x00, 0x01 of a constant table with
// v_perm_b32 (selector bytes 0..3 index the second operand).
__device__ __forceinline__ int trits_of_field(uint32_t packed4, int field) {
  const uint32_t table = 0x000100FFu;  // byte0 = -1, byte1 = 0, byte2 = +1
  uint32_t sel = (packed4 >> (2 * field)) & 0x03030303u;
  return (int)__builtin_amdgcn_perm(0u, table, sel);
}

// Field `field` of a row's 16 packed bytes: 16 signed trits for the 16
// consecutive columns 16*field + 0..15 of a 64-column tile, as an MFMA operand.
__device__ __forceinline__ v4i unpack_field(const uint4& p, int field) {
  v4i r;
  r.x = trits_of_field(p.x, field);
  r.y = trits_of_field(p.y, field);
  r.z = trits_of_field(p.z, field);
  r.w = trits_of_field(p.w, field);
  return r;
}

__device__ __forceinline__ v4i as_v4i(const uint4& u) {
  v4i r;
  r.x = (int)u.x;
  r.y = (int)u.y;
  r.z = (int)u.z;
  r.w = (int)u.w;
  return r;
}

// Row key of the XOR swizzle for 16-byte chunks of token rows in LDS that
// MFMA B-operand reads take 16 rows at a time (lane l reads row l % 16 with
// ds_read_b128): chunk c of row r is stored at c ^ lds_row_key(r), the two
// 2-bit halves of r % 16 swapped.  Measured on gfx950 with rows of 256 and
// 512 bytes: the plain key r % 16 leaves a two-way bank conflict on every
// such read (8.8 against 5.1 CU cycles per ds_read_b128), this key none.
__device__ __forceinline__ int lds_row_key(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Raw buffer resource over `bytes` bytes at `base` (stride 0).  Loads through
// it return zero for any offset at or past `bytes` instead of touching memory,
// so tails and absent operands need no branch (a load inside a divergent
// branch is followed by its own wait, which serializes a batch of loads).
// The descriptor must be wave-uniform; offsets are per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same load marked non-temporal (cache policy bit 1: `nt` on gfx950), for
// weight bytes that one launch reads exactly once.  A plain read stream of
// 59-117 MB measured 5.2-5.7 TB/s with default loads and 5.9-6.5 TB/s with
// this bit, at every workgroup count tried.
__device__ __forceinline__ uint4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Per-token int8 code of one finite bf16 x: round_half_even(fl32(x * s)),
// for s = fl32(127 / max(amax, 1e-5)) and |x| <= amax.  Adding 1.5 * 2^23
// to the fp32 product rounds it to an integer in the low mantissa bits
// (ties to even: the sum's parity is the integer's, 1.5 * 2^23 being even),
// so the low byte of the sum is the code in two's complement.  The product
// is at most 127 * (1 + 2^-24) in magnitude, so every code lies in
// [-127, 127] and the clamp to [-128, 127] never binds.
__device__ __forceinline__ uint32_t act_code_bits(uint32_t bf16_in_high_half, float s) {
  return __float_as_uint(__fadd_rn(__fmul_rn(__uint_as_float(bf16_in_high_half), s), 12582912.0f));
}

// Codes of the eight bf16 of a 16-byte chunk, packed in element order into
// 8 bytes; their sum is added to `sum`.
__device__ __forceinline__ uint2 act_codes8(const uint4& v, float s, int& sum) {
  auto four = [&](uint32_t d0, uint32_t d1) {
    const uint32_t a0 = act_code_bits(d0 << 16, s), a1 = act_code_bits(d0 & 0xFFFF0000u, s);
    const uint32_t a2 = act_code_bits(d1 << 16, s), a3 = act_code_bits(d1 & 0xFFFF0000u, s);
    // v_perm_b32: selector bytes 0-3 pick bytes of the second operand, 4-7 of the first, 0x0c gives 0
    const uint32_t p01 = __builtin_amdgcn_perm(a1, a0, 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(a3, a2, 0x0c0c0400u);
    const uint32_t q = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    sum = __builtin_amdgcn_sdot4((int)q, 0x01010101, sum, false);
    return q;
  };
  const uint32_t lo = four(v.x, v.y);
  const uint32_t hi = four(v.z, v.w);
  return make_uint2(lo, hi);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running max of |bf16| magnitude bits over 16-byte chunks, two lanes of
// 16 bits at a time (v_pk_max_u16); magnitude bits order like the values.
__device__ __forceinline__ u16x2 absmax_step(u16x2 m, const uint4& v) {
  auto mag = [](uint32_t d) { return __builtin_bit_cast(u16x2, d & 0x7FFF7FFFu); };
  m = __builtin_elementwise_max(m, mag(v.x));
  m = __builtin_elementwise_max(m, mag(v.y));
  m = __builtin_elementwise_max(m, mag(v.z));
  return __builtin_elementwise_max(m, mag(v.w));
}

// One fp32 through the vector memory path: issued where it is written and
// waited for only where it is used (a scalar load of a kernel argument's
// target is otherwise sunk to its use, adding a round trip there).
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, offset, 0, 0));
}

// Reduction over aligned groups of `g` lanes (g a power of two up to 64) with
// DPP lane moves inside each 16-lane row (no LDS round trip) and, for groups
// wider than a row, cross-lane permutes.  After each step every lane of a
// block holds the block's reduction, so the mirrors pair blocks correctly:
// quad_perm [1,0,3,2] and [2,3,0,1] reduce quads, row_half_mirror (lane i of
// an 8-lane half row takes lane 7 - i) joins quad pairs, row_mirror (15 - i)
// joins the two halves of a row.  Every lane ends with its group's value.
template <bool kMax>
__device__ __forceinline__ int lane_group_reduce(int v, int g) {
  auto op = [](int a, int b) { return kMax ? max(a, b) : a + b; };
  if (g >= 2) v = op(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));
  if (g >= 4) v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));
  if (g >= 8) v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));
  if (g >= 16) v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));
  if (g >= 32) v = op(v, __shfl_xor(v, 16, 64));
  if (g >= 64) v = op(v, __shfl_xor(v, 32, 64));
  return v;
}

// Whole-wave reduction, wave-uniform result: DPP within rows, then the four
// row results read as scalars.
template <bool kMax>
__device__ __forceinline__ int wave_reduce(int v) {
  v = lane_group_reduce<kMax>(v, 16);
  const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return kMax ? max(max(r0, r1), max(r2, r3)) : (r0 + r1) + (r2 + r3);
}

// v_mfma_i32_16x16x64_i8: D[16][16] += A[16][64] * B[64][16].  Lane l supplies
// row l%16 of A and column l%16 of B, 16 int8 each, for the same 16 k-slots
// (lane group l/16); D lands as rows 4*(l/16) + i, column l%16 in element i.
__device__ __forceinline__ v4i mfma_16x16x64(const v4i& a, const v4i& b, const v4i& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): a loop
// whose index is a compile-time constant in every copy of the body.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// s_waitcnt immediate that waits until at most n vector memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_at_most(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ void add4(v4i& a, const v4i& b) {
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
}

// Epilogue of a 16-row tile product: the lane holds the int32 sums of rows
// row0 .. row0 + 3 for token `tok`; writes acc (if non-NULL) and y = bf16(acc
// * scale) (if non-NULL), rows past n skipped.
__device__ __forceinline__ void store_tile(const v4i& acc, int64_t row0, int64_t tok, int64_t n, float scale,
                                           int32_t* __restrict__ acc_out, uint16_t* __restrict__ y_out) {
  const int vals[4] = {acc.x, acc.y, acc.z, acc.w};
  // four consecutive outputs of one token: one 16-byte and one 8-byte store when aligned
  uint16_t* yp = y_out ? y_out + tok * n + row0 : nullptr;
  int32_t* ap = acc_out ? acc_out + tok * n + row0 : nullptr;
  if (row0 + 3 < n && (!yp || ((uintptr_t)yp & 7) == 0) && (!ap || ((uintptr_t)ap & 15) == 0)) {
    if (ap) *reinterpret_cast<int4*>(ap) = make_int4(vals[0], vals[1], vals[2], vals[3]);
    if (yp)
      *reinterpret_cast<uint2*>(yp) = make_uint2(f32x2_to_bf16x2((float)vals[0] * scale, (float)vals[1] * scale),
                                                 f32x2_to_bf16x2((float)vals[2] * scale, (float)vals[3] * scale));
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + i;
    if (row < n) {
      if (acc_out) acc_out[tok * n + row] = vals[i];
      if (y_out) y_out[tok * n + row] = f32_to_bf16_rne((float)vals[i] * scale);
    }
  }
}

}  // namespace bl
