// Device helpers shared by the BitLinear kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs; overflow
// rounds to infinity as IEEE requires).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
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

// v_mfma_i32_16x16x64_i8: D[16][16] += A[16][64] * B[64][16].  Lane l supplies
// row l%16 of A and column l%16 of B, 16 int8 each, for the same 16 k-slots
// (lane group l/16); D lands as rows 4*(l/16) + i, column l%16 in element i.
__device__ __forceinline__ v4i mfma_16x16x64(const v4i& a, const v4i& b, const v4i& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace bl
