// Per-token absmax int8 activation quantization for BitLinear W1.58A8.
//
// deepmox.com chapter 8, "A low-bit model is a whole-stack design": activations
// take a separate per-token 8-bit path; onilabs.co, "A Two-Billion Ternary
// Bet": they are quantized dynamically.  For each token (row) i:
//   a = max_j |x[i][j]|,  s = fl32(127 / max(a, 1e-5)),
//   xq[i][j] = clamp(round_half_even(fl32(x[i][j] * s)), -128, 127),  alpha[i] = a.
//
// One workgroup per row.  Pass 1 reads the bf16 row with 128-bit loads and
// reduces the absmax exactly (integer max of the magnitude bits, which orders
// non-negative floats); pass 2 re-reads the row (an L2 hit) and writes int8.
// HBM-bound: 2k bytes in, k + 4 bytes out per row.
#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t quant_pair(uint32_t two_bf16, float s) {
  float lo = __uint_as_float(two_bf16 << 16);
  float hi = __uint_as_float(two_bf16 & 0xFFFF0000u);
  float ql = fminf(fmaxf(__builtin_rintf(__fmul_rn(lo, s)), -128.0f), 127.0f);
  float qh = fminf(fmaxf(__builtin_rintf(__fmul_rn(hi, s)), -128.0f), 127.0f);
  return ((uint32_t)(int)ql & 0xFFu) | (((uint32_t)(int)qh & 0xFFu) << 8);
}

__global__ __launch_bounds__(kQuantThreads) void k_quant_act(const uint4* __restrict__ x, int64_t k,
                                                              uint2* __restrict__ xq, float* __restrict__ alpha) {
  __shared__ uint32_t wave_max[kQuantThreads / 64];
  const int64_t row = blockIdx.x;
  const int64_t k8 = k / 8;  // 8 bf16 per 128-bit load
  const uint4* src = x + row * k8;
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < k8; i += kQuantThreads) {
    uint4 v = src[i];
    m = max(m, max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu));
    m = max(m, max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
    m = max(m, max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu));
    m = max(m, max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t amax_bits = wave_max[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) amax_bits = max(amax_bits, wave_max[w]);
  const float amax = __uint_as_float(amax_bits << 16);
  const float s = 127.0f / fmaxf(amax, 1e-5f);  // IEEE division
  uint2* dst = xq + row * k8;
  for (int64_t i = threadIdx.x; i < k8; i += kQuantThreads) {
    uint4 v = src[i];
    uint32_t b0 = quant_pair(v.x, s) | (quant_pair(v.y, s) << 16);
    uint32_t b1 = quant_pair(v.z, s) | (quant_pair(v.w, s) << 16);
    dst[i] = make_uint2(b0, b1);
  }
  if (threadIdx.x == 0) alpha[row] = amax;
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* alpha, hipStream_t s) {
  hipLaunchKernelGGL(k_quant_act, dim3((unsigned)m), dim3(kQuantThreads), 0, s, reinterpret_cast<const uint4*>(x), k,
                     reinterpret_cast<uint2*>(xq), alpha);
  return hipGetLastError();
}

}  // namespace bl
