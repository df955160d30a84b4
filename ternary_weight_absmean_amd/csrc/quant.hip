// Per-token absmax int8 activation quantization for BitLinear W1.58A8.
//
// deepmox.com chapter 8, "A low-bit model is a whole-stack design": activations
// take a separate per-token 8-bit path; onilabs.co, "A Two-Billion Ternary
// Bet": they are quantized dynamically.  For each token (row) i:
//   a = max_j |x[i][j]|,  s = fl32(127 / max(a, 1e-5)),
//   xq[i][j] = clamp(round_half_even(fl32(x[i][j] * s)), -128, 127),  alpha[i] = a.
//
// The absmax is reduced exactly as an integer max of the magnitude bits
// (they order non-negative floats like the values).  HBM-bound: 2k bytes in,
// k + 4 bytes out per row.
#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kQuantThreads = 256;

// One workgroup per token row.  Rows of up to 256 * kC chunks of 8 bf16 (kC
// up to 16: 32768 columns) are held in registers between the absmax and the
// quantization (one read of the row); longer rows (kC = 0) are read twice,
// the second time from L2.
// Loads go through a buffer resource over the row, so chunks past k read as
// zero and need no branch.  The int8 code is formed by adding 1.5 * 2^23 to
// the fp32 product x * s (round half to even into the low byte); for finite
// inputs |x * s| <= 127 * (1 + 2^-24), so the clamp to [-128, 127] never
// binds and is not applied.
template <int kC>
__global__ __launch_bounds__(kQuantThreads) void k_quant_act(const uint4* __restrict__ x, int64_t k,
                                                              uint2* __restrict__ xq, float* __restrict__ alpha) {
  __shared__ int wave_max[kQuantThreads / 64];
  const int64_t row = blockIdx.x;
  const int k8 = (int)(k / 8);  // 8 bf16 per 128-bit load
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rsrc = buffer_rsrc(x + row * k8, (uint32_t)(k8 * 16));
  uint4 v[kC > 0 ? kC : 1];
  u16x2 m2 = {0, 0};
  if (kC > 0) {
#pragma unroll
    for (int c = 0; c < kC; ++c) v[c] = buffer_load16(rsrc, (uint32_t)((tid + c * kQuantThreads) * 16));
#pragma unroll
    for (int c = 0; c < kC; ++c) m2 = absmax_step(m2, v[c]);
  } else {
    for (int i = tid; i < k8; i += kQuantThreads) m2 = absmax_step(m2, buffer_load16(rsrc, (uint32_t)(i * 16)));
  }
  const int wm = wave_reduce<true>((int)max(m2.x, m2.y));
  if ((tid & 63) == 0) wave_max[tid >> 6] = wm;
  __syncthreads();
  int amax_bits = wave_max[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) amax_bits = max(amax_bits, wave_max[w]);
  const float amax = __uint_as_float((uint32_t)amax_bits << 16);
  const float s = 127.0f / fmaxf(amax, 1e-5f);  // IEEE division
  uint2* dst = xq + row * k8;
  int unused = 0;
  if (kC > 0) {
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const int i = tid + c * kQuantThreads;
      if (i < k8) dst[i] = act_codes8(v[c], s, unused);
    }
  } else {
    for (int i = tid; i < k8; i += kQuantThreads) dst[i] = act_codes8(buffer_load16(rsrc, (uint32_t)(i * 16)), s, unused);
  }
  if (tid == 0) alpha[row] = amax;
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* alpha, hipStream_t s) {
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* q = reinterpret_cast<uint2*>(xq);
  const int64_t chunks = (k / 8 + kQuantThreads - 1) / kQuantThreads;  // per thread
  if (!grid_fits(m, kQuantThreads)) return kErrGridTooLarge;
  if (chunks <= 2)
    hipLaunchKernelGGL(k_quant_act<2>, dim3((unsigned)m), dim3(kQuantThreads), 0, s, xv, k, q, alpha);
  else if (chunks <= 4)
    hipLaunchKernelGGL(k_quant_act<4>, dim3((unsigned)m), dim3(kQuantThreads), 0, s, xv, k, q, alpha);
  else if (chunks <= 8)
    hipLaunchKernelGGL(k_quant_act<8>, dim3((unsigned)m), dim3(kQuantThreads), 0, s, xv, k, q, alpha);
  else if (chunks <= 16)
    hipLaunchKernelGGL(k_quant_act<16>, dim3((unsigned)m), dim3(kQuantThreads), 0, s, xv, k, q, alpha);
  else
    hipLaunchKernelGGL(k_quant_act<0>, dim3((unsigned)m), dim3(kQuantThreads), 0, s, xv, k, q, alpha);
  return hipGetLastError();
}

}  // namespace bl
