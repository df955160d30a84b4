// Weight preparation for BitLinear W1.58A8 (BitNet b1.58 absmean ternarization).
//
// bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution", section
// "The BitLinear Layer and AbsMean Quantization": gamma is the mean absolute
// value of the entire weight matrix; every weight is divided by gamma + 1e-5,
// rounded to the nearest integer and clamped to [-1, 1].  deepmox.com chapter 8,
// "A low-bit model is a whole-stack design": four ternary values per 8-bit unit.
//
// gamma must be identical wherever it is computed, because a one-ulp change
// flips every weight that sits within rounding distance of the +-0.5 decision
// boundary.  A floating-point sum depends on its order, so the sum of |w| is
// formed exactly: each |w| = sig * 2^(e-150) (e the biased exponent, sig the
// significand with its hidden bit), and sig is added into a 64-bit integer bin
// per exponent.  Integer addition is order-independent, so any grid and any
// atomic interleaving gives the same bins.  One thread then evaluates
// sum_e bins[e] * 2^(e-150) / (n*k) exactly in multi-word integer arithmetic
// and rounds it once to fp32 (nearest, ties to even).
//
// Kernels (all HBM-bound streaming passes except the one-thread fold):
//   k_zero_bins        256 x u64 <- 0
//   k_absmean_bins     read w once; per-wave LDS bins; one global atomic per
//                      non-empty bin per workgroup
//   k_gamma_fold       exact mean -> gamma (device memory; no host readback)
//   k_ternarize_pack   read w again; one thread per 16-byte row chunk of a
//                      16x64 tile; IEEE fp32 divide, round-half-even, clamp
//   k_unpack           packed -> int8 trits (inspection helper)
#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kBins = 256;
constexpr int kBinThreads = 256;
constexpr int kBinWaves = kBinThreads / 64;

__global__ void k_zero_bins(unsigned long long* bins) { bins[threadIdx.x] = 0ull; }

__device__ __forceinline__ void bin_abs(unsigned long long* lbins, float v) {
  uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
  uint32_t e = b >> 23;
  uint32_t sig = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  atomicAdd(&lbins[e], (unsigned long long)sig);
}

__global__ __launch_bounds__(kBinThreads) void k_absmean_bins(const float4* __restrict__ w4, int64_t n4,
                                                               unsigned long long* __restrict__ bins) {
  __shared__ unsigned long long lbins[kBinWaves][kBins];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  for (int i = tid; i < kBinWaves * kBins; i += kBinThreads) (&lbins[0][0])[i] = 0ull;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kBinThreads;
  for (int64_t i = (int64_t)blockIdx.x * kBinThreads + tid; i < n4; i += stride) {
    float4 v = w4[i];
    bin_abs(lbins[wave], v.x);
    bin_abs(lbins[wave], v.y);
    bin_abs(lbins[wave], v.z);
    bin_abs(lbins[wave], v.w);
  }
  __syncthreads();
  unsigned long long s = 0;
#pragma unroll
  for (int wv = 0; wv < kBinWaves; ++wv) s += lbins[wv][tid];
  if (s) atomicAdd(&bins[tid], s);
}

// ---------------------------------------------------------------- exact fold

constexpr int kLimbs = 22;  // 16-bit limbs: 352 bits > 2^(64 + 253)

// bit `pos` of a little-endian 16-bit-limb integer
__device__ __forceinline__ uint32_t limb_bit(const uint32_t* q, int pos) {
  return (q[pos >> 4] >> (pos & 15)) & 1u;
}

__global__ void k_gamma_fold(const unsigned long long* __restrict__ bins, unsigned long long count,
                             float* __restrict__ gamma) {
  if (threadIdx.x != 0) return;
  // X = sum_e bins[e] * 2^(max(e,1) - 1) = sum |w| * 2^149, as 16-bit limbs
  uint32_t x[kLimbs];
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) x[i] = 0;
  for (int e = 0; e < kBins - 1; ++e) {
    unsigned long long v = bins[e];
    if (v == 0) continue;
    int sh = e ? e - 1 : 0;
    int q = sh >> 4, r = sh & 15;
    unsigned long long lo = v << r;
    unsigned long long hi = r ? (v >> (64 - r)) : 0ull;
    x[q + 0] += (uint32_t)(lo & 0xFFFFu);
    x[q + 1] += (uint32_t)((lo >> 16) & 0xFFFFu);
    x[q + 2] += (uint32_t)((lo >> 32) & 0xFFFFu);
    x[q + 3] += (uint32_t)((lo >> 48) & 0xFFFFu);
    x[q + 4] += (uint32_t)(hi & 0xFFFFu);
  }
  uint32_t carry = 0;
  for (int i = 0; i < kLimbs; ++i) {
    uint32_t t = x[i] + carry;
    x[i] = t & 0xFFFFu;
    carry = t >> 16;
  }
  // Q = floor(X / count), R = X mod count (count < 2^40, so rem << 16 < 2^56)
  uint32_t qv[kLimbs];
  unsigned long long rem = 0;
  for (int i = kLimbs - 1; i >= 0; --i) {
    unsigned long long cur = (rem << 16) | x[i];
    qv[i] = (uint32_t)(cur / count);
    rem = cur % count;
  }
  int nb = 0;  // bit length of Q
  for (int i = kLimbs - 1; i >= 0; --i) {
    if (qv[i]) {
      nb = 16 * i + (32 - __clz(qv[i]));
      break;
    }
  }
  // keep 24 significant bits; mean = mant * 2^(shift - 149)
  int shift = nb > 24 ? nb - 24 : 0;
  uint32_t mant = 0;
  for (int b = 23; b >= 0; --b) mant = (mant << 1) | (shift + b < kLimbs * 16 ? limb_bit(qv, shift + b) : 0u);
  bool up;
  if (shift == 0) {
    unsigned long long twice = rem << 1;  // rem < 2^40
    up = twice > count || (twice == count && (mant & 1u));
  } else {
    bool round_bit = limb_bit(qv, shift - 1);
    bool sticky = rem != 0;
    for (int b = 0; b < shift - 1 && !sticky; ++b) sticky = limb_bit(qv, b);
    up = round_bit && (sticky || (mant & 1u));
  }
  // fp32 encoding of mant * 2^(shift-149): (shift << 23) + mant, also across
  // the carry when rounding reaches 2^24 and for subnormals (shift = 0).
  uint32_t bits = ((uint32_t)shift << 23) + mant + (up ? 1u : 0u);
  *gamma = __uint_as_float(bits);
}

// ---------------------------------------------------------------- ternarize + pack

constexpr int kPackThreads = 256;

// Thread per (row, 64-column tile): reads the 64 fp32 weights of that row
// segment (256 contiguous bytes) and writes its 16 packed bytes.  Column
// 16*f + b of the segment goes to byte b, bits 2f..2f+1, as code q + 1.
__global__ __launch_bounds__(kPackThreads) void k_ternarize_pack(const float* __restrict__ w, int64_t n, int64_t k,
                                                                  const float* __restrict__ gamma_ptr,
                                                                  uint4* __restrict__ packed) {
  const int64_t kt_count = k / kTileCols;
  const int64_t n_pad = (n + kTileRows - 1) / kTileRows * kTileRows;
  const int64_t idx = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (idx >= n_pad * kt_count) return;
  const int64_t row = idx / kt_count;
  const int64_t kt = idx % kt_count;
  uint4* dst = packed + ((row / kTileRows) * kt_count + kt) * (kTileBytes / 16) + (row % kTileRows);
  if (row >= n) {
    *dst = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
    return;
  }
  const float denom = *gamma_ptr + 1e-5f;
  const float4* src = reinterpret_cast<const float4*>(w + row * k + kt * kTileCols);
  uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      float4 v = src[f * 4 + b4];
      float c[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float r = __builtin_rintf(c[j] / denom);  // IEEE division, then round half to even
        r = fminf(fmaxf(r, -1.0f), 1.0f);
        uint32_t code = (uint32_t)((int)r + 1);
        word[b4] |= code << (8 * j + 2 * f);
      }
    }
  }
  *dst = make_uint4(word[0], word[1], word[2], word[3]);
}

__global__ __launch_bounds__(kPackThreads) void k_unpack(const uint4* __restrict__ packed, int64_t n, int64_t k,
                                                          int8_t* __restrict__ q) {
  const int64_t kt_count = k / kTileCols;
  const int64_t idx = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (idx >= n * kt_count) return;
  const int64_t row = idx / kt_count;
  const int64_t kt = idx % kt_count;
  const uint4 p = packed[((row / kTileRows) * kt_count + kt) * (kTileBytes / 16) + (row % kTileRows)];
  uint4* dst = reinterpret_cast<uint4*>(q + row * k + kt * kTileCols);
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    v4i t = unpack_field(p, f);
    dst[f] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
  }
}

}  // namespace

hipError_t launch_zero_bins(unsigned long long* bins, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_bins, dim3(1), dim3(kBins), 0, s, bins);
  return hipGetLastError();
}

hipError_t launch_absmean_bins(const float* w, int64_t count, unsigned long long* bins, hipStream_t s) {
  const int64_t n4 = count / 4;
  int64_t blocks = (n4 + kBinThreads - 1) / kBinThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_absmean_bins, dim3((unsigned)blocks), dim3(kBinThreads), 0, s,
                     reinterpret_cast<const float4*>(w), n4, bins);
  return hipGetLastError();
}

hipError_t launch_gamma_fold(const unsigned long long* bins, int64_t count, float* gamma, hipStream_t s) {
  hipLaunchKernelGGL(k_gamma_fold, dim3(1), dim3(64), 0, s, bins, (unsigned long long)count, gamma);
  return hipGetLastError();
}

hipError_t launch_ternarize_pack(const float* w, int64_t n, int64_t k, const float* gamma, uint8_t* packed,
                                 hipStream_t s) {
  const int64_t n_pad = (n + kTileRows - 1) / kTileRows * kTileRows;
  const int64_t threads = n_pad * (k / kTileCols);
  const int64_t blocks = (threads + kPackThreads - 1) / kPackThreads;
  hipLaunchKernelGGL(k_ternarize_pack, dim3((unsigned)blocks), dim3(kPackThreads), 0, s, w, n, k, gamma,
                     reinterpret_cast<uint4*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* q, hipStream_t s) {
  const int64_t threads = n * (k / kTileCols);
  const int64_t blocks = (threads + kPackThreads - 1) / kPackThreads;
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)blocks), dim3(kPackThreads), 0, s,
                     reinterpret_cast<const uint4*>(packed), n, k, q);
  return hipGetLastError();
}

}  // namespace bl
