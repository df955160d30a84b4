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
// Kernels (all HBM-bound streaming passes except the fold):
//   k_zero_bins        clear the 256 bins of the workspace
//   k_absmean_bins     read w once; exponent bins per workgroup (registers
//                      and LDS), added into the workspace's bins (64-bit
//                      integer atomics, 256 per workgroup)
//   k_gamma_fold       exact mean of the binned sum -> gamma (device memory;
//                      no host readback)
//   k_ternarize_pack   read w again; lane per float4, 16 lanes per 64-column
//                      row segment; the rounding of w / (gamma + 1e-5) as an
//                      exact threshold test
//   k_unpack           packed -> int8 trits (inspection helper)
//
// The allocation-free form of the packer keeps its bins in `scratch`, a
// static device array of this file (one copy per GPU, at its own address on
// each); the host side looks its address up once per device.
#include <mutex>

#include "device_util.h"
#include "internal.h"

// The packer's 256 exponent bins for callers that cannot allocate a
// workspace.  In host code this name is a stand-in for the symbol, not a
// device address: kernels receive the address static_pack_bins() looked up.
static __device__ __align__(256) unsigned long long scratch[256];

namespace bl {
namespace {

constexpr int kBins = 256;
constexpr int kBinThreads = 512;
constexpr int kBinLoads = 8;    // float4 loads per thread per iteration (in flight together)
constexpr int kWindow = 16;     // exponents accumulated in registers

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Exact sum of |w| by exponent.  |w| = sig * 2^(e-150) with e the biased
// exponent and sig the significand (hidden bit included for e > 0); the
// bins hold sum sig per exponent, so that sum |w| = sum_e bins[e] *
// 2^(max(e, 1) - 150).  Most values of a weight matrix fall within a few
// binades of its largest, so each lane adds sig << (e - e0) into one 64-bit
// register for e in the wave's window [e0, e0 + 16), e0 taken from the
// wave's first values; that register equals sum sig * 2^(e - e0), i.e. the
// bin e0 contribution of the window, and is split into its low and high 32
// bits for bins e0 and e0 + 32.  Values outside the window (and subnormals)
// go to LDS bins by atomic add.  Each workgroup then adds its 256 bins into
// the workspace's bins (cleared by k_zero_bins) with 64-bit integer atomics.
// All additions are of integers, so the result does not depend on the grid
// or the order.  At most 2^17 threads and count <= 2^39: at most 2^22 values
// per lane of at most 2^39 each, and no bin total exceeds
// count * 2^24 + 2^49 < 2^64.
__global__ __launch_bounds__(kBinThreads) void k_absmean_bins(const float4* __restrict__ w4, int64_t n4,
                                                               unsigned long long* __restrict__ ws) {
  __shared__ unsigned long long lbins[kBins];
  const int tid = threadIdx.x;
  if (tid < kBins) lbins[tid] = 0ull;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kBinThreads * kBinLoads;
  int e0 = -1;  // window base, chosen from the first batch
  unsigned long long acc = 0ull;
  auto add = [&](float v) {
    const uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
    const int e = (int)(b >> 23);
    const uint32_t sig = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    const uint32_t d = (uint32_t)(e - e0);
    if (d < (uint32_t)kWindow) {
      acc += (unsigned long long)sig << d;
    } else if (sig) {
      atomicAdd(&lbins[e], (unsigned long long)sig);
    }
  };
  for (int64_t base = (int64_t)blockIdx.x * kBinThreads * kBinLoads; base < n4; base += stride) {
    float4 v[kBinLoads];
#pragma unroll
    for (int j = 0; j < kBinLoads; ++j) {
      const int64_t i = base + j * kBinThreads + tid;
      v[j] = w4[i < n4 ? i : n4 - 1];
      if (i >= n4) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (e0 < 0) {
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < kBinLoads; ++j)
        mx = max(mx, max(max(__float_as_uint(v[j].x) & 0x7FFFFFFFu, __float_as_uint(v[j].y) & 0x7FFFFFFFu),
                         max(__float_as_uint(v[j].z) & 0x7FFFFFFFu, __float_as_uint(v[j].w) & 0x7FFFFFFFu)));
      const int emax = wave_reduce<true>((int)(mx >> 23));
      e0 = min(max(emax - (kWindow - 4), 1), kBins - 2 - 32);  // e0 >= 1, e0 + 32 <= 253
    }
#pragma unroll
    for (int j = 0; j < kBinLoads; ++j) {
      add(v[j].x);
      add(v[j].y);
      add(v[j].z);
      add(v[j].w);
    }
  }
  if (e0 >= 0) {  // wave-uniform: the wave saw at least one batch
    const unsigned long long lo = wave_sum_u64(acc & 0xFFFFFFFFull);
    const unsigned long long hi = wave_sum_u64(acc >> 32);
    if ((tid & 63) == 0) {
      if (lo) atomicAdd(&lbins[e0], lo);
      if (hi) atomicAdd(&lbins[e0 + 32], hi);
    }
  }
  __syncthreads();
  if (tid < kBins && lbins[tid]) atomicAdd(&ws[tid], lbins[tid]);
}

__global__ __launch_bounds__(kBins) void k_zero_bins(unsigned long long* __restrict__ ws) { ws[threadIdx.x] = 0ull; }

// ---------------------------------------------------------------- exact fold

constexpr int kLimbs = 22;  // 16-bit limbs: 352 bits > 2^(64 + 253)

// bit `pos` of a little-endian 16-bit-limb integer
__device__ __forceinline__ uint32_t limb_bit(const uint32_t* q, int pos) {
  return (q[pos >> 4] >> (pos & 15)) & 1u;
}

// floor(cur / d) and cur mod d for cur < 2^56, 0 < d < 2^40: a double
// estimate (relative error below 2^-52, so within one of the quotient), then
// integer correction.
__device__ __forceinline__ uint32_t div_step(unsigned long long cur, unsigned long long d, unsigned long long& rem) {
  long long q = (long long)((double)cur / (double)d);
  long long r = (long long)cur - q * (long long)d;
  while (r < 0) {
    --q;
    r += (long long)d;
  }
  while (r >= (long long)d) {
    ++q;
    r -= (long long)d;
  }
  rem = (unsigned long long)r;
  return (uint32_t)q;
}

// One workgroup of 256 threads: thread e adds the value bins[e] *
// 2^(max(e,1) - 1) into 16-bit limbs of X = sum |w| * 2^149 (LDS atomics;
// each limb sum stays below 2^25); one thread then propagates the carries,
// divides by the element count (long division by limbs) and rounds the
// quotient once to fp32, nearest with ties to even.
__global__ __launch_bounds__(kBins) void k_gamma_fold(const unsigned long long* __restrict__ ws,
                                                      unsigned long long count, float* __restrict__ gamma) {
  __shared__ uint32_t xl[kLimbs];
  const int e = threadIdx.x;
  if (e < kLimbs) xl[e] = 0;
  const unsigned long long v = ws[e];
  __syncthreads();
  if (v != 0 && e < kBins - 1) {
    const int sh = e ? e - 1 : 0;
    const int q = sh >> 4, r = sh & 15;
    const unsigned long long lo = v << r;
    const unsigned long long hi = r ? (v >> (64 - r)) : 0ull;
    atomicAdd(&xl[q + 0], (uint32_t)(lo & 0xFFFFu));
    atomicAdd(&xl[q + 1], (uint32_t)((lo >> 16) & 0xFFFFu));
    atomicAdd(&xl[q + 2], (uint32_t)((lo >> 32) & 0xFFFFu));
    atomicAdd(&xl[q + 3], (uint32_t)((lo >> 48) & 0xFFFFu));
    atomicAdd(&xl[q + 4], (uint32_t)(hi & 0xFFFFu));
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint32_t x[kLimbs];
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) x[i] = xl[i];
  uint32_t carry = 0;
  for (int i = 0; i < kLimbs; ++i) {
    const uint32_t t = x[i] + carry;
    x[i] = t & 0xFFFFu;
    carry = t >> 16;
  }
  // Q = floor(X / count), R = X mod count (count < 2^40, so rem << 16 < 2^56)
  uint32_t qv[kLimbs];
  unsigned long long rem = 0;
  for (int i = kLimbs - 1; i >= 0; --i) qv[i] = div_step((rem << 16) | x[i], count, rem);
  int nb = 0;  // bit length of Q
  for (int i = kLimbs - 1; i >= 0; --i) {
    if (qv[i]) {
      nb = 16 * i + (32 - __clz(qv[i]));
      break;
    }
  }
  // keep 24 significant bits; mean = mant * 2^(shift - 149)
  const int shift = nb > 24 ? nb - 24 : 0;
  uint32_t mant = 0;
  for (int b = 23; b >= 0; --b) mant = (mant << 1) | (shift + b < kLimbs * 16 ? limb_bit(qv, shift + b) : 0u);
  bool up;
  if (shift == 0) {
    const unsigned long long twice = rem << 1;  // rem < 2^40
    up = twice > count || (twice == count && (mant & 1u));
  } else {
    const bool round_bit = limb_bit(qv, shift - 1);
    // sticky: the remainder, or any quotient bit below the round bit
    bool sticky = rem != 0;
    const int below = shift - 1;  // bits 0 .. below-1
    for (int i = 0; i < (below >> 4) && !sticky; ++i) sticky = qv[i] != 0;
    if (!sticky && (below & 15)) sticky = (qv[below >> 4] & ((1u << (below & 15)) - 1u)) != 0;
    up = round_bit && (sticky || (mant & 1u));
  }
  // fp32 encoding of mant * 2^(shift-149): (shift << 23) + mant, also across
  // the carry when rounding reaches 2^24 and for subnormals (shift = 0).
  const uint32_t bits = ((uint32_t)shift << 23) + mant + (up ? 1u : 0u);
  *gamma = __uint_as_float(bits);
}

// ---------------------------------------------------------------- ternarize + pack

constexpr int kPackThreads = 256;

// Lane per 4 consecutive weights (one float4): 16 lanes cover one row of a
// 64-column tile and a wave covers 4 consecutive tiles of one row, so each
// wave-wide load reads 1 KiB contiguously.  Column c of the tile goes to byte
// c % 16, bits 2*(c/16): lane j (columns 4j..4j+3) fills field j / 4 of bytes
// 4*(j%4) .. 4*(j%4)+3, i.e. dword j % 4 of the row's 16 packed bytes.  The
// four lanes j = d, d+4, d+8, d+12 of dword d are OR-combined with DPP row
// rotations, and lanes 0..3 of each 16 store the dwords.  Rows past n get
// code 1 (trit 0).  Code = q + 1, q = clamp(round_half_even(w / (gamma +
// 1e-5)), -1, 1) with IEEE fp32 division, evaluated as the equivalent
// threshold test below.  Each thread handles kPackIter float4 slots, all
// loads issued first.
// glu_f > 0: w is a gate+up matrix [2 * glu_f][k] (gate rows first) and the
// packed row tiles alternate gate and up: packed tile 2t holds gate rows
// 16t..16t+15, tile 2t + 1 the up rows 16t..16t+15 (glu_f % 16 == 0).
constexpr int kPackIter = 4;  // float4 loads per thread, issued together
__global__ __launch_bounds__(kPackThreads) void k_ternarize_pack(const float4* __restrict__ w4, int64_t n, int64_t k,
                                                                  const float* __restrict__ gamma_ptr,
                                                                  uint32_t* __restrict__ packed, int64_t glu_f) {
  const int64_t k4 = k / 4;
  const int64_t n_pad = (n + kTileRows - 1) / kTileRows * kTileRows;
  const int64_t total = n_pad * k4;  // float4 slots of the padded matrix
  // q = clamp(rint(fl(w / d)), -1, 1) with d = fl(gamma + 1e-5) is +-1 exactly
  // when fl(|w| / d) > 0.5 (0.5 itself rounds to 0, ties to even).  The fp32
  // value above d / 2 is d / 2 + ulp(d / 2), whose quotient is 0.5 + 2^-24 / m
  // (m in [1, 2) the significand of d): beyond the midpoint 0.5 + 2^-25, so it
  // rounds above 0.5; and |w| <= d / 2 gives a quotient of at most 0.5.  So
  // for finite w the code is sign(w) when |w| > d / 2 (exact in fp32) and 0
  // otherwise -- the same bits as the correctly rounded division.
  const float half_d = (*gamma_ptr + 1e-5f) * 0.5f;
  int64_t idx[kPackIter];
  float4 v[kPackIter];
#pragma unroll
  for (int it = 0; it < kPackIter; ++it) {
    idx[it] = ((int64_t)blockIdx.x * kPackIter + it) * kPackThreads + threadIdx.x;
    const bool real = idx[it] < total && idx[it] / k4 < n;
    v[it] = w4[real ? idx[it] : 0];
  }
#pragma unroll
  for (int it = 0; it < kPackIter; ++it) {
    if (idx[it] >= total) break;  // whole 16-lane groups leave together (k4 is a multiple of 16)
    const int64_t row = idx[it] / k4;
    const int64_t c4 = idx[it] % k4;  // float4 within the row
    const int j = (int)(c4 & 15);     // lane within the tile row
    const int64_t kt = c4 >> 4;
    uint32_t part;
    if (row < n) {
      const float c[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
      part = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t code = fabsf(c[i]) > half_d ? (c[i] < 0.0f ? 0u : 2u) : 1u;
        part |= code << (8 * i + 2 * (j >> 2));
      }
    } else {
      part = 0x01010101u << (2 * (j >> 2));
    }
    // OR over the four lanes of the same dword (lane offsets 4 and 8 within the 16-lane row)
    part |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)part, 0x124, 0xF, 0xF, false);  // row_ror:4
    part |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)part, 0x128, 0xF, 0xF, false);  // row_ror:8
    int64_t prow = row;  // row of the packed matrix
    if (glu_f > 0) {
      const bool up = row >= glu_f;
      const int64_t r = up ? row - glu_f : row;
      prow = (r / kTileRows) * (2 * kTileRows) + (up ? kTileRows : 0) + r % kTileRows;
    }
    if (j < 4) packed[(((prow / kTileRows) * (k / kTileCols) + kt) * kTileRows + (prow % kTileRows)) * 4 + j] = part;
  }
}

// Packed q^T ([k][n]) from packed q ([n][k]), n % 64 == 0.  A workgroup
// turns the 64 x 64 trit block of q at rows 64 bj.., columns 64 bt.. (row
// tiles 4 bj..4 bj + 3 of column tile bt, 1 KiB) into the block of q^T at rows
// 64 bt.., columns 64 bj.. (row tiles 4 bt.. of column tile bj), through LDS as
// one code per byte.  Thread d of each 64 reads and writes dword d of one
// 256-byte tile: row d / 4, bytes 4 (d % 4)..+3, i.e. columns 16 f + 4 (d % 4) + i.
__global__ __launch_bounds__(256) void k_pack_transposed(const uint32_t* __restrict__ packed, int64_t n, int64_t k,
                                                         uint32_t* __restrict__ packed_t) {
  __shared__ uint8_t codes[64][64 + 4];  // [row of q in the block][column of q in the block]
  const int tid = threadIdx.x;
  const int64_t col_blocks = k / 64;
  const int64_t bj = (int64_t)blockIdx.x / col_blocks;
  const int64_t bt = (int64_t)blockIdx.x % col_blocks;
  const int s = tid >> 6, d = tid & 63;
  const int r = 16 * s + d / 4, b0 = 4 * (d % 4);
  const uint32_t w = packed[((4 * bj + s) * col_blocks + bt) * 64 + d];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) codes[r][16 * f + b0 + i] = (uint8_t)((w >> (8 * i + 2 * f)) & 3u);
  __syncthreads();
  // row r of the q^T block is column r of the q block; its byte b0 + i, field
  // f holds column 16 f + b0 + i of q^T = row 16 f + b0 + i of q
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) out |= (uint32_t)codes[16 * f + b0 + i][r] << (8 * i + 2 * f);
  packed_t[((4 * bt + s) * (n / 64) + bj) * 64 + d] = out;
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

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned long long* g_scratch_ptr[kMaxDevices];  // address of `scratch` on each device, once looked up

}  // namespace

hipError_t static_pack_bins(hipStream_t s, unsigned long long** bins) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the array's address on `dev`: looked up with that device current
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e == hipSuccess && p == nullptr) e = hipErrorInvalidSymbol;
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<unsigned long long*>(p);
  }
  *bins = g_scratch_ptr[dev];
  return hipSuccess;
}

int absmean_blocks(int64_t count) {
  const int64_t n4 = count / 4;
  int64_t blocks = (n4 + kBinThreads * kBinLoads - 1) / (kBinThreads * kBinLoads);
  if (blocks > kAbsmeanMaxBlocks) blocks = kAbsmeanMaxBlocks;
  return blocks < 1 ? 1 : (int)blocks;
}

hipError_t launch_absmean_bins(const float* w, int64_t count, unsigned long long* ws, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_bins, dim3(1), dim3(kBins), 0, s, ws);
  hipLaunchKernelGGL(k_absmean_bins, dim3((unsigned)absmean_blocks(count)), dim3(kBinThreads), 0, s,
                     reinterpret_cast<const float4*>(w), count / 4, ws);
  return hipGetLastError();
}

hipError_t launch_gamma_fold(const unsigned long long* ws, int64_t count, float* gamma, hipStream_t s) {
  hipLaunchKernelGGL(k_gamma_fold, dim3(1), dim3(kBins), 0, s, ws, (unsigned long long)count, gamma);
  return hipGetLastError();
}

hipError_t launch_ternarize_pack(const float* w, int64_t n, int64_t k, const float* gamma, uint8_t* packed,
                                 hipStream_t s, int64_t glu_f) {
  const int64_t n_pad = (n + kTileRows - 1) / kTileRows * kTileRows;
  const int64_t threads = n_pad * (k / 4);
  const int64_t blocks = (threads + kPackThreads * kPackIter - 1) / (kPackThreads * kPackIter);
  if (!grid_fits(blocks, kPackThreads)) return kErrGridTooLarge;
  hipLaunchKernelGGL(k_ternarize_pack, dim3((unsigned)blocks), dim3(kPackThreads), 0, s,
                     reinterpret_cast<const float4*>(w), n, k, gamma, reinterpret_cast<uint32_t*>(packed), glu_f);
  return hipGetLastError();
}

hipError_t launch_pack_transposed(const uint8_t* packed, int64_t n, int64_t k, uint8_t* packed_t, hipStream_t s) {
  const int64_t blocks = (n / 64) * (k / 64);
  if (!grid_fits(blocks, 256)) return kErrGridTooLarge;
  hipLaunchKernelGGL(k_pack_transposed, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(packed), n, k, reinterpret_cast<uint32_t*>(packed_t));
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* q, hipStream_t s) {
  const int64_t threads = n * (k / kTileCols);
  const int64_t blocks = (threads + kPackThreads - 1) / kPackThreads;
  if (!grid_fits(blocks, kPackThreads)) return kErrGridTooLarge;
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)blocks), dim3(kPackThreads), 0, s,
                     reinterpret_cast<const uint4*>(packed), n, k, q);
  return hipGetLastError();
}

}  // namespace bl
