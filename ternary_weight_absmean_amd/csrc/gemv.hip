// Decode product for BitLinear W1.58A8 (m <= 16 tokens): packed ternary W x int8 x.
//
// deepmox.com chapter 8, "A low-bit model is a whole-stack design": decode
// time goes to moving the weights; the GPU path keeps them packed at four
// trits per byte, moves them on chip, unpacks and computes with the 8-bit
// activations.  bako.co, "The BitLinear Layer and AbsMean Quantization": the
// ternary product is integer add/subtract; here the unpacked trits feed the
// int8 matrix cores, which perform exactly those integer sums (a trit of 0
// contributes 0, +-1 adds or subtracts x).
//
// The kernel is bound by HBM: every packed byte is read once, 0.25 byte per
// weight, and nothing else is large.  Work decomposition:
//   * one workgroup (4 waves) per 16-row tile of W and per 16-token block;
//   * the waves split K: wave w takes 1 KiB groups w, w+4, ... (a group is
//     four consecutive 16x64 tiles, contiguous in the packed layout), so each
//     wave-wide 128-bit load reads 1 KiB of HBM with no gaps;
//   * lane l holds row l%16 of tile (4*group + l/16): 16 bytes = 64 trits;
//     field f of those bytes is columns 16f..16f+15 of that tile, turned into
//     signed int8 with one v_perm per 4 trits, and multiplied with the same 16
//     activation bytes (one 128-bit load) in v_mfma_i32_16x16x64_i8, whose
//     B column l%16 is token l%16 of the block;
//   * the waves' 16x16 int32 partial sums are added in LDS (integer, so the
//     order does not matter) and wave 0 applies the epilogue
//     y = bf16(acc * gamma * alpha / 127).
// Loads for a batch of kGroupsPerBatch groups are issued before any of them
// is consumed, keeping several KiB per wave in flight.
#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = kGemvWaves * 64;
constexpr int kGroupsPerBatch = 4;

__global__ __launch_bounds__(kGemvThreads) void k_gemv(const uint4* __restrict__ packed,
                                                       const float* __restrict__ gamma_ptr,
                                                       const int8_t* __restrict__ xq,
                                                       const float* __restrict__ alpha, int64_t m, int64_t n,
                                                       int64_t k, int32_t* __restrict__ acc_out,
                                                       uint16_t* __restrict__ y_out) {
  __shared__ v4i partial[kGemvWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row_tile = blockIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.y * 16;
  const int64_t kt_count = k / kTileCols;
  const int64_t groups = (kt_count + 3) / 4;
  const int sub = lane >> 4;   // tile within a group
  const int col = lane & 15;   // A row (weight row) and B column (token)
  const int64_t tok = tok0 + col;
  const bool has_tok = tok < m;
  const uint4* wbase = packed + row_tile * kt_count * (kTileBytes / 16);
  const uint4* xrow = reinterpret_cast<const uint4*>(xq + (has_tok ? tok : 0) * k);

  v4i acc = {0, 0, 0, 0};
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t g0 = wave; g0 < groups; g0 += (int64_t)kGemvWaves * kGroupsPerBatch) {
    uint4 a[kGroupsPerBatch];
    uint4 b[kGroupsPerBatch][4];
#pragma unroll
    for (int u = 0; u < kGroupsPerBatch; ++u) {
      const int64_t g = g0 + (int64_t)u * kGemvWaves;
      const int64_t kt = 4 * g + sub;
      const bool valid = g < groups && kt < kt_count;
      a[u] = zero;
      if (valid) a[u] = wbase[4 * g * 16 + lane];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        b[u][f] = zero;
        if (valid && has_tok) b[u][f] = xrow[kt * 4 + f];
      }
    }
#pragma unroll
    for (int u = 0; u < kGroupsPerBatch; ++u) {
#pragma unroll
      for (int f = 0; f < 4; ++f) acc = mfma_16x16x64(unpack_field(a[u], f), as_v4i(b[u][f]), acc);
    }
  }
  partial[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kGemvWaves; ++w) {
    v4i p = partial[w][lane];
    acc.x += p.x;
    acc.y += p.y;
    acc.z += p.z;
    acc.w += p.w;
  }
  if (!has_tok) return;
  // lane holds rows 4*(lane/16) + i of the tile for token `tok`
  const float scale = (*gamma_ptr * alpha[tok]) / 127.0f;
  const int64_t row0 = row_tile * kTileRows + 4 * sub;
  const int vals[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + i;
    if (row < n) {
      if (acc_out) acc_out[tok * n + row] = vals[i];
      if (y_out) y_out[tok * n + row] = f32_to_bf16_rne((float)vals[i] * scale);
    }
  }
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                       int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s) {
  if ((m + 15) / 16 > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + kTileRows - 1) / kTileRows), (unsigned)((m + 15) / 16));
  hipLaunchKernelGGL(k_gemv, grid, dim3(kGemvThreads), 0, s, reinterpret_cast<const uint4*>(packed), gamma, xq,
                     alpha, m, n, k, acc, y);
  return hipGetLastError();
}

// Until the LDS-tiled GEMM lands, larger m runs the same kernel over
// 16-token blocks (grid.y).
hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                       int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s) {
  return launch_gemv(packed, gamma, xq, alpha, m, n, k, acc, y, s);
}

}  // namespace bl
