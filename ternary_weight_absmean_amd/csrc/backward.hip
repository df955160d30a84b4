// Straight-through backward of the BitLinear: the input gradient.
//
// bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution", section
// "Training Dynamics: The Straight-Through Estimator": the backward pass
// treats the rounding step as the identity, so the gradient passes through
// the quantized weights.  With the dequantized weights gamma * q, the input
// gradient is dx = gamma * dy q: a product that contracts over the n output
// rows of q, with a bf16 gradient dy and an fp32 result.
//
// k_bwd_x is the GEMM dx[i][t] = gamma * sum_j dy[i][j] q^T[t][j], reading
// q^T packed in the same tiled 2-bit layout as q (rows t, columns j), so that
// it has the shape of the forward product with bf16 activations:
//   * the matrix cores run v_mfma_f32_16x16x32_bf16: A = 16 rows of q^T as bf16
//     values -1, 0, +1 (exact), B = 16 tokens of dy, fp32 accumulation;
//   * a workgroup (4 waves along the rows of q^T) owns 256 rows x 64 tokens;
//     each wave 64 rows x 64 tokens = 4 x 4 MFMA tiles;
//   * each step covers 256 columns j: a wave loads its 64 rows' packed bytes
//     into registers (1 KiB per 16 rows: lane (r, s) holds row r of column
//     tile s, 64 trits), and MFMA (f, h) takes, per lane, the 8 trits of bytes
//     8h..8h+7 of field f (columns 64 s + 16 f + 8 h + e) -- eight MFMAs per
//     step.  The trits become bf16 with two v_perm lookups per 2 values, once
//     per row block, reused for the 4 token blocks;
//   * dy's tile (64 tokens x 256 columns x 2 bytes) is copied to LDS by DMA,
//     double-buffered; 16-byte chunk c of token row r is stored at chunk
//     c ^ (r % 16), so the 16 tokens of a B read fall in distinct banks.
// Tails: rows of q^T past k and tokens past m are never stored; columns past
// n read as zero gradient (and the trits there are multiplied by zero).
#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStepK = 256;                 // columns j per step
constexpr int kChunks = kStepK * 2 / 16;    // 16-byte chunks of a token row per step (bf16)
constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mfma_bf16(const uint4& a, const uint4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Four 2-bit codes (one per byte of cw, values 0..2) -> four bf16 values
// q = code - 1 in two dwords: byte selectors [c, c + 4] pick the low and high
// byte of the bf16 pattern from two constant words (0xBF80, 0x0000, 0x3F80).
__device__ __forceinline__ uint2 codes_to_bf16(uint32_t cw) {
  constexpr uint32_t kLo = 0x00800080u;  // low bytes for codes 0, 1, 2
  constexpr uint32_t kHi = 0x003F00BFu;  // high bytes
  const uint32_t sel0 = __builtin_amdgcn_perm(cw, cw, 0x01010000u) + 0x04000400u;
  const uint32_t sel1 = __builtin_amdgcn_perm(cw, cw, 0x03030202u) + 0x04000400u;
  return make_uint2(__builtin_amdgcn_perm(kHi, kLo, sel0), __builtin_amdgcn_perm(kHi, kLo, sel1));
}

template <int kTB, int kRB>
__global__ __launch_bounds__(256, 2) void k_bwd_x(const uint8_t* __restrict__ packed_t,
                                                  const float* __restrict__ gamma_ptr,
                                                  const uint16_t* __restrict__ dy, int64_t m, int64_t n, int64_t k,
                                                  int64_t blocks_n, float* __restrict__ dx) {
  constexpr int kBM = 16 * kTB;                        // tokens per workgroup
  constexpr int kWN = 16 * kRB;                        // rows of q^T per wave
  constexpr int kBN = kWaves * kWN;                    // rows of q^T per workgroup
  constexpr int kXDma = kBM * kChunks * 16 / 1024 / kWaves;  // 1 KiB DMA loads per wave per step
  __shared__ uint4 xs0[kBM * kChunks];
  __shared__ uint4 xs1[kBM * kChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane >> 4;
  const int col = lane & 15;

  // the XCD-grouped tile order of the forward GEMM
  constexpr int64_t kGroupN = 8;
  const int64_t tiles = (int64_t)gridDim.x;
  const int64_t blocks_m = tiles / blocks_n;
  const int64_t full = tiles / kXcds * kXcds;
  const int64_t t = (int64_t)blockIdx.x >= full
                        ? (int64_t)blockIdx.x
                        : (int64_t)(blockIdx.x % kXcds) * (tiles / kXcds) + blockIdx.x / kXcds;
  const int64_t group = t / (kGroupN * blocks_m);
  const int64_t first_bn = group * kGroupN;
  const int64_t group_n = min(kGroupN, blocks_n - first_bn);
  const int64_t local = t - group * kGroupN * blocks_m;
  const int64_t r0 = (first_bn + local % group_n) * kBN;  // first row of q^T
  const int64_t m0 = (local / group_n) * kBM;             // first token
  const int kt_count = (int)(n / kTileCols);              // column tiles of q^T
  const int64_t row_tiles = k / kTileRows;                // row tiles of q^T
  const int steps = (kt_count + 3) / 4;
  const int full_steps = kt_count / 4;
  const int64_t rt0 = r0 / kTileRows;
  const int tiles_here = (int)min((int64_t)(kBN / kTileRows), row_tiles - rt0);
  const int tokens_here = (int)min((int64_t)kBM, m - m0);
  const uint32_t row_bytes = (uint32_t)(2 * n);

  const __amdgpu_buffer_rsrc_t wrsrc =
      buffer_rsrc(packed_t + rt0 * kt_count * kTileBytes, (uint32_t)(tiles_here * kt_count * kTileBytes));
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(dy + m0 * n, (uint32_t)tokens_here * row_bytes);

  // DMA: lane i of a 1 KiB load writes LDS bytes 16i.. of it = token row
  // 2 * load + i / 32, stored chunk i % 32, which holds source chunk
  // (i % 32) ^ (row % 16)
  const int dma_row0 = wave * kXDma * 2 + (lane >> 5);
  auto load_x = [&](int s, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXDma; ++j) {
      const int row = dma_row0 + 2 * j;
      const int c = (lane & 31) ^ (row & 15);
      const uint32_t col_byte = (uint32_t)(s * kStepK * 2 + 16 * c);
      const uint32_t off = (s < full_steps || col_byte < row_bytes) ? (uint32_t)row * row_bytes + col_byte
                                                                     : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrsrc, (__attribute__((address_space(3))) void*)(dst + (wave * kXDma + j) * 64), 16, off, 0, 0, 0);
    }
  };
  const uint32_t w_off0 = (uint32_t)(wave * kRB * kt_count) * kTileBytes + (uint32_t)col * 16u;
  auto load_w = [&](int s, uint4* r) __attribute__((always_inline)) {
    const uint32_t kt = (uint32_t)min(4 * s + sub, kt_count - 1);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      r[rb] = buffer_load16(wrsrc, w_off0 + ((uint32_t)(rb * kt_count) + kt) * kTileBytes);
  };

  f32x4 acc[kRB][kTB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) acc[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 w_cur[kRB], w_next[kRB];
  load_w(0, w_cur);
  load_x(0, xs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto compute = [&](const uint4* xbuf) __attribute__((always_inline)) {
    // token row tb*16 + col; chunk 8*sub + 2*f + h stored at that ^ col
    const uint4* xt = xbuf + col * kChunks;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 b[kTB];
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) b[tb] = xt[tb * 16 * kChunks + ((8 * sub + 2 * f + h) ^ col)];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const uint32_t c0 = ((h ? w_cur[rb].z : w_cur[rb].x) >> (2 * f)) & 0x03030303u;
          const uint32_t c1 = ((h ? w_cur[rb].w : w_cur[rb].y) >> (2 * f)) & 0x03030303u;
          const uint2 lo = codes_to_bf16(c0), hi = codes_to_bf16(c1);
          const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int tb = 0; tb < kTB; ++tb) acc[rb][tb] = mfma_bf16(a, b[tb], acc[rb][tb]);
        }
      }
    }
  };

  for (int s = 0; s + 1 < steps; ++s) {
    uint4* rd = (s & 1) ? xs1 : xs0;
    uint4* wr = (s & 1) ? xs0 : xs1;
    load_w(s + 1, w_next);
    load_x(s + 1, wr);
    compute(rd);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA into wr has landed
    __syncthreads();                // ... and every other wave's, and nobody reads rd any more
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) w_cur[rb] = w_next[rb];
  }
  compute(((steps - 1) & 1) ? xs1 : xs0);

  const float gamma = *gamma_ptr;
  const bool vec_ok = ((uintptr_t)dx % 16) == 0;
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
    const int64_t tok = m0 + tb * 16 + col;
    if (tok >= m) continue;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int64_t row0 = r0 + wave * kWN + rb * 16 + 4 * sub;  // four consecutive t of this token
      if (row0 >= k) continue;                                    // k % 64 == 0: all four or none
      const f32x4 v = acc[rb][tb];
      float* out = dx + tok * k + row0;
      if (vec_ok) {
        *reinterpret_cast<float4*>(out) = make_float4(v.x * gamma, v.y * gamma, v.z * gamma, v.w * gamma);
      } else {
        out[0] = v.x * gamma;
        out[1] = v.y * gamma;
        out[2] = v.z * gamma;
        out[3] = v.w * gamma;
      }
    }
  }
}

}  // namespace

hipError_t launch_backward_x(const uint8_t* packed_t, const float* gamma, const uint16_t* dy, int64_t m, int64_t n,
                             int64_t k, float* dx, hipStream_t s) {
  // 256 rows of q^T x 64 tokens per workgroup
  const int64_t blocks_n = (k + 255) / 256, blocks = blocks_n * ((m + 63) / 64);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_bwd_x<4, 4>), dim3((unsigned)blocks), dim3(256), 0, s, packed_t, gamma, dy, m, n, k,
                     blocks_n, dx);
  return hipGetLastError();
}

}  // namespace bl
