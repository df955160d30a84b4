// Straight-through backward of the BitLinear: input and weight gradients.
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
//   * a workgroup (4 waves along the rows of q^T) owns 128 rows x 64 tokens;
//     each wave 32 rows x 64 tokens = 2 x 4 MFMA tiles;
//   * each step covers 256 columns j: a wave loads its 32 rows' packed bytes
//     into registers (1 KiB per 16 rows: lane (r, s) holds row r of column
//     tile s, 64 trits), and MFMA (f, h) takes, per lane, the 8 trits of bytes
//     8h..8h+7 of field f (columns 64 s + 16 f + 8 h + e) -- eight MFMAs per
//     step.  The trits become bf16 with two v_perm lookups per 2 values, once
//     per row block, reused for the 4 token blocks;
//   * dy's tile (64 tokens x 256 columns x 2 bytes) is copied to LDS by DMA,
//     double-buffered; 16-byte chunk c of token row r is stored at chunk
//     c ^ lds_row_key(r), so the B reads of 16 tokens are free of bank
//     conflicts.
// Tails: rows of q^T past k and tokens past m are never stored; columns past
// n read as zero gradient (and the trits there are multiplied by zero).
//
// The weight gradient dw[j][t] = sum_i alpha_i dy[i][j] xq[i][t] / 127
// contracts over the tokens, the row index of both inputs, so a preparation
// kernel first writes them token-contiguous into the caller's workspace:
// a = alpha_i * dy[i][j] (a product of two bf16 values: 16 significant bits,
// exact in fp32) split into a_hi = bf16(a) and a_lo = a - a_hi (at most 8
// significant bits: exact in bf16), transposed to [n][m_pad]; and xq
// converted to bf16 (exact) and transposed to [k][m_pad]; tokens past m are
// zero.  k_bwd_w then runs two bf16 MFMAs per tile pair (a_hi and a_lo with
// the same xq), so every product is exact and only the fp32 accumulation
// order differs from the exact sum; the sum is divided by 127 at the end.
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
  // (i % 32) ^ lds_row_key(row)
  const int dma_row0 = wave * kXDma * 2 + (lane >> 5);
  auto load_x = [&](int s, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXDma; ++j) {
      const int row = dma_row0 + 2 * j;
      const int c = (lane & 31) ^ lds_row_key(row);
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
    // token row tb*16 + col; chunk 8*sub + 2*f + h stored at that ^ key
    const uint4* xt = xbuf + col * kChunks;
    const int key = lds_row_key(col);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 b[kTB];
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) b[tb] = xt[tb * 16 * kChunks + ((8 * sub + 2 * f + h) ^ key)];
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
      // one field at a time: keeps the live operand registers (and so the
      // unrolled step pair) within the register file
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // two distinct LDS buffers named at compile time in an unrolled step pair:
  // the compiler then knows the DMA into one cannot touch the reads of the
  // other and does not wait for it before reading
  auto step = [&](int s, const uint4* rd, uint4* wr) __attribute__((always_inline)) {
    load_w(s + 1, w_next);
    load_x(s + 1, wr);
    compute(rd);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA into wr has landed
    __syncthreads();                // ... and every other wave's, and nobody reads rd any more
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) w_cur[rb] = w_next[rb];
  };
  int s = 0;
  for (; s + 2 < steps; s += 2) {
    step(s, xs0, xs1);
    step(s + 1, xs1, xs0);
  }
  if (s + 1 < steps) {
    step(s, xs0, xs1);
    compute(xs1);
  } else {
    compute(xs0);
  }

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

constexpr int kPrepTile = 64;

// One 64 x 64 block of the workspace per workgroup.  Blocks [0, nb) take
// gradient columns j (a_hi and a_lo rows), the rest the activation columns t.
__global__ __launch_bounds__(256) void k_bwd_w_prep(const uint16_t* __restrict__ dy, const int8_t* __restrict__ xq,
                                                    const float* __restrict__ alpha, int64_t m, int64_t n, int64_t k,
                                                    int64_t m_pad, uint16_t* __restrict__ a_hi,
                                                    uint16_t* __restrict__ a_lo, uint16_t* __restrict__ x_t) {
  __shared__ uint16_t hi_s[kPrepTile][kPrepTile + 2];
  __shared__ uint16_t lo_s[kPrepTile][kPrepTile + 2];
  const int tid = threadIdx.x;
  const int64_t token_blocks = m_pad / kPrepTile;
  const int64_t nb = (n / kPrepTile) * token_blocks;
  const bool grad = (int64_t)blockIdx.x < nb;
  const int64_t b = grad ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - nb;
  const int64_t c0 = (b / token_blocks) * kPrepTile;  // first column (j or t)
  const int64_t i0 = (b % token_blocks) * kPrepTile;  // first token
  // read: thread -> (token row, 16 consecutive columns), 4 rows per pass
  const int rr = tid >> 2, cc = 16 * (tid & 3);
  const int64_t i = i0 + rr;
  if (grad) {
    const float al = i < m ? alpha[i] : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      uint16_t h = 0, l = 0;
      if (i < m) {
        const float a = __uint_as_float((uint32_t)dy[i * n + c0 + cc + e] << 16) * al;  // exact
        h = f32_to_bf16_rne(a);
        l = (uint16_t)(__float_as_uint(a - __uint_as_float((uint32_t)h << 16)) >> 16);  // exact
      }
      hi_s[rr][cc + e] = h;
      lo_s[rr][cc + e] = l;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = i < m ? (float)xq[i * k + c0 + cc + e] : 0.0f;
      hi_s[rr][cc + e] = (uint16_t)(__float_as_uint(v) >> 16);  // |v| <= 128: exact in bf16
    }
  }
  __syncthreads();
  // write: thread -> (column, 16 consecutive tokens) of the transposed block
  const int wc = tid >> 2, wt = 16 * (tid & 3);
  uint16_t* dst = grad ? a_hi : x_t;
  uint32_t h8[8], l8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h8[e] = (uint32_t)hi_s[wt + 2 * e][wc] | ((uint32_t)hi_s[wt + 2 * e + 1][wc] << 16);
    l8[e] = (uint32_t)lo_s[wt + 2 * e][wc] | ((uint32_t)lo_s[wt + 2 * e + 1][wc] << 16);
  }
  const int64_t off = (c0 + wc) * m_pad + i0 + wt;
  *reinterpret_cast<uint4*>(dst + off) = make_uint4(h8[0], h8[1], h8[2], h8[3]);
  *reinterpret_cast<uint4*>(dst + off + 8) = make_uint4(h8[4], h8[5], h8[6], h8[7]);
  if (grad) {
    *reinterpret_cast<uint4*>(a_lo + off) = make_uint4(l8[0], l8[1], l8[2], l8[3]);
    *reinterpret_cast<uint4*>(a_lo + off + 8) = make_uint4(l8[4], l8[5], l8[6], l8[7]);
  }
}

constexpr int kWStep = 32;           // tokens per step (one MFMA)
constexpr int kWRow = kWStep / 8;  // 16-byte chunks per LDS row (64 bytes, unpadded)
// LDS slot of chunk c of operand row r: c ^ ((r >> 1) & 3) within the row.
// Measured on gfx950 for this kernel's reads (lane l reads chunk l / 16 of
// row l % 16 of a 16-row block): no bank conflicts, against 2.3 conflict
// cycles per ds_read_b128 with the rows padded to 80 bytes.
__device__ __forceinline__ int wslot(int r, int c) { return r * kWRow + (c ^ ((r >> 1) & 3)); }

// dw = (a_hi + a_lo) x_t^T / 127 over the token-contiguous workspace.  A
// workgroup (2 x 2 waves) owns 128 rows j x 128 columns t; a wave 64 x 64 =
// 4 x 4 tiles, two MFMAs per tile per step (a_hi, a_lo).  The three operand
// tiles (128 x 32 tokens each) go through LDS via registers, double-buffered.
__global__ __launch_bounds__(256, 2) void k_bwd_w(const uint16_t* __restrict__ a_hi, const uint16_t* __restrict__ a_lo,
                                                  const uint16_t* __restrict__ x_t, int64_t m_pad, int64_t n,
                                                  int64_t k, int64_t blocks_t, float* __restrict__ dw) {
  __shared__ uint4 sh[2][3][128 * kWRow];  // [buffer][a_hi, a_lo, x_t][wslot(row, chunk)]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave >> 1, wt = wave & 1;
  const int sub = lane >> 4, col = lane & 15;
  // the XCD-grouped tile order of the forward GEMM: an XCD's resident
  // workgroups cover about 8 j-blocks x 8 t-blocks and share their operand
  // slices in its L2 at each step
  constexpr int64_t kGroupJ = 8;
  const int64_t tiles = (int64_t)gridDim.x;
  const int64_t blocks_j = tiles / blocks_t;
  const int64_t full = tiles / kXcds * kXcds;
  const int64_t tt = (int64_t)blockIdx.x >= full
                         ? (int64_t)blockIdx.x
                         : (int64_t)(blockIdx.x % kXcds) * (tiles / kXcds) + blockIdx.x / kXcds;
  const int64_t group = tt / (kGroupJ * blocks_t);
  const int64_t first_j = group * kGroupJ;
  const int64_t group_j = min(kGroupJ, blocks_j - first_j);
  const int64_t local = tt - group * kGroupJ * blocks_t;
  const int64_t j0 = (first_j + local % group_j) * 128;
  const int64_t t0 = (local / group_j) * 128;
  const int steps = (int)(m_pad / kWStep);
  // staging: each operand tile is 128 rows x 64 bytes = 512 pieces of 16 bytes; thread -> pieces tid, tid + 256
  const int pr0 = tid >> 2, pc = tid & 3;
  const int rows_j = (int)min((int64_t)128, n - j0), rows_t = (int)min((int64_t)128, k - t0);
  auto load = [&](int s, uint4 (&v)[3][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = pr0 + 64 * h;
      const int64_t tok = (int64_t)s * kWStep + 8 * pc;
      v[0][h] = r < rows_j ? *reinterpret_cast<const uint4*>(a_hi + (j0 + r) * m_pad + tok) : make_uint4(0, 0, 0, 0);
      v[1][h] = r < rows_j ? *reinterpret_cast<const uint4*>(a_lo + (j0 + r) * m_pad + tok) : make_uint4(0, 0, 0, 0);
      v[2][h] = r < rows_t ? *reinterpret_cast<const uint4*>(x_t + (t0 + r) * m_pad + tok) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf, const uint4 (&v)[3][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int o = 0; o < 3; ++o)
#pragma unroll
      for (int h = 0; h < 2; ++h) sh[buf][o][wslot(pr0 + 64 * h, pc)] = v[o][h];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 v[3][2];
  load(0, v);
  store(0, v);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < steps) load(s + 1, v);
    // operands: lane (row col, token group sub) -> 8 tokens 8 sub..8 sub + 7 of its row
    uint4 bt[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) bt[b] = sh[buf][2][wslot(wt * 64 + b * 16 + col, sub)];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int r = wslot(wj * 64 + a * 16 + col, sub);
      const uint4 ah = sh[buf][0][r], al = sh[buf][1][r];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[a][b] = mfma_bf16(ah, bt[b], acc[a][b]);
        acc[a][b] = mfma_bf16(al, bt[b], acc[a][b]);
      }
    }
    if (s + 1 < steps) store(buf ^ 1, v);
    __syncthreads();
  }
  // lane holds rows 4 sub..4 sub + 3 (j) of column col (t) of each tile
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t t = t0 + wt * 64 + b * 16 + col;
      const int64_t j = j0 + wj * 64 + a * 16 + 4 * sub;
      if (t >= k) continue;
      const float vals[4] = {acc[a][b].x, acc[a][b].y, acc[a][b].z, acc[a][b].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i < n) dw[(j + i) * k + t] = vals[i] / 127.0f;
    }
}

}  // namespace

hipError_t launch_backward_x(const uint8_t* packed_t, const float* gamma, const uint16_t* dy, int64_t m, int64_t n,
                             int64_t k, float* dx, hipStream_t s) {
  // 128 rows of q^T x 64 tokens per workgroup (measured faster than 256 x 64)
  const int64_t blocks_n = (k + 127) / 128, blocks = blocks_n * ((m + 63) / 64);
  if (!grid_fits(blocks, 256)) return kErrGridTooLarge;
  hipLaunchKernelGGL((k_bwd_x<4, 2>), dim3((unsigned)blocks), dim3(256), 0, s, packed_t, gamma, dy, m, n, k,
                     blocks_n, dx);
  return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  if (!grid_fits(blocks, 256)) return kErrGridTooLarge;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, count);
  return hipGetLastError();
}

size_t backward_w_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const int64_t m_pad = (m + 63) / 64 * 64;
  return (size_t)(2 * n + k) * (size_t)m_pad * 2;
}

hipError_t launch_backward_w(const uint16_t* dy, const int8_t* xq, const float* alpha, int64_t m, int64_t n, int64_t k,
                             float* dw, void* workspace, hipStream_t s) {
  const int64_t m_pad = (m + 63) / 64 * 64;
  uint16_t* a_hi = reinterpret_cast<uint16_t*>(workspace);
  uint16_t* a_lo = a_hi + n * m_pad;
  uint16_t* x_t = a_lo + n * m_pad;
  const int64_t prep_blocks = (n / kPrepTile + k / kPrepTile) * (m_pad / kPrepTile);
  const int64_t blocks_t = (k + 127) / 128, blocks = ((n + 127) / 128) * blocks_t;
  if (!grid_fits(prep_blocks, 256) || !grid_fits(blocks, 256)) return kErrGridTooLarge;
  hipLaunchKernelGGL(k_bwd_w_prep, dim3((unsigned)prep_blocks), dim3(256), 0, s, dy, xq, alpha, m, n, k, m_pad, a_hi,
                     a_lo, x_t);
  hipLaunchKernelGGL(k_bwd_w, dim3((unsigned)blocks), dim3(256), 0, s, a_hi, a_lo, x_t, m_pad, n, k, blocks_t, dw);
  return hipGetLastError();
}

}  // namespace bl
