// Decode products for BitLinear W1.58A8 (up to 64 tokens): packed ternary W x int8 x.
//
// deepmox.com chapter 8, "A low-bit model is a whole-stack design": decode
// time goes to moving the weights; the GPU path keeps them packed at four
// trits per byte, moves them on chip, unpacks them and computes with the
// 8-bit activations.  bako.co, "The BitLinear Layer and AbsMean Quantization":
// the ternary product is integer add/subtract; here the unpacked values feed
// the int8 matrix cores, which perform exactly those integer sums.
//
// The kernels are bound by HBM (or, for the small matrices of a 2B-shaped
// model, by launch latency): every packed byte is read once (0.25 byte per
// weight) and nothing else is large.  Shared decomposition:
//   * a workgroup owns one or more 16-row tiles of W and a block of up to 16
//     tokens;
//   * its waves split K by 1 KiB groups (four consecutive 16x64 tiles,
//     contiguous in the packed layout), so each wave-wide 128-bit load reads
//     1 KiB of HBM with no gaps;
//   * lane l holds row l%16 of tile (4*group + l/16): 16 bytes = 64 trits.
//     Field f (bits 2f..2f+1 of each byte) is columns 16f..16f+15 of the
//     tile, multiplied in v_mfma_i32_16x16x64_i8 with the same 16 activation
//     bytes; B column l%16 is token l%16 of the block;
//   * the waves' 16x16 int32 partial sums are added in LDS (integer,
//     order-free) and the epilogue writes y = bf16(acc * gamma * alpha / 127).
//
// Kernels:
//   k_bitlinear_m1     one token, quantization fused; each wave quantizes only
//                      the columns it multiplies (single-token decode)
//   k_bitlinear_tok    2..16 tokens (m * k small), one wave per token
//                      quantizes the block, quantization fused
//   k_bitlinear_fused  a few tokens of rows past 8192 (m * k small), or one
//                      of rows past 28672, block quantization fused
//   k_gemv_lds         2..64 tokens, int8 activations given, staged in LDS
//                      (16 tokens per workgroup, or 64 on large matrices)
//   k_gemv_ring        2..16 tokens on rows of 8192 and more, int8
//                      activations given, streamed through an LDS ring by DMA
//   k_gemv_direct      one token, int8 activations given
// The fused kernels feed the MFMA with the raw codes c = q + 1 and correct
// with the token's activation sum: sum q*x = sum c*x - sum x.  Masking a
// byte with 0x03, 0x0C, 0x30 gives 1, 4 and 16 times fields 0, 1, 2, and
// (b >> 2) & 0x30 gives 16 times field 3, so four accumulators hold c*x
// scaled by 1, 4, 16, 16 and are divided exactly at the end (20 VALU ops per
// 1 KiB group instead of 44 for a signed table lookup).  The others convert
// codes to signed trits with v_perm.
#include <utility>

#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kWaves = 4;
constexpr int kGroupsPerBatch = 4;
constexpr int kLdsBudget = 163840;  // LDS per workgroup (and per CU) on gfx950
constexpr int kLdsRowPad = 16;          // row stride k + 16 bytes spreads the 16 token rows over the banks

__device__ __forceinline__ v4i mask4(const uint4& a, uint32_t mask, int shift) {
  v4i r;
  r.x = (int)((a.x >> shift) & mask);
  r.y = (int)((a.y >> shift) & mask);
  r.z = (int)((a.z >> shift) & mask);
  r.w = (int)((a.w >> shift) & mask);
  return r;
}

// Gated outputs h[tok][col0 .. col0 + 3] = bf16(relu(g)^2 * u) from the exact
// products of four gate rows (g) and the four matching up rows (u).
__device__ __forceinline__ void store_glu_tile(const v4i& g, const v4i& u, int64_t col0, int64_t tok, int64_t f,
                                               float scale, uint16_t* __restrict__ h_out) {
  const float h[4] = {glu_value(g.x, u.x, scale), glu_value(g.y, u.y, scale), glu_value(g.z, u.z, scale),
                      glu_value(g.w, u.w, scale)};
  uint16_t* hp = h_out + tok * f + col0;
  if (col0 + 3 < f && ((uintptr_t)hp & 7) == 0) {
    *reinterpret_cast<uint2*>(hp) = make_uint2(f32x2_to_bf16x2(h[0], h[1]), f32x2_to_bf16x2(h[2], h[3]));
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (col0 + i < f) hp[i] = f32_to_bf16_rne(h[i]);
}

// Partial reduction of `v` over the `g = min(tpr, 64)` lanes of a token row
// group inside one wave; lanes with (tid % g) == 0 then write the group's value
// to scratch[tid / g].  A row's value is the max/sum of its tpr/g entries.
template <bool kMax>
__device__ __forceinline__ void group_partial(int v, int tpr, int* scratch) {
  const int g = tpr < 64 ? tpr : 64;
  v = lane_group_reduce<kMax>(v, g);
  if ((threadIdx.x % g) == 0) scratch[threadIdx.x / g] = v;
}

template <bool kMax>
__device__ __forceinline__ int row_total(int row, int tpr, const int* scratch) {
  const int g = tpr < 64 ? tpr : 64;
  const int per_row = tpr / g;  // 1..8 entries per row
  int r = scratch[row * per_row];
  for (int i = 1; i < per_row; ++i) r = kMax ? max(r, scratch[row * per_row + i]) : r + scratch[row * per_row + i];
  return r;
}


// Whole BitLinear for a block of up to 16 tokens: per-token absmax int8
// quantization (same arithmetic as bl_quant_act) into LDS, then the codes x
// int8 product with four scaled accumulators, then the bf16 rescale.
// Latency-ordered: the activation loads and the first weight loads are issued
// first; the absmax and the activation sum each take one LDS round.  A
// workgroup handles kRT consecutive 16-row tiles, so the quantization is
// amortized over them; the weight loads of all its tiles form one stream,
// prefetched a batch ahead, with one buffer resource per tile (reads past a
// tile, or of a tile past n, return zero codes).
// kGlu (kRT even): gate+up matrix with alternating gate/up row tiles; wave w
// gates the tile pairs (2p, 2p + 1) with p = w, w + kW, ... into y_out ([m][n / 2]).
template <int kRT, int kW, bool kGlu = false>
__global__ __launch_bounds__(kW * 64) void k_bitlinear_fused(const uint4* __restrict__ packed,
                                                              const float* __restrict__ gamma_ptr,
                                                              const uint4* __restrict__ x, float* __restrict__ alpha,
                                                              int8_t* __restrict__ xq_out, int64_t m, int64_t n,
                                                              int64_t k, int32_t* __restrict__ acc_out,
                                                              uint16_t* __restrict__ y_out) {
  constexpr int kT = kW * 64;           // threads
  constexpr int kXC = kW >= 8 ? 8 : 4;  // bf16 chunks of 8 per thread held between the quantizer passes
  extern __shared__ uint4 xs_raw[];  // [rows][k + kLdsRowPad] int8 activations of this token block
  int8_t* xs = reinterpret_cast<int8_t*>(xs_raw);
  __shared__ v4i partial[kRT][kW][64];
  __shared__ int red_max[kT / 16];
  __shared__ int red_sum[kT / 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile0 = (int64_t)blockIdx.x * kRT;
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  const int tiles_here = (int)min((int64_t)kRT, row_tiles - tile0);
  const int64_t tok0 = (int64_t)blockIdx.y * 16;
  const int rows = (int)min((int64_t)16, m - tok0);
  const int kt_count = (int)(k / kTileCols);
  const int groups = (kt_count + 3) / 4;
  const int my_groups = (groups - wave + kW - 1) / kW;
  const int sub = lane >> 4;
  const int col = lane & 15;
  const bool first_block = blockIdx.x == 0;

  // ---- activation loads (first: loads retire in order), then the first weight batch
  int rp = 1;
  while (rp < rows) rp <<= 1;
  const int tpr = kT / rp;  // threads per token row
  const int my_row = tid / tpr;
  const int j0 = tid % tpr;
  const bool row_ok = my_row < rows;
  const int64_t k8 = k / 8;
  const int64_t ldx = k + kLdsRowPad;
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(x + tok0 * k8, (uint32_t)(rows * k8 * 16));
  const bool cached = (k8 + tpr - 1) / tpr <= kXC;
  uint4 xr[kXC];
  if (cached) {
#pragma unroll
    for (int c = 0; c < kXC; ++c) {
      const int64_t i = j0 + (int64_t)c * tpr;
      xr[c] = buffer_load16(xrsrc, row_ok && i < k8 ? (uint32_t)((my_row * k8 + i) * 16) : kOutOfRange);
    }
  }
  const uint32_t tile_bytes = (uint32_t)(kt_count * kTileBytes);
  auto tile_rsrc = [&](int rt) {
    return buffer_rsrc(packed + (tile0 + rt) * kt_count * (kTileBytes / 16), rt < tiles_here ? tile_bytes : 0u);
  };
  auto w_off = [&](int gi) { return (uint32_t)((wave + gi * kW) * 1024 + lane * 16); };
  uint4 a_cur[kGroupsPerBatch];
  {
    const __amdgpu_buffer_rsrc_t r0 = tile_rsrc(0);
#pragma unroll
    for (int u = 0; u < kGroupsPerBatch; ++u) a_cur[u] = buffer_load16_stream(r0, w_off(u));
  }
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  // keep these loads here, in flight while the activations are reduced
  __builtin_amdgcn_sched_barrier(0);

  // ---- quantize the token block into LDS
  // Longer rows are read twice, kBatchX chunks per thread at a time (loads
  // issued together; offsets past the row, or of rows past the block, read
  // as zero): one dependent load per chunk measured several times slower.
  constexpr int kBatchX = 8;
  auto load_batch = [&](int64_t i0, uint4 (&v)[kBatchX]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBatchX; ++u) {
      const int64_t i = i0 + (int64_t)u * tpr;
      v[u] = buffer_load16(xrsrc, i < k8 ? (uint32_t)((my_row * k8 + i) * 16) : kOutOfRange);
    }
  };
  u16x2 m2 = {0, 0};
  if (cached) {
#pragma unroll
    for (int c = 0; c < kXC; ++c) m2 = absmax_step(m2, xr[c]);
  } else {
    for (int64_t i0 = j0; i0 < k8; i0 += (int64_t)kBatchX * tpr) {
      uint4 v[kBatchX];
      load_batch(i0, v);
#pragma unroll
      for (int u = 0; u < kBatchX; ++u) m2 = absmax_step(m2, v[u]);
    }
  }
  group_partial<true>((int)max(m2.x, m2.y), tpr, red_max);
  __syncthreads();
  const float amax = __uint_as_float((uint32_t)row_total<true>(my_row, tpr, red_max) << 16);
  const float s = 127.0f / fmaxf(amax, 1e-5f);  // IEEE division, as in bl_quant_act
  int sum = 0;
  if (row_ok) {
    uint2* dst = reinterpret_cast<uint2*>(xs + (int64_t)my_row * ldx);
    uint2* gdst = (first_block && xq_out) ? reinterpret_cast<uint2*>(xq_out + (tok0 + my_row) * k) : nullptr;
    if (cached) {
#pragma unroll
      for (int c = 0; c < kXC; ++c) {
        const int64_t i = j0 + (int64_t)c * tpr;
        if (i < k8) {
          const uint2 q = act_codes8(xr[c], s, sum);
          dst[i] = q;
          if (gdst) gdst[i] = q;
        }
      }
    }
    if (j0 == 0 && first_block && alpha) alpha[tok0 + my_row] = amax;
  }
  if (!cached) {
    uint2* dst = reinterpret_cast<uint2*>(xs + (int64_t)my_row * ldx);
    uint2* gdst = (first_block && xq_out && row_ok) ? reinterpret_cast<uint2*>(xq_out + (tok0 + my_row) * k) : nullptr;
    for (int64_t i0 = j0; i0 < k8; i0 += (int64_t)kBatchX * tpr) {
      uint4 v[kBatchX];
      load_batch(i0, v);
#pragma unroll
      for (int u = 0; u < kBatchX; ++u) {
        const int64_t i = i0 + (int64_t)u * tpr;
        if (row_ok && i < k8) {
          const uint2 q = act_codes8(v[u], s, sum);
          dst[i] = q;
          if (gdst) gdst[i] = q;
        }
      }
    }
  }
  group_partial<false>(sum, tpr, red_sum);
  __syncthreads();

  // ---- weight stream: codes times activations, four scaled accumulators per tile
  const bool has_tok = col < rows;
  const int8_t* xrow = xs + (int64_t)(has_tok ? col : 0) * ldx;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    v4i acc1 = {0, 0, 0, 0}, acc4 = acc1, acc16a = acc1, acc16b = acc1;
    const __amdgpu_buffer_rsrc_t cur_rsrc = tile_rsrc(rt);
    const __amdgpu_buffer_rsrc_t next_rsrc = tile_rsrc(rt + 1);  // empty past the last tile
    for (int gi = 0; gi < my_groups; gi += kGroupsPerBatch) {
      const bool same = gi + kGroupsPerBatch < my_groups;
      const int ngi = same ? gi + kGroupsPerBatch : 0;
      uint4 a_next[kGroupsPerBatch];
#pragma unroll
      for (int u = 0; u < kGroupsPerBatch; ++u)
        a_next[u] = buffer_load16_stream(same ? cur_rsrc : next_rsrc, w_off(ngi + u));
#pragma unroll
      for (int u = 0; u < kGroupsPerBatch; ++u) {
        // tiles past k carry zero codes, so any in-bounds activation bytes will do
        const int kt = min(4 * (wave + (gi + u) * kW) + sub, kt_count - 1);
        const uint4* xt = reinterpret_cast<const uint4*>(xrow) + kt * 4;
        uint4 b[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) b[f] = xt[f];
        acc1 = mfma_16x16x64(mask4(a_cur[u], 0x03030303u, 0), as_v4i(b[0]), acc1);
        acc4 = mfma_16x16x64(mask4(a_cur[u], 0x0C0C0C0Cu, 0), as_v4i(b[1]), acc4);
        acc16a = mfma_16x16x64(mask4(a_cur[u], 0x30303030u, 0), as_v4i(b[2]), acc16a);
        acc16b = mfma_16x16x64(mask4(a_cur[u], 0x30303030u, 2), as_v4i(b[3]), acc16b);
      }
#pragma unroll
      for (int u = 0; u < kGroupsPerBatch; ++u) a_cur[u] = a_next[u];
    }
    if (my_groups == 0 && rt + 1 < kRT) {  // keep the stream aligned: nothing was loaded for this tile
#pragma unroll
      for (int u = 0; u < kGroupsPerBatch; ++u) a_cur[u] = buffer_load16_stream(next_rsrc, w_off(u));
    }
    // exact: acc4 holds 4x, acc16a/b 16x the code sums
    v4i part = acc1;
    part.x += (acc4.x >> 2) + (acc16a.x >> 4) + (acc16b.x >> 4);
    part.y += (acc4.y >> 2) + (acc16a.y >> 4) + (acc16b.y >> 4);
    part.z += (acc4.z >> 2) + (acc16a.z >> 4) + (acc16b.z >> 4);
    part.w += (acc4.w >> 2) + (acc16a.w >> 4) + (acc16b.w >> 4);
    partial[rt][wave][lane] = part;
  }
  __syncthreads();
  // wave w finishes row tiles w, w + 4, ... for the block's tokens
  if (!has_tok) return;
  const int xsum = row_total<false>(col, kT / rp, red_sum);  // sum q*x = sum c*x - sum x
  const float row_amax = __uint_as_float((uint32_t)row_total<true>(col, kT / rp, red_max) << 16);
  const float scale = (gamma * row_amax) / 127.0f;
  auto tile_sum = [&](int rt) {
    v4i acc = partial[rt][0][lane];
#pragma unroll
    for (int w = 1; w < kW; ++w) add4(acc, partial[rt][w][lane]);
    acc.x -= xsum;
    acc.y -= xsum;
    acc.z -= xsum;
    acc.w -= xsum;
    return acc;
  };
  if constexpr (kGlu) {
    static_assert(kRT % 2 == 0, "gate/up tiles come in pairs");
#pragma unroll
    for (int p = 0; p < kRT / 2; ++p) {
      if (p % kW != wave || 2 * p >= tiles_here) continue;
      store_glu_tile(tile_sum(2 * p), tile_sum(2 * p + 1), (tile0 / 2 + p) * kTileRows + 4 * sub, tok0 + col, n / 2,
                     scale, y_out);
    }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    if (rt % kW != wave || rt >= tiles_here) continue;
    store_tile(tile_sum(rt), (tile0 + rt) * kTileRows + 4 * sub, tok0 + col, n, scale, acc_out, y_out);
  }
}

// Whole BitLinear for a block of up to kW (8 or 16) tokens on rows of up to
// 8192 columns, in one launch of kW waves.  Wave r quantizes token r of the
// block from registers (kXC 16-byte bf16 chunks per lane: the row's absmax
// and activation sum are whole-wave reductions, no LDS round) and writes its
// int8 codes into LDS row r.  Every weight load of the workgroup (kRT row
// tiles x the 1 KiB groups w, w + kW, ... of wave w) is issued right after
// the activation loads, so the HBM latency of the weights overlaps the
// quantization.  After one barrier each wave multiplies its groups with B
// operands read from LDS (four scaled accumulators per row tile, as in
// k_bitlinear_fused); the waves' partial sums of a row tile then meet in
// LDS.  Waves past the block's tokens only multiply.  kGlu (kRT even):
// gate+up matrix with alternating gate/up row tiles, y_out is h ([m][n / 2]).
template <int kRT, int kXC, int kW, bool kGlu = false>
__global__ __launch_bounds__(kW * 64) void k_bitlinear_tok(const uint4* __restrict__ packed,
                                                         const float* __restrict__ gamma_ptr,
                                                         const uint4* __restrict__ x, float* __restrict__ alpha,
                                                         int8_t* __restrict__ xq_out, int m, int n, int k,
                                                         int32_t* __restrict__ acc_out, uint16_t* __restrict__ y_out) {
  static_assert(kW == 8 || kW == 16, "one wave per token of the block");
  constexpr int kJ = (2 * kXC + kW - 1) / kW;  // groups per wave and row tile (ceil(k / 256) <= 2 kXC)
  extern __shared__ uint4 xs_raw[];            // [kW][k + kLdsRowPad] codes, then [kRT][kW][64] partial sums
  __shared__ int tok_sum[16];
  __shared__ int tok_amax[16];
  int8_t* xs = reinterpret_cast<int8_t*>(xs_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane >> 4;
  const int col = lane & 15;
  const int tile0 = (int)blockIdx.x * kRT;
  const int row_tiles = (n + kTileRows - 1) / kTileRows;
  const int tiles_here = min(kRT, row_tiles - tile0);
  const int tok0 = (int)blockIdx.y * kW;
  const int rows = min(kW, m - tok0);
  const int kt_count = k / kTileCols;
  const int groups = (kt_count + 3) / 4;
  const int k8 = k / 8;
  const int ldx = k + kLdsRowPad;
  const bool first_block = blockIdx.x == 0;

  // ---- token row `wave`: chunks lane, lane + 64, ...; reads past the row,
  // or by a wave without a token, return zero
  const __amdgpu_buffer_rsrc_t xrsrc =
      buffer_rsrc(x + (int64_t)(tok0 + min(wave, rows - 1)) * k8, wave < rows ? (uint32_t)k * 2u : 0u);
  uint4 xr[kXC];
#pragma unroll
  for (int i = 0; i < kXC; ++i) xr[i] = buffer_load16(xrsrc, (uint32_t)(lane + 64 * i) * 16u);
  // ---- weights: lane (col, sub) of group g holds row col of tile 4g + sub;
  // tiles past k, and row tiles past n, read as zero codes
  const __amdgpu_buffer_rsrc_t wrsrc = buffer_rsrc(packed + (int64_t)tile0 * kt_count * (kTileBytes / 16),
                                                   (uint32_t)(tiles_here * kt_count * kTileBytes));
  uint4 a[kJ][kRT];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int kt = 4 * (wave + kW * j) + sub;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      a[j][rt] = buffer_load16_stream(
          wrsrc, kt < kt_count ? (uint32_t)((rt * kt_count + kt) * kTileBytes + col * 16) : kOutOfRange);
  }
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- quantize token `wave` into LDS row `wave` (and xq, alpha once)
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < kXC; ++i) m2 = absmax_step(m2, xr[i]);
  const int amax_bits = wave_reduce<true>((int)max(m2.x, m2.y));
  const float amax = __uint_as_float((uint32_t)amax_bits << 16);
  const float s = 127.0f / fmaxf(amax, 1e-5f);  // IEEE division, as in bl_quant_act
  int sum = 0;
  if (wave < rows) {
    uint2* dst = reinterpret_cast<uint2*>(xs + wave * ldx);
    uint2* gdst = first_block && xq_out ? reinterpret_cast<uint2*>(xq_out + (int64_t)(tok0 + wave) * k) : nullptr;
#pragma unroll
    for (int i = 0; i < kXC; ++i) {
      const int c = lane + 64 * i;
      if (c < k8) {
        const uint2 q = act_codes8(xr[i], s, sum);
        dst[c] = q;
        if (gdst) gdst[c] = q;
      }
    }
    if (first_block && alpha && lane == 0) alpha[tok0 + wave] = amax;
  }
  sum = wave_reduce<false>(sum);
  if (lane == 0) {
    tok_sum[wave] = sum;
    tok_amax[wave] = amax_bits;
  }
  __syncthreads();

  // ---- products: token col's 16 bytes of field f of tile 4g + sub
  const int8_t* xrow = xs + min(col, kW - 1) * ldx;  // B columns past the block: any row (not stored)
  v4i acc[kRT][4];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[rt][f] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int g = wave + kW * j;
    if (g >= groups) break;  // wave-uniform
    // tiles past k carry zero codes, so any in-bounds activation bytes will do
    const int kt = min(4 * g + sub, kt_count - 1);
    const uint4* xt = reinterpret_cast<const uint4*>(xrow + kt * kTileCols);
    uint4 b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) b[f] = xt[f];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      acc[rt][0] = mfma_16x16x64(mask4(a[j][rt], 0x03030303u, 0), as_v4i(b[0]), acc[rt][0]);
      acc[rt][1] = mfma_16x16x64(mask4(a[j][rt], 0x0C0C0C0Cu, 0), as_v4i(b[1]), acc[rt][1]);
      acc[rt][2] = mfma_16x16x64(mask4(a[j][rt], 0x30303030u, 0), as_v4i(b[2]), acc[rt][2]);
      acc[rt][3] = mfma_16x16x64(mask4(a[j][rt], 0x30303030u, 2), as_v4i(b[3]), acc[rt][3]);
    }
  }
  // the waves with groups (all of them once groups >= 16) leave their partial
  // sums where the codes were
  const int nw = min(kW, groups);
  __syncthreads();
  v4i* partial = reinterpret_cast<v4i*>(xs_raw);  // [kRT][kW][64]
  if (wave < nw) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      // exact: acc[1] holds 4x, acc[2] and acc[3] 16x the code sums
      v4i part = acc[rt][0];
      part.x += (acc[rt][1].x >> 2) + ((acc[rt][2].x + acc[rt][3].x) >> 4);
      part.y += (acc[rt][1].y >> 2) + ((acc[rt][2].y + acc[rt][3].y) >> 4);
      part.z += (acc[rt][1].z >> 2) + ((acc[rt][2].z + acc[rt][3].z) >> 4);
      part.w += (acc[rt][1].w >> 2) + ((acc[rt][2].w + acc[rt][3].w) >> 4);
      partial[(rt * kW + wave) * 64 + lane] = part;
    }
  }
  __syncthreads();
  if (col >= rows) return;
  const int xsum = tok_sum[col];  // sum q*x = sum c*x - sum x
  const float scale = (gamma * __uint_as_float((uint32_t)tok_amax[col] << 16)) / 127.0f;
  auto tile_sum = [&](int rt) {
    v4i t = partial[(rt * kW) * 64 + lane];
    for (int w = 1; w < nw; ++w) add4(t, partial[(rt * kW + w) * 64 + lane]);
    t.x -= xsum;
    t.y -= xsum;
    t.z -= xsum;
    t.w -= xsum;
    return t;
  };
  if constexpr (kGlu) {
    static_assert(kRT % 2 == 0, "gate/up tiles come in pairs");
#pragma unroll
    for (int p = 0; p < kRT / 2; ++p) {
      if (p != wave || 2 * p >= tiles_here) continue;
      store_glu_tile(tile_sum(2 * p), tile_sum(2 * p + 1), (int64_t)(tile0 / 2 + p) * kTileRows + 4 * sub, tok0 + col,
                     n / 2, scale, y_out);
    }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    if (rt != wave || rt >= tiles_here) continue;
    store_tile(tile_sum(rt), (int64_t)(tile0 + rt) * kTileRows + 4 * sub, tok0 + col, n, scale, acc_out, y_out);
  }
}

constexpr int kM1MaxSlots = 7;  // 16-byte bf16 chunks per lane at 8 waves (own groups only: rows up to k = 28672)

// BitLinear for one token (kM = 1), quantization fused.  The kernel also
// takes up to kM = 4 tokens of short rows, a form no longer launched (the
// token-block kernel is faster there); the source keeps it because the
// one-token instance compiles to faster code from it (measured 3.77
// against 3.90 us per launch on the 2B-shaped stack).  Wave w of the kWv (4, or 8 for long rows) multiplies
// the 256-column groups w, w + kWv, ... and quantizes exactly those, for every token, into its own
// LDS region, which only it reads.  The tokens' absmaxes come from per-wave
// maxima of the own groups exchanged through LDS (one barrier).  Slot i of
// lane l holds chunk (l % 32) of the wave's own group rank 2i + l / 32, so
// all 64 lanes quantize.  Each wave subtracts the activation sums of its own
// columns from its partial products, so the waves' partials add up to
// sum q*x; one barrier then combines them.  A workgroup handles kRT
// consecutive 16-row tiles, reusing the quantized tokens; the weight loads
// of all its tiles form one stream, prefetched a batch ahead.  kC = slots
// per lane (ceil(own groups / 2)).  kGlu: the matrix is a gate+up matrix
// packed with alternating gate/up row tiles and kRT = 2, so the workgroup's
// two tiles are the gate and up rows of the same 16 outputs; wave 0 writes
// h = bf16(relu(g)^2 * u) into y_out ([m][n / 2]).
template <int kRT, int kC, int kM, bool kGlu = false, int kWv = kWaves>
__global__ __launch_bounds__(kWv * 64) void k_bitlinear_m1(const uint4* __restrict__ packed,
                                                               const float* __restrict__ gamma_ptr,
                                                               const uint4* __restrict__ x, float* __restrict__ alpha,
                                                               int8_t* __restrict__ xq_out, int m, int n, int k,
                                                               int32_t* __restrict__ acc_out,
                                                               uint16_t* __restrict__ y_out) {
  constexpr int kW = kWv;
  constexpr int kB = kGroupsPerBatch;  // weight groups per batch (larger batches measured no faster)
  extern __shared__ uint4 xw_raw[];    // [wave][own group rank][token][256 bytes]
  __shared__ v4i partial[kRT][kW][64];
  __shared__ int wave_max[kW][kM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile0 = blockIdx.x * kRT;
  const int row_tiles = (n + kTileRows - 1) / kTileRows;
  const int tiles_here = min(kRT, row_tiles - tile0);
  const int kt_count = k / kTileCols;
  const int groups = (kt_count + 3) / 4;
  const int my_groups = (groups - wave + kW - 1) / kW;
  const int max_groups = (groups + kW - 1) / kW;
  const int sub = lane >> 4;
  const int col = lane & 15;
  const int tc = min(col, kM - 1);  // token of this lane's MFMA column (columns past the block repeat one)
  const int half = lane >> 5;
  const int r = lane & 31;

  // activations first (loads retire in order), then the first weight batch.
  // Slot i of lane l: chunk l % 32 of own group rank 2i + l / 32 (group
  // w + kW * rank), for every token; ranks past this wave's share, tokens
  // past m and columns past k read as zero.
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(x, (uint32_t)(m * k * 2));
  uint4 xr[kM][kC];
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const int rank = 2 * i + half;
    const int g = wave + kW * rank;
#pragma unroll
    for (int t = 0; t < kM; ++t)
      xr[t][i] = buffer_load16(xrsrc, rank < my_groups && g * 32 + r < k / 8 ? (uint32_t)(t * k * 2 + g * 512 + r * 16)
                                                                          : kOutOfRange);
  }
  // Weights: one resource per row tile, so that groups past k (and a whole
  // tile past n) read as zero codes instead of the next tile's bytes.
  const uint32_t tile_bytes = (uint32_t)(kt_count * kTileBytes);
  auto tile_rsrc = [&](int rt) {
    return buffer_rsrc(packed + (size_t)(tile0 + rt) * kt_count * (kTileBytes / 16), rt < tiles_here ? tile_bytes : 0u);
  };
  // this wave's gi-th group within a row tile
  auto w_off = [&](int gi) { return (uint32_t)((wave + gi * kW) * 1024 + lane * 16); };
  uint4 a_cur[kB];
  {
    const __amdgpu_buffer_rsrc_t r0 = tile_rsrc(0);
#pragma unroll
    for (int u = 0; u < kB; ++u) a_cur[u] = buffer_load16_stream(r0, w_off(u));
  }
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  // keep these loads here, in flight while the activations are reduced
  __builtin_amdgcn_sched_barrier(0);

  // per-token absmax: this wave's columns, then the waves' maxima through LDS
  float amax[kM], s[kM];
#pragma unroll
  for (int t = 0; t < kM; ++t) {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < kC; ++i) m2 = absmax_step(m2, xr[t][i]);
    const int mx = wave_reduce<true>((int)max(m2.x, m2.y));
    if (lane == 0) wave_max[wave][t] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kM; ++t) {
    int mx = wave_max[0][t];
#pragma unroll
    for (int w = 1; w < kW; ++w) mx = max(mx, wave_max[w][t]);
    amax[t] = __uint_as_float((uint32_t)mx << 16);
    s[t] = 127.0f / fmaxf(amax[t], 1e-5f);  // IEEE division, as in bl_quant_act
  }

  // quantize this wave's own groups: (rank, token) lands at byte
  // 256 * (rank * kM + token) + 8 r of the wave's region
  int8_t* region = reinterpret_cast<int8_t*>(xw_raw) + wave * max_groups * kM * 256;
  const bool first_block = blockIdx.x == 0;
  int sum[kM];
#pragma unroll
  for (int t = 0; t < kM; ++t) sum[t] = 0;
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    if (2 * i >= my_groups) break;  // wave-uniform
    const int rank = 2 * i + half;
    if (rank < my_groups) {
      const int chunk = (wave + kW * rank) * 32 + r;
#pragma unroll
      for (int t = 0; t < kM; ++t) {
        const uint2 q = act_codes8(xr[t][i], s[t], sum[t]);
        reinterpret_cast<uint2*>(region + (rank * kM + t) * 256)[r] = q;
        if (first_block && xq_out && t < m && chunk < k / 8) reinterpret_cast<uint2*>(xq_out + (int64_t)t * k)[chunk] = q;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kM; ++t) sum[t] = wave_reduce<false>(sum[t]);
  if (first_block && wave == 0 && lane < m && lane < kM && alpha) {
    float a = amax[0];
#pragma unroll
    for (int t = 1; t < kM; ++t) a = lane == t ? amax[t] : a;
    alpha[lane] = a;
  }
  // this lane's token: its activation sum and absmax (uniform values, selected)
  int my_sum = sum[0];
  float my_amax = amax[0];
#pragma unroll
  for (int t = 1; t < kM; ++t) {
    my_sum = tc == t ? sum[t] : my_sum;
    my_amax = tc == t ? amax[t] : my_amax;
  }
  // this wave's own LDS writes are complete before its reads below
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)

#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    v4i acc1 = {0, 0, 0, 0}, acc4 = acc1, acc16a = acc1, acc16b = acc1;
    const __amdgpu_buffer_rsrc_t cur_rsrc = tile_rsrc(rt);
    const __amdgpu_buffer_rsrc_t next_rsrc = tile_rsrc(rt + 1);  // empty past the last tile
    for (int gi = 0; gi < my_groups; gi += kB) {
      // next batch: more groups of this tile, else the first groups of the next
      const bool same = gi + kB < my_groups;
      const int ngi = same ? gi + kB : 0;
      uint4 a_next[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        a_next[u] = buffer_load16_stream(same ? cur_rsrc : next_rsrc, w_off(ngi + u));
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        // groups past this wave's share carry zero codes; any region slot will do
        const int gl = min(gi + u, max_groups - 1);
        const uint4* xt = reinterpret_cast<const uint4*>(region + (gl * kM + tc) * 256) + 4 * sub;
        uint4 b[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) b[f] = xt[f];
        acc1 = mfma_16x16x64(mask4(a_cur[u], 0x03030303u, 0), as_v4i(b[0]), acc1);
        acc4 = mfma_16x16x64(mask4(a_cur[u], 0x0C0C0C0Cu, 0), as_v4i(b[1]), acc4);
        acc16a = mfma_16x16x64(mask4(a_cur[u], 0x30303030u, 0), as_v4i(b[2]), acc16a);
        acc16b = mfma_16x16x64(mask4(a_cur[u], 0x30303030u, 2), as_v4i(b[3]), acc16b);
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) a_cur[u] = a_next[u];
    }
    if (my_groups == 0 && rt + 1 < kRT) {  // keep the stream aligned: nothing was loaded for this tile
#pragma unroll
      for (int u = 0; u < kB; ++u) a_cur[u] = buffer_load16_stream(next_rsrc, w_off(u));
    }
    // exact: acc4 holds 4x, acc16a/b 16x the code sums; minus this wave's x sum
    v4i part = acc1;
    part.x += (acc4.x >> 2) + (acc16a.x >> 4) + (acc16b.x >> 4) - my_sum;
    part.y += (acc4.y >> 2) + (acc16a.y >> 4) + (acc16b.y >> 4) - my_sum;
    part.z += (acc4.z >> 2) + (acc16a.z >> 4) + (acc16b.z >> 4) - my_sum;
    part.w += (acc4.w >> 2) + (acc16a.w >> 4) + (acc16b.w >> 4) - my_sum;
    partial[rt][wave][lane] = part;
  }
  __syncthreads();
  // wave w finishes row tiles w, w + kW, ...; MFMA column c is token c
  if (col >= m || col >= kM) return;
  const float scale = (gamma * my_amax) / 127.0f;
  if constexpr (kGlu) {
    static_assert(kRT == 2, "a gate tile and its up tile per workgroup");
    if (wave != 0) return;
    v4i g = partial[0][0][lane], u = partial[1][0][lane];
#pragma unroll
    for (int w = 1; w < kW; ++w) {
      add4(g, partial[0][w][lane]);
      add4(u, partial[1][w][lane]);
    }
    store_glu_tile(g, u, (int64_t)(tile0 / 2) * kTileRows + 4 * sub, col, n / 2, scale, y_out);
    return;
  }
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    if (rt % kW != wave || rt >= tiles_here) continue;
    v4i acc = partial[rt][0][lane];
#pragma unroll
    for (int w = 1; w < kW; ++w) add4(acc, partial[rt][w][lane]);
    store_tile(acc, (int64_t)(tile0 + rt) * kTileRows + 4 * sub, col, n, scale, acc_out, y_out);
  }
}

// Product with int8 activations given for one token (bl_linear with m = 1,
// and bl_bitlinear's fallback for rows longer than the fused kernels take).  Waves
// split K by 1 KiB groups as above; each lane loads its activation bytes
// (16 per field) straight from global memory as MFMA B operands and reuses
// them for the kRT row tiles of the workgroup, so activation traffic per
// weight byte falls as 4 * tokens / (16 * kRT).  Codes become signed trits
// with v_perm.  kB groups per wave form a batch; the next batch's loads are
// issued before the current batch's products.
// kGlu (kRT even): gate+up matrix with alternating gate/up row tiles; the
// pairs (2p, 2p + 1) are gated into y_out ([m][n / 2]).
template <int kRT, int kB, int kW, bool kGlu = false>
__global__ __launch_bounds__(kW * 64) void k_gemv_direct(const uint4* __restrict__ packed,
                                                          const float* __restrict__ gamma_ptr,
                                                          const int8_t* __restrict__ xq,
                                                          const float* __restrict__ alpha, int64_t m, int64_t n,
                                                          int64_t k, int32_t* __restrict__ acc_out,
                                                          uint16_t* __restrict__ y_out) {
  __shared__ v4i partial[kRT][kW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t tile0 = (int64_t)blockIdx.x * kRT;
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  const int tiles_here = (int)min((int64_t)kRT, row_tiles - tile0);
  const int64_t tok0 = (int64_t)blockIdx.y * 16;
  const int kt_count = (int)(k / kTileCols);
  const int groups = (kt_count + 3) / 4;
  const int sub = lane >> 4;
  const int col = lane & 15;
  const int64_t tok = tok0 + col;
  const bool has_tok = tok < m;
  const int rows = (int)min((int64_t)16, m - tok0);
  // resources over each row tile and over this token block; offsets past
  // either read as zero (tail groups, absent tokens, tiles past n), and a
  // zero activation byte makes the product zero whatever the trit
  const uint32_t tile_bytes = (uint32_t)(kt_count * kTileBytes);
  __amdgpu_buffer_rsrc_t wrsrc[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
    wrsrc[rt] = buffer_rsrc(packed + (tile0 + rt) * kt_count * (kTileBytes / 16), rt < tiles_here ? tile_bytes : 0u);
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(xq + tok0 * k, (uint32_t)(rows * k));
  // scales read now (a load at the epilogue would add a memory round trip)
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  const float alpha_tok = buffer_load_f32(buffer_rsrc(alpha + tok0, (uint32_t)(rows * 4)), has_tok ? col * 4 : kOutOfRange);

  auto load_batch = [&](int g0, uint4 (&a)[kRT][kB], uint4 (&b)[kB][4]) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int g = g0 + u * kW;
      const int kt = 4 * g + sub;
      const bool valid = kt < kt_count && has_tok;
#pragma unroll
      for (int f = 0; f < 4; ++f)
        b[u][f] = buffer_load16(xrsrc, valid ? (uint32_t)(col * k + kt * kTileCols + 16 * f) : kOutOfRange);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        a[rt][u] = buffer_load16_stream(wrsrc[rt], g < groups ? (uint32_t)(g * 1024 + lane * 16) : kOutOfRange);
    }
  };
  v4i acc[kRT][2];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) acc[rt][0] = acc[rt][1] = v4i{0, 0, 0, 0};
  uint4 a_cur[kRT][kB], b_cur[kB][4];
  load_batch(wave, a_cur, b_cur);
  for (int g0 = wave; g0 < groups; g0 += kW * kB) {
    uint4 a_nxt[kRT][kB], b_nxt[kB][4];
    load_batch(g0 + kW * kB, a_nxt, b_nxt);  // past the end: out of range, no memory access
#pragma unroll
    for (int u = 0; u < kB; ++u) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[rt][f & 1] = mfma_16x16x64(unpack_field(a_cur[rt][u], f), as_v4i(b_cur[u][f]), acc[rt][f & 1]);
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
#pragma unroll
      for (int f = 0; f < 4; ++f) b_cur[u][f] = b_nxt[u][f];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) a_cur[rt][u] = a_nxt[rt][u];
    }
  }
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    add4(acc[rt][0], acc[rt][1]);
    partial[rt][wave][lane] = acc[rt][0];
  }
  __syncthreads();
  // wave w finishes row tiles w, w + kW, ...
  if (!has_tok) return;
  const float scale = (gamma * alpha_tok) / 127.0f;
  if constexpr (kGlu) {
    static_assert(kRT % 2 == 0, "gate/up tiles come in pairs");
#pragma unroll
    for (int p = 0; p < kRT / 2; ++p) {
      if (p % kW != wave || 2 * p >= tiles_here) continue;
      v4i g = partial[2 * p][0][lane], u = partial[2 * p + 1][0][lane];
#pragma unroll
      for (int w = 1; w < kW; ++w) {
        add4(g, partial[2 * p][w][lane]);
        add4(u, partial[2 * p + 1][w][lane]);
      }
      store_glu_tile(g, u, (tile0 / 2 + p) * kTileRows + 4 * sub, tok, n / 2, scale, y_out);
    }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    if (rt % kW != wave || rt >= tiles_here) continue;
    v4i sum = partial[rt][0][lane];
#pragma unroll
    for (int w = 1; w < kW; ++w) add4(sum, partial[rt][w][lane]);
    store_tile(sum, (tile0 + rt) * kTileRows + 4 * sub, tok, n, scale, acc_out, y_out);
  }
}


// Product with int8 activations given, 2 <= m <= 16 tokens, activations
// staged through LDS.  Loaded straight from global memory as MFMA B operands
// (k_gemv_direct), a wave's activation load touches 32 cache lines (16
// token rows x 2 lines) for 1 KiB, so the L1 line rate bounds the kernel
// near 2.5 TB/s of weights at 16 tokens.  Here the workgroup copies the
// token block in column chunks of kC = kW * kGW * 256 bytes per token, with
// loads that read each token row contiguously, into LDS (row stride kC + 16
// bytes: the 16 rows of a B operand read fall in distinct banks); the waves
// then read their B operands from LDS.  Per chunk, wave w multiplies groups
// w, w + kW, ... of the chunk (kGW of them) for the kRT row tiles of the
// workgroup.  The next chunk's activations and weights are loaded into
// registers while the current chunk is multiplied; two barriers per chunk
// guard the single LDS buffer.  Codes become signed trits with v_perm.
// kGlu (kRT even): gate+up matrix with alternating gate/up row tiles; the
// (tile pair, token block) items are gated into y_out ([m][n / 2]).
template <int kRT, int kW, int kGW, int kTB, bool kGlu = false>
__global__ __launch_bounds__(kW * 64) void k_gemv_lds(const uint4* __restrict__ packed,
                                                       const float* __restrict__ gamma_ptr,
                                                       const int8_t* __restrict__ xq,
                                                       const float* __restrict__ alpha, int64_t m, int64_t n,
                                                       int64_t k, int32_t* __restrict__ acc_out,
                                                       uint16_t* __restrict__ y_out) {
  constexpr int kT = kW * 64;
  constexpr int kC = kW * kGW * 256;          // columns per chunk
  constexpr int kLd = kC + 16;                // LDS row stride
  constexpr int kRowsX = 16 * kTB;            // token rows staged
  constexpr int kPieces = kRowsX * kC / 16;   // 16-byte pieces per chunk
  constexpr int kXLoads = kPieces / kT;       // per thread
  constexpr int kAcc = kTB == 1 ? 2 : 1;      // independent accumulator chains per (tile, token block)
  static_assert(kPieces % kT == 0, "chunk must split evenly over the threads");
  static_assert(kRT * kTB * kW * 1024 <= kRowsX * kLd, "partial sums reuse the activation buffer");
  __shared__ uint4 xs_raw[kRowsX * kLd / 16];
  int8_t* xs = reinterpret_cast<int8_t*>(xs_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile0 = (int64_t)blockIdx.x * kRT;
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  const int tiles_here = (int)min((int64_t)kRT, row_tiles - tile0);
  const int64_t tok0 = (int64_t)blockIdx.y * kRowsX;
  const int rows = (int)min((int64_t)kRowsX, m - tok0);
  const int kt_count = (int)(k / kTileCols);
  const int groups = (kt_count + 3) / 4;
  const int chunks = (int)((k + kC - 1) / kC);
  const int sub = lane >> 4;
  const int col = lane & 15;

  const uint32_t tile_bytes = (uint32_t)(kt_count * kTileBytes);
  __amdgpu_buffer_rsrc_t wrsrc[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
    wrsrc[rt] = buffer_rsrc(packed + (tile0 + rt) * kt_count * (kTileBytes / 16), rt < tiles_here ? tile_bytes : 0u);
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(xq + tok0 * k, (uint32_t)(rows * k));
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(alpha + tok0, (uint32_t)(rows * 4));
  float alpha_tok[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb)
    alpha_tok[tb] = buffer_load_f32(arsrc, 16 * tb + col < rows ? (uint32_t)((16 * tb + col) * 4) : kOutOfRange);

  // piece p of a chunk: token row p / (kC / 16), 16 bytes at column 16 * (p % (kC / 16))
  auto load_x = [&](int c, uint4 (&v)[kXLoads]) {
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int p = tid + i * kT;
      const int r = p / (kC / 16);
      const int64_t colx = (int64_t)c * kC + 16 * (p % (kC / 16));
      v[i] = buffer_load16(xrsrc, colx < k ? (uint32_t)(r * k + colx) : kOutOfRange);
    }
  };
  // this wave's u-th group of chunk c (global group index)
  auto group_of = [&](int c, int u) { return c * (kW * kGW) + wave + u * kW; };
  auto load_w = [&](int c, uint4 (&a)[kRT][kGW]) {
#pragma unroll
    for (int u = 0; u < kGW; ++u) {
      const int g = group_of(c, u);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        a[rt][u] = buffer_load16_stream(wrsrc[rt], g < groups ? (uint32_t)(g * 1024 + lane * 16) : kOutOfRange);
    }
  };

  v4i acc[kRT][kTB][kAcc];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
      for (int j = 0; j < kAcc; ++j) acc[rt][tb][j] = v4i{0, 0, 0, 0};
  uint4 xv[kXLoads];
  uint4 a_cur[kRT][kGW];
  load_x(0, xv);
  load_w(0, a_cur);
  for (int c = 0; c < chunks; ++c) {
    __syncthreads();  // the previous chunk's B operands have been read
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int p = tid + i * kT;
      *reinterpret_cast<uint4*>(xs + (p / (kC / 16)) * kLd + 16 * (p % (kC / 16))) = xv[i];
    }
    __syncthreads();
    uint4 a_nxt[kRT][kGW];
    if (c + 1 < chunks) {
      load_x(c + 1, xv);
      load_w(c + 1, a_nxt);
    }
#pragma unroll
    for (int u = 0; u < kGW; ++u) {
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        // local tile 4 * (wave + u * kW) + sub of this chunk, field f, token row 16 tb + col
        const int8_t* xt = xs + (16 * tb + col) * kLd + (4 * (wave + u * kW) + sub) * kTileCols;
        uint4 b[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) b[f] = *reinterpret_cast<const uint4*>(xt + 16 * f);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
          for (int f = 0; f < 4; ++f)
            acc[rt][tb][f % kAcc] = mfma_16x16x64(unpack_field(a_cur[rt][u], f), as_v4i(b[f]), acc[rt][tb][f % kAcc]);
        }
      }
    }
    if (c + 1 < chunks) {
#pragma unroll
      for (int u = 0; u < kGW; ++u) {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) a_cur[rt][u] = a_nxt[rt][u];
      }
    }
  }
  // the waves' partial sums, in the activation buffer once everyone is done with it
  __syncthreads();
  v4i* partial = reinterpret_cast<v4i*>(xs_raw);  // [kRT][kTB][kW][64]
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
      v4i a = acc[rt][tb][0];
      if (kAcc == 2) add4(a, acc[rt][tb][kAcc - 1]);
      partial[((rt * kTB + tb) * kW + wave) * 64 + lane] = a;
    }
  __syncthreads();
  auto pair_sum = [&](int rt, int tb) {
    const int pair = rt * kTB + tb;
    v4i sum = partial[(pair * kW) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kW; ++w) add4(sum, partial[(pair * kW + w) * 64 + lane]);
    return sum;
  };
  if constexpr (kGlu) {
    static_assert(kRT % 2 == 0, "gate/up tiles come in pairs");
#pragma unroll
    for (int p = 0; p < kRT / 2; ++p)
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const int item = p * kTB + tb;
        if (item % kW != wave || 2 * p >= tiles_here || 16 * tb + col >= rows) continue;
        const float scale = (gamma * alpha_tok[tb]) / 127.0f;
        store_glu_tile(pair_sum(2 * p, tb), pair_sum(2 * p + 1, tb), (tile0 / 2 + p) * kTileRows + 4 * sub,
                       tok0 + 16 * tb + col, n / 2, scale, y_out);
      }
    return;
  }
  // wave w finishes the (row tile, token block) pairs w, w + kW, ...
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
      const int pair = rt * kTB + tb;
      if (pair % kW != wave || rt >= tiles_here || 16 * tb + col >= rows) continue;
      v4i sum = partial[(pair * kW) * 64 + lane];
#pragma unroll
      for (int w = 1; w < kW; ++w) add4(sum, partial[(pair * kW + w) * 64 + lane]);
      const float scale = (gamma * alpha_tok[tb]) / 127.0f;
      store_tile(sum, (tile0 + rt) * kTileRows + 4 * sub, tok0 + 16 * tb + col, n, scale, acc_out, y_out);
    }
}


// Product with int8 activations given, 2 <= m <= 16 tokens, long rows: the
// token block's activations stream through a ring of kS 1024-column LDS
// buffers filled by DMA (buffer loads that write LDS, no registers) kS - 1
// chunks ahead, so the loads of kS - 1 chunks are in flight while one is
// multiplied; one barrier per chunk.  kW = 4 * kRT waves: wave w multiplies
// 256-column group w % 4 of every chunk for row tile w / 4 of the workgroup
// (one non-temporal 1 KiB weight load per chunk, in a register ring beside
// the LDS ring), and the four waves of a tile add their partial sums through
// LDS at the end.  Token rows are 1024 bytes apart in a buffer, so stored
// 16-byte piece p of row r holds source piece p ^ (r % 16): the 16 token rows
// of a B operand read fall in distinct banks.  Pieces past k and rows past m
// read as zero, so the trits of a partial last group (whose codes past k are
// zero, i.e. -1) meet zero activations.  The chunk loop is unrolled by the
// ring size so that every buffer is named at compile time.
// kGlu (kRT = 2): gate+up matrix with alternating gate/up row tiles; wave 0
// gates the tile pair into y_out ([m][n / 2]).
template <int kRT, bool kGlu = false, int kS = 4>
__global__ __launch_bounds__(kRT * 256) void k_gemv_ring(const uint4* __restrict__ packed,
                                                        const float* __restrict__ gamma_ptr,
                                                        const int8_t* __restrict__ xq,
                                                        const float* __restrict__ alpha, int64_t m, int64_t n,
                                                        int64_t k, int32_t* __restrict__ acc_out,
                                                        uint16_t* __restrict__ y_out) {
  constexpr int kW = 4 * kRT;
  constexpr int kCC = 1024;          // columns per chunk
  constexpr int kPieces = kCC / 16;  // 16-byte pieces per token row and chunk
  constexpr int kDma = 16 / kW;      // token rows this wave copies per chunk, one 1 KiB DMA each
  static_assert(16 % kW == 0, "the 16 token rows split evenly over the waves");
  static_assert(!kGlu || kRT == 2, "a gate tile and its up tile per workgroup");
  static_assert(kS >= 3 && kS <= 8, "ring depth");
  // the ring: kS distinct LDS objects (each named at compile time below)
  __shared__ uint4 xs0[16 * kPieces], xs1[16 * kPieces], xs2[16 * kPieces], xs3[16 * kPieces];
  __shared__ uint4 xs4[kS > 4 ? 16 * kPieces : 1], xs5[kS > 5 ? 16 * kPieces : 1];
  __shared__ uint4 xs6[kS > 6 ? 16 * kPieces : 1], xs7[kS > 7 ? 16 * kPieces : 1];
  __shared__ v4i partial[kRT][4][64];
  auto ring = [&](auto slot) -> uint4* {
    constexpr int i = decltype(slot)::value;
    if constexpr (i == 0) return xs0;
    else if constexpr (i == 1) return xs1;
    else if constexpr (i == 2) return xs2;
    else if constexpr (i == 3) return xs3;
    else if constexpr (i == 4) return xs4;
    else if constexpr (i == 5) return xs5;
    else if constexpr (i == 6) return xs6;
    else return xs7;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int my_rt = wave >> 2;
  const int my_g = wave & 3;
  const int sub = lane >> 4;
  const int col = lane & 15;
  const int64_t tile0 = (int64_t)blockIdx.x * kRT;
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  const int tiles_here = (int)min((int64_t)kRT, row_tiles - tile0);
  const int64_t tok0 = (int64_t)blockIdx.y * 16;
  const int rows = (int)min((int64_t)16, m - tok0);
  const int kt_count = (int)(k / kTileCols);
  const int chunks = (int)((k + kCC - 1) / kCC);
  const uint32_t kk = (uint32_t)k;

  const __amdgpu_buffer_rsrc_t wrsrc =
      buffer_rsrc(packed + (tile0 + my_rt) * kt_count * (kTileBytes / 16),
                  my_rt < tiles_here ? (uint32_t)(kt_count * kTileBytes) : 0u);
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(xq + tok0 * k, (uint32_t)(rows * k));
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  const float alpha_tok =
      buffer_load_f32(buffer_rsrc(alpha + tok0, (uint32_t)(rows * 4)), col < rows ? (uint32_t)(col * 4) : kOutOfRange);

  // chunk c: this wave's token rows into dst by DMA, its weight group into w
  auto load_chunk = [&](int c, uint4* dst, uint4& w) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const int row = wave * kDma + j;
      const uint32_t col_byte = (uint32_t)c * kCC + 16u * (uint32_t)(lane ^ (row & 15));
      const uint32_t off = col_byte < kk ? (uint32_t)row * kk + col_byte : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (__attribute__((address_space(3))) void*)(dst + row * kPieces),
                                               16, off, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // one issue order for every chunk: the wait counts depend on it
    w = buffer_load16_stream(wrsrc, (uint32_t)((c * 4 + my_g) * 1024 + lane * 16));
  };

  v4i acc0 = {0, 0, 0, 0}, acc1 = acc0;
  auto compute = [&](const uint4* buf, const uint4& w) __attribute__((always_inline)) {
    // token col, column tile sub of group my_g: pieces 16 * my_g + 4 * sub + f
    const uint4* xt = buf + col * kPieces;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const v4i b = as_v4i(xt[(16 * my_g + 4 * sub + f) ^ col]);
      if (f & 1)
        acc1 = mfma_16x16x64(unpack_field(w, f), b, acc1);
      else
        acc0 = mfma_16x16x64(unpack_field(w, f), b, acc0);
    }
  };
  // chunk c: this wave's LDS reads of chunk c - 1 have completed and its DMA
  // and weights of chunk c (issued before those of chunks c + 1 and c + 2)
  // have landed; after the barrier that holds for every wave, so chunk c is
  // in LDS and the buffer of chunk c - 1 is free for chunk c + 3.  (A bare
  // s_barrier with its own wait: __syncthreads() carries a release fence,
  // which would wait for every DMA this wave has in flight, the later
  // chunks' included.  The scheduling barriers keep every LDS access and
  // MFMA on its side of it.)
  auto step = [&](int c, const uint4* rd, const uint4& w_rd, uint4* wr, uint4& w_wr) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most((kS - 2) * (kDma + 1)) & ~(15 << 8));  // and lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(c + kS - 1, wr, w_wr);
    // nothing of this chunk's arithmetic moves above the barrier (its weight
    // register would then be waited for early, with the later loads)
    __builtin_amdgcn_sched_barrier(0);
    compute(rd, w_rd);
  };
  // issue order as in the loop: each chunk's DMA, then its weights
  uint4 w[kS];
  static_for<kS - 1>([&](auto i) {
    load_chunk(decltype(i)::value, ring(i), w[decltype(i)::value]);
    __builtin_amdgcn_sched_barrier(0);
  });
  // chunks past the last read as zero: the ring runs in whole turns (at
  // least one: k > 0, and the loads above stay ahead of the loop)
  int c = 0;
  do {
    static_for<kS>([&](auto i) {
      constexpr int cur = decltype(i)::value, prev = (cur + kS - 1) % kS;
      step(c + cur, ring(i), w[cur], ring(std::integral_constant<int, prev>{}), w[prev]);
    });
    c += kS;
  } while (c < chunks);
  __builtin_amdgcn_s_waitcnt(0);  // the last (all-zero) loads have landed before the wave can exit

  add4(acc0, acc1);
  partial[my_rt][my_g][lane] = acc0;
  __syncthreads();
  if (my_g != 0 || col >= rows) return;
  auto tile_sum = [&](int rt) {
    v4i sum = partial[rt][0][lane];
#pragma unroll
    for (int g = 1; g < 4; ++g) add4(sum, partial[rt][g][lane]);
    return sum;
  };
  const float scale = (gamma * alpha_tok) / 127.0f;
  if constexpr (kGlu) {
    if (wave != 0 || tiles_here < 2) return;
    store_glu_tile(tile_sum(0), tile_sum(1), (tile0 / 2) * kTileRows + 4 * sub, tok0 + col, n / 2, scale, y_out);
    return;
  }
  if (my_rt >= tiles_here) return;
  store_tile(tile_sum(my_rt), (tile0 + my_rt) * kTileRows + 4 * sub, tok0 + col, n, scale, acc_out, y_out);
}

}  // namespace

size_t gemv_lds_bytes(int64_t m, int64_t k) { return (size_t)(m < 16 ? m : 16) * (size_t)(k + kLdsRowPad); }

namespace {

// LDS of k_bitlinear_fused<kRT, kW> besides the token block
constexpr size_t fused_static_lds(int rt, int w) { return (size_t)rt * w * 1024 + 2 * (size_t)(w * 4) * 4; }

constexpr int kFusedWaves = 8;

// Row tiles per workgroup of k_bitlinear_fused (0: the token block does not
// fit in LDS).  It takes the rows the other fused kernels do not hold (one
// token of more than 28672 columns, 2-3 tokens of more than 8192), with
// eight waves; two row tiles per workgroup once there are ~4 per CU (one
// token) or ~2 (several).
int fused_plan(int64_t m, int64_t n, int64_t k) {
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  int rt = m == 1 ? (row_tiles >= 1024 ? 2 : 1) : (row_tiles >= 512 ? 2 : 1);
  const size_t dyn = gemv_lds_bytes(m, k);
  while (rt > 1 && dyn + fused_static_lds(rt, kFusedWaves) > (size_t)kLdsBudget) rt /= 2;
  if (dyn + fused_static_lds(rt, kFusedWaves) > (size_t)kLdsBudget) return 0;
  return rt;
}

}  // namespace

constexpr int64_t kFusedMaxTokenColumns = 32767;  // m * k beyond which a block's quantization costs too much


namespace {

// kGlu: gate+up matrix of n rows, alternating gate/up tiles; y is h [m][n / 2]
// and every workgroup takes an even number of row tiles.
constexpr int64_t kRingMinK = 8192;  // rows from which 2..16 tokens take k_gemv_ring

template <bool kGlu>
hipError_t launch_gemv_impl(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                            int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s) {
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  // at most one workgroup of up to 1024 threads per row tile, at most 4 token blocks
  if (!grid_fits(row_tiles, 1024) || (m + 15) / 16 > 65535) return kErrGridTooLarge;
  const uint4* p = reinterpret_cast<const uint4*>(packed);
  if ((m > 32 || (m > 16 && k < kRingMinK)) && row_tiles >= 512) {
    // 32 or 64 tokens per workgroup: the unpacked weights serve 2 or 4 token
    // blocks (pays on matrices of many row tiles; elsewhere the token blocks
    // go to separate workgroups below, whose activation bytes per CU are
    // fewer: measured 17.4 -> 12.1 us for 64 tokens on a 2560 x 6912
    // matrix).  Up to 32 tokens: two row tiles per workgroup (2B-shaped
    // gate+up at 17-32 tokens: 8.8-9.4 against 11.3-11.4 us in 16-token
    // workgroups; rows of 8192 and more keep the LDS ring there); 64: four
    // (12.1 against 13.6 us with two)
    if (m <= 32) {
      const dim3 grid((unsigned)((row_tiles + 1) / 2), (unsigned)((m + 31) / 32));
      hipLaunchKernelGGL((k_gemv_lds<2, 4, 1, 2, kGlu>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
    } else {
      const dim3 grid((unsigned)((row_tiles + 3) / 4), (unsigned)((m + 63) / 64));
      hipLaunchKernelGGL((k_gemv_lds<4, 4, 1, 4, kGlu>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
    }
    return hipGetLastError();
  }
  if (m >= 2) {
    // one workgroup per 16-token block; two row tiles per workgroup once
    // there are ~2 per CU, or once one tile per workgroup would make 256
    // workgroups or more (2B-shaped rows at 17-64 tokens: 9.8 -> 7.7 us for
    // 64 tokens on 240 row tiles, 9.2 -> 8.7 for 17 on 160; a single block
    // of 160 row tiles measured slower with two); rows of 8192 and more
    // stream through the LDS ring (measured 10-25% faster on 70B-shaped
    // matrices at 4-16 tokens; no gain on 2560- and 6912-column rows)
    const int rt = kGlu || row_tiles >= 512 || (k < kRingMinK && row_tiles * ((m + 15) / 16) >= 256) ? 2 : 1;
    const dim3 grid((unsigned)((row_tiles + rt - 1) / rt), (unsigned)((m + 15) / 16));
    if (k >= kRingMinK) {
      // four row tiles (sixteen waves) per workgroup once there are ~8 per CU:
      // half the activation bytes per weight byte (measured 34 -> 28 us for
      // 16 tokens on a 57344 x 8192 matrix)
      if (!kGlu && row_tiles >= 2048) {
        const dim3 grid4((unsigned)((row_tiles + 3) / 4), (unsigned)((m + 15) / 16));
        hipLaunchKernelGGL((k_gemv_ring<4>), grid4, dim3(1024), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
      } else if (rt == 2) {
        hipLaunchKernelGGL((k_gemv_ring<2, kGlu>), grid, dim3(512), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
      } else {
        hipLaunchKernelGGL((k_gemv_ring<1>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
      }
    } else if (rt == 2) {
      hipLaunchKernelGGL((k_gemv_lds<2, 4, 4, 1, kGlu>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
    } else {
      hipLaunchKernelGGL((k_gemv_lds<1, 4, 4, 1>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
    }
    return hipGetLastError();
  }
  // one token: its activation bytes are few, so each lane loads its own
  const int rt = row_tiles >= 2048 ? 4 : row_tiles >= 512 || kGlu ? 2 : 1;
  const dim3 grid((unsigned)((row_tiles + rt - 1) / rt), (unsigned)((m + 15) / 16));
  if (rt == 4)
    hipLaunchKernelGGL((k_gemv_direct<4, 2, 4, kGlu>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
  else if (rt == 2)
    hipLaunchKernelGGL((k_gemv_direct<2, 2, 4, kGlu>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
  else
    hipLaunchKernelGGL((k_gemv_direct<1, 4, 4>), grid, dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, acc, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                       int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s) {
  return launch_gemv_impl<false>(packed, gamma, xq, alpha, m, n, k, acc, y, s);
}

hipError_t launch_gemv_glu(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                           int64_t f, int64_t k, uint16_t* h, hipStream_t s) {
  return launch_gemv_impl<true>(packed, gamma, xq, alpha, m, 2 * f, k, nullptr, h, s);
}

namespace {

typedef void (*M1Kernel)(const uint4*, const float*, const uint4*, float*, int8_t*, int, int, int, int32_t*,
                         uint16_t*);
struct M1Config {
  int rt = 0;
  int waves = kWaves;
  M1Kernel kernel = nullptr;  // none for several tokens, or rows needing more slots per lane than it has
};

template <int kRT, bool kGlu>
M1Kernel m1_pick(int64_t groups, int& waves) {
  const int64_t slots = ((groups + kWaves - 1) / kWaves + 1) / 2;
  waves = kWaves;
  if (slots <= 2) return k_bitlinear_m1<kRT, 2, 1, kGlu>;
  if (slots <= 5) return k_bitlinear_m1<kRT, 5, 1, kGlu>;
  // long rows: eight waves, so each streams half as many groups (measured
  // 4.9 TB/s against 4.3 with four on rows of 28672)
  if (((groups + 7) / 8 + 1) / 2 <= kM1MaxSlots) {
    waves = 8;
    return k_bitlinear_m1<kRT, kM1MaxSlots, 1, kGlu, 8>;
  }
  return nullptr;
}

// The gated form always takes two row tiles (a gate tile and its up tile)
// per workgroup.
M1Config m1_config_glu(int64_t m, int64_t groups) {
  if (m != 1) return M1Config{};
  M1Config c;
  c.rt = 2;
  c.kernel = m1_pick<2, true>(groups, c.waves);
  return c;
}

M1Config m1_config(int64_t m, int64_t groups, int64_t row_tiles) {
  if (m != 1) return M1Config{};
  // two row tiles per workgroup (the quantized tokens are reused) for short
  // rows once there are more than ~2 tiles per CU, for longer rows once there
  // are ~4 (measured on 8192-column rows: 5.6 TB/s against 5.1 with one)
  const int rt = (row_tiles >= 512 && groups <= 16) || row_tiles >= 1024 ? 2 : 1;
  M1Config c;
  c.rt = rt;
  c.kernel = rt == 2 ? m1_pick<2, false>(groups, c.waves) : m1_pick<1, false>(groups, c.waves);
  return c;
}

}  // namespace

// One launch per BitLinear where the quantization is cheap enough to fuse:
// k_bitlinear_m1 for one token (rows up to 28672), k_bitlinear_tok for 2-16
// tokens with m * k <= 65536, rows up to 8192 and few workgroups (below),
// k_bitlinear_fused for the rest with m * k <= 32767 (one token of longer
// rows, 2-3 tokens of longer rows or of many row tiles).  Larger blocks go
// through the quantizer and the GEMV kernels.
namespace {

constexpr int64_t kTokMaxK = 8192;  // rows k_bitlinear_tok holds (16 tokens x k codes in LDS, k / 512 chunks per lane)

// Row tiles per workgroup of k_bitlinear_tok: four on matrices of 512+ (the
// block's quantization shared by more weights: 16 tokens on 864 row tiles of
// 2560 columns, 6.9 against 8.2 us with two), else one (two for gate+up pairs).
int tok_row_tiles(int64_t row_tiles, bool glu) { return row_tiles >= 512 ? 4 : glu ? 2 : 1; }

// Every workgroup of k_bitlinear_tok (and of k_bitlinear_fused) quantizes its
// whole token block (about 4.5 VALU operations per activation), so one launch
// pays off while that repeated work is small: m * k up to 65536 (2B-shaped
// matrices: 16 tokens of 2560 columns 5.2 against 6.0 us for the quantizer +
// product pair, of 6912 columns 8.5 against 7.7 us; 32 tokens of 2560 no
// faster), and a bound on the activations quantized over all workgroups:
// 2^24, or 2^23 for rows of 8192 and more, whose quantizer + LDS-ring pair is
// faster (70B-shaped gate+up, 8192-column rows: 26.5 against 30.2 us at 2
// tokens, 26.3 against 29.8 at 4, 26.8 against 36.7 at 8; the block-quantizing
// kernel at 3 tokens 31.4 against 26.0).
int64_t max_repeated_quantization(int64_t k) { return k >= kRingMinK ? (int64_t)1 << 23 : (int64_t)1 << 24; }

bool tok_applies(int64_t m, int64_t n, int64_t k, bool glu) {
  if (m < 2 || m > 16 || k > kTokMaxK || m * k > 65536) return false;
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  const int rt = tok_row_tiles(row_tiles, glu);
  return (row_tiles + rt - 1) / rt * m * k <= max_repeated_quantization(k);
}

template <bool kGlu>
hipError_t launch_tok(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                      int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, hipStream_t s) {
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  // eight waves (one per token) for up to 8 tokens (3.7 against 4.1 us at 2)
  const int rt = tok_row_tiles(row_tiles, kGlu);
  const dim3 grid((unsigned)((row_tiles + rt - 1) / rt));
  const uint4* p = reinterpret_cast<const uint4*>(packed);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int mi = (int)m, ni = (int)n, ki = (int)k;
  const int64_t c = (k + 511) / 512;
  auto go = [&](auto kern, int w) {
    const size_t lds = std::max((size_t)w * (size_t)(k + kLdsRowPad), (size_t)rt * w * 1024);
    hipLaunchKernelGGL(kern, grid, dim3(w * 64), lds, s, p, gamma, xv, alpha, xq, mi, ni, ki, acc, y);
    return hipGetLastError();
  };
  auto pick = [&](auto xc) {
    constexpr int kXC = decltype(xc)::value;
    if (m <= 8) {
      if (rt == 4) return go(k_bitlinear_tok<4, kXC, 8, kGlu>, 8);
      if (rt == 2) return go(k_bitlinear_tok<2, kXC, 8, kGlu>, 8);
      if constexpr (!kGlu) return go(k_bitlinear_tok<1, kXC, 8>, 8);
    } else {
      if (rt == 4) return go(k_bitlinear_tok<4, kXC, 16, kGlu>, 16);
      if (rt == 2) return go(k_bitlinear_tok<2, kXC, 16, kGlu>, 16);
      if constexpr (!kGlu) return go(k_bitlinear_tok<1, kXC, 16>, 16);
    }
    return hipErrorInvalidValue;
  };
#define BL_TOK_CASE(XC) \
  if (c <= XC) return pick(std::integral_constant<int, XC>{});
  BL_TOK_CASE(2)
  BL_TOK_CASE(4)
  BL_TOK_CASE(6)
  BL_TOK_CASE(8)
  BL_TOK_CASE(12)
  BL_TOK_CASE(16)
#undef BL_TOK_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool gemv_fused_applies(int64_t m, int64_t n, int64_t k) {
  if (tok_applies(m, n, k, false)) return true;
  if (m < 1 || m > 16) return false;
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  if (m1_config(m, (k / kTileCols + 3) / 4, row_tiles).kernel) return true;
  if (m > 1 && m * k > kFusedMaxTokenColumns) return false;
  const int rt = fused_plan(m, n, k);
  // several tokens: the same bound on repeated quantization as k_bitlinear_tok
  if (m > 1 && rt > 0 && (row_tiles + rt - 1) / rt * m * k > max_repeated_quantization(k)) return false;
  return rt > 0;
}

namespace {

// Block-quantizing kernel for the gated form: two row tiles (a gate tile and
// its up tile) per workgroup, if the token block leaves room for them.
bool fused_glu_fits(int64_t m, int64_t k) {
  return gemv_lds_bytes(m, k) + fused_static_lds(2, kFusedWaves) <= (size_t)kLdsBudget;
}

}  // namespace

bool gemv_fused_glu_applies(int64_t m, int64_t f, int64_t k) {
  if (f >= 16 && f % 16 == 0 && tok_applies(m, 2 * f, k, true)) return true;
  if (m < 1 || m > 16 || f < 16 || f % 16 != 0) return false;
  if (m1_config_glu(m, (k / kTileCols + 3) / 4).kernel) return true;
  if (m > 1 && m * k > kFusedMaxTokenColumns) return false;
  if (m > 1 && f / kTileRows * m * k > max_repeated_quantization(k)) return false;  // two row tiles per workgroup
  return fused_glu_fits(m, k);
}

hipError_t launch_gemv_fused_glu(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t f,
                                 int64_t k, int8_t* xq, float* alpha, uint16_t* h, hipStream_t s) {
  if (!gemv_fused_glu_applies(m, f, k)) return hipErrorInvalidValue;
  if (tok_applies(m, 2 * f, k, true)) return launch_tok<true>(packed, gamma, x, m, 2 * f, k, xq, alpha, nullptr, h, s);
  const int64_t groups = (k / kTileCols + 3) / 4;
  const int64_t row_tiles = 2 * f / kTileRows;
  const M1Config c = m1_config_glu(m, groups);
  const uint4* p = reinterpret_cast<const uint4*>(packed);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  if (c.kernel) {
    const size_t lds = (size_t)c.waves * (size_t)((groups + c.waves - 1) / c.waves) * 256;
    const dim3 grid((unsigned)(row_tiles / 2));
    hipLaunchKernelGGL(c.kernel, grid, dim3(64 * c.waves), lds, s, p, gamma, xv, alpha, xq, (int)m, (int)(2 * f),
                       (int)k, nullptr, h);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(row_tiles / 2), (unsigned)((m + 15) / 16));
  const size_t lds = gemv_lds_bytes(m, k);
  const int64_t n = 2 * f;
  hipLaunchKernelGGL((k_bitlinear_fused<2, kFusedWaves, true>), grid, dim3(64 * kFusedWaves), lds, s, p, gamma, xv,
                     alpha, xq, m, n, k, nullptr, h);
  return hipGetLastError();
}

hipError_t launch_gemv_fused(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n,
                             int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, hipStream_t s) {
  if (!gemv_fused_applies(m, n, k)) return hipErrorInvalidValue;
  if (tok_applies(m, n, k, false)) return launch_tok<false>(packed, gamma, x, m, n, k, xq, alpha, acc, y, s);
  const M1Config c = m1_config(m, (k / kTileCols + 3) / 4, (n + kTileRows - 1) / kTileRows);
  if (c.kernel) {
    const int64_t groups = (k / kTileCols + 3) / 4;
    const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
    const size_t lds = (size_t)c.waves * (size_t)((groups + c.waves - 1) / c.waves) * 256;
    const dim3 grid((unsigned)((row_tiles + c.rt - 1) / c.rt));
    hipLaunchKernelGGL(c.kernel, grid, dim3(64 * c.waves), lds, s, reinterpret_cast<const uint4*>(packed), gamma,
                       reinterpret_cast<const uint4*>(x), alpha, xq, (int)m, (int)n, (int)k, acc, y);
    return hipGetLastError();
  }
  const int rt = fused_plan(m, n, k);
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  const dim3 grid((unsigned)((row_tiles + rt - 1) / rt), (unsigned)((m + 15) / 16));
  const uint4* p = reinterpret_cast<const uint4*>(packed);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const size_t lds = gemv_lds_bytes(m, k);
  if (rt == 2)
    hipLaunchKernelGGL((k_bitlinear_fused<2, kFusedWaves>), grid, dim3(64 * kFusedWaves), lds, s, p, gamma, xv, alpha,
                       xq, m, n, k, acc, y);
  else
    hipLaunchKernelGGL((k_bitlinear_fused<1, kFusedWaves>), grid, dim3(64 * kFusedWaves), lds, s, p, gamma, xv, alpha,
                       xq, m, n, k, acc, y);
  return hipGetLastError();
}

}  // namespace bl
