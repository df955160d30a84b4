// Prefill product for BitLinear W1.58A8 (more tokens than the decode kernels
// take): packed ternary W x int8 x.
//
// deepmox.com chapter 8, "A low-bit model is a whole-stack design": the packed
// weights move on chip, are unpacked there and multiplied with the 8-bit
// activations; bako.co, "The BitLinear Layer and AbsMean Quantization": the
// ternary product is integer add/subtract, here carried out by the int8
// matrix cores (v_mfma_i32_16x16x64_i8) on the unpacked values.
//
// With many tokens the product is a dense contraction (2*m*n*k int8 ops over
// n*k/4 + m*k bytes), bound by the matrix cores, not by HBM.  Tiling:
//   * a workgroup (4 waves side by side along n) owns 256 weight rows x 128
//     or 64 tokens, or 128 rows x 64 tokens (the largest tile that leaves
//     enough workgroups); each wave owns 64 or 32 rows x all the workgroup's
//     tokens, i.e. 4 x 8, 4 x 4 or 2 x 4 MFMA tiles of 16 x 16.  No two
//     waves share weight rows, so each packed byte is unpacked once per
//     workgroup;
//   * K advances 256 columns per step.  The weights never pass through LDS:
//     each wave loads its 64 rows' packed bytes straight into registers (one
//     1 KiB load per 16 rows per step: 16 rows x 4 tiles of 64 columns) and
//     unpacks them there -- 2-bit codes are 4x smaller than int8, so this is
//     the cheap operand to fetch per wave;
//   * the activation tile (tokens x 256 bytes) is shared by the four waves
//     through LDS, double-buffered, and copied there by DMA (buffer loads
//     that write LDS directly: no registers, no LDS store instructions);
//     16-byte chunk c of token row r is stored at chunk c ^ lds_row_key(r)
//     of that row, so the 128-bit reads of 16 token rows are free of bank
//     conflicts;
//   * the MFMA A operand is the raw code c = q + 1 of one 2-bit field
//     ((p >> 2f) & 0x03030303), so the product is sum c*x; the token's sum of
//     x turns it into sum q*x.  The sums come from the B operands already in
//     registers: wave w adds up field w (4 dot4 per token block and step);
//   * next step's DMA and weight loads are issued before this step's MFMAs;
//     one barrier per step.
// Tails: raw buffer resources return zero past the end of the weight row
// tiles and token rows; column tails beyond k are masked to zero, so code 0
// (or token 0) contributes nothing and the activation sums stay exact.
#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kWaves = 4;
constexpr int kStepK = 256;             // columns per step
constexpr int kXRow = kStepK / 16;     // 16-byte chunks per token row in LDS
constexpr int kXcds = 8;                // accelerator complex dies, each with its own L2

// kTB, kRB: 16-token (4 or 8) and 16-row (2 or 4) MFMA blocks per wave.
// kFixedBuffers: the step loop is unrolled by two so that every LDS read and
// every DMA names one of the two activation buffers at compile time; the
// compiler then knows that the DMA into one buffer cannot touch the reads of
// the other and does not wait for the DMA before reading.  Without it (fewer
// registers: more workgroups per CU) each step's reads wait for the DMA just
// issued.
// kGlu: the matrix is a gate+up matrix packed with alternating gate/up row
// tiles; a wave's row blocks 2p and 2p + 1 are then the gate and up rows of
// the same 16 outputs, and the epilogue writes h = bf16(relu(g)^2 * u) into
// y_out ([m][n / 2]); acc_out is unused.
template <int kTB, int kRB, bool kFixedBuffers, bool kGlu = false>
__global__ __launch_bounds__(256, 2) void k_gemm(const uint8_t* __restrict__ packed, const float* __restrict__ gamma_ptr,
                                                 const int8_t* __restrict__ xq, const float* __restrict__ alpha,
                                                 int64_t m, int64_t n, int64_t k, int64_t blocks_n,
                                                 int32_t* __restrict__ acc_out, uint16_t* __restrict__ y_out) {
  constexpr int kBM = 16 * kTB;                       // tokens per workgroup
  constexpr int kWN = 16 * kRB;                       // weight rows per wave
  constexpr int kBN = kWaves * kWN;                   // weight rows per workgroup
  constexpr int kXDma = kBM * kStepK / 1024 / kWaves; // 1 KiB LDS-DMA loads per wave per step
  __shared__ uint4 xs0[kBM * kXRow];  // activation tile buffers: two distinct LDS objects
  __shared__ uint4 xs1[kBM * kXRow];
  __shared__ int row_sum[kBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int sub = lane >> 4;
  const int col = lane & 15;

  // Workgroups are dealt to the XCDs round-robin (id % 8).  Each XCD gets a
  // contiguous run of tiles in a grouped order: groups of kGroupN weight
  // blocks, token blocks outer and weight blocks inner within a group.  The
  // ~64 workgroups an XCD runs at once then cover about 8 weight blocks x 8
  // token blocks, whose operands both fit that XCD's 4 MB L2; each XCD reads
  // its share of the weights once and the activations once per group.
  constexpr int64_t kGroupN = 8;
  const int64_t tiles = (int64_t)gridDim.x;
  const int64_t blocks_m = tiles / blocks_n;
  const int64_t full = tiles / kXcds * kXcds;  // ids past the last full round keep their order
  const int64_t t = (int64_t)blockIdx.x >= full
                        ? (int64_t)blockIdx.x
                        : (int64_t)(blockIdx.x % kXcds) * (tiles / kXcds) + blockIdx.x / kXcds;
  const int64_t group = t / (kGroupN * blocks_m);
  const int64_t first_bn = group * kGroupN;
  const int64_t group_n = min(kGroupN, blocks_n - first_bn);
  const int64_t local = t - group * kGroupN * blocks_m;
  const int64_t bn = first_bn + local % group_n;
  const int64_t bm = local / group_n;
  const int64_t n0 = bn * kBN;
  const int64_t m0 = bm * kBM;
  const int kt_count = (int)(k / kTileCols);
  const int64_t row_tiles = (n + kTileRows - 1) / kTileRows;
  const int steps = (kt_count + 3) / 4;
  const int full_steps = kt_count / 4;  // steps whose four 64-column tiles all lie inside k
  const int64_t rt0 = n0 / kTileRows;
  const int tiles_here = (int)min((int64_t)(kBN / kTileRows), row_tiles - rt0);
  const int tokens_here = (int)min((int64_t)kBM, m - m0);
  const uint32_t kk = (uint32_t)k;

  // Raw buffer resources over this workgroup's weight row tiles and token
  // rows: reads past either end return zero.  All offsets fit in 32 bits.
  const __amdgpu_buffer_rsrc_t wrsrc =
      buffer_rsrc(packed + rt0 * kt_count * kTileBytes, (uint32_t)(tiles_here * kt_count * kTileBytes));
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(xq + m0 * k, (uint32_t)tokens_here * kk);

  // Activation tiles go global -> LDS by DMA (buffer_load ... lds): lane i of
  // a load writes LDS bytes 16i..16i+15 of that load's 1 KiB, i.e. token row
  // 4*load + i/16, stored chunk i%16.  Stored chunk p of row r holds source
  // chunk p ^ lds_row_key(r), so the lane fetches that one.
  const int dma_row0 = wave * kXDma * 4 + (lane >> 4);
  auto load_x = [&](int s, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXDma; ++j) {
      const int row = dma_row0 + 4 * j;
      const int c = (lane & 15) ^ lds_row_key(row);
      const uint32_t col_byte = (uint32_t)(s * kStepK + 16 * c);
      const uint32_t off = (s < full_steps || col_byte < kk) ? (uint32_t)row * kk + col_byte : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrsrc, (__attribute__((address_space(3))) void*)(dst + (wave * kXDma + j) * 64), 16, off, 0, 0, 0);
    }
  };
  // weights: row block rb of this wave, step s; lane = (tile sub, row col).
  // Past-the-end tiles of a partial step are clamped to the last tile: they
  // meet zero activations.
  const uint32_t w_off0 = (uint32_t)(wave * kRB * kt_count) * kTileBytes + (uint32_t)col * 16u;
  auto load_w = [&](int s, uint4* r) __attribute__((always_inline)) {
    const uint32_t kt = (uint32_t)min(4 * s + sub, kt_count - 1);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      r[rb] = buffer_load16(wrsrc, w_off0 + ((uint32_t)(rb * kt_count) + kt) * kTileBytes);
  };

  v4i acc[kRB][kTB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) acc[rb][tb] = v4i{0, 0, 0, 0};
  // Per-token activation sums, taken from the B operands already in
  // registers: wave w adds field w of every token block, so lane (col, sub)
  // holds, per token block tb, the sum over columns 16w..16w+15 of column tile
  // `sub` of every step for token tb*16 + col.
  int x_sum[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) x_sum[tb] = 0;
  if (tid < kBM) row_sum[tid] = 0;

  uint4 w_cur[kRB], w_next[kRB];
  load_w(0, w_cur);
  load_x(0, xs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto compute = [&](const uint4* xbuf) __attribute__((always_inline)) {
    // token row tb*16 + col, chunk 4*sub + f, stored at chunk (4*sub + f) ^ key
    const uint4* xt = xbuf + col * kXRow;
    const int key = lds_row_key(col);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      v4i b[kTB];
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) b[tb] = as_v4i(xt[tb * 16 * kXRow + ((4 * sub + f) ^ key)]);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        v4i a;
        a.x = (int)((w_cur[rb].x >> (2 * f)) & 0x03030303u);
        a.y = (int)((w_cur[rb].y >> (2 * f)) & 0x03030303u);
        a.z = (int)((w_cur[rb].z >> (2 * f)) & 0x03030303u);
        a.w = (int)((w_cur[rb].w >> (2 * f)) & 0x03030303u);
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) acc[rb][tb] = mfma_16x16x64(a, b[tb], acc[rb][tb]);
      }
      if (f == wave) {  // wave-uniform
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) {
          x_sum[tb] = __builtin_amdgcn_sdot4(b[tb].x, 0x01010101, x_sum[tb], false);
          x_sum[tb] = __builtin_amdgcn_sdot4(b[tb].y, 0x01010101, x_sum[tb], false);
          x_sum[tb] = __builtin_amdgcn_sdot4(b[tb].z, 0x01010101, x_sum[tb], false);
          x_sum[tb] = __builtin_amdgcn_sdot4(b[tb].w, 0x01010101, x_sum[tb], false);
        }
      }
    }
  };

  // one step: prefetch step s + 1 into wr, multiply the tile in rd
  auto step = [&](int s, const uint4* rd, uint4* wr) __attribute__((always_inline)) {
    load_w(s + 1, w_next);
    load_x(s + 1, wr);
    compute(rd);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA into wr has landed
    __syncthreads();                // ... and every other wave's, and nobody reads rd any more
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) w_cur[rb] = w_next[rb];
  };
  if constexpr (kFixedBuffers) {
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
  } else {
    for (int s = 0; s + 1 < steps; ++s) step(s, (s & 1) ? xs1 : xs0, (s & 1) ? xs0 : xs1);
    compute(((steps - 1) & 1) ? xs1 : xs0);
  }

  // per-token activation sums: add the four column-tile lanes of each token,
  // then the four waves' fields
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
    int v = x_sum[tb];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (sub == 0) atomicAdd(&row_sum[tb * 16 + col], v);
  }
  __syncthreads();

  const float gamma = *gamma_ptr;
  if constexpr (kGlu) {
    static_assert(kRB % 2 == 0, "gate/up row blocks come in pairs");
    const int64_t f = n / 2;
    const int64_t t0 = (n0 + wave * kWN) / (2 * kTileRows);  // gate tile of row blocks 0 and 1
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
      const int tok_local = tb * 16 + col;
      const int64_t tok = m0 + tok_local;
      if (tok >= m) continue;
      const int xsum = row_sum[tok_local];
      const float scale = (gamma * alpha[tok]) / 127.0f;
#pragma unroll
      for (int p = 0; p < kRB / 2; ++p) {
        const int64_t col0 = (t0 + p) * kTileRows + 4 * sub;  // four outputs of h
        if (col0 >= f) continue;
        const v4i& ga = acc[2 * p][tb];
        const v4i& ua = acc[2 * p + 1][tb];
        const float h[4] = {glu_value(ga.x - xsum, ua.x - xsum, scale), glu_value(ga.y - xsum, ua.y - xsum, scale),
                            glu_value(ga.z - xsum, ua.z - xsum, scale), glu_value(ga.w - xsum, ua.w - xsum, scale)};
        uint16_t* hp = y_out + tok * f + col0;  // f % 16 == 0: all four are inside the row
        if (((uintptr_t)hp & 7) == 0) {
          *reinterpret_cast<uint2*>(hp) = make_uint2(f32x2_to_bf16x2(h[0], h[1]), f32x2_to_bf16x2(h[2], h[3]));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) hp[i] = f32_to_bf16_rne(h[i]);
        }
      }
    }
    return;
  }
  // 4 consecutive outputs per lane: one 16-byte int32 / 8-byte bf16 store when
  // every row start is aligned for it
  const bool vec_ok = (n % 4) == 0 && ((uintptr_t)acc_out % 16) == 0 && ((uintptr_t)y_out % 8) == 0;
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
    const int tok_local = tb * 16 + col;
    const int64_t tok = m0 + tok_local;
    if (tok >= m) continue;
    const int xsum = row_sum[tok_local];
    const float scale = (gamma * alpha[tok]) / 127.0f;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      // this lane's four consecutive output rows row0..row0+3 for token tok
      const int64_t row0 = n0 + wave * kWN + rb * 16 + 4 * sub;
      const int vals[4] = {acc[rb][tb].x - xsum, acc[rb][tb].y - xsum, acc[rb][tb].z - xsum, acc[rb][tb].w - xsum};
      if (vec_ok && row0 + 3 < n) {
        if (acc_out) *reinterpret_cast<int4*>(acc_out + tok * n + row0) = make_int4(vals[0], vals[1], vals[2], vals[3]);
        if (y_out) {
          const uint32_t lo = f32x2_to_bf16x2((float)vals[0] * scale, (float)vals[1] * scale);
          const uint32_t hi = f32x2_to_bf16x2((float)vals[2] * scale, (float)vals[3] * scale);
          *reinterpret_cast<uint2*>(y_out + tok * n + row0) = make_uint2(lo, hi);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = row0 + i;
          if (row < n) {
            if (acc_out) acc_out[tok * n + row] = vals[i];
            if (y_out) y_out[tok * n + row] = f32_to_bf16_rne((float)vals[i] * scale);
          }
        }
      }
    }
  }
}

}  // namespace

namespace {

// Tile of the GEMM for an m x n product: the largest that still gives the
// chip enough workgroups -- 256 rows x 128 tokens with >= 4 per CU, else
// 256 x 64 with >= 2 per CU, else 128 x 64.
struct GemmTile {
  int64_t rows, toks;
};
GemmTile gemm_tile(int64_t m, int64_t n) {
  auto count = [&](int64_t rows, int64_t toks) { return ((n + rows - 1) / rows) * ((m + toks - 1) / toks); };
  if (count(256, 128) >= 1024) return {256, 128};
  if (count(256, 64) >= 512) return {256, 64};
  return {128, 64};
}

int64_t gemm_blocks(int64_t m, int64_t n) {
  const GemmTile t = gemm_tile(m, n);
  return ((n + t.rows - 1) / t.rows) * ((m + t.toks - 1) / t.toks);
}

template <bool kGlu>
hipError_t launch_gemm_impl(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                            int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s) {
  // Fixed buffers (unrolled steps, more registers) where they measured
  // faster: always for 128 x 64 tiles (same occupancy either way), for
  // 256 x 64 tiles only with long rows (the extra registers cost a
  // workgroup per CU, which the short-row shapes need more); the 256 x 128
  // tile does not fit its registers unrolled.
  const uint8_t* p = packed;
  auto launch = [&](auto kern, int64_t rows, int64_t toks) {
    const int64_t blocks_n = (n + rows - 1) / rows, blocks = ((m + toks - 1) / toks) * blocks_n;
    if (!grid_fits(blocks, 256)) return kErrGridTooLarge;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, p, gamma, xq, alpha, m, n, k, blocks_n, acc, y);
    return hipSuccess;
  };
  hipError_t e;
  const GemmTile t = gemm_tile(m, n);
  if (t.toks == 128)
    e = launch(k_gemm<8, 4, false, kGlu>, 256, 128);
  else if (t.rows == 256)
    e = k >= 8192 ? launch(k_gemm<4, 4, true, kGlu>, 256, 64) : launch(k_gemm<4, 4, false, kGlu>, 256, 64);
  else
    e = launch(k_gemm<4, 2, true, kGlu>, 128, 64);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

bool gemm_fits(int64_t m, int64_t n) { return grid_fits(gemm_blocks(m, n), 256); }

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                       int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s) {
  return launch_gemm_impl<false>(packed, gamma, xq, alpha, m, n, k, acc, y, s);
}

hipError_t launch_gemm_glu(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                           int64_t f, int64_t k, uint16_t* h, hipStream_t s) {
  return launch_gemm_impl<true>(packed, gamma, xq, alpha, m, 2 * f, k, nullptr, h, s);
}

}  // namespace bl
