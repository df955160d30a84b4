// Five trits per byte: the denser weight code of BitLinear W1.58A8.
//
// bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution", section
// "The Information Theory of 1.58 Bits": a three-state weight carries
// log2(3), about 1.58, bits; deepmox.com chapter 1, "Why Smaller Weights Are
// Not the Whole Story", section "A different place to make efficiency
// decisions": the 2B4T model keeps its non-embedding weights in 0.4 GB, less
// than two bits per weight.  3^5 = 243 <= 256, so five trits fit one byte:
// 1.6 bits per weight, 20% fewer bytes than four trits per byte.
//
// Code: codes c_d = t_d + 1 (d = 0..4) form v = sum_d c_d * 3^(4-d) and the
// byte is b = ceil(256 v / 243), the base-3 fraction v / 243 scaled to a
// byte and rounded up.  Rounding up keeps b / 256 in [v / 243, (v + 1) / 243),
// so digit d is the carry out of the low byte when (b * 3^d mod 256) is
// multiplied by 3: c_0 = (3 b) >> 8, then p <- (3 p) & 0xFF, c_d = (3 p) >> 8.
// Layout: 16-row x 320-column super-tiles of 1024 bytes, column super-tile
// fastest; in a super-tile, column 80 g + 16 d + j of row r sits in byte
// 256 g + 16 r + j as digit d.  A wave's 128-bit load of a super-tile (lane l
// reads bytes 16 l..16 l + 15: group l / 16, row l % 16) is 1 KiB contiguous,
// and digit d of a lane's 16 bytes is the 16 consecutive columns
// 80 g + 16 d .. + 15 of its row: one MFMA operand (k-slot group l / 16).
//
// Decode without masks: a lane splits each of its four dwords into the even
// bytes (p_lo = bytes 0, 2 in 16-bit lanes) and the odd bytes (p_hi = bytes
// 1, 3).  t = 3 p then holds the digit codes of its two bytes in bytes 1 and
// 3 (t < 3 * 256 per 16-bit lane), and the low parts (bytes 0 and 2) are the
// next p.  t itself is the MFMA operand: the activation operand carries
// zeros in bytes 0 and 2 of every dword, so those bytes add nothing.  Per
// digit and dword: two multiplies and two ANDs; no byte shuffles.  Each
// digit takes two MFMAs (even and odd bytes), ten per 16 weight bytes.
#include "device_util.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kSuperCols = 320;
constexpr int kSuperBytes = 1024;
constexpr int kExpBytes = 640;  // LDS bytes of one super-tile's expanded activation codes

// ---------------------------------------------------------------- packer

// One thread per packed dword: bytes 4 q .. 4 q + 3 (q % 4) of group g, row r
// of super-tile (band, s); a 256-thread workgroup writes one super-tile.
// Digit d of byte j holds column 320 s + 80 g + 16 d + j, so each of the
// five digits is one float4 load of 4 consecutive columns.  The rounding of
// w / (gamma + 1e-5) is the exact threshold test |w| > d / 2 (as in the
// 2-bit packer).  Rows past n and columns past k hold trit 0.
__global__ __launch_bounds__(256) void k_ternarize_pack_b3(const float4* __restrict__ w4, int64_t n, int64_t k,
                                                           const float* __restrict__ gamma_ptr,
                                                           uint32_t* __restrict__ packed) {
  const int64_t supers = (k + kSuperCols - 1) / kSuperCols;
  const int64_t band = (int64_t)blockIdx.x / supers;
  const int64_t s = (int64_t)blockIdx.x % supers;
  const int q = threadIdx.x;
  const int g = q >> 6, r = (q >> 2) & 15, j0 = 4 * (q & 3);
  const int64_t row = band * kTileRows + r;
  const float half_d = (*gamma_ptr + 1e-5f) * 0.5f;
  const int64_t k4 = k / 4;
  float4 v[5];
#pragma unroll
  for (int d = 0; d < 5; ++d) {
    const int64_t col = s * kSuperCols + 80 * g + 16 * d + j0;  // 4 columns, all inside k or all past it
    v[d] = (row < n && col < k) ? w4[row * k4 + col / 4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  auto code = [&](float x) { return fabsf(x) > half_d ? (x < 0.0f ? 0u : 2u) : 1u; };
  uint32_t val[4] = {0, 0, 0, 0};  // base-3 value of bytes j0 .. j0 + 3
#pragma unroll
  for (int d = 0; d < 5; ++d) {
    val[0] = 3 * val[0] + code(v[d].x);
    val[1] = 3 * val[1] + code(v[d].y);
    val[2] = 3 * val[2] + code(v[d].z);
    val[3] = 3 * val[3] + code(v[d].w);
  }
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) out |= ((256u * val[i] + 242u) / 243u) << (8 * i);  // ceil(256 v / 243)
  packed[(int64_t)blockIdx.x * (kSuperBytes / 4) + q] = out;
}

// ---------------------------------------------------------------- decode

// Even (p_lo) and odd (p_hi) bytes of a dword in 16-bit lanes.
__device__ __forceinline__ uint32_t even_bytes(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x0c020c00u); }
__device__ __forceinline__ uint32_t odd_bytes(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x0c030c01u); }

// BitLinear for one token (blockIdx.y) of five-trits-per-byte weights,
// quantization fused: the single-token kernel of the 2-bit code with the
// base-3 decode.  Wave w of kW multiplies super-tiles w, w + kW, ... of every
// row band of the workgroup and quantizes exactly those columns of the token
// into its own LDS region, expanded for the even/odd operands: for group g,
// digit d, 16 bytes [0, x_0, 0, x_2, 0, x_4, ...] then [0, x_1, 0, x_3, ...]
// (x_j the code of column 80 g + 16 d + j).  The token's absmax comes from
// the waves' maxima through LDS (one barrier); each wave subtracts the
// activation sum of its own columns (the MFMAs take the codes c = t + 1), and
// one barrier combines the waves.  Slot i of lane l holds 16-byte bf16 chunk
// 64 i + l of the wave's own columns (40 per super-tile); chunks past k read
// as zero.  kRT consecutive row bands per workgroup share the quantized token;
// the stream runs super-tile outer, band inner, so each super-tile's
// activation operands are read from LDS once for all bands (measured 7-14%
// faster than band outer; four super-tiles per batch instead of two, and
// four waves on rows of up to 40 super-tiles, measured no faster).
template <int kRT, int kC, int kW>
__global__ __launch_bounds__(kW * 64) void k_bitlinear_b3(const uint4* __restrict__ packed,
                                                          const float* __restrict__ gamma_ptr,
                                                          const uint4* __restrict__ x, float* __restrict__ alpha,
                                                          int8_t* __restrict__ xq_out, int n, int k,
                                                          int32_t* __restrict__ acc_out, uint16_t* __restrict__ y_out) {
  constexpr int kB = 2;  // super-tiles per prefetch batch (4 measured slower)
  extern __shared__ uint4 xe_raw[];  // [wave][own super-tile rank][640 bytes]
  __shared__ v4i partial[kRT][kW][64];
  __shared__ int wave_max[kW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok = blockIdx.y;
  const int band0 = blockIdx.x * kRT;
  const int bands = (n + kTileRows - 1) / kTileRows;
  const int bands_here = min(kRT, bands - band0);
  const int supers = (k + kSuperCols - 1) / kSuperCols;
  const int my_supers = (supers - wave + kW - 1) / kW;
  const int max_supers = (supers + kW - 1) / kW;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int k8 = k / 8;

  // activations first (loads retire in order): chunk c = 64 i + lane of the
  // wave's own columns is chunk c % 40 of own super-tile c / 40
  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(x + (int64_t)tok * k8, (uint32_t)(k * 2));
  uint4 xr[kC];
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const int c = 64 * i + lane;
    const int rank = c / 40;
    const int chunk = (wave + kW * rank) * 40 + c % 40;  // 16-byte bf16 chunk of the row
    xr[i] = buffer_load16(xrsrc, rank < my_supers && chunk < k8 ? (uint32_t)chunk * 16u : kOutOfRange);
  }
  // weights: one resource per row band, so that a band past n, and a
  // super-tile past this wave's share, read as zero bytes; a zero byte
  // decodes to codes 0, which add nothing to the products
  const uint32_t band_bytes = (uint32_t)supers * kSuperBytes;
  auto band_rsrc = [&](int rt) {
    return buffer_rsrc(packed + (size_t)(band0 + rt) * supers * (kSuperBytes / 16), rt < bands_here ? band_bytes : 0u);
  };
  auto w_off = [&](int gi) { return (uint32_t)((wave + gi * kW) * kSuperBytes + lane * 16); };
  uint4 a_cur[kB];
  {
    const __amdgpu_buffer_rsrc_t r0 = band_rsrc(0);
#pragma unroll
    for (int u = 0; u < kB; ++u) a_cur[u] = buffer_load16_stream(r0, w_off(u));
  }
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  __builtin_amdgcn_sched_barrier(0);

  // the token's absmax: this wave's columns, then the waves' maxima
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < kC; ++i) m2 = absmax_step(m2, xr[i]);
  const int wmax = wave_reduce<true>((int)max(m2.x, m2.y));
  if (lane == 0) wave_max[wave] = wmax;
  __syncthreads();
  int mx = wave_max[0];
#pragma unroll
  for (int w = 1; w < kW; ++w) mx = max(mx, wave_max[w]);
  const float amax = __uint_as_float((uint32_t)mx << 16);
  const float s = 127.0f / fmaxf(amax, 1e-5f);  // IEEE division, as in bl_quant_act

  // quantize own chunks into the expanded LDS layout; chunk e (0..39) of a
  // super-tile is columns 8 e .. 8 e + 7: group e / 10, digit (e % 10) / 2,
  // bytes j0 = 8 (e % 2) .. + 7 of that 16-column run
  uint8_t* region = reinterpret_cast<uint8_t*>(xe_raw) + wave * max_supers * kExpBytes;
  const bool first_block = blockIdx.x == 0;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const int c = 64 * i + lane;
    const int rank = c / 40;
    if (rank < my_supers) {
      const int e = c % 40;
      const int chunk = (wave + kW * rank) * 40 + e;
      const uint2 q = act_codes8(xr[i], s, sum);  // codes of columns 8 e .. 8 e + 7 (zero past k)
      uint8_t* dst = region + rank * kExpBytes + (e / 2) * 32 + (e % 2) * 8;
      // even-column operand bytes [0, x0, 0, x2, 0, x4, 0, x6], odd-column [0, x1, 0, x3, ...]
      const uint2 lo = make_uint2(__builtin_amdgcn_perm(q.x, 0u, 0x060c040cu), __builtin_amdgcn_perm(q.y, 0u, 0x060c040cu));
      const uint2 hi = make_uint2(__builtin_amdgcn_perm(q.x, 0u, 0x070c050cu), __builtin_amdgcn_perm(q.y, 0u, 0x070c050cu));
      *reinterpret_cast<uint2*>(dst) = lo;
      *reinterpret_cast<uint2*>(dst + 16) = hi;
      if (first_block && xq_out && chunk < k8) reinterpret_cast<uint2*>(xq_out + (int64_t)tok * k)[chunk] = q;
    }
  }
  sum = wave_reduce<false>(sum);
  if (first_block && wave == 0 && lane == 0 && alpha) alpha[tok] = amax;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes before its reads

  // super-tile outer, row band inner: a super-tile's activation operands are
  // read from LDS once and serve every band of the workgroup
  v4i acc[kRT][2];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) acc[rt][0] = acc[rt][1] = v4i{0, 0, 0, 0};
  uint4 w_cur[kRT][kB];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const __amdgpu_buffer_rsrc_t r = band_rsrc(rt);
#pragma unroll
    for (int u = 0; u < kB; ++u) w_cur[rt][u] = rt == 0 ? a_cur[u] : buffer_load16_stream(r, w_off(u));
  }
  for (int gi = 0; gi < my_supers; gi += kB) {
    uint4 w_nxt[kRT][kB];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const __amdgpu_buffer_rsrc_t r = band_rsrc(rt);
#pragma unroll
      for (int u = 0; u < kB; ++u) w_nxt[rt][u] = buffer_load16_stream(r, w_off(gi + kB + u));
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int gl = min(gi + u, max_supers - 1);
      const uint8_t* xb = region + gl * kExpBytes + g * 5 * 32;
      v4i blo[5], bhi[5];
#pragma unroll
      for (int d = 0; d < 5; ++d) {
        blo[d] = as_v4i(*reinterpret_cast<const uint4*>(xb + d * 32));
        bhi[d] = as_v4i(*reinterpret_cast<const uint4*>(xb + d * 32 + 16));
      }
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const uint4 a = w_cur[rt][u];
        uint32_t plo[4] = {even_bytes(a.x), even_bytes(a.y), even_bytes(a.z), even_bytes(a.w)};
        uint32_t phi[4] = {odd_bytes(a.x), odd_bytes(a.y), odd_bytes(a.z), odd_bytes(a.w)};
#pragma unroll
        for (int d = 0; d < 5; ++d) {
          v4i tlo, thi;
          tlo.x = (int)(plo[0] + (plo[0] << 1));
          tlo.y = (int)(plo[1] + (plo[1] << 1));
          tlo.z = (int)(plo[2] + (plo[2] << 1));
          tlo.w = (int)(plo[3] + (plo[3] << 1));
          thi.x = (int)(phi[0] + (phi[0] << 1));
          thi.y = (int)(phi[1] + (phi[1] << 1));
          thi.z = (int)(phi[2] + (phi[2] << 1));
          thi.w = (int)(phi[3] + (phi[3] << 1));
          acc[rt][0] = mfma_16x16x64(tlo, blo[d], acc[rt][0]);
          acc[rt][1] = mfma_16x16x64(thi, bhi[d], acc[rt][1]);
          if (d < 4) {
            plo[0] = (uint32_t)tlo.x & 0x00FF00FFu;
            plo[1] = (uint32_t)tlo.y & 0x00FF00FFu;
            plo[2] = (uint32_t)tlo.z & 0x00FF00FFu;
            plo[3] = (uint32_t)tlo.w & 0x00FF00FFu;
            phi[0] = (uint32_t)thi.x & 0x00FF00FFu;
            phi[1] = (uint32_t)thi.y & 0x00FF00FFu;
            phi[2] = (uint32_t)thi.z & 0x00FF00FFu;
            phi[3] = (uint32_t)thi.w & 0x00FF00FFu;
          }
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int u = 0; u < kB; ++u) w_cur[rt][u] = w_nxt[rt][u];
  }
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    v4i part = acc[rt][0];
    add4(part, acc[rt][1]);
    part.x -= sum;
    part.y -= sum;
    part.z -= sum;
    part.w -= sum;
    partial[rt][wave][lane] = part;
  }
  __syncthreads();
  if (col != 0) return;  // MFMA column 0 carries the token (all columns hold it)
  const float scale = (gamma * amax) / 127.0f;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    if (rt % kW != wave || rt >= bands_here) continue;
    v4i acc = partial[rt][0][lane];
#pragma unroll
    for (int w = 1; w < kW; ++w) add4(acc, partial[rt][w][lane]);
    store_tile(acc, (int64_t)(band0 + rt) * kTileRows + 4 * g, tok, n, scale, acc_out, y_out);
  }
}

// The same product for matrices with many row bands: wave w of the kW owns
// the whole row band blockIdx.x * kW + w (all its super-tiles), so the
// stream needs no cross-wave sums and no barrier after the quantization;
// the workgroup quantizes the token once, into one expanded copy in LDS
// that every wave reads.  Chunk c of the row goes to thread c % (64 kW),
// slot c / (64 kW); the token's absmax and activation sum are reduced over
// the workgroup through LDS (two barriers, both before the stream).
template <int kW, int kC>
__global__ __launch_bounds__(kW * 64) void k_bitlinear_b3_band(const uint4* __restrict__ packed,
                                                               const float* __restrict__ gamma_ptr,
                                                               const uint4* __restrict__ x, float* __restrict__ alpha,
                                                               int8_t* __restrict__ xq_out, int n, int k,
                                                               int32_t* __restrict__ acc_out,
                                                               uint16_t* __restrict__ y_out) {
  constexpr int kT = kW * 64;
  constexpr int kB = 4;  // super-tiles per prefetch batch
  extern __shared__ uint4 xe_raw[];  // [super-tile][640 bytes]
  __shared__ int red[2][kW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok = blockIdx.y;
  const int bands = (n + kTileRows - 1) / kTileRows;
  const int band = blockIdx.x * kW + wave;
  const int supers = (k + kSuperCols - 1) / kSuperCols;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int k8 = k / 8;

  const __amdgpu_buffer_rsrc_t xrsrc = buffer_rsrc(x + (int64_t)tok * k8, (uint32_t)(k * 2));
  uint4 xr[kC];
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const int c = (int)threadIdx.x + kT * i;
    xr[i] = buffer_load16(xrsrc, c < k8 ? (uint32_t)c * 16u : kOutOfRange);
  }
  // this wave's band: one resource (a band past n reads zero bytes, whose
  // codes 0 add nothing), super-tiles in order
  const __amdgpu_buffer_rsrc_t wrsrc =
      buffer_rsrc(packed + (size_t)band * supers * (kSuperBytes / 16), band < bands ? (uint32_t)supers * kSuperBytes : 0u);
  auto w_off = [&](int st) { return (uint32_t)(st * kSuperBytes + lane * 16); };
  uint4 a_cur[kB];
#pragma unroll
  for (int u = 0; u < kB; ++u) a_cur[u] = buffer_load16_stream(wrsrc, w_off(u));
  const float gamma = buffer_load_f32(buffer_rsrc(gamma_ptr, 4), 0);
  __builtin_amdgcn_sched_barrier(0);

  u16x2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < kC; ++i) m2 = absmax_step(m2, xr[i]);
  int v = wave_reduce<true>((int)max(m2.x, m2.y));
  if (lane == 0) red[0][wave] = v;
  __syncthreads();
  int mx = red[0][0];
#pragma unroll
  for (int w = 1; w < kW; ++w) mx = max(mx, red[0][w]);
  const float amax = __uint_as_float((uint32_t)mx << 16);
  const float s = 127.0f / fmaxf(amax, 1e-5f);  // IEEE division, as in bl_quant_act

  uint8_t* region = reinterpret_cast<uint8_t*>(xe_raw);
  const bool first_block = blockIdx.x == 0;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const int c = (int)threadIdx.x + kT * i;
    if (c < supers * 40) {  // chunks of the padded last super-tile are zero codes
      const uint2 q = act_codes8(xr[i], s, sum);
      const int st = c / 40, e = c % 40;
      uint8_t* dst = region + st * kExpBytes + (e / 2) * 32 + (e % 2) * 8;
      const uint2 lo = make_uint2(__builtin_amdgcn_perm(q.x, 0u, 0x060c040cu), __builtin_amdgcn_perm(q.y, 0u, 0x060c040cu));
      const uint2 hi = make_uint2(__builtin_amdgcn_perm(q.x, 0u, 0x070c050cu), __builtin_amdgcn_perm(q.y, 0u, 0x070c050cu));
      *reinterpret_cast<uint2*>(dst) = lo;
      *reinterpret_cast<uint2*>(dst + 16) = hi;
      if (first_block && xq_out && c < k8) reinterpret_cast<uint2*>(xq_out + (int64_t)tok * k)[c] = q;
    }
  }
  v = wave_reduce<false>(sum);
  if (lane == 0) red[1][wave] = v;
  if (first_block && wave == 0 && lane == 0 && alpha) alpha[tok] = amax;
  __syncthreads();
  int xsum = red[1][0];
#pragma unroll
  for (int w = 1; w < kW; ++w) xsum += red[1][w];

  v4i acc0 = {0, 0, 0, 0}, acc1 = acc0;
  for (int st = 0; st < supers; st += kB) {
    uint4 a_nxt[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) a_nxt[u] = buffer_load16_stream(wrsrc, w_off(st + kB + u));  // past the row: zero
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int sl = min(st + u, supers - 1);  // past the row: zero codes, any operands
      const uint8_t* xb = region + sl * kExpBytes + g * 5 * 32;
      const uint4 a = a_cur[u];
      uint32_t plo[4] = {even_bytes(a.x), even_bytes(a.y), even_bytes(a.z), even_bytes(a.w)};
      uint32_t phi[4] = {odd_bytes(a.x), odd_bytes(a.y), odd_bytes(a.z), odd_bytes(a.w)};
#pragma unroll
      for (int d = 0; d < 5; ++d) {
        v4i tlo, thi;
        tlo.x = (int)(plo[0] + (plo[0] << 1));
        tlo.y = (int)(plo[1] + (plo[1] << 1));
        tlo.z = (int)(plo[2] + (plo[2] << 1));
        tlo.w = (int)(plo[3] + (plo[3] << 1));
        thi.x = (int)(phi[0] + (phi[0] << 1));
        thi.y = (int)(phi[1] + (phi[1] << 1));
        thi.z = (int)(phi[2] + (phi[2] << 1));
        thi.w = (int)(phi[3] + (phi[3] << 1));
        acc0 = mfma_16x16x64(tlo, as_v4i(*reinterpret_cast<const uint4*>(xb + d * 32)), acc0);
        acc1 = mfma_16x16x64(thi, as_v4i(*reinterpret_cast<const uint4*>(xb + d * 32 + 16)), acc1);
        if (d < 4) {
          plo[0] = (uint32_t)tlo.x & 0x00FF00FFu;
          plo[1] = (uint32_t)tlo.y & 0x00FF00FFu;
          plo[2] = (uint32_t)tlo.z & 0x00FF00FFu;
          plo[3] = (uint32_t)tlo.w & 0x00FF00FFu;
          phi[0] = (uint32_t)thi.x & 0x00FF00FFu;
          phi[1] = (uint32_t)thi.y & 0x00FF00FFu;
          phi[2] = (uint32_t)thi.z & 0x00FF00FFu;
          phi[3] = (uint32_t)thi.w & 0x00FF00FFu;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) a_cur[u] = a_nxt[u];
  }
  if (col != 0 || band >= bands) return;
  add4(acc0, acc1);
  acc0.x -= xsum;
  acc0.y -= xsum;
  acc0.z -= xsum;
  acc0.w -= xsum;
  store_tile(acc0, (int64_t)band * kTileRows + 4 * g, tok, n, (gamma * amax) / 127.0f, acc_out, y_out);
}

}  // namespace
}  // namespace bl

namespace bl {

size_t packed_bytes_b3(int64_t n, int64_t k) {
  return (size_t)((n + kTileRows - 1) / kTileRows * kTileRows) * (size_t)((k + 319) / 320 * 64);
}

hipError_t launch_ternarize_pack_b3(const float* w, int64_t n, int64_t k, const float* gamma, uint8_t* packed,
                                    hipStream_t s) {
  const int64_t blocks = (n + kTileRows - 1) / kTileRows * ((k + 319) / 320);
  if (!grid_fits(blocks, 256)) return kErrGridTooLarge;
  hipLaunchKernelGGL(k_ternarize_pack_b3, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(w),
                     n, k, gamma, reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

namespace {

typedef void (*B3Kernel)(const uint4*, const float*, const uint4*, float*, int8_t*, int, int, int32_t*, uint16_t*);

template <int kRT>
B3Kernel b3_pick(int waves, int64_t slots) {
  if (waves == 4) return slots <= 2 ? k_bitlinear_b3<kRT, 2, 4> : nullptr;
  if (slots <= 2) return k_bitlinear_b3<kRT, 2, 8>;
  if (slots <= 4) return k_bitlinear_b3<kRT, 4, 8>;
  if (slots <= 8) return k_bitlinear_b3<kRT, 8, 8>;
  if (slots <= 16) return k_bitlinear_b3<kRT, 16, 8>;
  return nullptr;
}

}  // namespace

hipError_t launch_bitlinear_b3(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n,
                               int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, hipStream_t s) {
  if (k > kB3MaxK || m > 65535) return kErrGridTooLarge;
  const int64_t supers = (k + 319) / 320, bands = (n + kTileRows - 1) / kTileRows;
  if (bands >= 2048 && supers <= 51) {
    // a whole band per wave, eight waves per workgroup: on the 70B-shaped
    // gate+up (3584 bands of 26 super-tiles) 29.4 against 33.6 us for the
    // split-row kernel below
    const int64_t slots = (supers * 40 + 511) / 512;
    auto kern = slots <= 2 ? k_bitlinear_b3_band<8, 2> : k_bitlinear_b3_band<8, 4>;
    const dim3 grid((unsigned)((bands + 7) / 8), (unsigned)m);
    if (!grid_fits(grid.x, 512)) return kErrGridTooLarge;
    hipLaunchKernelGGL(kern, grid, dim3(512), (size_t)supers * kExpBytes, s, reinterpret_cast<const uint4*>(packed),
                       gamma, reinterpret_cast<const uint4*>(x), alpha, xq, (int)n, (int)k, acc, y);
    return hipGetLastError();
  }
  // four waves for short rows, eight (each quantizing and streaming half as
  // many super-tiles) for longer ones; two row bands per workgroup (sharing
  // the quantized token) once there are ~2-4 per CU
  const int waves = supers <= 12 ? 4 : 8;
  const int64_t max_supers = (supers + waves - 1) / waves;
  const int64_t slots = (40 * max_supers + 63) / 64;
  const int rt = (bands >= 512 && k <= 4096) || bands >= 1024 ? 2 : 1;
  const B3Kernel kern = rt == 2 ? b3_pick<2>(waves, slots) : b3_pick<1>(waves, slots);
  if (!kern) return kErrGridTooLarge;
  const dim3 grid((unsigned)((bands + rt - 1) / rt), (unsigned)m);
  if (!grid_fits(grid.x, 64 * waves)) return kErrGridTooLarge;
  const size_t lds = (size_t)waves * (size_t)max_supers * kExpBytes;
  hipLaunchKernelGGL(kern, grid, dim3(64 * waves), lds, s, reinterpret_cast<const uint4*>(packed), gamma,
                     reinterpret_cast<const uint4*>(x), alpha, xq, (int)n, (int)k, acc, y);
  return hipGetLastError();
}

}  // namespace bl
