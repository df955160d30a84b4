// Internal declarations of the BitLinear W1.58A8 HIP library (gfx950).
// Launchers are called only by the C ABI in abi.hip after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// Packed layout: 16-row x 64-column tiles of 256 bytes, column tile fastest.
constexpr int kTileRows = 16;
constexpr int kTileCols = 64;
constexpr int kTileBytes = 256;

// A launch of `blocks` workgroups of `threads` work-items fits the device:
// the grid's total work-item count must stay below 2^32.  Launchers return
// kErrGridTooLarge (before any HIP call) for a shape that would not fit; the
// C ABI reports it as BL_ERR_SHAPE.
constexpr hipError_t kErrGridTooLarge = hipErrorInvalidConfiguration;
inline bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 1 && blocks <= ((int64_t)1 << 32) / threads - 1;
}

// Weight packer (absmean exponent bins -> exact gamma -> ternarize + pack).
// The workspace holds the 256 exponent bins (u64) of the whole matrix; the
// absmean workgroups add into them with integer atomics (cleared first).
constexpr int kAbsmeanMaxBlocks = 256;
constexpr size_t kPackWorkspaceBytes = 256 * sizeof(unsigned long long);
hipError_t launch_absmean_bins(const float* w, int64_t count, unsigned long long* ws, hipStream_t s);
hipError_t launch_gamma_fold(const unsigned long long* ws, int64_t count, float* gamma, hipStream_t s);
// Device address of the library's static 2 KiB bin array (kPackWorkspaceBytes)
// on the device of stream `s`, for the allocation-free packer; looked up once
// per device (thread-safe), then cached.
hipError_t static_pack_bins(hipStream_t s, unsigned long long** bins);
// glu_f > 0: w is [2 * glu_f][k] gate rows then up rows, packed with
// alternating gate/up 16-row tiles (n == 2 * glu_f, glu_f % 16 == 0).
hipError_t launch_ternarize_pack(const float* w, int64_t n, int64_t k, const float* gamma, uint8_t* packed,
                                 hipStream_t s, int64_t glu_f = 0);
// Packed q^T ([k][n]) from packed q ([n][k]); n % 64 == 0.
hipError_t launch_pack_transposed(const uint8_t* packed, int64_t n, int64_t k, uint8_t* packed_t, hipStream_t s);
// Straight-through backward: dx = gamma * dy q from packed q^T; dw = dy^T (alpha / 127 qx).
hipError_t launch_backward_x(const uint8_t* packed_t, const float* gamma, const uint16_t* dy, int64_t m, int64_t n,
                             int64_t k, float* dx, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t s);
size_t backward_w_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_backward_w(const uint16_t* dy, const int8_t* xq, const float* alpha, int64_t m, int64_t n, int64_t k,
                             float* dw, void* workspace, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* q, hipStream_t s);

// Five trits per byte (base 3): 16-row x 320-column super-tiles of 1 KiB.
// The fused single-token decode holds a row's activations on chip: k up to
// kB3MaxK (25 super-tiles per wave of eight); m tokens run as m passes.
constexpr int64_t kB3MaxK = 64000;
constexpr int64_t kB3MaxM = 64;
size_t packed_bytes_b3(int64_t n, int64_t k);
hipError_t launch_ternarize_pack_b3(const float* w, int64_t n, int64_t k, const float* gamma, uint8_t* packed,
                                    hipStream_t s);
hipError_t launch_bitlinear_b3(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n,
                               int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, hipStream_t s);

// Per-token absmax int8 quantizer.
hipError_t launch_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* alpha, hipStream_t s);

// Ternary x int8 products: GEMV-style kernels that stream the weights once
// per 16 or 64 tokens (up to 16 tokens, and up to 64 unless the matrix has
// enough rows to keep the GEMM's larger tiles busy), else the LDS-tiled GEMM.
inline bool gemv_serves(int64_t m, int64_t n) { return m <= 16 || (m <= 64 && (n + 15) / 16 < 2048); }
hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                       int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s);
// Fused per-token quantization + product for a small token block
// (gemv_fused_applies: one token, or m * k small); writes xq/alpha (if non-NULL)
// exactly as launch_quant_act would.
bool gemv_fused_applies(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_fused(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n,
                             int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                       int64_t n, int64_t k, int32_t* acc, uint16_t* y, hipStream_t s);
// The GEMM's grid fits the device for an m x n product.
bool gemm_fits(int64_t m, int64_t n);

// Squared-ReLU gated products from gate+up weights packed with alternating
// gate/up row tiles (n = 2f rows): h[i][j] = bf16(relu(g)^2 * u), g and u the
// rescaled products of gate row j and up row j; h is [m][f].
hipError_t launch_gemv_glu(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                           int64_t f, int64_t k, uint16_t* h, hipStream_t s);
hipError_t launch_gemm_glu(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                           int64_t f, int64_t k, uint16_t* h, hipStream_t s);
// One kernel for quantization + gated product, where the single-token (or
// few-token, short-row) kernel applies.
bool gemv_fused_glu_applies(int64_t m, int64_t f, int64_t k);
hipError_t launch_gemv_fused_glu(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t f,
                                 int64_t k, int8_t* xq, float* alpha, uint16_t* h, hipStream_t s);

}  // namespace bl
