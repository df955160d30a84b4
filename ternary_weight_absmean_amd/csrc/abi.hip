// C ABI of the BitLinear W1.58A8 library: argument validation and dispatch.
// Declarations, argument meaning, layouts and error behaviour: include/bitlinear.h.
#include "../../include/bitlinear.h"
#include "internal.h"

namespace {

constexpr int64_t kLimit40 = (int64_t)1 << 40;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool valid_k(int64_t k) { return k >= 64 && k <= BL_MAX_K && k % 64 == 0; }

bool product_ok(int64_t a, int64_t b) { return a == 0 || b < kLimit40 / a; }

// A launch grid beyond the device's work-item limit is a shape error (the
// launchers detect it before any HIP call); any other failure is the runtime's.
bl_status from_hip(hipError_t e) {
  return e == hipSuccess ? BL_OK : e == bl::kErrGridTooLarge ? BL_ERR_SHAPE : BL_ERR_HIP;
}

// Largest weight count the packer takes: its grid covers n * k / 16 work-items.
constexpr int64_t kMaxPackWeights = (int64_t)1 << 35;

}  // namespace

extern "C" {

size_t bl_packed_bytes(int64_t n, int64_t k) {
  if (n < 0 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k)) return 0;
  return (size_t)((n + 15) / 16 * 16) * (size_t)(k / 4);
}

size_t bl_ternarize_pack_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k)) return 0;
  return bl::kPackWorkspaceBytes;
}

bl_status bl_ternarize_pack(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!w || !packed || !gamma || !workspace) return BL_ERR_NULL;
  if (n < 1 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k) || n * k > kMaxPackWeights) return BL_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(workspace, 16)) return BL_ERR_ALIGN;
  if (workspace_bytes < bl_ternarize_pack_workspace_bytes(n, k)) return BL_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* bins = (unsigned long long*)workspace;
  hipError_t e = bl::launch_absmean_bins(w, n * k, bins, s);
  if (e == hipSuccess) e = bl::launch_gamma_fold(bins, n * k, gamma, s);
  if (e == hipSuccess) e = bl::launch_ternarize_pack(w, n, k, gamma, packed, s);
  return from_hip(e);
}

bl_status bl_ternarize_pack_noalloc(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma,
                                    void* stream) {
  if (!w || !packed || !gamma) return BL_ERR_NULL;
  if (n < 1 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k) || n * k > kMaxPackWeights) return BL_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4)) return BL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* bins = nullptr;  // the static array's device address, never its host-side name
  hipError_t e = bl::static_pack_bins(s, &bins);
  if (e == hipSuccess) e = bl::launch_absmean_bins(w, n * k, bins, s);
  if (e == hipSuccess) e = bl::launch_gamma_fold(bins, n * k, gamma, s);
  if (e == hipSuccess) e = bl::launch_ternarize_pack(w, n, k, gamma, packed, s);
  return from_hip(e);
}

size_t bl_packed_bytes_b3(int64_t n, int64_t k) {
  if (n < 0 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k)) return 0;
  return bl::packed_bytes_b3(n, k);
}

bl_status bl_ternarize_pack_b3(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!w || !packed || !gamma || !workspace) return BL_ERR_NULL;
  if (n < 1 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k) || n * k > kMaxPackWeights) return BL_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(workspace, 16)) return BL_ERR_ALIGN;
  if (workspace_bytes < bl_ternarize_pack_workspace_bytes(n, k)) return BL_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* bins = (unsigned long long*)workspace;
  hipError_t e = bl::launch_absmean_bins(w, n * k, bins, s);
  if (e == hipSuccess) e = bl::launch_gamma_fold(bins, n * k, gamma, s);
  if (e == hipSuccess) e = bl::launch_ternarize_pack_b3(w, n, k, gamma, packed, s);
  return from_hip(e);
}

bl_status bl_bitlinear_b3(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n,
                          int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, void* stream) {
  if (m < 0 || m > BL_B3_MAX_M || n < 0 || n > BL_MAX_N || !valid_k(k) || k > BL_B3_MAX_K || !product_ok(n + 16, k))
    return BL_ERR_SHAPE;
  if (m == 0 || n == 0) return BL_OK;  // empty tensors may carry NULL pointers
  if (!packed || !gamma || !x || !xq || !alpha || (!acc && !y)) return BL_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(xq, 16) || !aligned(gamma, 4) || !aligned(alpha, 4) ||
      (acc && !aligned(acc, 4)) || (y && !aligned(y, 2)))
    return BL_ERR_ALIGN;
  return from_hip(bl::launch_bitlinear_b3(packed, gamma, x, m, n, k, xq, alpha, acc, y, (hipStream_t)stream));
}

bl_status bl_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* alpha, void* stream) {
  if (m < 0 || m > BL_MAX_M || !valid_k(k) || !product_ok(m, k)) return BL_ERR_SHAPE;
  if (m == 0) return BL_OK;  // empty tensors may carry NULL pointers
  if (!x || !xq || !alpha) return BL_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(alpha, 4)) return BL_ERR_ALIGN;
  return from_hip(bl::launch_quant_act(x, m, k, xq, alpha, (hipStream_t)stream));
}

bl_status bl_linear(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                    int64_t n, int64_t k, int32_t* acc, uint16_t* y, void* stream) {
  if (m < 0 || m > BL_MAX_M || n < 0 || n > BL_MAX_N || !valid_k(k) || !product_ok(m, k) || !product_ok(n + 16, k) ||
      !product_ok(m, n))
    return BL_ERR_SHAPE;
  if (m == 0 || n == 0) return BL_OK;  // empty tensors may carry NULL pointers
  if (!packed || !gamma || !xq || !alpha || (!acc && !y)) return BL_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(xq, 16) || !aligned(gamma, 4) || !aligned(alpha, 4) ||
      (acc && !aligned(acc, 4)) || (y && !aligned(y, 2)))
    return BL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (bl::gemv_serves(m, n)) return from_hip(bl::launch_gemv(packed, gamma, xq, alpha, m, n, k, acc, y, s));
  return from_hip(bl::launch_gemm(packed, gamma, xq, alpha, m, n, k, acc, y, s));
}

bl_status bl_bitlinear(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                       int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, void* stream) {
  if (m < 0 || m > BL_MAX_M || n < 0 || n > BL_MAX_N || !valid_k(k) || !product_ok(m, k) || !product_ok(n + 16, k) ||
      !product_ok(m, n))
    return BL_ERR_SHAPE;
  if (m == 0) return BL_OK;  // empty tensors may carry NULL pointers
  if (!x || !xq || !alpha || (n > 0 && (!packed || !gamma || (!acc && !y)))) return BL_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(alpha, 4) || (n > 0 && (!aligned(packed, 16) ||
      !aligned(gamma, 4) || (acc && !aligned(acc, 4)) || (y && !aligned(y, 2)))))
    return BL_ERR_ALIGN;
  if (n > 0 && !bl::gemv_serves(m, n) && !bl::gemm_fits(m, n)) return BL_ERR_SHAPE;  // before the quantizer runs
  hipStream_t s = (hipStream_t)stream;
  if (n > 0 && bl::gemv_fused_applies(m, n, k))
    return from_hip(bl::launch_gemv_fused(packed, gamma, x, m, n, k, xq, alpha, acc, y, s));
  hipError_t e = bl::launch_quant_act(x, m, k, xq, alpha, s);
  if (e != hipSuccess || n == 0) return from_hip(e);
  if (bl::gemv_serves(m, n)) return from_hip(bl::launch_gemv(packed, gamma, xq, alpha, m, n, k, acc, y, s));
  return from_hip(bl::launch_gemm(packed, gamma, xq, alpha, m, n, k, acc, y, s));
}

bl_status bl_ternarize_pack_glu(const float* w, int64_t f, int64_t k, uint8_t* packed, float* gamma, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!w || !packed || !gamma || !workspace) return BL_ERR_NULL;
  if (f < 16 || f % 16 != 0 || 2 * f > BL_MAX_N || !valid_k(k) || !product_ok(2 * f + 16, k) ||
      2 * f * k > kMaxPackWeights)
    return BL_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(workspace, 16)) return BL_ERR_ALIGN;
  if (workspace_bytes < bl_ternarize_pack_workspace_bytes(2 * f, k)) return BL_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* bins = (unsigned long long*)workspace;
  hipError_t e = bl::launch_absmean_bins(w, 2 * f * k, bins, s);
  if (e == hipSuccess) e = bl::launch_gamma_fold(bins, 2 * f * k, gamma, s);
  if (e == hipSuccess) e = bl::launch_ternarize_pack(w, 2 * f, k, gamma, packed, s, f);
  return from_hip(e);
}

namespace {

bl_status check_glu_product(int64_t m, int64_t f, int64_t k) {
  if (m < 0 || m > BL_MAX_M || f < 16 || f % 16 != 0 || 2 * f > BL_MAX_N || !valid_k(k) || !product_ok(m, k) ||
      !product_ok(2 * f + 16, k) || !product_ok(m, 2 * f))
    return BL_ERR_SHAPE;
  return BL_OK;
}

}  // namespace

bl_status bl_linear_glu(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha, int64_t m,
                        int64_t f, int64_t k, uint16_t* h, void* stream) {
  if (bl_status st = check_glu_product(m, f, k)) return st;
  if (m == 0) return BL_OK;  // empty tensors may carry NULL pointers
  if (!packed || !gamma || !xq || !alpha || !h) return BL_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(xq, 16) || !aligned(gamma, 4) || !aligned(alpha, 4) || !aligned(h, 2))
    return BL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (bl::gemv_serves(m, 2 * f)) return from_hip(bl::launch_gemv_glu(packed, gamma, xq, alpha, m, f, k, h, s));
  return from_hip(bl::launch_gemm_glu(packed, gamma, xq, alpha, m, f, k, h, s));
}

bl_status bl_bitlinear_glu(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t f,
                           int64_t k, int8_t* xq, float* alpha, uint16_t* h, void* stream) {
  if (bl_status st = check_glu_product(m, f, k)) return st;
  if (m == 0) return BL_OK;
  if (!packed || !gamma || !x || !xq || !alpha || !h) return BL_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(xq, 16) || !aligned(gamma, 4) || !aligned(alpha, 4) ||
      !aligned(h, 2))
    return BL_ERR_ALIGN;
  if (!bl::gemv_serves(m, 2 * f) && !bl::gemm_fits(m, 2 * f)) return BL_ERR_SHAPE;  // before the quantizer runs
  hipStream_t s = (hipStream_t)stream;
  if (bl::gemv_fused_glu_applies(m, f, k))
    return from_hip(bl::launch_gemv_fused_glu(packed, gamma, x, m, f, k, xq, alpha, h, s));
  hipError_t e = bl::launch_quant_act(x, m, k, xq, alpha, s);
  if (e != hipSuccess) return from_hip(e);
  if (bl::gemv_serves(m, 2 * f)) return from_hip(bl::launch_gemv_glu(packed, gamma, xq, alpha, m, f, k, h, s));
  return from_hip(bl::launch_gemm_glu(packed, gamma, xq, alpha, m, f, k, h, s));
}

bl_status bl_pack_transposed(const uint8_t* packed, int64_t n, int64_t k, uint8_t* packed_t, void* stream) {
  if (n < 64 || n % 64 != 0 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k)) return BL_ERR_SHAPE;
  if (!packed || !packed_t) return BL_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(packed_t, 16)) return BL_ERR_ALIGN;
  return from_hip(bl::launch_pack_transposed(packed, n, k, packed_t, (hipStream_t)stream));
}

bl_status bl_bitlinear_backward_x(const uint8_t* packed_t, const float* gamma, const uint16_t* dy, int64_t m,
                                  int64_t n, int64_t k, float* dx, void* stream) {
  if (m < 0 || m > BL_MAX_M || n < 64 || n % 64 != 0 || n > BL_MAX_BACKWARD_N || !valid_k(k) || !product_ok(m, n) ||
      !product_ok(m, k) || !product_ok(n + 16, k))
    return BL_ERR_SHAPE;
  if (m == 0) return BL_OK;
  if (!packed_t || !gamma || !dy || !dx) return BL_ERR_NULL;
  if (!aligned(packed_t, 16) || !aligned(gamma, 4) || !aligned(dy, 16) || !aligned(dx, 4)) return BL_ERR_ALIGN;
  return from_hip(bl::launch_backward_x(packed_t, gamma, dy, m, n, k, dx, (hipStream_t)stream));
}

size_t bl_backward_w_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || m > BL_MAX_M || n < 64 || n % 64 != 0 || n > BL_MAX_BACKWARD_N || !valid_k(k) || !product_ok(m + 64, n) ||
      !product_ok(m + 64, k))
    return 0;
  return bl::backward_w_workspace_bytes(m, n, k);
}

bl_status bl_bitlinear_backward_w(const uint16_t* dy, const int8_t* xq, const float* alpha, int64_t m, int64_t n,
                                  int64_t k, float* dw, void* workspace, size_t workspace_bytes, void* stream) {
  if (m < 0 || m > BL_MAX_M || n < 64 || n % 64 != 0 || n > BL_MAX_BACKWARD_N || !valid_k(k) || !product_ok(m + 64, n) ||
      !product_ok(m + 64, k) || !product_ok(n, k))
    return BL_ERR_SHAPE;
  if (!dy && m > 0) return BL_ERR_NULL;
  if (!dw || (m > 0 && (!xq || !alpha || !workspace))) return BL_ERR_NULL;
  if (!aligned(dy, 2) || !aligned(alpha, 4) || !aligned(dw, 4) || !aligned(workspace, 16)) return BL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (m == 0) return from_hip(bl::launch_fill_zero(dw, n * k, s));  // empty sum
  if (workspace_bytes < bl::backward_w_workspace_bytes(m, n, k)) return BL_ERR_WORKSPACE;
  return from_hip(bl::launch_backward_w(dy, xq, alpha, m, n, k, dw, workspace, s));
}

bl_status bl_unpack_ternary(const uint8_t* packed, int64_t n, int64_t k, int8_t* q, void* stream) {
  if (n < 0 || n > BL_MAX_N || !valid_k(k) || !product_ok(n + 16, k)) return BL_ERR_SHAPE;
  if (n == 0) return BL_OK;
  if (!packed || !q) return BL_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(q, 16)) return BL_ERR_ALIGN;
  return from_hip(bl::launch_unpack(packed, n, k, q, (hipStream_t)stream));
}

const char* bl_status_string(bl_status s) {
  switch (s) {
    case BL_OK: return "BL_OK";
    case BL_ERR_NULL: return "BL_ERR_NULL: a required pointer is NULL";
    case BL_ERR_SHAPE: return "BL_ERR_SHAPE: m, n or k outside the supported range";
    case BL_ERR_ALIGN: return "BL_ERR_ALIGN: a pointer is not aligned as required";
    case BL_ERR_WORKSPACE: return "BL_ERR_WORKSPACE: workspace too small";
    case BL_ERR_HIP: return "BL_ERR_HIP: the HIP runtime rejected a launch";
  }
  return "unknown bl_status";
}

}  // extern "C"
