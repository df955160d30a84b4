/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitLinear W1.58A8 library.
 *
 * The layer is the BitNet b1.58 BitLinear: weights are absmean-ternarized to
 * {-1, 0, +1} and stored packed at 2 bits each; activations are quantized per
 * token to int8 by absmax; the product is accumulated in int32 and rescaled to
 * bf16.  Sources, on the BitNet b1.58 pages:
 *   [P1] bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution",
 *        section "The BitLinear Layer and AbsMean Quantization": gamma is the
 *        mean absolute value of the entire weight matrix; each weight is
 *        divided by (gamma + 1e-5), rounded to the nearest integer and clamped
 *        to [-1, 1]; with ternary weights the matrix product reduces to
 *        integer additions and subtractions.
 *   [P2] deepmox.com chapter 8, "A low-bit model is a whole-stack design":
 *        weights take the three values -1, 0, +1; activations use a separate
 *        per-token 8-bit path (W1.58A8); the GPU path packs four ternary values
 *        per 8-bit storage unit, moves packed weights from HBM on chip,
 *        unpacks them and computes with the 8-bit activations.
 *   [P3] onilabs.co, "A Two-Billion Ternary Bet": activations are quantized
 *        dynamically; scale factors are staged for mixed-precision compute;
 *        the 2B4T model uses squared ReLU in its feed-forward block (as does
 *        [P2], same section).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronizes; it only enqueues work
 *     on `stream` (a hipStream_t; NULL means the null stream) and returns.
 *   - Tensors are dense and row-major.  W is [n][k] (n output features,
 *     k input features), activations are [m][k] (m tokens), outputs [m][n].
 *   - k must be a positive multiple of 64 and at most BL_MAX_K (2^22);
 *     m <= BL_MAX_M (2^23) and n <= BL_MAX_N (2^26); m and n may be 0
 *     (nothing is enqueued) except where stated; n * k, m * k and m * n must
 *     stay below 2^40.  A shape inside these limits whose launch grid would
 *     still exceed the device's 2^32 work-items (a very large m * n product)
 *     returns BL_ERR_SHAPE as well, before anything is enqueued.
 *   - Pointers that are read or written with 128-bit accesses (w, packed, x,
 *     xq, workspace) must be 16-byte aligned; alpha, gamma and acc 4-byte,
 *     y 2-byte aligned.
 *   - Validation happens on the host before anything is enqueued; a failing
 *     check returns its code and enqueues nothing.  Shapes are checked first;
 *     an empty problem (m or n = 0) then returns BL_OK at once, so empty
 *     tensors may pass NULL pointers.  A failed kernel launch
 *     returns BL_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronization.  Entry points are thread-safe; the only global
 *     mutable state is the device array of bl_ternarize_pack_noalloc (see
 *     there).  Calls on one stream execute in order.
 *   - Inputs must be finite (no Inf or NaN).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BL_MAX_K (1 << 22)
#define BL_MAX_M (1 << 23)
#define BL_MAX_N (1 << 26)
#define BL_MAX_BACKWARD_N (1 << 24)

/* Status codes.  bl_status is a plain int, so that any value a caller
 * passes back (bl_status_string) is well defined in C and C++ alike. */
typedef int bl_status;
enum {
    BL_OK = 0,
    BL_ERR_NULL = 1,      /* a required pointer is NULL                          */
    BL_ERR_SHAPE = 2,     /* m, n or k outside the supported range               */
    BL_ERR_ALIGN = 3,     /* a pointer is not aligned as required                */
    BL_ERR_WORKSPACE = 4, /* workspace smaller than bl_ternarize_pack_workspace_bytes */
    BL_ERR_HIP = 5        /* the HIP runtime rejected a launch                   */
};

/* Size in bytes of the packed ternary buffer for an [n][k] weight matrix:
 * ceil(n/16)*16 * k/4 (four trits per byte [P2]; rows padded to 16).
 * Returns 0 for an invalid shape. */
size_t bl_packed_bytes(int64_t n, int64_t k);

/* Device workspace needed by bl_ternarize_pack: a fixed 2 KiB (256 exponent
 * bins of 64-bit integers, into which the absmean pass adds).  Returns 0 for
 * an invalid shape. */
size_t bl_ternarize_pack_workspace_bytes(int64_t n, int64_t k);

/* Weight preparation [P1]: gamma = mean |w| over all n*k weights, computed
 * exactly and rounded once to fp32 (nearest, ties to even); then every weight
 * becomes q = clamp(round_half_even(w / fl32(gamma + 1e-5f)), -1, 1), the
 * division in correctly rounded fp32; q is stored packed.
 *   w         [n][k] fp32, read only.
 *   packed    out, bl_packed_bytes(n, k) bytes.  Layout: 2-bit code q + 1
 *             (0, 1, 2; 3 never occurs).  The matrix is cut into tiles of 16
 *             rows x 64 columns; tile (i, j) starts at byte
 *             256 * (i * (k/64) + j); inside it, row r owns bytes 16r..16r+15,
 *             and column 64j + t of that row sits in byte 16r + (t % 16) at
 *             bits 2*(t/16)..2*(t/16)+1.  Rows n..ceil(n/16)*16-1 hold code 1.
 *   gamma     out, one fp32 on the device (gamma, without eps).
 *   workspace device scratch of workspace_bytes >= the size above; its
 *             contents on entry do not matter and are clobbered.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (n < 1, bad k, or n*k > 2^35: 34 G
 *         weights, 137 GB of fp32 input), BL_ERR_ALIGN, BL_ERR_WORKSPACE,
 *         BL_ERR_HIP. */
bl_status bl_ternarize_pack(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma,
                            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * bl_ternarize_pack (same gamma, same packed bytes), without a workspace
 * argument.  The 2 KiB of exponent bins live in a static device array of the
 * library, one per GPU, held until the process ends; it covers every shape
 * bl_ternarize_pack takes (n*k <= 2^35), and larger shapes are rejected with
 * BL_ERR_SHAPE.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress, with that device current); later calls allocate and
 * free nothing.  Each call clears the bins on `stream` (with a kernel) before
 * using them, so leftovers of an earlier call do not matter, but two calls
 * that overlap on one GPU (on different streams, or from different host
 * threads) share the array and race: serialize them.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP (also when the
 *         array's address cannot be obtained). */
bl_status bl_ternarize_pack_noalloc(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma,
                                    void* stream);

/* Per-token absmax int8 activation quantization [P2, P3]: for each row i,
 * a = max_j |x[i][j]|, s = fl32(127 / max(a, 1e-5f)),
 * xq[i][j] = clamp(round_half_even(fl32(x[i][j] * s)), -128, 127), alpha[i] = a.
 *   x      [m][k] bf16 (raw 16-bit patterns), read only.
 *   xq     out [m][k] int8.
 *   alpha  out [m] fp32 (the per-token absmax, exactly a bf16 value).
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* alpha, void* stream);

/* Ternary x int8 product with rescale [P1, P3]:
 *   acc[i][j] = sum_t xq[i][t] * q[j][t]          (exact, int32)
 *   y[i][j]   = bf16(acc[i][j] * gamma * alpha[i] / 127)   (fp32 evaluation,
 *               within one bf16 ulp of the exactly rounded value; acc = 0
 *               gives +0)
 *   packed/gamma as written by bl_ternarize_pack for an [n][k] matrix;
 *   xq/alpha as written by bl_quant_act for [m][k] activations.
 *   acc    out [m][n] int32, or NULL to skip it.
 *   y      out [m][n] bf16 bit patterns, or NULL to skip it (not both NULL).
 * The kernel is chosen from m, n and k: decode kernels that stream the
 * weights once per block of 16 (or 64) tokens for up to 64 tokens, the tiled
 * int8 matrix-core GEMM beyond; results do not depend on the choice.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_linear(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha,
                    int64_t m, int64_t n, int64_t k, int32_t* acc, uint16_t* y, void* stream);

/* The whole layer in one call [P1, P2, P3]: per-token absmax int8
 * quantization of x followed by the ternary product and rescale, with exactly
 * the results of bl_quant_act followed by bl_linear.  For one token, and for
 * up to 16 tokens while m * k is at most 65536 (rows up to 8192; 32767
 * beyond) and the activations quantized over all workgroups stay below 2^24
 * (2^23 for rows of 8192 and more), a single kernel does both steps (each
 * workgroup quantizes the tokens it multiplies); otherwise the two kernels
 * run back to back on `stream`.  Results do not depend on the choice.
 *   x      [m][k] bf16 (raw 16-bit patterns), read only.
 *   xq     out [m][k] int8 (the quantized activations; also used as staging).
 *   alpha  out [m] fp32 (per-token absmax).
 *   acc, y as in bl_linear (either may be NULL, not both).
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_bitlinear(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                       int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, void* stream);

/* ---- Five trits per byte ----
 * The denser weight code: [P4] bako.co, "BitNet b1.58 and the 1-Bit AI
 * Architecture Revolution", section "The Information Theory of 1.58 Bits" (a
 * three-state weight carries log2(3), about 1.58, bits) and [P5] deepmox.com
 * chapter 1, "Why Smaller Weights Are Not the Whole Story", section "A
 * different place to make efficiency decisions" (the 2B4T model keeps its
 * non-embedding weights below two bits per weight).  3^5 = 243 <= 256, so
 * five trits share one byte: 1.6 bits per weight, 20% fewer bytes to move
 * per decoded token than the 2-bit code, for the same gamma, trits and
 * results. */

#define BL_B3_MAX_K 64000
#define BL_B3_MAX_M 64

/* Size in bytes of the five-trits-per-byte buffer for an [n][k] matrix:
 * ceil(n/16)*16 rows of ceil(k/320)*64 bytes.  Returns 0 for an invalid shape. */
size_t bl_packed_bytes_b3(int64_t n, int64_t k);

/* Weight preparation in the five-trits-per-byte code [P1, P4, P5]: the same
 * gamma and trits as bl_ternarize_pack, stored as follows.  Five trits t_0..t_4
 * with codes c_d = t_d + 1 form v = sum_d c_d * 3^(4-d); the byte is
 * ceil(256 * v / 243) (so v = floor(243 * b / 256), and digit d is also
 * floor(3 * ((b * 3^d) mod 256) / 256)).  The matrix is cut into super-tiles
 * of 16 rows x 320 columns, 1024 bytes each, column super-tile fastest
 * (super-tile (i, s) at byte 1024 * (i * ceil(k/320) + s)); inside one,
 * column 80 g + 16 d + j (g < 4, d < 5, j < 16) of row r sits in byte
 * 256 g + 16 r + j as digit d.  Columns past k and rows past n hold trit 0.
 *   w, gamma, workspace as for bl_ternarize_pack; packed has
 *   bl_packed_bytes_b3(n, k) bytes.
 * Errors: as bl_ternarize_pack. */
bl_status bl_ternarize_pack_b3(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma,
                               void* workspace, size_t workspace_bytes, void* stream);

/* The whole layer from five-trits-per-byte weights, for decoding [P1, P2, P3,
 * P4]: per-token absmax int8 quantization of x (xq, alpha written exactly as
 * bl_quant_act would) and the ternary product with the bf16 rescale, with
 * exactly the results of bl_quant_act followed by bl_linear on the 2-bit
 * packing of the same trits.  One kernel per call; every token is its own
 * pass over the weights, so the call is meant for few tokens (m up to
 * BL_B3_MAX_M) and rows up to BL_B3_MAX_K columns (a row's activations are
 * held on chip).
 *   packed/gamma from bl_ternarize_pack_b3 for an [n][k] matrix;
 *   x [m][k] bf16; xq out [m][k] int8; alpha out [m] fp32;
 *   acc, y as in bl_linear (either may be NULL, not both).
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (m > BL_B3_MAX_M, k > BL_B3_MAX_K, or
 *         as bl_bitlinear), BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_bitlinear_b3(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t n,
                          int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y, void* stream);

/* ---- Gated feed-forward front half: gate+up BitLinear + squared ReLU ----
 * A feed-forward block with f hidden units has one gate+up BitLinear of 2f
 * output rows (rows 0..f-1 the gate, rows f..2f-1 the up projection; one
 * gamma for the whole matrix) followed by squared-ReLU gating [P2, P3]:
 *   h[i][j] = bf16(relu(g)^2 * u),  g = acc[i][j] * s,  u = acc[i][f + j] * s,
 *   s = gamma * alpha[i] / 127,
 * with acc the exact int32 products as in bl_linear.  g and u are not rounded
 * to bf16 first; h is evaluated in fp32 (within one bf16 ulp of the exactly
 * rounded value) and relu(g) = 0 gives +0 * u (so -0 for negative u).
 * f must be a positive multiple of 16. */

/* Weight preparation for a gate+up matrix: exactly bl_ternarize_pack of the
 * [2f][k] matrix w (gamma of all 2f*k weights), except that the packed row
 * tiles alternate: packed row tile 2t holds gate rows 16t..16t+15 and packed
 * row tile 2t+1 holds up rows 16t..16t+15 (rows f+16t.. of w), so that both
 * halves of 16 outputs sit next to each other.  packed has
 * bl_packed_bytes(2f, k) bytes; bl_unpack_ternary(packed, 2f, k) returns the
 * rows in that packed order.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (f not a positive multiple of 16, bad k,
 *         2f*k > 2^35), BL_ERR_ALIGN, BL_ERR_WORKSPACE, BL_ERR_HIP. */
bl_status bl_ternarize_pack_glu(const float* w, int64_t f, int64_t k, uint8_t* packed, float* gamma,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Gated product from quantized activations: packed/gamma from
 * bl_ternarize_pack_glu, xq/alpha from bl_quant_act ([m][k]).
 *   h      out [m][f] bf16 bit patterns.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_linear_glu(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* alpha,
                        int64_t m, int64_t f, int64_t k, uint16_t* h, void* stream);

/* The gated front half in one call: per-token quantization of x (xq and
 * alpha written exactly as bl_quant_act would) and the gated product, with
 * exactly the results of bl_quant_act followed by bl_linear_glu.  The token
 * counts that bl_bitlinear serves with a single kernel take one here too.
 *   x      [m][k] bf16; xq out [m][k] int8; alpha out [m] fp32;
 *   h      out [m][f] bf16 bit patterns.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_bitlinear_glu(const uint8_t* packed, const float* gamma, const uint16_t* x, int64_t m, int64_t f,
                           int64_t k, int8_t* xq, float* alpha, uint16_t* h, void* stream);

/* ---- Straight-through backward ----
 * [P1], section "Training Dynamics: The Straight-Through Estimator": the
 * backward pass treats the rounding step as the identity, so gradients pass
 * through the quantized weights to full-precision shadow weights, which are
 * ternarized again at the next forward pass (bl_ternarize_pack).  Both
 * quantizers are the identity in the backward pass and gamma, alpha are
 * constants; with the dequantized forward y = xhat What^T (xhat = alpha / 127
 * * xq, What = gamma * q):
 *   dx[i][t] = gamma * sum_j dy[i][j] * q[j][t]
 *   dw[j][t] = sum_i dy[i][j] * alpha[i] * xq[i][t] / 127
 * dy is bf16 [m][n]; dx and dw are fp32, accumulated in fp32 in any order
 * (within (n + 2) * 2^-24 * sum |terms| of the exact value for dx). */

/* The packed form of q^T ([k][n], the layout of bl_ternarize_pack with rows t
 * and columns j) from the packed form of q ([n][k]): the operand of
 * bl_bitlinear_backward_x, which contracts over the rows of q.  n must be a
 * positive multiple of 64; packed_t has bl_packed_bytes(k, n) bytes.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_pack_transposed(const uint8_t* packed, int64_t n, int64_t k, uint8_t* packed_t, void* stream);

/* Input gradient dx = gamma * dy q.
 *   packed_t  from bl_pack_transposed of the layer's packed weights; gamma
 *             the layer's gamma (device).
 *   dy        [m][n] bf16 bit patterns (16-byte aligned).
 *   dx        out [m][k] fp32.
 * n must be a multiple of 64 and at most BL_MAX_BACKWARD_N (2^24).
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_bitlinear_backward_x(const uint8_t* packed_t, const float* gamma, const uint16_t* dy, int64_t m,
                                  int64_t n, int64_t k, float* dx, void* stream);

/* Device workspace of bl_bitlinear_backward_w: 2 * (2n + k) * ceil(m/64)*64
 * bytes (the gradient, scaled by alpha and split into two bf16 parts, and the
 * int8 activations as bf16, both stored token-contiguous).  Returns 0 for an
 * invalid shape. */
size_t bl_backward_w_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Weight gradient for the shadow weights: dw[j][t] = sum_i dy[i][j] *
 * alpha[i] * xq[i][t] / 127.  alpha[i] * dy[i][j] (two bf16 values) is split
 * exactly into two bf16 parts, so every product is exact; the sums are fp32.
 *   dy         [m][n] bf16 bit patterns; xq [m][k] int8 and alpha [m] fp32 as
 *              written by bl_quant_act / bl_bitlinear for the layer's input.
 *   dw         out [n][k] fp32 (overwritten; zero for m = 0).
 *   workspace  device scratch of workspace_bytes >= bl_backward_w_workspace_bytes;
 *              contents on entry do not matter and are clobbered.
 * n must be a multiple of 64 and at most BL_MAX_BACKWARD_N.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_WORKSPACE, BL_ERR_HIP. */
bl_status bl_bitlinear_backward_w(const uint16_t* dy, const int8_t* xq, const float* alpha, int64_t m, int64_t n,
                                  int64_t k, float* dw, void* workspace, size_t workspace_bytes, void* stream);

/* Unpack a packed buffer back to trits (test and inspection helper [P2]):
 * q[j][t] in {-1, 0, 1} for the n real rows.  A code 3 (never produced by
 * bl_ternarize_pack) decodes as 0.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bl_unpack_ternary(const uint8_t* packed, int64_t n, int64_t k, int8_t* q, void* stream);

/* Static, human-readable name of a status code. */
const char* bl_status_string(bl_status s);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
