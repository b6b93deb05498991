/*
 * kq.h — quantized scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the SDPA quantization scheme of the NVIDIA blog
 * "Optimizing FLUX.1 Kontext for Image Editing with Low-Precision Quantization",
 * section "Workflow and Quantization" (its four bullets and Fig. 4):
 *   - Q, K and V are quantized per-tensor FP8 or per-block FP4 (first bullet);
 *   - BMM1 = Q K^T runs on FP8 inputs and accumulates in higher precision (second bullet);
 *   - softmax runs in FP32 with no quantization (third bullet);
 *   - BMM2 = P V runs with per-tensor FP8 (fourth bullet);
 *   - the quantization nodes are FakeQuantize (quantize, then dequantize) operations and the
 *     scales are static, fixed by post-training calibration (workflow step 4).
 * Token positions for the rotary embedding follow lpnh.cn "Flux.1 Kontext deep dive",
 * sections 1 and 3: target-image tokens at (0, h, w), context-image tokens at (i, h, w).
 *
 * Formats: FP8 is OCP E4M3 ("E4M3FN": bias 7, max 448, NaN = S.1111.111, no infinities).
 * FP4 is OCP MX E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in blocks of 32 consecutive
 * elements along the last dimension, each block with an E8M0 scale byte (2^(byte-127)).
 * Every encoder rounds to nearest with ties to the even code, saturates to the largest finite
 * magnitude, and keeps the input's sign bit (negative values that round to zero give -0).
 *
 * Conventions for every entry point below:
 *   - Pointers named *_dev or documented as device pointers are device memory owned by the
 *     caller; the library allocates nothing and is reentrant.  Its only global state is a
 *     per-device cache of the compute-unit count (written once, read-only after).
 *   - Device buffers must be 16-byte aligned unless stated otherwise.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); no call synchronizes.
 *     A fault inside a kernel surfaces at the caller's next synchronization.
 *   - Arguments are validated before any HIP call.  KQ_ERR_INVALID_ARG: a NULL or misaligned
 *     pointer, a negative or zero size, a non-finite or non-positive scale.
 *     KQ_ERR_UNSUPPORTED: a valid request outside what the kernels implement (for example
 *     d != 128 for attention).  KQ_ERR_HIP: the kernel launch failed (hipGetLastError).
 *     No exception crosses this interface and nothing aborts.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KQ_OK = 0,
  KQ_ERR_INVALID_ARG = -1,
  KQ_ERR_UNSUPPORTED = -2,
  KQ_ERR_HIP = -3
} kq_status;

/* Layout flags for FP8 outputs. */
enum {
  KQ_LAYOUT_ROWS = 0,       /* same as the input: [rows][d], d contiguous                     */
  KQ_LAYOUT_TRANSPOSED = 1  /* per (batch, head) transposed: [B*H][d][kq_vt_ld(N)], tokens
                               contiguous, columns N .. kq_vt_ld(N)-1 written as zero          */
};

/* Rotary-embedding descriptor for kq_quantize_fp4_block.
 * cos_sin: device float32 [n_tokens][d/2][2] = (cos, sin) of the angle of each adjacent pair
 * (build it with kq_rope3_table); row r of the input is token r % n_tokens. */
typedef struct {
  const float* cos_sin;
  int64_t n_tokens;
} kq_rope3;

/* Human-readable name of a status code (static string). */
const char* kq_status_string(kq_status status);

/* Row stride, in bytes, of the transposed FP8 layout for a sequence of n_tokens tokens:
 * n_tokens rounded up to a multiple of 128 (the attention kernel's key tile), or -1 if
 * n_tokens < 1. */
int64_t kq_vt_ld(int64_t n_tokens);

/* Host-only.  Static per-tensor FP8 scale from a calibrated amax (blog section "Workflow and
 * Quantization", FP8 per-tensor bullets; workflow step 4): *scale = fl32(amax / 448) and
 * *inv_scale = fl32(448 / amax), both single IEEE float32 divisions; amax == 0 gives 1 and 1.
 * INVALID_ARG for NULL outputs or a negative or non-finite amax. */
kq_status kq_fp8_scales_from_amax(float amax, float* scale, float* inv_scale);

/* Host-only.  Builds the 3-axis rotary table for integer token positions (lpnh.cn "Flux.1
 * Kontext deep dive", sections 1 and 3).  positions: host int32 [n_tokens][3] (image index,
 * h, w); table: host float32 [n_tokens][64][2].  The head dimension 128 is cut into axis
 * slices of widths 16, 56, 56; pair k of axis a (width d_a) turns by pos_a / theta^(2k/d_a),
 * evaluated in double precision (pow, cos, sin of the C library) and rounded to float32.
 * INVALID_ARG for NULL pointers, n_tokens < 1 or theta <= 0. */
kq_status kq_rope3_table(const int32_t* positions, int64_t n_tokens, double theta, float* table);

/* Calibration (blog workflow step 4, read as a max calibrator):
 * *amax_dev = max(*amax_dev, max_i |x_i|) over n bf16 values.  x_bf16: device bf16 [n];
 * amax_dev: device float32 scalar, 4-byte aligned, which the caller
 * initializes (to 0 for a fresh calibration) — successive calls keep a running maximum.
 * Inputs must be free of NaN.  n == 0 enqueues nothing. */
kq_status kq_amax_calibrate(const void* x_bf16, int64_t n, float* amax_dev, hipStream_t stream);

/* Per-tensor FP8 quantization, the BMM input quantizer (blog bullets 2 and 4):
 * y = E4M3(fl32(x * inv_scale)) for a bf16 tensor of rows x d.
 * layout KQ_LAYOUT_ROWS: y is uint8 [rows][d]; n_tokens is ignored (pass 0 or rows).
 * layout KQ_LAYOUT_TRANSPOSED: rows = (B*H) * n_tokens and y is uint8 [B*H][d][kq_vt_ld(n_tokens)]
 * (the layout kq_attn_quant_fwd reads V in); requires d == 128.
 * Requires d % 16 == 0 and inv_scale finite and > 0. */
kq_status kq_quantize_fp8_tensor(const void* x_bf16, int64_t rows, int d, int64_t n_tokens,
                                 float inv_scale, uint8_t* y_e4m3, int layout,
                                 hipStream_t stream);

/* Per-block FP4 quantization (blog first bullet and Fig. 4), optionally preceded by the
 * 3-axis rotary embedding (rope != NULL) and optionally followed by per-tensor FP8 of the
 * dequantized values.  For each row of d elements (d % 32 == 0; d == 128 with a rotary
 * table) and each block of 32:
 *   x'   = rope ? rotate(x) : x, in float32, each product and sum rounded separately;
 *   e    = clamp(floor(log2(max |x'|)) - 2, -127, 127)  (e = -127 for an all-zero block);
 *   code = E2M1(x' / 2^e);  dq = E2M1value(code) * 2^e  (exact in bf16).
 * codes:  device uint8 [rows][d/2], two codes per byte, even element in the low nibble.
 * scales: device uint8 [rows][d/32], E8M0 byte e + 127 (1-byte aligned).
 * dq_bf16_or_null: device bf16 [rows][d] or NULL.
 * fp8_or_null: device uint8 [rows][d] = E4M3(fl32(dq * inv_scale8)) or NULL; inv_scale8 is
 * ignored when fp8_or_null is NULL.
 * rope: the table must hold n_tokens rows; rows must be a multiple of n_tokens. */
kq_status kq_quantize_fp4_block(const void* x_bf16, int64_t rows, int d, uint8_t* codes,
                                uint8_t* scales_e8m0, void* dq_bf16_or_null,
                                uint8_t* fp8_or_null, float inv_scale8,
                                const kq_rope3* rope_or_null, hipStream_t stream);

/* Fused quantized attention forward (blog bullets 2-4, Fig. 4), one (batch, head) per
 * B*H slice, no mask, d = 128:
 *   BMM1 on E4M3 Q, K with float32 accumulation; t = raw * c1, c1 = s_q s_k sm_scale log2(e);
 *   float32 softmax with an integer row offset M = ceil(max t) kept online, p = exp2(t - M);
 *   P quantized to E4M3 with the static per-tensor scale 1/448 (code = E4M3(448 p));
 *   BMM2 on the E4M3 P and V codes with float32 accumulation;
 *   O = acc * (s_v / 448) / sum(p), the row sum taken over the unquantized float32 p.
 * q8, k8: device uint8 [B*H][N][128].  v8: v_layout KQ_LAYOUT_ROWS → [B*H][N][128] is
 * UNSUPPORTED; v_layout KQ_LAYOUT_TRANSPOSED → [B*H][128][kq_vt_ld(N)] with zero padding, as
 * kq_quantize_fp8_tensor writes it.  s_q, s_k, s_v: per-tensor scales (kq_fp8_scales_from_amax);
 * sm_scale: softmax scale (1/sqrt(128) for these models).
 * o_f32: device float32 [B*H][N][128].  row_stats_or_null: device float32 [B*H][N][2] =
 * (M, sum(p)) per query row, or NULL.
 * Any finite scales: |t| is at most c1 * 448^2 * 128; when that bound reaches 2^20 the kernel
 * forms each exp2 argument in the definition's order, fl32(raw c1) - M_kb, instead of one
 * fused multiply-add (slower; only inputs scaled far beyond unit range get there). */
kq_status kq_attn_quant_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                            int v_layout, int B, int H, int N, int d, float s_q, float s_k,
                            float s_v, float sm_scale, float* o_f32, float* row_stats_or_null,
                            hipStream_t stream);

/* Bytes of device workspace kq_attn_quant_fwd_ws uses for this shape on the current device
 * (0 when the launch fills whole rounds of compute units and needs none).  Same argument
 * rules as kq_attn_quant_fwd; d must be 128.  Host-only apart from one device-attribute query
 * per device. */
kq_status kq_attn_workspace_size(int B, int H, int N, int d, size_t* bytes);

/* kq_attn_quant_fwd with a caller-owned device workspace (16-byte aligned, at least
 * kq_attn_workspace_size bytes for the same shape and device; NULL runs kq_attn_quant_fwd).
 * The attention of one 256-row query block runs on one compute unit; when the query blocks
 * leave the last round of the device's compute units partly idle, each block of that round is
 * split along the keys into consecutive ranges that run on the idle units, and a second kernel
 * merges their partial results (accumulator, row sum and integer row offset per range) by the
 * same exact power-of-two rescaling the online softmax uses.  The outputs equal
 * kq_attn_quant_fwd's up to float32 summation order.  A workspace smaller than required is
 * KQ_ERR_INVALID_ARG.  Two calls sharing a workspace must be ordered (same stream). */
kq_status kq_attn_quant_fwd_ws(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                               int v_layout, int B, int H, int N, int d, float s_q, float s_k,
                               float s_v, float sm_scale, float* o_f32,
                               float* row_stats_or_null, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* kq_attn_quant_fwd_ws with Q given in bf16 and quantized inside the attention kernel (blog
 * bullets 1-4, Fig. 4: the per-tensor FP8 FakeQuantize of Q feeding the first matmul).  Each
 * element's code is E4M3(clamp(fl32(x * inv_scale_q), -448, 448)), nearest even: the codes
 * kq_quantize_fp8_tensor writes with the same inv_scale_q, so O and the row statistics equal,
 * bit for bit, those of quantizing Q with it and calling kq_attn_quant_fwd_ws.  Every Q element
 * is read once, so this saves the quantizer's pass over Q and its FP8 copy.
 * q_bf16: device bf16 [B*H][N][128], 16-byte aligned.  inv_scale_q: finite, > 0 (the
 * quantizer's scale, kq_fp8_scales_from_amax); s_q still enters c1 as in kq_attn_quant_fwd.
 * Every other argument, rule and error as kq_attn_quant_fwd_ws. */
kq_status kq_attn_quant_fwd_qbf16(const void* q_bf16, float inv_scale_q, const uint8_t* k8,
                                  const uint8_t* v8, int v_layout, int B, int H, int N, int d,
                                  float s_q, float s_k, float s_v, float sm_scale, float* o_f32,
                                  float* row_stats_or_null, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* SVD-Quant in FP4 for a projection GEMM (blog section "Workflow and Quantization", which names
 * SVD-Quant in FP4 beside PTQ in FP8 and FP4; the page gives none of its steps, so this is the
 * method's plainest form).  Offline, the bf16 weights W [N][K] are split into rank-r bf16
 * factors L_up [N][r], L_down [r][K] (from W's SVD) and the bf16 residual
 * R = W - L_up L_down, whose MXFP4 codes and scales come from kq_quantize_fp4_block like any
 * weight's.  Per forward:
 *   kq_svdquant_down:        T = bf16(A L_down^T), A [M][K] bf16 activations, T [M][r] bf16
 *                            (each value the float32 sum rounded once, nearest even);
 *   kq_gemm_mxfp4_svdquant:  C = dq(A4) dq(R4)^T + T L_up^T, float32 accumulation, C float32
 *                            [M][N] (the _bf16 form rounds C once to bf16, nearest even);
 *                            A4, R4 as kq_gemm_mxfp4's operands.
 * Device pointers, 16-byte aligned (scales 4-byte).  r % 16 == 0 with r <= 64 (down) and
 * r <= 256 (GEMM), K % 64 == 0 (down) and K % 128 == 0 (GEMM); otherwise KQ_ERR_UNSUPPORTED,
 * as are sizes whose byte offsets pass 2^31.  Other rules as kq_gemm_mxfp4. */
kq_status kq_svdquant_down(const void* a_bf16, const void* l_down_bf16, int64_t M, int64_t K,
                           int rank, void* t_bf16, hipStream_t stream);
/* The activation pass of a forward in one read of A: kq_svdquant_down's T, and A's MXFP4 codes
 * [M][K/2] and E8M0 scales [M][K/32], equal bit for bit to kq_quantize_fp4_block's on A
 * (a_codes 16-byte aligned).  Same rules as kq_svdquant_down. */
kq_status kq_svdquant_activations(const void* a_bf16, const void* l_down_bf16, int64_t M,
                                  int64_t K, int rank, uint8_t* a_codes, uint8_t* a_scales,
                                  void* t_bf16, hipStream_t stream);

/* The offline weight step (host only; no HIP call): from the bf16 weights w [N][K] (host
 * memory), the rank-r bf16 factors l_up [N][r] = U_r S_r and l_down [r][K] = V_r^T of W's
 * leading singular triplets, and the bf16 residual [N][K] = W - l_up l_down (with the rounded
 * factors), every value rounded once to nearest even.  The triplets come from a randomized
 * range finder (fixed seed, r + 8 columns, 4 power-iteration rounds) and a one-sided Jacobi
 * SVD of the projected matrix, in float64: deterministic, and equal to an exact SVD's up to
 * the bf16 rounding wherever singular value r stands clear of singular value r + 9.  Caller-
 * owned host buffers; 1 <= rank <= min(N, K) else KQ_ERR_INVALID_ARG, non-finite weights
 * KQ_ERR_INVALID_ARG, N K > 2^32 KQ_ERR_UNSUPPORTED.  Factor signs are arbitrary (the product
 * is what counts). */
kq_status kq_svdquant_factorize(const uint16_t* w_bf16, int64_t N, int64_t K, int rank,
                                uint16_t* l_up_bf16, uint16_t* l_down_bf16,
                                uint16_t* residual_bf16);
kq_status kq_gemm_mxfp4_svdquant(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const uint8_t* r_codes, const uint8_t* r_scales, int64_t M,
                                 int64_t N, int64_t K, const void* t_bf16,
                                 const void* l_up_bf16, int rank, float* c_f32,
                                 hipStream_t stream);
kq_status kq_gemm_mxfp4_svdquant_bf16(const uint8_t* a_codes, const uint8_t* a_scales,
                                      const uint8_t* r_codes, const uint8_t* r_scales, int64_t M,
                                      int64_t N, int64_t K, const void* t_bf16,
                                      const void* l_up_bf16, int rank, void* c_bf16,
                                      hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kq_attn_quant_fwd_ws with the key-split workspace
 * taken from a static device array of the library instead of the caller.  Same arguments,
 * rules and results (bit for bit) as kq_attn_quant_fwd_ws given a workspace of
 * kq_attn_workspace_size bytes.  The array holds 256 x 256 x 132 floats (33 MiB: the partial
 * results of 256 query blocks' key ranges, every plan of a 256-compute-unit device); a shape
 * whose plan needs more on the current device is KQ_ERR_UNSUPPORTED.  It allocates nothing:
 * the array exists once per GPU until the process ends, and its device address is looked up
 * once per device (hipGetSymbolAddress; a failure is KQ_ERR_HIP).  Every call on a GPU shares
 * that GPU's array and overwrites what it needs before reading it (nothing has to start at
 * zero); calls that overlap on one GPU (different streams, or host threads without ordering)
 * race on it. */
kq_status kq_attn_quant_fwd_noalloc(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                                    int v_layout, int B, int H, int N, int d, float s_q,
                                    float s_k, float s_v, float sm_scale, float* o_f32,
                                    float* row_stats_or_null, hipStream_t stream);

/* Attention with a native MXFP4 BMM1 (a hardware-native variant; the blog keeps both
 * products in FP8, so this one is not its numerics): Q and K stay in the per-block FP4 form
 * kq_quantize_fp4_block writes (E2M1 codes + an E8M0 scale per 32 elements of d, RoPE
 * applied before quantization where used), and BMM1 multiplies their dequantized values on
 * the matrix cores with float32 accumulation, without the per-tensor FP8 step:
 *   raw = sum_d dq(q)_d dq(k)_d, dq = E2M1value * 2^(scale byte - 127);
 *   t = raw * c1, c1 = sm_scale log2(e) (rounded once to float32);
 * then softmax, P and BMM2 exactly as kq_attn_quant_fwd (V per-tensor FP8 with scale s_v).
 * q_codes, k_codes: device uint8 [B*H][N][64]; q_scales, k_scales: device uint8 [B*H][N][4]
 * (4-byte aligned); v8, v_layout, o_f32, row_stats_or_null as kq_attn_quant_fwd; workspace as
 * kq_attn_quant_fwd_ws (NULL: no key split; size from kq_attn_workspace_size).
 * Precondition for parity with the definition: |t| < 2^20, which holds when
 * sm_scale log2(e) 128 max|dq(q)| max|dq(k)| < 2^20 (the E8M0 scales are data, so the library
 * cannot check it).  Beyond it the fused exp2 argument may put 448 p past the E4M3 range; the
 * codes then saturate at 448 (no NaN while t is finite), and the output drifts from the
 * definition. */
kq_status kq_attn_mxfp4_fwd(const uint8_t* q_codes, const uint8_t* q_scales,
                            const uint8_t* k_codes, const uint8_t* k_scales, const uint8_t* v8,
                            int v_layout, int B, int H, int N, int d, float s_v, float sm_scale,
                            float* o_f32, float* row_stats_or_null, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Literal FakeQuantize of the normalized P ("R1"; blog bullet 4 and Fig. 4 read as a
 * FakeQuantize node on the FP32 softmax output with a calibrated per-tensor scale), two
 * passes over the keys (each of them split along the keys when a workspace is given):
 *   pass 1: M = ceil(max t), l = sum exp2(t - M) per row (t as in kq_attn_quant_fwd);
 *   pass 2: P = exp2(t - M) / l, codes = E4M3(P * 448 / amax_P) saturated at 448,
 *           O = (sum codes E4M3(v)) * (amax_P / 448) * s_v.
 * amax_P is the static calibrated maximum of P over the tensor (kq_attn_r1_amax).
 * Same arguments and rules as kq_attn_quant_fwd.  row_stats4: device float32 [B*H][N][4]
 * (16-byte aligned), written by pass 1 as (M, l, max_j exp2(t - M), 0) per row.  workspace:
 * as kq_attn_quant_fwd_ws (NULL: no key split; size from kq_attn_workspace_size), used by each
 * pass in turn; the partial results of the second pass share the row's M and merge by plain
 * summation. */

/* Pass 1 alone (calibration): fills row_stats4, writes no output. */
kq_status kq_attn_r1_stats(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                           int v_layout, int B, int H, int N, int d, float s_q, float s_k,
                           float s_v, float sm_scale, float* row_stats4, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* amax_dev[0] = max(amax_dev[0], max over `rows` rows of row_stats4 of fl32(max p / l)): the
 * largest normalized probability.  The caller zero-initializes amax_dev for a fresh
 * calibration; rows = B*H*N.  amax_dev must hold +0 or a positive value: the device takes the
 * maximum with unsigned atomics on the float bits. */
kq_status kq_attn_r1_amax(const float* row_stats4, int64_t rows, float* amax_dev,
                          hipStream_t stream);

/* Both passes with the static amax_P (finite, > 0); o_f32 as kq_attn_quant_fwd. */
kq_status kq_attn_r1_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, int v_layout,
                         int B, int H, int N, int d, float s_q, float s_k, float s_v,
                         float sm_scale, float amax_p, float* o_f32, float* row_stats4,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Quantized projection GEMMs: C = A B^T for the linear layers around the attention, with
 * per-tensor FP8 (W8A8) or per-block FP4 post-training quantization of both operands (blog
 * section "Workflow and Quantization", the quantization config and its PTQ paragraph).
 * A: activations [M][K], one row per token; B: weights [N][K], one row per output feature;
 * both K-contiguous.  c_f32: device float32 [M][N], fully overwritten.  Products are taken on
 * the matrix cores with float32 accumulation (summation order unspecified).
 * Sizes: M, N, K >= 1; N % 4 == 0; (max(M, N) + 512) * (bytes per operand row) < 2^31;
 * otherwise KQ_ERR_UNSUPPORTED (sizes < 1: KQ_ERR_INVALID_ARG). */

/* FP8: a8 device uint8 [M][K], b8 device uint8 [N][K], E4M3 codes (kq_quantize_fp8_tensor with
 * KQ_LAYOUT_ROWS writes them); s_a, s_b their per-tensor scales;
 * C = s_a s_b sum_k E4M3(a8)_mk E4M3(b8)_nk.  K % 64 == 0. */
kq_status kq_gemm_fp8(const uint8_t* a8, const uint8_t* b8, int64_t M, int64_t N, int64_t K,
                      float s_a, float s_b, float* c_f32, hipStream_t stream);

/* MXFP4: a_codes device uint8 [M][K/2], b_codes [N][K/2], E2M1 codes two per byte (even
 * element in the low nibble); a_scales [M][K/32], b_scales [N][K/32] E8M0 bytes (4-byte
 * aligned), one per 32 consecutive k (kq_quantize_fp4_block writes both);
 * C = sum_k dq(a)_mk dq(b)_nk with dq = E2M1value * 2^(scale byte - 127).  K % 128 == 0. */
kq_status kq_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales,
                        const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                        int64_t K, float* c_f32, hipStream_t stream);

/* The same two products with C delivered in bf16, the activation type of the transformer the
 * projections sit in: c_bf16 device bf16 [M][N] (16-byte aligned), fully overwritten, each
 * element the float32 result above rounded once to bf16 (round to nearest even).  Arguments,
 * sizes and errors as kq_gemm_fp8 / kq_gemm_mxfp4. */
kq_status kq_gemm_fp8_bf16(const uint8_t* a8, const uint8_t* b8, int64_t M, int64_t N, int64_t K,
                           float s_a, float s_b, void* c_bf16, hipStream_t stream);
kq_status kq_gemm_mxfp4_bf16(const uint8_t* a_codes, const uint8_t* a_scales,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                             int64_t N, int64_t K, void* c_bf16, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
