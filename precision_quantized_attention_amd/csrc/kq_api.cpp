// C-ABI entry points of libkq: argument validation (before any HIP call), the host-side scale
// and rotary-table rules, and dispatch to the HIP kernels.  See include/kq.h for the contract.

#include "../../include/kq.h"
#include "kq_launch.h"

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool finite_pos(float x) { return isfinite(x) && x > 0.0f; }
kq_status from_hip(hipError_t e) { return e == hipSuccess ? KQ_OK : KQ_ERR_HIP; }

constexpr int64_t kVtAlign = 128;
constexpr int kAxes[3] = {16, 56, 56};

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

struct SplitPlan {
  int nfull, rem, split;
};

// Attention workgroups are 256-row query blocks, one per CU at a time.  When the blocks do not
// fill the last round of the device's CUs, the `rem` blocks of that round are split along the
// keys into `split` = floor(cus / rem) ranges (at most one per key tile), so the round runs
// on (nearly) all CUs for 1/split of the time.
SplitPlan plan_split(int64_t nblocks, int ntiles, int cus) {
  SplitPlan pl{(int)nblocks, 0, 0};
  if (cus <= 0) return pl;
  const int64_t rounds = nblocks / cus, rem = nblocks - rounds * cus;
  if (rem == 0) return pl;
  const int split = (int)std::min<int64_t>(cus / rem, ntiles);
  if (split < 2) return pl;
  pl.nfull = (int)(rounds * cus);
  pl.rem = (int)rem;
  pl.split = split;
  return pl;
}

// Validation shared by the attention entry points; fills p (without the split fields).
kq_status attn_params(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, int v_layout,
                      int B, int H, int N, int d, float s_q, float s_k, float s_v,
                      float sm_scale, float* o_f32, float* row_stats_or_null,
                      kq::AttnParams* p) {
  if (q8 == nullptr || k8 == nullptr || v8 == nullptr || o_f32 == nullptr) return KQ_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || d < 1) return KQ_ERR_INVALID_ARG;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o_f32, 16))
    return KQ_ERR_INVALID_ARG;
  if (row_stats_or_null != nullptr && !aligned(row_stats_or_null, 8)) return KQ_ERR_INVALID_ARG;
  if (!finite_pos(s_q) || !finite_pos(s_k) || !finite_pos(s_v) || !finite_pos(sm_scale))
    return KQ_ERR_INVALID_ARG;
  if (v_layout != KQ_LAYOUT_ROWS && v_layout != KQ_LAYOUT_TRANSPOSED) return KQ_ERR_INVALID_ARG;
  if (d != 128 || v_layout != KQ_LAYOUT_TRANSPOSED) return KQ_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)B * H;
  const int64_t nqb = ((int64_t)N + kq::kAttnRowsPerBlock - 1) / kq::kAttnRowsPerBlock;
  // per-(b, h) byte offsets are 32-bit: N * 128 and 128 * kq_vt_ld(N) below 2^31
  if (bh * nqb > INT32_MAX || kq_vt_ld(N) * 128 >= ((int64_t)1 << 31)) return KQ_ERR_UNSUPPORTED;
  const double c1 = (double)s_q * (double)s_k * (double)sm_scale * 1.4426950408889634;
  if (!isfinite(c1) || !isfinite((float)c1) || (float)c1 <= 0.0f) return KQ_ERR_INVALID_ARG;
  p->q = q8;
  p->q_bf16 = nullptr;
  p->q_inv = 0.0f;
  p->k = k8;
  p->q_scales = p->k_scales = nullptr;
  p->vt = v8;
  p->o = o_f32;
  p->stats = row_stats_or_null;
  p->bh = (int)bh;
  p->n = N;
  p->ldv = kq_vt_ld(N);
  p->c1 = (float)c1;
  p->s_v = s_v;
  // |t| = |raw c1| <= c1 448^2 d over E4M3 codes: past 2^20 the kernel forms the exp2 argument
  // unfused (see the attention kernel)
  p->wide_scores = (double)p->c1 * 448.0 * 448.0 * 128.0 >= 1048576.0;
  p->nfull = (int)(bh * nqb);
  p->rem = 0;
  p->split = 0;
  p->ws = nullptr;
  p->stats4 = nullptr;
  p->r1_stats = nullptr;
  p->r1_inv_p = p->r1_s_p = 0.0f;
  return KQ_OK;
}

SplitPlan attn_plan(int B, int H, int N) {
  const int64_t nqb = ((int64_t)N + kq::kAttnRowsPerBlock - 1) / kq::kAttnRowsPerBlock;
  return plan_split((int64_t)B * H * nqb, (N + 63) / 64, device_cus());
}

// Key split of the last round through a caller workspace (NULL: none).
kq_status attn_workspace(int B, int H, int N, void* workspace, size_t workspace_bytes,
                         kq::AttnParams* p) {
  if (workspace == nullptr) return KQ_OK;
  if (!aligned(workspace, 16)) return KQ_ERR_INVALID_ARG;
  const SplitPlan pl = attn_plan(B, H, N);
  if (pl.split == 0) return KQ_OK;
  if (workspace_bytes < kq::attn_workspace_bytes(pl.rem, pl.split)) return KQ_ERR_INVALID_ARG;
  p->nfull = pl.nfull;
  p->rem = pl.rem;
  p->split = pl.split;
  p->ws = static_cast<float*>(workspace);
  return KQ_OK;
}

// Shared validation of the projection GEMMs: sizes, the K granule of one k-step, N a multiple
// of 4 (float4 stores of C) and 32-bit buffer offsets for the last tile's prefetches.
kq_status gemm_params(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                      void* c, int64_t k_granule, int64_t row_bytes, kq::GemmParams* p) {
  if (a == nullptr || b == nullptr || c == nullptr || M < 1 || N < 1 || K < 1)
    return KQ_ERR_INVALID_ARG;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16)) return KQ_ERR_INVALID_ARG;
  if (K % k_granule != 0 || N % 4 != 0) return KQ_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if ((std::max(M, N) + 512) * row_bytes >= lim || K >= lim) return KQ_ERR_UNSUPPORTED;
  p->a = a;
  p->b = b;
  p->c = c;
  p->m = (int)M;
  p->n = (int)N;
  p->k = (int)K;
  p->a_scales = p->b_scales = nullptr;
  p->scale = 1.0f;
  p->out_bf16 = false;
  p->rank = 0;
  p->t = nullptr;
  p->l_up = nullptr;
  return KQ_OK;
}

kq_status gemm_fp8(const uint8_t* a8, const uint8_t* b8, int64_t M, int64_t N, int64_t K,
                   float s_a, float s_b, void* c, bool out_bf16, hipStream_t stream) {
  if (!finite_pos(s_a) || !finite_pos(s_b) || !finite_pos(s_a * s_b)) return KQ_ERR_INVALID_ARG;
  kq::GemmParams p;
  const kq_status st = gemm_params(a8, b8, M, N, K, c, 64, K, &p);
  if (st != KQ_OK) return st;
  p.scale = s_a * s_b;
  p.out_bf16 = out_bf16;
  return from_hip(kq::launch_gemm(p, false, stream));
}

kq_status gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                     const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                     bool out_bf16, hipStream_t stream) {
  if (a_scales == nullptr || b_scales == nullptr) return KQ_ERR_INVALID_ARG;
  if (!aligned(a_scales, 4) || !aligned(b_scales, 4)) return KQ_ERR_INVALID_ARG;
  kq::GemmParams p;
  const kq_status st = gemm_params(a_codes, b_codes, M, N, K, c, 128, K / 2, &p);
  if (st != KQ_OK) return st;
  p.a_scales = a_scales;
  p.b_scales = b_scales;
  p.out_bf16 = out_bf16;
  return from_hip(kq::launch_gemm(p, true, stream));
}

}  // namespace

extern "C" {

const char* kq_status_string(kq_status status) {
  switch (status) {
    case KQ_OK: return "ok";
    case KQ_ERR_INVALID_ARG: return "invalid argument";
    case KQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KQ_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

int64_t kq_vt_ld(int64_t n_tokens) {
  if (n_tokens < 1) return -1;
  return (n_tokens + kVtAlign - 1) / kVtAlign * kVtAlign;
}

kq_status kq_fp8_scales_from_amax(float amax, float* scale, float* inv_scale) {
  if (scale == nullptr || inv_scale == nullptr) return KQ_ERR_INVALID_ARG;
  if (!isfinite(amax) || amax < 0.0f) return KQ_ERR_INVALID_ARG;
  if (amax == 0.0f) {
    *scale = 1.0f;
    *inv_scale = 1.0f;
    return KQ_OK;
  }
  volatile float a = amax;              // keep each division a single float32 operation
  *scale = a / 448.0f;
  *inv_scale = 448.0f / a;
  return KQ_OK;
}

kq_status kq_rope3_table(const int32_t* positions, int64_t n_tokens, double theta, float* table) {
  if (positions == nullptr || table == nullptr || n_tokens < 1) return KQ_ERR_INVALID_ARG;
  if (!(theta > 0.0) || !isfinite(theta)) return KQ_ERR_INVALID_ARG;
  for (int64_t n = 0; n < n_tokens; ++n) {
    int j = 0;
    for (int a = 0; a < 3; ++a) {
      const double p = (double)positions[n * 3 + a];
      const int da = kAxes[a];
      for (int k = 0; k < da / 2; ++k) {
        const double w = 1.0 / pow(theta, (2.0 * k) / da);
        const double ang = p * w;
        table[(n * 64 + j) * 2 + 0] = (float)cos(ang);
        table[(n * 64 + j) * 2 + 1] = (float)sin(ang);
        ++j;
      }
    }
  }
  return KQ_OK;
}

kq_status kq_amax_calibrate(const void* x_bf16, int64_t n, float* amax_dev, hipStream_t stream) {
  if (x_bf16 == nullptr || amax_dev == nullptr || n < 0) return KQ_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(amax_dev, 4)) return KQ_ERR_INVALID_ARG;
  if (n == 0) return KQ_OK;
  return from_hip(kq::launch_amax_bf16(static_cast<const uint16_t*>(x_bf16), n, amax_dev, stream));
}

kq_status kq_quantize_fp8_tensor(const void* x_bf16, int64_t rows, int d, int64_t n_tokens,
                                 float inv_scale, uint8_t* y_e4m3, int layout,
                                 hipStream_t stream) {
  if (x_bf16 == nullptr || y_e4m3 == nullptr || rows < 1 || d < 1) return KQ_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(y_e4m3, 16) || !finite_pos(inv_scale))
    return KQ_ERR_INVALID_ARG;
  if (d % 16 != 0) return KQ_ERR_UNSUPPORTED;
  if (layout == KQ_LAYOUT_ROWS) {
    return from_hip(kq::launch_fp8_rows(static_cast<const uint16_t*>(x_bf16), rows * d,
                                        inv_scale, y_e4m3, stream));
  }
  if (layout != KQ_LAYOUT_TRANSPOSED) return KQ_ERR_INVALID_ARG;
  if (n_tokens < 1 || rows % n_tokens != 0) return KQ_ERR_INVALID_ARG;
  if (d != 128) return KQ_ERR_UNSUPPORTED;
  const int64_t bh = rows / n_tokens;
  if (bh > 65535) return KQ_ERR_UNSUPPORTED;
  return from_hip(kq::launch_fp8_transposed(static_cast<const uint16_t*>(x_bf16), bh, n_tokens,
                                            kq_vt_ld(n_tokens), inv_scale, y_e4m3, stream));
}

kq_status kq_quantize_fp4_block(const void* x_bf16, int64_t rows, int d, uint8_t* codes,
                                uint8_t* scales_e8m0, void* dq_bf16_or_null,
                                uint8_t* fp8_or_null, float inv_scale8,
                                const kq_rope3* rope_or_null, hipStream_t stream) {
  if (x_bf16 == nullptr || codes == nullptr || scales_e8m0 == nullptr || rows < 1 || d < 1)
    return KQ_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(codes, 16)) return KQ_ERR_INVALID_ARG;
  if (dq_bf16_or_null != nullptr && !aligned(dq_bf16_or_null, 16)) return KQ_ERR_INVALID_ARG;
  if (fp8_or_null != nullptr && (!aligned(fp8_or_null, 16) || !finite_pos(inv_scale8)))
    return KQ_ERR_INVALID_ARG;
  if (d % 32 != 0) return KQ_ERR_UNSUPPORTED;
  const float* table = nullptr;
  int64_t tokens = 1;
  if (rope_or_null != nullptr) {
    if (rope_or_null->cos_sin == nullptr || rope_or_null->n_tokens < 1) return KQ_ERR_INVALID_ARG;
    if (!aligned(rope_or_null->cos_sin, 16)) return KQ_ERR_INVALID_ARG;
    if (rows % rope_or_null->n_tokens != 0) return KQ_ERR_INVALID_ARG;
    if (d != 128 || rows >= ((int64_t)1 << 32)) return KQ_ERR_UNSUPPORTED;
    table = rope_or_null->cos_sin;
    tokens = rope_or_null->n_tokens;
  }
  if (rows * (int64_t)d / 8 > (int64_t)UINT32_MAX * 256) return KQ_ERR_UNSUPPORTED;
  return from_hip(kq::launch_fp4_block(static_cast<const uint16_t*>(x_bf16), rows, d, codes,
                                       scales_e8m0, static_cast<uint16_t*>(dq_bf16_or_null),
                                       fp8_or_null, inv_scale8, table, tokens, stream));
}

kq_status kq_attn_quant_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                            int v_layout, int B, int H, int N, int d, float s_q, float s_k,
                            float s_v, float sm_scale, float* o_f32, float* row_stats_or_null,
                            hipStream_t stream) {
  kq::AttnParams p;
  const kq_status st = attn_params(q8, k8, v8, v_layout, B, H, N, d, s_q, s_k, s_v, sm_scale,
                                   o_f32, row_stats_or_null, &p);
  if (st != KQ_OK) return st;
  return from_hip(kq::launch_attn_fp8(p, stream));
}

kq_status kq_attn_workspace_size(int B, int H, int N, int d, size_t* bytes) {
  if (bytes == nullptr || B < 1 || H < 1 || N < 1 || d < 1) return KQ_ERR_INVALID_ARG;
  if (d != 128) return KQ_ERR_UNSUPPORTED;
  const SplitPlan pl = attn_plan(B, H, N);
  *bytes = kq::attn_workspace_bytes(pl.rem, pl.split);
  return KQ_OK;
}

kq_status kq_attn_quant_fwd_ws(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                               int v_layout, int B, int H, int N, int d, float s_q, float s_k,
                               float s_v, float sm_scale, float* o_f32,
                               float* row_stats_or_null, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  kq::AttnParams p;
  const kq_status st = attn_params(q8, k8, v8, v_layout, B, H, N, d, s_q, s_k, s_v, sm_scale,
                                   o_f32, row_stats_or_null, &p);
  if (st != KQ_OK) return st;
  const kq_status sw = attn_workspace(B, H, N, workspace, workspace_bytes, &p);
  if (sw != KQ_OK) return sw;
  return from_hip(kq::launch_attn_fp8(p, stream));
}

kq_status kq_attn_quant_fwd_qbf16(const void* q_bf16, float inv_scale_q, const uint8_t* k8,
                                  const uint8_t* v8, int v_layout, int B, int H, int N, int d,
                                  float s_q, float s_k, float s_v, float sm_scale, float* o_f32,
                                  float* row_stats_or_null, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (!finite_pos(inv_scale_q)) return KQ_ERR_INVALID_ARG;
  kq::AttnParams p;
  // q_bf16 takes q8's checks (non-null, 16-byte aligned); the kernel reads it instead
  const kq_status st = attn_params(static_cast<const uint8_t*>(q_bf16), k8, v8, v_layout, B, H, N,
                                   d, s_q, s_k, s_v, sm_scale, o_f32, row_stats_or_null, &p);
  if (st != KQ_OK) return st;
  // per-(b, h) Q bytes N * 256 are addressed with 32-bit offsets (N < 2^24 holds above)
  p.q = nullptr;
  p.q_bf16 = static_cast<const uint16_t*>(q_bf16);
  p.q_inv = inv_scale_q;
  const kq_status sw = attn_workspace(B, H, N, workspace, workspace_bytes, &p);
  if (sw != KQ_OK) return sw;
  return from_hip(kq::launch_attn_fp8(p, stream));
}

kq_status kq_attn_quant_fwd_noalloc(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                                    int v_layout, int B, int H, int N, int d, float s_q,
                                    float s_k, float s_v, float sm_scale, float* o_f32,
                                    float* row_stats_or_null, hipStream_t stream) {
  kq::AttnParams p;
  const kq_status st = attn_params(q8, k8, v8, v_layout, B, H, N, d, s_q, s_k, s_v, sm_scale,
                                   o_f32, row_stats_or_null, &p);
  if (st != KQ_OK) return st;
  const SplitPlan pl = attn_plan(B, H, N);
  if (pl.split != 0) {
    void* ws = nullptr;
    size_t cap = 0;
    if (kq::attn_static_workspace(&ws, &cap) != hipSuccess) return KQ_ERR_HIP;
    if (kq::attn_workspace_bytes(pl.rem, pl.split) > cap) return KQ_ERR_UNSUPPORTED;
    p.nfull = pl.nfull;
    p.rem = pl.rem;
    p.split = pl.split;
    p.ws = static_cast<float*>(ws);
  }
  return from_hip(kq::launch_attn_fp8(p, stream));
}

kq_status kq_gemm_fp8(const uint8_t* a8, const uint8_t* b8, int64_t M, int64_t N, int64_t K,
                      float s_a, float s_b, float* c_f32, hipStream_t stream) {
  return gemm_fp8(a8, b8, M, N, K, s_a, s_b, c_f32, false, stream);
}

kq_status kq_gemm_fp8_bf16(const uint8_t* a8, const uint8_t* b8, int64_t M, int64_t N, int64_t K,
                           float s_a, float s_b, void* c_bf16, hipStream_t stream) {
  return gemm_fp8(a8, b8, M, N, K, s_a, s_b, c_bf16, true, stream);
}

kq_status kq_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales,
                        const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                        int64_t K, float* c_f32, hipStream_t stream) {
  return gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, M, N, K, c_f32, false, stream);
}

kq_status kq_gemm_mxfp4_bf16(const uint8_t* a_codes, const uint8_t* a_scales,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                             int64_t N, int64_t K, void* c_bf16, hipStream_t stream) {
  return gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, M, N, K, c_bf16, true, stream);
}

static kq_status svdquant_pass(const void* a_bf16, const void* l_down_bf16, int64_t M, int64_t K,
                               int rank, void* t_bf16, uint8_t* a_codes, uint8_t* a_scales,
                               hipStream_t stream) {
  if (a_bf16 == nullptr || l_down_bf16 == nullptr || t_bf16 == nullptr || M < 1 || K < 1 ||
      rank < 1)
    return KQ_ERR_INVALID_ARG;
  if (!aligned(a_bf16, 16) || !aligned(l_down_bf16, 16) || !aligned(t_bf16, 16))
    return KQ_ERR_INVALID_ARG;
  if (K % 64 != 0 || rank % 16 != 0 || rank > 64) return KQ_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;           // 32-bit buffer ranges and offsets
  if ((M + 32) * K * 2 >= lim || (int64_t)rank * K * 2 >= lim) return KQ_ERR_UNSUPPORTED;
  return from_hip(kq::launch_lowrank_down(static_cast<const uint16_t*>(a_bf16),
                                          static_cast<const uint16_t*>(l_down_bf16), (int)M,
                                          (int)K, rank, static_cast<uint16_t*>(t_bf16), a_codes,
                                          a_scales, stream));
}

kq_status kq_svdquant_down(const void* a_bf16, const void* l_down_bf16, int64_t M, int64_t K,
                           int rank, void* t_bf16, hipStream_t stream) {
  return svdquant_pass(a_bf16, l_down_bf16, M, K, rank, t_bf16, nullptr, nullptr, stream);
}

kq_status kq_svdquant_activations(const void* a_bf16, const void* l_down_bf16, int64_t M,
                                  int64_t K, int rank, uint8_t* a_codes, uint8_t* a_scales,
                                  void* t_bf16, hipStream_t stream) {
  if (a_codes == nullptr || a_scales == nullptr || !aligned(a_codes, 16))
    return KQ_ERR_INVALID_ARG;
  return svdquant_pass(a_bf16, l_down_bf16, M, K, rank, t_bf16, a_codes, a_scales, stream);
}

static kq_status gemm_svdquant(const uint8_t* a_codes, const uint8_t* a_scales,
                               const uint8_t* r_codes, const uint8_t* r_scales, int64_t M,
                               int64_t N, int64_t K, const void* t_bf16, const void* l_up_bf16,
                               int rank, void* c, bool out_bf16, hipStream_t stream) {
  if (t_bf16 == nullptr || l_up_bf16 == nullptr || rank < 1) return KQ_ERR_INVALID_ARG;
  if (!aligned(t_bf16, 16) || !aligned(l_up_bf16, 16)) return KQ_ERR_INVALID_ARG;
  if (a_scales == nullptr || r_scales == nullptr) return KQ_ERR_INVALID_ARG;
  if (!aligned(a_scales, 4) || !aligned(r_scales, 4)) return KQ_ERR_INVALID_ARG;
  kq::GemmParams p;
  const kq_status st = gemm_params(a_codes, r_codes, M, N, K, c, 128, K / 2, &p);
  if (st != KQ_OK) return st;
  if (rank % 16 != 0 || rank > 256) return KQ_ERR_UNSUPPORTED;
  p.a_scales = a_scales;
  p.b_scales = r_scales;
  p.out_bf16 = out_bf16;
  p.rank = rank;
  p.t = static_cast<const uint16_t*>(t_bf16);
  p.l_up = static_cast<const uint16_t*>(l_up_bf16);
  return from_hip(kq::launch_gemm(p, true, stream));
}

kq_status kq_gemm_mxfp4_svdquant(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const uint8_t* r_codes, const uint8_t* r_scales, int64_t M,
                                 int64_t N, int64_t K, const void* t_bf16,
                                 const void* l_up_bf16, int rank, float* c_f32,
                                 hipStream_t stream) {
  return gemm_svdquant(a_codes, a_scales, r_codes, r_scales, M, N, K, t_bf16, l_up_bf16, rank,
                       c_f32, false, stream);
}

kq_status kq_gemm_mxfp4_svdquant_bf16(const uint8_t* a_codes, const uint8_t* a_scales,
                                      const uint8_t* r_codes, const uint8_t* r_scales, int64_t M,
                                      int64_t N, int64_t K, const void* t_bf16,
                                      const void* l_up_bf16, int rank, void* c_bf16,
                                      hipStream_t stream) {
  return gemm_svdquant(a_codes, a_scales, r_codes, r_scales, M, N, K, t_bf16, l_up_bf16, rank,
                       c_bf16, true, stream);
}

kq_status kq_attn_mxfp4_fwd(const uint8_t* q_codes, const uint8_t* q_scales,
                            const uint8_t* k_codes, const uint8_t* k_scales, const uint8_t* v8,
                            int v_layout, int B, int H, int N, int d, float s_v, float sm_scale,
                            float* o_f32, float* row_stats_or_null, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  kq::AttnParams p;
  const kq_status st = attn_params(q_codes, k_codes, v8, v_layout, B, H, N, d, 1.0f, 1.0f, s_v,
                                   sm_scale, o_f32, row_stats_or_null, &p);
  if (st != KQ_OK) return st;
  if (q_scales == nullptr || k_scales == nullptr) return KQ_ERR_INVALID_ARG;
  if (!aligned(q_scales, 4) || !aligned(k_scales, 4)) return KQ_ERR_INVALID_ARG;
  p.q_scales = q_scales;
  p.wide_scores = false;   // raw carries the E8M0 scales: the documented precondition bounds it
  p.k_scales = k_scales;
  const kq_status sw = attn_workspace(B, H, N, workspace, workspace_bytes, &p);
  if (sw != KQ_OK) return sw;
  return from_hip(kq::launch_attn_fp8(p, stream));
}

kq_status kq_attn_r1_stats(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                           int v_layout, int B, int H, int N, int d, float s_q, float s_k,
                           float s_v, float sm_scale, float* row_stats4, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  kq::AttnParams p;
  // row_stats4 stands in for the output in the shared checks (the first pass writes no O)
  const kq_status st = attn_params(q8, k8, v8, v_layout, B, H, N, d, s_q, s_k, s_v, sm_scale,
                                   row_stats4, nullptr, &p);
  if (st != KQ_OK) return st;
  if (!aligned(row_stats4, 16)) return KQ_ERR_INVALID_ARG;
  const kq_status sw = attn_workspace(B, H, N, workspace, workspace_bytes, &p);
  if (sw != KQ_OK) return sw;
  p.o = nullptr;
  p.stats4 = row_stats4;
  return from_hip(kq::launch_attn_fp8(p, stream));
}

kq_status kq_attn_r1_amax(const float* row_stats4, int64_t rows, float* amax_dev,
                          hipStream_t stream) {
  if (row_stats4 == nullptr || amax_dev == nullptr || rows < 1) return KQ_ERR_INVALID_ARG;
  if (!aligned(row_stats4, 16) || !aligned(amax_dev, 4)) return KQ_ERR_INVALID_ARG;
  return from_hip(kq::launch_r1_amax(row_stats4, rows, amax_dev, stream));
}

kq_status kq_attn_r1_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, int v_layout,
                         int B, int H, int N, int d, float s_q, float s_k, float s_v,
                         float sm_scale, float amax_p, float* o_f32, float* row_stats4,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!finite_pos(amax_p) || row_stats4 == nullptr || !aligned(row_stats4, 16))
    return KQ_ERR_INVALID_ARG;
  const float s_p = amax_p / 448.0f, inv_p = 448.0f / amax_p;
  if (!finite_pos(s_p) || !finite_pos(inv_p)) return KQ_ERR_INVALID_ARG;
  kq::AttnParams p;
  const kq_status st = attn_params(q8, k8, v8, v_layout, B, H, N, d, s_q, s_k, s_v, sm_scale,
                                   o_f32, nullptr, &p);
  if (st != KQ_OK) return st;
  const kq_status sw = attn_workspace(B, H, N, workspace, workspace_bytes, &p);
  if (sw != KQ_OK) return sw;
  kq::AttnParams p1 = p;
  p1.o = nullptr;
  p1.stats4 = row_stats4;
  const hipError_t e = kq::launch_attn_fp8(p1, stream);
  if (e != hipSuccess) return KQ_ERR_HIP;
  p.r1_stats = row_stats4;
  p.r1_inv_p = inv_p;
  p.r1_s_p = s_p;
  return from_hip(kq::launch_attn_fp8(p, stream));
}

}  // extern "C"
