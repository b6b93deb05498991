// Internal launchers shared by the C-ABI layer (kq_api.cpp) and the kernel files.
// Arguments arrive here already validated; each launcher enqueues its kernels on `stream`
// and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, float* amax, hipStream_t stream);

hipError_t launch_fp8_rows(const uint16_t* x, int64_t n, float inv_scale, uint8_t* y,
                           hipStream_t stream);

hipError_t launch_fp8_transposed(const uint16_t* x, int64_t bh, int64_t n_tokens, int64_t ld,
                                 float inv_scale, uint8_t* y, hipStream_t stream);

hipError_t launch_fp4_block(const uint16_t* x, int64_t rows, int d, uint8_t* codes,
                            uint8_t* scales, uint16_t* dq, uint8_t* fp8, float inv_scale8,
                            const float* rope_table, int64_t rope_tokens, hipStream_t stream);

struct AttnParams {
  const uint8_t* q;       // [BH][N][128] E4M3, or [BH][N][64] packed E2M1 (q_scales set)
  const uint16_t* q_bf16; // FP8 BMM1 only: [BH][N][128] bf16 Q quantized in the kernel (q unused), or nullptr
  float q_inv;            // with q_bf16: the per-tensor 1 / s_q the codes are formed with
  const uint8_t* k;       // [BH][N][128] E4M3, or [BH][N][64] packed E2M1
  const uint8_t* q_scales;  // MXFP4 BMM1: [BH][N][4] E8M0; nullptr: FP8 BMM1
  const uint8_t* k_scales;  // MXFP4 BMM1: [BH][N][4] E8M0
  const uint8_t* vt;      // [BH][128][ldv] E4M3, zero beyond N
  float* o;               // [BH][N][128]
  float* stats;           // [BH][N][2] or nullptr
  int bh;
  int n;
  int64_t ldv;
  float c1;               // s_q * s_k * sm_scale * log2(e) (MXFP4: sm_scale * log2(e)), rounded once
  float s_v;
  bool wide_scores;       // |t| may reach 2^20: the exp2 argument is formed unfused (FP8 only)
  // Key split of the last, partial round of query blocks (split == 0: none).  Query blocks
  // [0, nfull) run whole; each of the `rem` blocks after them runs as `split` workgroups over
  // consecutive key ranges, writing partial results to `ws`, merged by a second kernel.
  int nfull;
  int rem;
  int split;
  float* ws;              // [rem * split][256][128] partial acc, then [rem * split][256][4] stats
  // Literal FakeQuantize of the normalized P (R1), two passes.
  float* stats4;          // first pass: [BH][N][4] = (M, l, max p, 0) per row, or nullptr
  const float* r1_stats;  // second pass: the first pass's stats4 (nullptr: not R1)
  float r1_inv_p;         // 448 / amax_P
  float r1_s_p;           // amax_P / 448
};

// Query rows per attention workgroup (the unit of the split).
constexpr int kAttnRowsPerBlock = 256;

// Bytes of workspace for `rem * split` partial query blocks.
constexpr size_t attn_workspace_bytes(int rem, int split) {
  return (size_t)rem * split * kAttnRowsPerBlock * (128 + 4) * sizeof(float);
}

hipError_t launch_attn_fp8(const AttnParams& p, hipStream_t stream);

// The static key-split workspace: partial results of up to 256 query blocks' key ranges, the
// most a 256-compute-unit device's plan uses (rem * split <= compute units).
constexpr size_t kAttnStaticWorkspaceBytes = attn_workspace_bytes(1, 256);

// Device address and size of the static workspace on the current device (looked up once per
// device with hipGetSymbolAddress).
hipError_t attn_static_workspace(void** ptr, size_t* bytes);

hipError_t launch_r1_amax(const float* row_stats4, int64_t rows, float* amax, hipStream_t stream);

struct GemmParams {
  const uint8_t* a;         // [M][K] E4M3 codes, or [M][K/2] packed E2M1 codes
  const uint8_t* b;         // [N][K] / [N][K/2]
  const uint8_t* a_scales;  // [M][K/32] E8M0 (FP4 only)
  const uint8_t* b_scales;  // [N][K/32] E8M0 (FP4 only)
  void* c;                  // [M][N] float32, or bf16 when out_bf16
  int m, n, k;
  float scale;              // s_a * s_b (FP8), 1 (FP4)
  bool out_bf16;            // C rounded to bf16 (round to nearest even) instead of float32
  // SVD-Quant branch (FP4 only; rank 0: none): C += T L_up^T before the MXFP4 sum
  int rank;                 // multiple of 16
  const uint16_t* t;        // [M][rank] bf16
  const uint16_t* l_up;     // [N][rank] bf16
};

// C = A B^T; K % 64 == 0 (FP8) or K % 128 == 0 (FP4), N % 4 == 0.
hipError_t launch_gemm(const GemmParams& p, bool fp4, hipStream_t stream);

// T = bf16(A L_down^T) for the SVD-Quant branch: A [m][k], L_down [rank][k], T [m][rank], all
// bf16; k % 64 == 0, rank % 16 == 0, rank <= 64.  With a_codes (and a_scales) the same pass also
// writes A's MXFP4 codes [m][k/2] and E8M0 scales [m][k/32] (kq_quantize_fp4_block's output).
hipError_t launch_lowrank_down(const uint16_t* a, const uint16_t* l_down, int m, int k, int rank,
                               uint16_t* t, uint8_t* a_codes, uint8_t* a_scales,
                               hipStream_t stream);

}  // namespace kq
