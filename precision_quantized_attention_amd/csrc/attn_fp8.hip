// Fused quantized attention forward for gfx950: FP8 (E4M3) Q/K/V/P, FP32 softmax, FP32 output —
// the SDPA quantization of the NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with
// Low-Precision Quantization", section "Workflow and Quantization" (bullets 2-4, Fig. 4).
//
// Softmax reading: per query row, an integer offset M = ceil(running max of t) with
// t = raw * c1 (c1 = s_q s_k sm_scale log2 e); p = exp2(t - M) lies in (0, 1]; P is quantized
// with the static per-tensor scale 1/448 as E4M3(448 p); the row sum is taken over the
// unquantized float32 p.  When M grows, the accumulator and the row sum are rescaled by the
// exact power of two 2^(M_old - M_new), and P values already quantized keep their codes:
// E4M3 rounding commutes with power-of-two scaling in its normal range, so the result equals
// the full-row definition up to float32 accumulation order and the E4M3 subnormal range.
//
// Matrix cores.  BMM1 must accumulate in higher precision (blog bullet 2).  gfx950's FP8
// MFMA sums its products in groups of 8 along k and truncates every product of a group to
// 2^-13 of the group's largest one before the float32 accumulate; with the outlier channels
// of diffusion-transformer activations that shifts scores by ~1e-2 in the exp2 domain.  The
// bf16 MFMA keeps ~24 bits, and every E4M3 value is exact in bf16, so BMM1 runs on
// v_mfma_f32_32x32x16_bf16 fed with the E4M3 values of Q and K (converted on chip, the FP8
// codes stay the interface) — the same products, summed without truncation.  BMM2 keeps the
// FP8 MFMA (v_mfma_f32_32x32x64_f8f6f4): there the truncation only touches products of tiny
// probabilities, far below the output tolerance.
//
// Work decomposition (CDNA4, wave64): workgroup = 4 waves = 128 query rows of one
// (batch, head); wave = 32 query rows; key tiles of 64 keys.  Per tile the workgroup stages
// K (converted to bf16, [64][128]) and V^T (FP8, [128][64]) in LDS, double buffered, one
// barrier per tile.  Both products are computed transposed so each lane owns one query row:
//   S^T (keys x queries) = K · Q^T      A = K rows from LDS, B = Q (registers, loaded once)
//   O^T (d x queries)   += V^T · P^T    A = V^T rows from LDS, B = P (registers)
// so the S accumulator of lane (r, g) holds 32 scores of query r, which is exactly the B
// operand layout P needs for the second product: no cross-lane shuffles of P, and the row
// max / row sum need one exchange between lanes r and r + 32.  The K rows fed to the first
// product are permuted (krow below) so that lane group g ends up holding the 32 consecutive
// keys 32g .. 32g + 31 of the tile; V^T then supplies them as one contiguous 32-byte run.

#include "kq_launch.h"

#include <math.h>

namespace kq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kBM = 128;        // query rows per workgroup
constexpr int kBN = 64;         // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKRow = kD * 2;   // bytes per bf16 K row in LDS
constexpr float kLog2_448 = 8.807354922057604f;

// LDS swizzles of 16-byte chunks (XOR on the chunk index) so that the operand reads of any
// 8 consecutive lanes hit 8 different 16-byte slots of a 128-byte bank window.
__device__ __forceinline__ int kswz(int row) {
  return (row & 3) | (((row >> 5) & 1) << 2) | (((row >> 2) & 1) << 3);
}
__device__ __forceinline__ int vswz(int row) { return (row >> 1) & 3; }

// Buffer resource over `bytes` bytes from `base`: loads past the end return zeros (the
// hardware range check), which pads the last key tile and the last query block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
}

// 4 E4M3 codes (one dword) -> 4 bf16 values (two dwords), exact.
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
  const v2bf lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  const v2bf hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
  // format codes 0, 0: both operands OCP E4M3; no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i cat8(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}
__device__ __forceinline__ v8bf as_bf16x8(uint4 v) { return __builtin_bit_cast(v8bf, v); }

__global__ void __launch_bounds__(kThreads, 2) attn_fp8_kernel(AttnParams a, int nqb) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][kBN * kKRow];   // bf16 K tiles
  __shared__ __attribute__((aligned(16))) uint8_t Vs[2][kD * kBN];      // FP8 V^T tiles

  // XCD-aware order: consecutive dispatch slots go round-robin over the 8 XCDs, so give each
  // XCD a contiguous range of (head, query-block) pairs and keep a head's K/V in one L2.
  const int bid = blockIdx.x, total = gridDim.x;
  const int xcd = bid & 7, local = bid >> 3, per = total >> 3, rem = total & 7;
  const int logical = (xcd < rem) ? xcd * (per + 1) + local
                                  : rem * (per + 1) + (xcd - rem) * per + local;
  const int bh = logical / nqb, qb = logical - bh * nqb;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 31, g = l >> 5;
  const int N = a.n;
  const int q = qb * kBM + w * 32 + r;

  // Q operand (bf16 values of the E4M3 codes): step m covers d = 16m .. 16m + 15; lane (r, g)
  // supplies query q, d = 16m + 8g .. +7.  Rows past N read as zeros.
  v8bf qop[8];
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + (int64_t)bh * N * kD, (uint32_t)N * kD);
    const uint32_t qo = (uint32_t)q * kD + 8 * g;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint2 c = bload8(qr, qo + 16 * m);
      const uint2 lo = e4m3x4_to_bf16(c.x), hi = e4m3x4_to_bf16(c.y);
      qop[m] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  }

  // K row (within the tile) read by this lane for key block kb (see file comment).
  int kbase[2], ksw[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int krow = 32 * ((r >> 2) & 1) + 16 * kb + 4 * (r >> 3) + (r & 3);
    kbase[kb] = krow * kKRow;
    ksw[kb] = kswz(krow);
  }

  // Tile loader: each thread moves two 16-byte FP8 chunks of K (written as 2 x 16 bytes of
  // bf16 to LDS) and two 16-byte chunks of V^T per tile.
  const int kr0 = tid >> 3, kc = tid & 7;                  // K chunk tid: row, 16-byte column
  const int kr1 = kr0 + kThreads / 8;                      // K chunk tid + 256
  const int vd0 = tid >> 2, vc = tid & 3;                  // V^T chunk tid
  const int vd1 = vd0 + kThreads / 4;
  const int ks00 = kr0 * kKRow + (((2 * kc) ^ kswz(kr0)) << 4);
  const int ks01 = kr0 * kKRow + (((2 * kc + 1) ^ kswz(kr0)) << 4);
  const int ks10 = kr1 * kKRow + (((2 * kc) ^ kswz(kr1)) << 4);
  const int ks11 = kr1 * kKRow + (((2 * kc + 1) ^ kswz(kr1)) << 4);
  const int vs0 = vd0 * kBN + ((vc ^ vswz(vd0)) << 4), vs1 = vd1 * kBN + ((vc ^ vswz(vd1)) << 4);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + (int64_t)bh * N * kD, (uint32_t)N * kD);
  const uint32_t ko0 = kr0 * kD + kc * 16, ko1 = kr1 * kD + kc * 16;
  const uint8_t* Vg = a.vt + (int64_t)bh * kD * a.ldv;
  const uint8_t* vg0 = Vg + (int64_t)vd0 * a.ldv + vc * 16;
  const uint8_t* vg1 = Vg + (int64_t)vd1 * a.ldv + vc * 16;
  uint4 kx0, kx1, vx0, vx1;
#define KQ_GLOAD(k0)                                                 \
  {                                                                  \
    kx0 = bload16(krs, (uint32_t)(k0) * kD + ko0);                   \
    kx1 = bload16(krs, (uint32_t)(k0) * kD + ko1);                   \
    vx0 = *reinterpret_cast<const uint4*>(vg0 + (k0));               \
    vx1 = *reinterpret_cast<const uint4*>(vg1 + (k0));               \
  }
#define KQ_LSTORE(buf)                                                                   \
  {                                                                                      \
    uint8_t* kb_ = Ks[buf];                                                              \
    uint2 a_ = e4m3x4_to_bf16(kx0.x), b_ = e4m3x4_to_bf16(kx0.y);                        \
    uint2 c_ = e4m3x4_to_bf16(kx0.z), d_ = e4m3x4_to_bf16(kx0.w);                        \
    *reinterpret_cast<uint4*>(kb_ + ks00) = make_uint4(a_.x, a_.y, b_.x, b_.y);          \
    *reinterpret_cast<uint4*>(kb_ + ks01) = make_uint4(c_.x, c_.y, d_.x, d_.y);          \
    a_ = e4m3x4_to_bf16(kx1.x); b_ = e4m3x4_to_bf16(kx1.y);                              \
    c_ = e4m3x4_to_bf16(kx1.z); d_ = e4m3x4_to_bf16(kx1.w);                              \
    *reinterpret_cast<uint4*>(kb_ + ks10) = make_uint4(a_.x, a_.y, b_.x, b_.y);          \
    *reinterpret_cast<uint4*>(kb_ + ks11) = make_uint4(c_.x, c_.y, d_.x, d_.y);          \
    *reinterpret_cast<uint4*>(&Vs[buf][vs0]) = vx0;                                      \
    *reinterpret_cast<uint4*>(&Vs[buf][vs1]) = vx1;                                      \
  }

  v16f o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = 0.0f;
  float m_run = -INFINITY;   // integer-valued running offset M
  float lsum = 0.0f;         // partial row sum of 448 p over this lane's keys
  const float c1 = a.c1;

  const int ntiles = (N + kBN - 1) / kBN;
  KQ_GLOAD(0)
  KQ_LSTORE(0)
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const int k0 = j * kBN;
    if (j + 1 < ntiles) KQ_GLOAD(k0 + kBN)

    // ---- BMM1 (bf16 matrix cores on E4M3 values): S^T tile, 64 keys x 32 queries per wave
    v16f s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
    const uint8_t* kt = Ks[buf];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 kv =
            *reinterpret_cast<const uint4*>(kt + kbase[kb] + (((2 * m + g) ^ ksw[kb]) << 4));
        s[kb] = mfma_bf16(as_bf16x8(kv), qop[m], s[kb]);
      }
    }
    // lane (r, g): s[kb][i] = score of query r against key k0 + 32g + 16kb + i
    if (k0 + kBN > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + 32 * g + 16 * kb + i >= N) s[kb][i] = -INFINITY;
    }

    // ---- softmax (float32), integer offset in the exp2 domain
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m_run, ceilf(mx * c1));
    if (__any(mnew != m_run)) {
      const float alpha =
          (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, (int)(m_run - mnew));
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[c][i] *= alpha;
      m_run = mnew;
    }
    const float bias = kLog2_448 - m_run;
    v8i pop;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 0], c1, bias));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 1], c1, bias));
        const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 2], c1, bias));
        const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 3], c1, bias));
        lsum += (p0 + p1) + (p2 + p3);
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
        pop[4 * kb + i4] = wd;
      }
    }

    // ---- BMM2 (FP8 matrix cores): O^T += V^T · P^T, four 32-row blocks of d
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 32 * c + r;
      const uint8_t* vr = &Vs[buf][d * kBN];
      const int sw = vswz(d);
      const uint4 lo = *reinterpret_cast<const uint4*>(vr + (((2 * g) ^ sw) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(vr + (((2 * g + 1) ^ sw) << 4));
      o[c] = mfma_f8(cat8(lo, hi), pop, o[c]);
    }

    if (j + 1 < ntiles) KQ_LSTORE(buf ^ 1)
    __syncthreads();
  }
#undef KQ_GLOAD
#undef KQ_LSTORE

  // ---- epilogue: O = acc * s_v / sum(448 p); lane (r, g) holds d = 32c + 8(i/4) + 4g + i%4
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float scale = a.s_v / ltot;
  if (q < N) {
    float* op = a.o + ((int64_t)bh * N + q) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4 v = make_float4(o[c][4 * i4] * scale, o[c][4 * i4 + 1] * scale,
                               o[c][4 * i4 + 2] * scale, o[c][4 * i4 + 3] * scale);
        *reinterpret_cast<float4*>(op + 32 * c + 8 * i4 + 4 * g) = v;
      }
    if (a.stats != nullptr && g == 0) {
      float2 st = make_float2(m_run, ltot * (1.0f / 448.0f));
      *reinterpret_cast<float2*>(a.stats + ((int64_t)bh * N + q) * 2) = st;
    }
  }
}

}  // namespace

hipError_t launch_attn_fp8(const AttnParams& p, hipStream_t stream) {
  const int nqb = (p.n + kBM - 1) / kBM;
  const int64_t blocks = (int64_t)nqb * p.bh;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, nqb);
  return hipGetLastError();
}

}  // namespace kq
