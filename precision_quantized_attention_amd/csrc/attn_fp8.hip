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
// Work decomposition (CDNA4, wave64): workgroup = 8 waves = 256 query rows of one
// (batch, head), one workgroup per CU; wave = 32 query rows; key tiles of 64 keys.  Per tile
// the workgroup stages K (converted to bf16, [64][128]) and V^T (FP8, [128][64]) in LDS,
// double buffered.  The two waves sharing a SIMD run in ping-pong: while one issues matrix-core
// work the other runs its softmax on the VALU (see the schedule in the kernel).  Both products are computed transposed so each lane owns one query row:
//   S^T (keys x queries) = K · Q^T      A = K rows from LDS, B = Q (registers, loaded once)
//   O^T (d x queries)   += V^T · P^T    A = V^T rows from LDS, B = P (registers)
// so the S accumulator of lane (r, g) holds 32 scores of query r, which is exactly the B
// operand layout P needs for the second product: no cross-lane shuffles of P, and the row
// max / row sum need one exchange between lanes r and r + 32.  The K rows fed to the first
// product are permuted (krow_of_key) so that lane group g ends up holding the 32 consecutive
// keys 32g .. 32g + 31 of the tile; V^T then supplies them as one contiguous 32-byte run.
// LDS rows are padded by 16 bytes, which spreads the operand reads of any 8 (or 16)
// consecutive lanes over distinct 16-byte bank slots.

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
constexpr int kWaves = 8;                   // two groups of four waves, one wave per SIMD each
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;            // query rows per workgroup (32 per wave)
constexpr int kBN = 64;                     // keys per tile
constexpr int kKPitch = kD * 2 + 16;        // bf16 K row in LDS + 16 bytes of padding
constexpr int kVPitch = kBN + 16;           // FP8 V^T row in LDS + 16 bytes of padding
constexpr int kKStage = kBN * kKPitch;      // 17408 bytes
constexpr int kVStage = kD * kVPitch;       // 10240 bytes
constexpr float kLog2_448 = 8.807354922057604f;

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
// FP8 x FP8 with E8M0 block scales on the B operand (format codes 0, 0: both operands OCP
// E4M3; A unscaled, 127 = 1.0).  The 64 k-values form two scale blocks: bytes 0-15 of both
// lane groups are block 0 and bytes 16-31 block 1; lane group g supplies block g's scale.
__device__ __forceinline__ v16f mfma_f8_scaled(v8i a, v8i b, v16f c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

__device__ __forceinline__ v8i cat8(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}
__device__ __forceinline__ v8bf as_bf16x8(uint4 v) { return __builtin_bit_cast(v8bf, v); }

// max(x[l], x[l ^ 32]) for every lane l: v_permlane32_swap with both operands x leaves
// {x[l], x[l ^ 32]} in its two results (in an order that depends on the half of the wave).
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// LDS row of key kappa (0..63 within a tile): rows are stored in the order the first product
// consumes them — row 32kb + r feeds lane r of key block kb (see the file comment for the
// key permutation), so every operand read is a fixed per-lane base plus an immediate offset.
__device__ __forceinline__ int krow_of_key(int kappa) {
  return 32 * ((kappa >> 4) & 1) + 8 * ((kappa >> 2) & 3) + 4 * ((kappa >> 5) & 1) + (kappa & 3);
}

__global__ void __launch_bounds__(kThreads, 1) attn_fp8_kernel(AttnParams a, int nqb) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2 * kKStage];   // bf16 K tiles
  __shared__ __attribute__((aligned(16))) uint8_t Vs[2 * kVStage];   // FP8 V^T tiles

  // XCD-aware order: consecutive dispatch slots go round-robin over the 8 XCDs, so give each
  // XCD a contiguous range of (head, query-block) pairs and keep a head's K/V in one L2.
  const int bid = blockIdx.x, total = gridDim.x;
  const int xcd = bid & 7, local = bid >> 3, per = total >> 3, rem = total & 7;
  const int logical = (xcd < rem) ? xcd * (per + 1) + local
                                  : rem * (per + 1) + (xcd - rem) * per + local;
  // (the integer division runs on the vector unit; readfirstlane returns the values to scalar
  // registers so the buffer descriptors below stay scalar)
  const int bh = __builtin_amdgcn_readfirstlane(logical / nqb);
  const int qb = logical - bh * nqb;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 31, g = l >> 5;
  const int grp = w >> 2;                   // 0: waves 0-3, 1: waves 4-7 (one per SIMD each)
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

  // Operand read bases (bytes within a stage); block kb / step m / d-block c are immediates.
  const int kread = r * kKPitch + 16 * g;
  const int vread = r * kVPitch + 32 * g;

  // Tile staging: a K tile is 512 FP8 chunks of 16 bytes (64 keys x 8) and a V^T tile 512
  // chunks (128 d-rows x 4); each thread owns chunk `tid` of both.  Each group writes its half
  // during its own matrix-core phase, when its VALU is otherwise idle.
  const int kr = tid >> 3, kc = tid & 7;                   // key row, 16-byte column
  const int vd = tid >> 2, vc = tid & 3;                   // d row, 16-byte column
  const int kw = krow_of_key(kr) * kKPitch + 32 * kc;
  const int vw = vd * kVPitch + 16 * vc;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + (int64_t)bh * N * kD, (uint32_t)N * kD);
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(a.vt + (int64_t)bh * kD * a.ldv, (uint32_t)(kD * a.ldv));
  const uint32_t ko = kr * kD + kc * 16;
  const uint32_t vo = (uint32_t)(vd * a.ldv + vc * 16);
  uint4 kx, vx;
#define KQ_STAGE_K(buf)                                                                  \
  {                                                                                      \
    uint8_t* kb_ = Ks + (buf) * kKStage + kw;                                            \
    const uint2 a_ = e4m3x4_to_bf16(kx.x), b_ = e4m3x4_to_bf16(kx.y);                    \
    const uint2 c_ = e4m3x4_to_bf16(kx.z), d_ = e4m3x4_to_bf16(kx.w);                    \
    *reinterpret_cast<uint4*>(kb_) = make_uint4(a_.x, a_.y, b_.x, b_.y);                 \
    *reinterpret_cast<uint4*>(kb_ + 16) = make_uint4(c_.x, c_.y, d_.x, d_.y);            \
  }
#define KQ_STAGE_V(buf) { *reinterpret_cast<uint4*>(Vs + (buf) * kVStage + vw) = vx; }

  v16f o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = 0.0f;
  v16f s[2];
  v8i pop = {0, 0, 0, 0, 0, 0, 0, 0};       // P codes of the previous tile (none before tile 0)
  int pscale = 127;          // E8M0 scale of this lane group's P block (see the softmax)
  float m_ref = 0.0f;        // per-row reference offset (integer-valued), set on tile 0
  float m_top = -INFINITY;   // largest block offset seen (for the row statistics)
  float lsum = 0.0f;         // partial row sum of 448 p * 2^(M_kb - m_ref) over this lane's keys
  const float c1 = a.c1;
  const int ntiles = (N + kBN - 1) / kBN;

  // Ping-pong schedule.  Every wave alternates a matrix-core phase (BMM2 of the previous
  // tile, BMM1 of the current one, staging of the next tiles) and a VALU phase (softmax of the
  // current tile).  Group 1 runs half a period behind group 0, so on every SIMD one wave is in
  // its matrix-core phase while the other is in its VALU phase; workgroup barriers separate
  // the phases.  Phase 2j: group 0 MFMA(j), group 1 softmax(j-1); phase 2j+1: group 0
  // softmax(j), group 1 MFMA(j).  K(j) and V(j-1) are read in phases 2j and 2j+1; K(j+1) and
  // V(j) are written to the other buffers in the same two phases (half by each group) and are
  // complete before phase 2j+2.  Both groups pass 2 * ntiles + 3 barriers.
  kx = bload16(krs, ko);                       // K(0), all 512 chunks
  KQ_STAGE_K(0)
  *reinterpret_cast<uint4*>(Vs + kVStage + vw) = make_uint4(0, 0, 0, 0);   // "V(-1)" = 0
  kx = bload16(krs, (uint32_t)kBN * kD + ko);  // K(1): this thread's chunk
  vx = bload16(vrs, vo);                       // V(0)
  __syncthreads();
  if (grp == 1) __syncthreads();
  for (int j = 0; j <= ntiles; ++j) {
    // ---------------- matrix-core phase (one straight-line block; at j == 0 the P codes and
    // the V^T buffer are zero, at j == ntiles the scores are never used)
    const int cur = j & 1;
    {
      // Operand window: the 8 V^T reads of BMM2(j-1) and the first 4 K reads of BMM1(j) go
      // out first; then every MFMA is issued together with the read four K steps ahead, so the
      // LDS latency hides behind the matrix cores.  sched_barrier(0) pins this order.
      const uint8_t* vt_ = Vs + (cur ^ 1) * kVStage + vread;
      const uint8_t* kt_ = Ks + cur * kKStage + kread;
#define KQ_KREAD(t) (*reinterpret_cast<const uint4*>(kt_ + ((t) & 1) * 32 * kKPitch + 32 * ((t) >> 1)))
      uint4 vv[8], kv[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        vv[2 * c] = *reinterpret_cast<const uint4*>(vt_ + c * 32 * kVPitch);
        vv[2 * c + 1] = *reinterpret_cast<const uint4*>(vt_ + c * 32 * kVPitch + 16);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) kv[t] = KQ_KREAD(t);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {                     // BMM2(j-1): O^T += V^T · P^T
        o[c] = mfma_f8_scaled(cat8(vv[2 * c], vv[2 * c + 1]), pop, o[c], pscale);
        kv[4 + c] = KQ_KREAD(4 + c);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {                    // BMM1(j): S^T = K · Q^T, t = 2m + kb
        const int m = t >> 1, kb = t & 1;
        s[kb] = mfma_bf16(as_bf16x8(kv[t]), qop[m], m == 0 ? v16f{} : s[kb]);
        if (t + 8 < 16) kv[t + 8] = KQ_KREAD(t + 8);
        __builtin_amdgcn_sched_barrier(0);
      }
#undef KQ_KREAD
      // stage K(j+1) and V(j) from registers, then prefetch K(j+2) and V(j+1); past the end
      // the buffer loads return zeros and the stages they fill are never read
      KQ_STAGE_K(cur ^ 1)
      KQ_STAGE_V(cur)
      kx = bload16(krs, (uint32_t)(j + 2) * kBN * kD + ko);
      vx = bload16(vrs, vo + (uint32_t)(j + 1) * kBN);
    }
    __syncthreads();
    // ---------------- VALU phase: softmax of tile j
    if (j < ntiles) {
      const int k0 = j * kBN;
      // lane (r, g): s[kb][i] = score of query r against key k0 + 32g + 16kb + i
      if (k0 + kBN > N) {
        const int nv_ = N - k0 - 32 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (16 * kb + i >= nv_) s[kb][i] = -INFINITY;
      }
      // BMM2's P operand is E4M3 with an E8M0 block scale per 32-key block: block kb holds
      // the s[kb] values of both lanes of a row (bytes 0-15 / 16-31 of each lane's operand),
      // and lane group g supplies the scale of block g.  Each block is quantized against its
      // own integer offset M_kb = ceil(max t over the block) (so p <= 1 and 448 p fits E4M3)
      // and carries 2^(M_kb - m_ref) as its scale: no accumulator rescale when the running
      // maximum grows.  Codes differ from full-row ones by exact powers of two, which E4M3
      // rounding preserves in its normal range.
      float mx0 = s[0][0], mx1 = s[1][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        mx0 = fmaxf(mx0, s[0][i]);
        mx1 = fmaxf(mx1, s[1][i]);
      }
      mx0 = max_with_partner(mx0);
      mx1 = max_with_partner(mx1);
      float mb0 = ceilf(mx0 * c1), mb1 = ceilf(mx1 * c1);
      if (j == 0) {                    // row reference: the row's offset on the first tile
        const float mr = fmaxf(mb0, mb1);
        m_ref = (mr == -INFINITY) ? 0.0f : mr;
      }
      if (mx0 == -INFINITY) mb0 = m_ref;             // whole block masked: p = 0 below
      if (mx1 == -INFINITY) mb1 = m_ref;
      float d0 = mb0 - m_ref, d1 = mb1 - m_ref;
      if (__builtin_expect(__any(fmaxf(d0, d1) > 64.0f), 0)) {
        // keep 2^d far from float32 overflow: move the row reference up, rescale exactly
        const float up = fmaxf(fmaxf(d0, d1) - 32.0f, 0.0f);
        const float alpha = __builtin_amdgcn_ldexpf(1.0f, -(int)up);
        lsum *= alpha;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[c][i] *= alpha;
        m_ref += up;
        d0 -= up;
        d1 -= up;
      }
      d0 = fmaxf(d0, -126.0f);         // weights below 2^-126 of the reference: negligible
      d1 = fmaxf(d1, -126.0f);
      m_top = fmaxf(m_top, fmaxf(mb0, mb1));
      pscale = 127 + (int)(g ? d1 : d0);
      float part[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float bias = kLog2_448 - (kb ? mb1 : mb0);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 0], c1, bias));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 1], c1, bias));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 2], c1, bias));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * i4 + 3], c1, bias));
          const float q4 = (p0 + p1) + (p2 + p3);
          part[kb] = i4 ? part[kb] + q4 : q4;
          // both halves of the dword are written; the previous codes only stand in for the
          // untouched half of the first conversion
          int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pop[4 * kb + i4], false);
          wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
          pop[4 * kb + i4] = wd;
        }
      }
      const float part0 = part[0], part1 = part[1];
      lsum += __builtin_amdgcn_ldexpf(part0, (int)d0) + __builtin_amdgcn_ldexpf(part1, (int)d1);
    }
    __syncthreads();
  }
  if (grp == 0) __syncthreads();
#undef KQ_STAGE_K
#undef KQ_STAGE_V

  // ---- epilogue: O = acc * s_v / sum(448 p); lane (r, g) holds d = 32c + 8(i/4) + 4g + i%4
  const float ltot = lsum + __shfl_xor(lsum, 32);      // sum of 448 p relative to m_ref
  const float scale = a.s_v / ltot;
  const float m_row = fmaxf(m_top, __shfl_xor(m_top, 32));   // the row's M = ceil(max t)
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
      // (M, l) with l relative to the row's M
      float2 st = make_float2(m_row, __builtin_amdgcn_ldexpf(ltot * (1.0f / 448.0f), (int)(m_ref - m_row)));
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
