// Quantized projection GEMMs for gfx950: C = A · B^T with A the activations [M][K] (one row
// per token) and B the weights [N][K] (one row per output feature), both K-contiguous, C in
// float32 or rounded once to bf16 — the linear layers around the attention in the NVIDIA blog "Optimizing FLUX.1
// Kontext for Image Editing with Low-Precision Quantization" (section "Workflow and
// Quantization": per-tensor FP8 and per-block FP4 post-training quantization of the linear
// layers).
//   FP8 (W8A8): E4M3 codes, per-tensor scales: C = s_a s_b sum_k a_mk b_nk.
//   MXFP4: E2M1 codes two per byte (even element in the low nibble) with an E8M0 scale per 32
//   consecutive k, for both operands: C = sum_k dq(a)_mk dq(b)_nk.  The scales feed the scaled
//   MFMA directly.
//
// Work decomposition (CDNA4, wave64): workgroup = 8 waves (two per SIMD) = a 256 x 256 tile of
// C; wave (wm, wn) computes 64 (m) x 128 (n) = 2 x 4 tiles of 32 x 32 on the 32x32x64 f8f6f4
// MFMA (the scaled form for MXFP4, the unscaled one for FP8; 128 accumulator registers), with
// a step's six operand sub-tiles read from LDS before its first MFMA.  The product is computed
// transposed, D = B_sub · A_sub^T, so each lane owns one row m of C and stores runs of 4
// consecutive n.  A k-step moves 64 bytes of each operand row (64 FP8 or 128 FP4 elements)
// through LDS: rows padded to 80 bytes (conflict-free 16-byte operand reads), three stages so
// a step's tile is written two steps before it is multiplied and one barrier per step
// suffices; the HBM loads of a step are issued two steps before their LDS store (two register
// sets), and the two waves of a SIMD hide each other's operand reads.
//
// Operand layouts of the f8f6f4 MFMA (measured): for E4M3, lane (r, g) holds row r with
// k = 16g .. 16g+15 in bytes 0-15 and k = 32+16g .. in bytes 16-31; for E2M1, lane (r, g)
// holds k = 32g .. 32g+31 in 32 nibbles (low first) and supplies the scale of that 32-block.

#include "kq_launch.h"

namespace kq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 256;            // workgroup tile of C (M and N)
constexpr int kThreads = 512;         // 8 waves, two per SIMD
constexpr int kRowBytes = 64;         // bytes of one operand row per k-step
constexpr int kPitch = kRowBytes + 16;
constexpr int kOpStage = kTile * kPitch;            // 20480 bytes per operand
constexpr int kScStage = kTile * 4;                 // 4 E8M0 bytes per row per k-step (FP4)
constexpr int kStage = 2 * kOpStage + 2 * kScStage; // A, B codes + A, B scales
constexpr int kStages = 3;
constexpr int kGroupM = 8;            // tiles of M visited together (L2 reuse of B tiles)

#define KQ_FENCE() __builtin_amdgcn_sched_barrier(0)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// A wave holds 8 tiles of 32 x 32 (128 accumulator registers) and two waves share each SIMD.
// FP8 takes the unscaled form (zero scale operands select v_mfma_f32_32x32x64_f8f6f4).
template <bool kFP4>
__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c, int sa, int sb) {
  if (kFP4) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i cat8(uint4 lo, uint4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// One k-step of a wave's 128 (n) x 64 (m) tile: 4 sub-tiles of B rows (the MFMA's A side) and
// 2 of A rows (its B side), each 32 bytes per lane read from the LDS stage st = [A rows][B rows]
// codes, then [A rows][B rows] scale dwords.  FP8: lane (r, g) takes bytes 16g and 32 + 16g of
// its row (k = 16g.., 32+16g..); FP4: k-chunk h = 0, 1 at bytes 32h + 16g (k = 64h + 32g ..),
// with the scale byte of block 2h + g.
template <bool kFP4>
__device__ __forceinline__ void kstep(v16f (&acc)[4][2], const uint8_t* st, int rbase_n,
                                      int rbase_m, int sbase_n, int sbase_m, int g) {
  uint4 n[4][2], m[2][2];
  uint32_t sn[4], sm[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint8_t* pm = st + rbase_m + i * 32 * kPitch;
    m[i][0] = *reinterpret_cast<const uint4*>(pm);
    m[i][1] = *reinterpret_cast<const uint4*>(pm + 32);
    if (kFP4) sm[i] = *reinterpret_cast<const uint32_t*>(st + 2 * kOpStage + sbase_m + i * 32 * 4);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* pn = st + kOpStage + rbase_n + i * 32 * kPitch;
    n[i][0] = *reinterpret_cast<const uint4*>(pn);
    n[i][1] = *reinterpret_cast<const uint4*>(pn + 32);
    if (kFP4) sn[i] = *reinterpret_cast<const uint32_t*>(st + 2 * kOpStage + kScStage + sbase_n + i * 32 * 4);
  }
  // All operand reads are issued before the first MFMA (the empty asm needs every read's
  // result): one LDS round trip per step instead of one per sub-tile pair, which the compiler
  // would otherwise choose to save registers.
  {
#define KQ_V4(X_) (u32x4{(X_).x, (X_).y, (X_).z, (X_).w})
    asm volatile("" ::"v"(KQ_V4(n[0][0])), "v"(KQ_V4(n[0][1])), "v"(KQ_V4(n[1][0])),
                 "v"(KQ_V4(n[1][1])), "v"(KQ_V4(n[2][0])), "v"(KQ_V4(n[2][1])),
                 "v"(KQ_V4(n[3][0])), "v"(KQ_V4(n[3][1])), "v"(KQ_V4(m[0][0])),
                 "v"(KQ_V4(m[0][1])), "v"(KQ_V4(m[1][0])), "v"(KQ_V4(m[1][1])));
    if (kFP4) asm volatile("" ::"v"(sn[0]), "v"(sn[1]), "v"(sn[2]), "v"(sn[3]), "v"(sm[0]), "v"(sm[1]));
#undef KQ_V4
  }
  if (kFP4) {
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const int sa = (int)((sn[ni] >> (8 * (2 * h + g))) & 0xFF);
          const int sb = (int)((sm[mi] >> (8 * (2 * h + g))) & 0xFF);
          acc[ni][mi] = mfma<true>(cat8(n[ni][h], z), cat8(m[mi][h], z), acc[ni][mi], sa, sb);
        }
  } else {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        acc[ni][mi] = mfma<false>(cat8(n[ni][0], n[ni][1]), cat8(m[mi][0], m[mi][1]),
                                  acc[ni][mi], 127, 127);
  }
}

// Two float32 values -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32) in one dword.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <bool kFP4, bool kBf16>
__global__ void __launch_bounds__(kThreads, 1) gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage];
  const int tiles_m = (p.m + kTile - 1) / kTile, tiles_n = (p.n + kTile - 1) / kTile;
  const int total = tiles_m * tiles_n;
  // XCD-aware order: each XCD takes a contiguous range of tiles, visited in groups of kGroupM
  // tiles of M per tile of N so concurrent workgroups share A and B tiles in the XCD's L2
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3, per = total >> 3, rm = total & 7;
  const int logical = (xcd < rm) ? xcd * (per + 1) + local : rm * (per + 1) + (xcd - rm) * per + local;
  const int gsz = kGroupM * tiles_n;
  const int first_m = (logical / gsz) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int mt = __builtin_amdgcn_readfirstlane(first_m + (logical % gsz) % gm);
  const int nt = __builtin_amdgcn_readfirstlane((logical % gsz) / gm);

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 31, g = l >> 5;
  const int wm = w & 3, wn = w >> 2;                   // wave tile: m 64 wm .., n 128 wn ..
  const int row_bytes = kFP4 ? p.k / 2 : p.k;          // bytes per operand row
  const int nsteps = row_bytes / kRowBytes;
  const int sc_bytes = p.k / 32;                       // E8M0 bytes per row (FP4)

  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.a, (uint32_t)p.m * row_bytes);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(p.b, (uint32_t)p.n * row_bytes);

  // staging: each operand tile is 256 rows x 4 chunks of 16 bytes; thread t owns chunks t and
  // t + 512 of both (rows t/4 and t/4 + 128, chunk t % 4); for FP4, threads 0-255 stage the
  // scale dword of A row t and threads 256-511 that of B row t - 256
  const int crow = tid >> 2, cchunk = tid & 3;
  const uint32_t goff_a = (uint32_t)(mt * kTile + crow) * row_bytes + 16 * cchunk;
  const uint32_t goff_b = (uint32_t)(nt * kTile + crow) * row_bytes + 16 * cchunk;
  const uint32_t row128 = 128u * row_bytes;
  const int loff = crow * kPitch + 16 * cchunk;
  const bool sc_a = __builtin_amdgcn_readfirstlane(tid) < 256;
  const __amdgpu_buffer_rsrc_t scr =
      make_rsrc(sc_a ? p.a_scales : p.b_scales, (uint32_t)(sc_a ? p.m : p.n) * sc_bytes);
  const uint32_t soff = (uint32_t)((sc_a ? mt : nt) * kTile + (tid & 255)) * sc_bytes;
  const int sloff = 2 * kOpStage + (sc_a ? 0 : kScStage) + 4 * (tid & 255);

  uint4 xa0[2], xa1[2], xb0[2], xb1[2];
  uint32_t xs[2] = {0, 0};
#define KQ_LOAD(s, R)                                                     \
  {                                                                       \
    const uint32_t o_ = (uint32_t)(s) * kRowBytes;                        \
    xa0[R] = bload16(ar, goff_a + o_);                                    \
    xa1[R] = bload16(ar, goff_a + row128 + o_);                           \
    xb0[R] = bload16(br, goff_b + o_);                                    \
    xb1[R] = bload16(br, goff_b + row128 + o_);                           \
    if (kFP4) xs[R] = bload4(scr, soff + 4 * (uint32_t)(s));              \
  }
#define KQ_STORE(stage, R)                                                \
  {                                                                       \
    uint8_t* st_ = lds + (stage) * kStage;                                \
    *reinterpret_cast<uint4*>(st_ + loff) = xa0[R];                       \
    *reinterpret_cast<uint4*>(st_ + loff + 128 * kPitch) = xa1[R];        \
    *reinterpret_cast<uint4*>(st_ + kOpStage + loff) = xb0[R];            \
    *reinterpret_cast<uint4*>(st_ + kOpStage + loff + 128 * kPitch) = xb1[R]; \
    if (kFP4) *reinterpret_cast<uint32_t*>(st_ + sloff) = xs[R];          \
  }

  const int rbase_n = (wn * 128 + r) * kPitch + 16 * g;
  const int rbase_m = (wm * 64 + r) * kPitch + 16 * g;
  const int sbase_n = (wn * 128 + r) * 4, sbase_m = (wm * 64 + r) * 4;

  v16f acc[4][2];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ni][mi][i] = 0.0f;

  // Step s stores register set s % 2 (step s + 2, fetched in step s - 2) into stage (s + 2) % 3
  // (read last in step s - 1), fetches step s + 4 into the same set and multiplies stage s % 3
  // (stored in step s - 2).  Past the last step the fetches read bytes of the next rows (or
  // zeros past the end) into stages nothing reads.
  KQ_LOAD(0, 0);
  KQ_STORE(0, 0);
  KQ_LOAD(1, 1);
  KQ_STORE(1, 1);
  KQ_LOAD(2, 0);
  KQ_LOAD(3, 1);
  __syncthreads();
  int st_mul = 0, st_wr = 2;
  for (int s = 0; s < nsteps; s += 2) {
    KQ_STORE(st_wr, 0);
    KQ_LOAD(s + 4, 0);
    KQ_FENCE();
    kstep<kFP4>(acc, lds + st_mul * kStage, rbase_n, rbase_m, sbase_n, sbase_m, g);
    __syncthreads();
    st_mul = st_mul == 2 ? 0 : st_mul + 1;
    st_wr = st_wr == 2 ? 0 : st_wr + 1;
    if (s + 1 < nsteps) {
      KQ_STORE(st_wr, 1);
      KQ_LOAD(s + 5, 1);
      KQ_FENCE();
      kstep<kFP4>(acc, lds + st_mul * kStage, rbase_n, rbase_m, sbase_n, sbase_m, g);
      __syncthreads();
      st_mul = st_mul == 2 ? 0 : st_mul + 1;
      st_wr = st_wr == 2 ? 0 : st_wr + 1;
    }
  }
#undef KQ_LOAD
#undef KQ_STORE

  // epilogue: lane (r, g) owns row m = mt*256 + wm*64 + 32 mi + r and, for each sub-tile ni,
  // columns n = nt*256 + wn*128 + 32 ni + 8q + 4g .. +3 (q = 0..3): a float4, or 4 bf16
  const float scale = p.scale;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int m = mt * kTile + wm * 64 + 32 * mi + r;
    if (m >= p.m) continue;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nt * kTile + wn * 128 + 32 * ni + 8 * q + 4 * g;
        if (n < p.n) {
          const v16f& c = acc[ni][mi];
          const float c0 = c[4 * q] * scale, c1 = c[4 * q + 1] * scale;
          const float c2 = c[4 * q + 2] * scale, c3 = c[4 * q + 3] * scale;
          const int64_t off = (int64_t)m * p.n + n;
          if constexpr (kBf16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.c) + off) =
                make_uint2(bf16x2_rne(c0, c1), bf16x2_rne(c2, c3));
          else
            *reinterpret_cast<float4*>(static_cast<float*>(p.c) + off) = make_float4(c0, c1, c2, c3);
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, bool fp4, hipStream_t stream) {
  const int tiles = ((p.m + kTile - 1) / kTile) * ((p.n + kTile - 1) / kTile);
  if (fp4 && p.out_bf16)
    hipLaunchKernelGGL((gemm_kernel<true, true>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else if (fp4)
    hipLaunchKernelGGL((gemm_kernel<true, false>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else if (p.out_bf16)
    hipLaunchKernelGGL((gemm_kernel<false, true>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<false, false>), dim3(tiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kq
