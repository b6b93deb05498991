// Calibration and quantization kernels for gfx950 (HBM-bound: coalesced 16-byte accesses,
// one pass over the input, no reuse).
//
// The quantizers follow the NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with
// Low-Precision Quantization", section "Workflow and Quantization": per-tensor FP8 (E4M3)
// for the BMM inputs, per-block FP4 for Q/K/V in the FP4 variant (Fig. 4), FakeQuantize
// semantics, static scales from a max calibrator.  Encoders are bit-exact: E4M3 uses the
// hardware conversion v_cvt_pk_fp8_f32 (round to nearest even, OCP encoding) on inputs
// clamped to +-448, which turns it into the saturating conversion; E2M1 uses gfx950's
// v_cvt_scalef32_pk_fp4_{bf16,f32}, which divides by 2^(E - 127) (E = the exponent field of
// its float scale operand, 0 .. 254; the mantissa is ignored) and rounds to the nearest E2M1
// value, ties to the even code, saturating at +-6 and keeping the sign of zero, and
// v_cvt_scalef32_pk_{bf16,f32}_fp4, which multiplies back exactly (both directions measured
// against the E2M1 definition on every finite bf16 value and every E).  The FP32 denormal
// mode is left at "preserve", so power-of-two rescaling stays exact.

#include "kq_launch.h"
#include "kq_fp4.h"

#include <algorithm>

#pragma clang fp contract(off)

namespace kq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once: do not keep in the caches)
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// clamp to +-448 in one v_med3_f32 (inputs are never NaN: finite bf16 times a finite scale)
__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// Four floats -> four E4M3 bytes (byte i = value i), after the per-tensor scale.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float inv) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a * inv), sat448(b * inv), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c * inv), sat448(d * inv), w, true);
  return (uint32_t)w;
}

// 8 bf16 (one uint4) -> 8 E4M3 bytes (uint2)
__device__ __forceinline__ uint2 e4m3x8(uint4 v, float inv) {
  uint2 r;
  r.x = e4m3x4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y), inv);
  r.y = e4m3x4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w), inv);
  return r;
}

// ------------------------------------------------------------------ amax
// max |x| over bf16 magnitudes: for non-NaN values the 15-bit magnitude field orders like
// |x|, and a non-negative float32 orders like its bit pattern, so the running maximum is an
// unsigned atomic max on the float bits.  At most two workgroups per CU, grid-stride, kU loads
// of 16 bytes in flight per thread, a packed 16-bit max per dword; each workgroup issues its
// atomic only if the stored maximum is below its own (the stored value only grows, so
// skipping then changes nothing), which keeps the atomics on the one result word few.

template <int kT, int kU>
__global__ void __launch_bounds__(kT) amax_bf16_kernel(const uint16_t* __restrict__ x,
                                                       int64_t n, float* amax) {
  const int64_t n8 = n >> 3;
  const uint4* x8 = reinterpret_cast<const uint4*>(x);
  u16x2 m = {0, 0};
  const int64_t stride = (int64_t)gridDim.x * kT * kU;
  for (int64_t base = (int64_t)blockIdx.x * kT * kU + threadIdx.x; base < n8; base += stride) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = base + u * kT;
      v[u] = i < n8 ? ld_stream(x8 + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) m = mag_max(mag_max(mag_max(mag_max(m, v[u].x), v[u].y), v[u].z), v[u].w);
  }
  uint32_t r = max((uint32_t)m[0], (uint32_t)m[1]);
  // tail (n not a multiple of 8): first workgroup only
  if (blockIdx.x == 0) {
    for (int64_t t = (n8 << 3) + threadIdx.x; t < n; t += kT) r = max(r, (uint32_t)(x[t] & 0x7FFFu));
  }
  // wave reduction, then one atomic per workgroup at most
  for (int off = 32; off > 0; off >>= 1) r = max(r, (uint32_t)__shfl_xor((int)r, off));
  __shared__ uint32_t wmax[kT / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t bmax = wmax[0];
    for (int w = 1; w < kT / 64; ++w) bmax = max(bmax, wmax[w]);
    unsigned int* dst = reinterpret_cast<unsigned int*>(amax);
    if ((bmax << 16) > __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(dst, bmax << 16);
  }
}

// ------------------------------------------------------------------ FP8, row layout
// Grid-stride over 16-byte chunks (8 bf16 -> 8 E4M3 bytes), kRowsU chunks per thread per
// step, with the next step's loads issued before this step's conversions and stores, so
// 2 kRowsU x 16 bytes per thread are in flight; consecutive lanes take consecutive chunks in
// every load and store.  Loads are non-temporal (read once).
constexpr int kRowsU = 4;

__global__ void __launch_bounds__(kThreads) fp8_rows_kernel(const uint16_t* __restrict__ x,
                                                            int64_t n, float inv,
                                                            uint8_t* __restrict__ y) {
  const int64_t n8 = n >> 3;
  const uint4* x8 = reinterpret_cast<const uint4*>(x);
  uint2* y8 = reinterpret_cast<uint2*>(y);
  const int64_t stride = (int64_t)gridDim.x * kThreads * kRowsU;
  int64_t base = (int64_t)blockIdx.x * (kThreads * kRowsU) + threadIdx.x;
  uint4 v[kRowsU];
#pragma unroll
  for (int u = 0; u < kRowsU; ++u) {
    const int64_t i = base + u * kThreads;
    v[u] = i < n8 ? ld_stream(x8 + i) : make_uint4(0, 0, 0, 0);
  }
  for (; base < n8; base += stride) {
    uint4 nv[kRowsU];
#pragma unroll
    for (int u = 0; u < kRowsU; ++u) {
      const int64_t i = base + stride + u * kThreads;
      nv[u] = i < n8 ? ld_stream(x8 + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRowsU; ++u) {
      const int64_t i = base + u * kThreads;
      if (i < n8) y8[i] = e4m3x8(v[u], inv);
    }
#pragma unroll
    for (int u = 0; u < kRowsU; ++u) v[u] = nv[u];
  }
}

// ------------------------------------------------------------------ FP8, transposed layout
// One workgroup per (batch*head, 128-token tile).  In each of two passes a thread takes 4
// consecutive tokens 4tq .. 4tq+3 and the 8 channels 8dc .. 8dc+7 (4 loads of 16 bytes; 16
// consecutive lanes cover whole 256-byte token rows), converts them, transposes the 4 x 8
// E4M3 bytes in registers (v_perm_b32) into 8 dwords, one per channel holding the 4 tokens,
// and writes them to LDS; then every thread reads 16-byte segments of the transposed rows and
// writes them out (each 128-token row segment a whole 128-byte line, so no line is shared
// with another workgroup).  Tokens >= N become 0.  The LDS tile holds, for channel d, the
// dwords of token quads in 16-byte granules whose position is XOR-swizzled with (d / 8) % 8,
// so the 64 lanes of a write pass (16 channel groups x 4 quads) spread over all banks and every
// 16-byte read stays aligned.
constexpr int kTT = 128;         // tokens per tile (kq_vt_ld pads the rows to a multiple)

__device__ __forceinline__ int tq_slot(int d, int tq) {
  return 4 * ((tq >> 2) ^ ((d >> 3) & 7)) + (tq & 3);
}

__global__ void __launch_bounds__(kThreads) fp8_transposed_kernel(const uint16_t* __restrict__ x,
                                                                  int64_t n_tokens, int64_t ld,
                                                                  float inv,
                                                                  uint8_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[128][kTT / 4];
  const int64_t bh = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kTT;
  const uint16_t* xs = x + bh * n_tokens * 128;
  uint4 v[2][4];                 // both passes' loads in flight before any conversion
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = threadIdx.x + pass * kThreads;
    const int dc = idx & 15, tq = idx >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t tok = t0 + 4 * tq + j;
      v[pass][j] = tok < n_tokens ? ld_stream(xs + tok * 128 + 8 * dc) : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = threadIdx.x + pass * kThreads;
    const int dc = idx & 15, tq = idx >> 4;
    uint2 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = e4m3x8(v[pass][j], inv);
    // out[i] = byte i of b[0], b[1], b[2], b[3] (channel 8dc + i, tokens 4tq .. 4tq + 3)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w0 = h ? b[0].y : b[0].x, w1 = h ? b[1].y : b[1].x;
      const uint32_t w2 = h ? b[2].y : b[2].x, w3 = h ? b[3].y : b[3].x;
      const uint32_t a01 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);   // w0.0 w1.0 w0.1 w1.1
      const uint32_t b01 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);   // w0.2 w1.2 w0.3 w1.3
      const uint32_t a23 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
      const uint32_t b23 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
      const uint32_t o[4] = {__builtin_amdgcn_perm(a23, a01, 0x05040100u),
                             __builtin_amdgcn_perm(a23, a01, 0x07060302u),
                             __builtin_amdgcn_perm(b23, b01, 0x05040100u),
                             __builtin_amdgcn_perm(b23, b01, 0x07060302u)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 8 * dc + 4 * h + i;
        tile[d][tq_slot(d, tq)] = o[i];
      }
    }
  }
  __syncthreads();
  uint8_t* ys = y + bh * 128 * ld + t0;
#pragma unroll
  for (int u = 0; u < (128 * kTT / 16) / kThreads; ++u) {
    const int c = threadIdx.x + u * kThreads;
    const int d = c >> 3, q = c & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(&tile[d][tq_slot(d, 4 * q)]);
    *reinterpret_cast<uint4*>(ys + (int64_t)d * ld + 16 * q) = v;
  }
}

// ------------------------------------------------------------------ FP4 block (+RoPE, +dq, +FP8)
// Each thread takes 16-byte chunks (8 bf16); the 4 chunks of a 32-element block sit in 4
// consecutive lanes of the same load, so every load and store is contiguous across the wave
// and the block maximum is two quad-permute (DPP) max steps.  kFp4U chunks per thread, all
// loaded before any is converted.  The block's exponent e = clamp(floor(log2 amax) - 2, -127,
// 127) comes from the largest magnitude (an integer max on the float32 bit patterns: a
// non-negative float orders like its bits; bf16 magnitudes are the high halves), and the
// hardware conversions take 2^e as the float with exponent field e + 127.  Outputs per chunk:
// 4 bytes of codes (low nibble = even element), the block's E8M0 byte (first lane of the
// quad), and optionally 16 bytes of dequantized bf16 and 8 bytes of its per-tensor FP8.
constexpr int kFp4U = 4;

template <bool kRope, bool kDq, bool kFp8>
__global__ void __launch_bounds__(kThreads) fp4_block_kernel(
    const uint4* __restrict__ x, int64_t n16, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint4* __restrict__ dq, uint2* __restrict__ fp8, float inv8,
    const float4* __restrict__ rope, int64_t rope_tokens) {
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kFp4U) + threadIdx.x;
  uint4 v[kFp4U];
  float4 cs[kFp4U][2];
#pragma unroll
  for (int u = 0; u < kFp4U; ++u) {
    const int64_t i = base + u * kThreads;
    v[u] = i < n16 ? ld_stream(x + i) : make_uint4(0, 0, 0, 0);
    if constexpr (kRope) {
      // (cos, sin) of the chunk's 4 pairs: d = 128 (16 chunks per row), rows < 2^32 (host)
      const uint32_t row = (uint32_t)(i >> 4);
      const uint32_t tok = row % (uint32_t)rope_tokens;
      const float4* t = rope + (int64_t)tok * 32 + 2 * (int)(i & 15);
      cs[u][0] = i < n16 ? t[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      cs[u][1] = i < n16 ? t[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int u = 0; u < kFp4U; ++u) {
    const int64_t i = base + u * kThreads;
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float f[8];
    uint32_t am;
    if constexpr (kRope) {
      // RoPE-3 on the chunk's 4 adjacent pairs, each product and sum rounded on its own
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float4 t = cs[u][j];
        const float x0 = bf16_lo(w[2 * j]), x1 = bf16_hi(w[2 * j]);
        const float x2 = bf16_lo(w[2 * j + 1]), x3 = bf16_hi(w[2 * j + 1]);
        f[4 * j] = __fsub_rn(__fmul_rn(x0, t.x), __fmul_rn(x1, t.y));
        f[4 * j + 1] = __fadd_rn(__fmul_rn(x0, t.y), __fmul_rn(x1, t.x));
        f[4 * j + 2] = __fsub_rn(__fmul_rn(x2, t.z), __fmul_rn(x3, t.w));
        f[4 * j + 3] = __fadd_rn(__fmul_rn(x2, t.w), __fmul_rn(x3, t.z));
      }
      am = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = max(am, __float_as_uint(f[j]) & 0x7FFFFFFFu);
    } else {
      const u16x2 m = mag_max(mag_max(mag_max(mag_max(u16x2{0, 0}, w[0]), w[1]), w[2]), w[3]);
      am = max((uint32_t)m[0], (uint32_t)m[1]) << 16;
    }
    am = quad_max(am);
    const int e = mx_block_exponent(am);
    const float scale = mx_scale_operand(e);
    uint32_t c;
    if constexpr (kRope) c = e2m1x8_f32(f, scale);
    else c = e2m1x8_bf16(w, scale);
    if (i < n16) {
      codes[i] = c;
      if ((threadIdx.x & 3) == 0) scales[i >> 2] = (uint8_t)(e + 127);
      if constexpr (kDq) dq[i] = e2m1x8_to_bf16(c, scale);
      if constexpr (kFp8) {
        float y[8];
        e2m1x8_to_f32(c, scale, y);
        fp8[i] = make_uint2(e4m3x4(y[0], y[1], y[2], y[3], inv8), e4m3x4(y[4], y[5], y[6], y[7], inv8));
      }
    }
  }
}

int grid_for(int64_t items, int64_t per_block, int cap) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g > cap ? cap : g);
}

}  // namespace

hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, float* amax, hipStream_t stream) {
  // at most 512 workgroups of 512 threads (two per CU) with 13 loads of 16 bytes in flight per
  // thread: a Kontext tensor (26.7 M elements) is read in one pass of 503 workgroups, spread
  // evenly over the CUs.  Measured on it (cold reads): 9.55 us against 10.15 us for one
  // 1024-thread workgroup per CU looping over 4 loads (whose last pass leaves most CUs idle)
  // and 12.2-12.4 us past 512 workgroups (CUs with three).  Few atomics on the one result
  // word: those of thousands of small workgroups serialize on it and cost more than the loads.
  const int grid = grid_for(n / 8, 512 * 13, 512);
  hipLaunchKernelGGL((amax_bf16_kernel<512, 13>), dim3(grid), dim3(512), 0, stream, x, n, amax);
  return hipGetLastError();
}

hipError_t launch_fp8_rows(const uint16_t* x, int64_t n, float inv_scale, uint8_t* y,
                           hipStream_t stream) {
  // 2048 workgroups (8 per CU) striding over the tensor (measured best among exact-cover and
  // persistent shapes of 256 to 1024 threads and 1 to 8 chunks in flight)
  const int64_t per = (int64_t)kThreads * kRowsU * 8;       // elements per workgroup step
  const int64_t grid = std::min<int64_t>((n + per - 1) / per, 2048);
  hipLaunchKernelGGL(fp8_rows_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, n,
                     inv_scale, y);
  return hipGetLastError();
}

hipError_t launch_fp8_transposed(const uint16_t* x, int64_t bh, int64_t n_tokens, int64_t ld,
                                 float inv_scale, uint8_t* y, hipStream_t stream) {
  dim3 grid((unsigned)(ld / kTT), (unsigned)bh);
  hipLaunchKernelGGL(fp8_transposed_kernel, grid, dim3(kThreads), 0, stream, x, n_tokens, ld,
                     inv_scale, y);
  return hipGetLastError();
}

hipError_t launch_fp4_block(const uint16_t* x, int64_t rows, int d, uint8_t* codes,
                            uint8_t* scales, uint16_t* dq, uint8_t* fp8, float inv_scale8,
                            const float* rope_table, int64_t rope_tokens, hipStream_t stream) {
  const int64_t n16 = rows * d / 8;
  const dim3 g((unsigned)((n16 + kThreads * kFp4U - 1) / (kThreads * kFp4U))), t(kThreads);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t* cv = reinterpret_cast<uint32_t*>(codes);
  uint4* dv = reinterpret_cast<uint4*>(dq);
  uint2* fv = reinterpret_cast<uint2*>(fp8);
  const float4* rv = reinterpret_cast<const float4*>(rope_table);
#define KQ_FP4(R, D, F)                                                                       \
  hipLaunchKernelGGL((fp4_block_kernel<R, D, F>), g, t, 0, stream, xv, n16, cv, scales, dv,   \
                     fv, inv_scale8, rv, rope_tokens)
  const bool r = rope_table != nullptr, dd = dq != nullptr, f = fp8 != nullptr;
  if (r) {
    if (dd && f) KQ_FP4(true, true, true); else if (dd) KQ_FP4(true, true, false);
    else if (f) KQ_FP4(true, false, true); else KQ_FP4(true, false, false);
  } else {
    if (dd && f) KQ_FP4(false, true, true); else if (dd) KQ_FP4(false, true, false);
    else if (f) KQ_FP4(false, false, true); else KQ_FP4(false, false, false);
  }
#undef KQ_FP4
  return hipGetLastError();
}

}  // namespace kq
