// Calibration and quantization kernels for gfx950 (HBM-bound: coalesced 16-byte accesses,
// one pass over the input, no reuse).
//
// The quantizers follow the NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with
// Low-Precision Quantization", section "Workflow and Quantization": per-tensor FP8 (E4M3)
// for the BMM inputs, per-block FP4 for Q/K/V in the FP4 variant (Fig. 4), FakeQuantize
// semantics, static scales from a max calibrator.  Encoders are bit-exact: E4M3 uses the
// hardware conversion v_cvt_pk_fp8_f32 (round to nearest even, OCP encoding) on inputs
// clamped to +-448, which turns it into the saturating conversion; E2M1 is decided by
// comparing the exactly rescaled magnitude against the midpoints of the E2M1 value set.
// The FP32 denormal mode is left at "preserve", so power-of-two rescaling stays exact.

#include "kq_launch.h"

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

__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

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
// unsigned atomic max on the float bits.
// kT threads per workgroup, kU loads of 16 bytes in flight per thread per step.
template <int kT, int kU>
__global__ void __launch_bounds__(kT) amax_bf16_kernel(const uint16_t* __restrict__ x,
                                                       int64_t n, float* amax) {
  const int64_t n8 = n >> 3;
  const uint4* x8 = reinterpret_cast<const uint4*>(x);
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kT;
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  // fold each 32-bit word as two 16-bit magnitudes
#define KQ_FOLD(w) { uint32_t t_ = (w) & 0x7FFF7FFFu; m = max(m, max(t_ & 0xFFFFu, t_ >> 16)); }
  for (; i + (kU - 1) * stride < n8; i += kU * stride) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = ld_stream(x8 + i + u * stride);
#pragma unroll
    for (int u = 0; u < kU; ++u) { KQ_FOLD(v[u].x) KQ_FOLD(v[u].y) KQ_FOLD(v[u].z) KQ_FOLD(v[u].w) }
  }
  for (; i < n8; i += stride) {
    uint4 v = ld_stream(x8 + i);
    KQ_FOLD(v.x) KQ_FOLD(v.y) KQ_FOLD(v.z) KQ_FOLD(v.w)
  }
#undef KQ_FOLD
  // tail (n not a multiple of 8): first block only
  if (blockIdx.x == 0) {
    for (int64_t t = (n8 << 3) + threadIdx.x; t < n; t += kT) m = max(m, (uint32_t)(x[t] & 0x7FFFu));
  }
  // wave reduction then one atomic per workgroup
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[kT / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = wmax[0];
    for (int w = 1; w < kT / 64; ++w) b = max(b, wmax[w]);
    atomicMax(reinterpret_cast<unsigned int*>(amax), b << 16);
  }
}

// ------------------------------------------------------------------ FP8, row layout
__global__ void __launch_bounds__(kThreads) fp8_rows_kernel(const uint16_t* __restrict__ x,
                                                            int64_t n, float inv,
                                                            uint8_t* __restrict__ y) {
  const int64_t n8 = n >> 3;
  const uint4* x8 = reinterpret_cast<const uint4*>(x);
  uint2* y8 = reinterpret_cast<uint2*>(y);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    y8[i] = e4m3x8(ld_stream(x8 + i), inv);
  }
}

// ------------------------------------------------------------------ FP8, transposed layout
// One workgroup per (batch*head, 128-token tile): read 128 x 128 bf16 rows coalesced, convert,
// transpose through LDS, write 128 rows of 128 tokens coalesced (each row segment a whole
// 128-byte line, so no line is shared with another workgroup).  Tokens >= N become 0.
constexpr int kTT = 128;         // tokens per tile (kq_vt_ld pads the rows to a multiple)
constexpr int kTPad = 4;         // LDS row padding (bytes) against bank conflicts

__global__ void __launch_bounds__(kThreads) fp8_transposed_kernel(const uint16_t* __restrict__ x,
                                                                  int64_t n_tokens, int64_t ld,
                                                                  float inv,
                                                                  uint8_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[128][kTT + kTPad];
  const int64_t bh = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kTT;
  const uint16_t* xs = x + bh * n_tokens * 128;
#pragma unroll
  for (int u = 0; u < (kTT * 128 / 8) / kThreads; ++u) {
    const int c = threadIdx.x + u * kThreads;
    const int tok = c >> 4;
    const int d0 = (c & 15) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t0 + tok < n_tokens)
      v = ld_stream(xs + (t0 + tok) * 128 + d0);
    const uint2 b = e4m3x8(v, inv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[d0 + i][tok] = (uint8_t)(b.x >> (8 * i));
      tile[d0 + 4 + i][tok] = (uint8_t)(b.y >> (8 * i));
    }
  }
  __syncthreads();
  uint8_t* ys = y + bh * 128 * ld + t0;
#pragma unroll
  for (int u = 0; u < (128 * kTT / 16) / kThreads; ++u) {
    const int c = threadIdx.x + u * kThreads;
    const int d = c / (kTT / 16);
    const int q = c % (kTT / 16);
    uint4 v;
    v.x = *reinterpret_cast<const uint32_t*>(&tile[d][16 * q]);
    v.y = *reinterpret_cast<const uint32_t*>(&tile[d][16 * q + 4]);
    v.z = *reinterpret_cast<const uint32_t*>(&tile[d][16 * q + 8]);
    v.w = *reinterpret_cast<const uint32_t*>(&tile[d][16 * q + 12]);
    *reinterpret_cast<uint4*>(ys + (int64_t)d * ld + 16 * q) = v;
  }
}

// ------------------------------------------------------------------ FP4 block (+RoPE, +FP8)
// One thread per 8 consecutive elements; the 4 threads of a 32-element block are 4
// consecutive lanes and share the block maximum through two xor shuffles.
__device__ __forceinline__ uint32_t e2m1_code(float x, float inv_pow2) {
  const float q = fabsf(x) * inv_pow2;   // exact: multiplication by a power of two
  uint32_t c = (q > 0.25f) + (q >= 0.75f) + (q > 1.25f) + (q >= 1.75f) + (q > 2.5f) +
               (q >= 3.5f) + (q > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 0x8u);
}

// E2M1 magnitude code (0..7) -> value * 2^e, exact (denormals preserved), sign from `neg`.
__device__ __forceinline__ float e2m1_value(uint32_t code, int e) {
  const uint32_t c = code & 7u;
  const uint32_t E = c >> 1;
  const float mant = (E == 0) ? 0.5f * (float)(c & 1u) : 1.0f + 0.5f * (float)(c & 1u);
  const float v = __builtin_amdgcn_ldexpf(mant, e + (E == 0 ? 0 : (int)E - 1));
  return (code & 8u) ? -v : v;
}

__global__ void __launch_bounds__(kThreads) fp4_block_kernel(
    const uint16_t* __restrict__ x, int64_t n8, int d, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint4* __restrict__ dq, uint2* __restrict__ fp8, float inv8,
    const float* __restrict__ rope, int64_t rope_tokens) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= n8) return;   // n8 is a multiple of 4, so whole 4-lane groups leave together
  const uint4 v = ld_stream(reinterpret_cast<const uint4*>(x) + t);
  float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  if (rope != nullptr) {
    const int64_t e0 = t * 8;
    const int64_t row = e0 / d;
    const int64_t tok = row % rope_tokens;
    const int pair0 = (int)(e0 - row * d) >> 1;
    const float4* cs = reinterpret_cast<const float4*>(rope + (tok * (d / 2) + pair0) * 2);
    const float4 a = cs[0], b = cs[1];
    const float c[4] = {a.x, a.z, b.x, b.z};
    const float s[4] = {a.y, a.w, b.y, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = f[2 * j], x1 = f[2 * j + 1];
      f[2 * j] = __fsub_rn(__fmul_rn(x0, c[j]), __fmul_rn(x1, s[j]));
      f[2 * j + 1] = __fadd_rn(__fmul_rn(x0, s[j]), __fmul_rn(x1, c[j]));
    }
  }
  uint32_t am = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = max(am, __float_as_uint(f[j]) & 0x7FFFFFFFu);
  am = max(am, (uint32_t)__shfl_xor((int)am, 1));
  am = max(am, (uint32_t)__shfl_xor((int)am, 2));
  // e = clamp(floor(log2 amax) - 2, -127, 127); for a normal amax floor(log2) is the unbiased
  // exponent; a zero or subnormal amax has floor(log2) <= -127, so e clamps to -127.
  const int expf = (int)(am >> 23);
  const int e = max(expf - 129, -127);
  const float inv_pow2 = __uint_as_float((uint32_t)(127 - e) << 23);
  uint32_t packed = 0;
  uint32_t cv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    cv[j] = e2m1_code(f[j], inv_pow2);
    packed |= cv[j] << (4 * j);
  }
  codes[t] = packed;
  if ((t & 3) == 0) scales[t >> 2] = (uint8_t)(e + 127);
  if (dq != nullptr || fp8 != nullptr) {
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = e2m1_value(cv[j], e);
    if (dq != nullptr) {
      uint4 o;
      o.x = (__float_as_uint(y[0]) >> 16) | (__float_as_uint(y[1]) & 0xFFFF0000u);
      o.y = (__float_as_uint(y[2]) >> 16) | (__float_as_uint(y[3]) & 0xFFFF0000u);
      o.z = (__float_as_uint(y[4]) >> 16) | (__float_as_uint(y[5]) & 0xFFFF0000u);
      o.w = (__float_as_uint(y[6]) >> 16) | (__float_as_uint(y[7]) & 0xFFFF0000u);
      dq[t] = o;
    }
    if (fp8 != nullptr) {
      uint2 o;
      o.x = e4m3x4(y[0], y[1], y[2], y[3], inv8);
      o.y = e4m3x4(y[4], y[5], y[6], y[7], inv8);
      fp8[t] = o;
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
  // at most 256 workgroups of 1024 threads (one per CU), 4 loads of 16 bytes in flight per
  // thread: enough bytes in flight for HBM, and few atomics on the one result word (the
  // atomics of many small workgroups serialize on it and cost more than the loads)
  const int grid = grid_for(n / 8, 1024 * 4, 256);
  hipLaunchKernelGGL((amax_bf16_kernel<1024, 4>), dim3(grid), dim3(1024), 0, stream, x, n, amax);
  return hipGetLastError();
}

hipError_t launch_fp8_rows(const uint16_t* x, int64_t n, float inv_scale, uint8_t* y,
                           hipStream_t stream) {
  const int grid = grid_for(n / 8, kThreads * 2, 256 * 16);
  hipLaunchKernelGGL(fp8_rows_kernel, dim3(grid), dim3(kThreads), 0, stream, x, n, inv_scale, y);
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
  const int64_t n8 = rows * d / 8;
  const int64_t grid = (n8 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(fp4_block_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, n8, d,
                     reinterpret_cast<uint32_t*>(codes), scales, reinterpret_cast<uint4*>(dq),
                     reinterpret_cast<uint2*>(fp8), inv_scale8, rope_table, rope_tokens);
  return hipGetLastError();
}

}  // namespace kq
