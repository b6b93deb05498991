// Test-only probe: one matrix-core instruction per wave on caller-given operands, so a test can
// compare what gfx950's FP8 matrix instructions return with a model of how they add their
// products.  Not part of libkq; built beside the tests.
//
// Every instance is one wave of 64 lanes.  Instance i reads A[i] ([M][K] E4M3 codes, row-major),
// B[i] ([N][K] E4M3 codes: row n is column n of the product's right operand), C[i] ([M][N]
// float32 accumulator input) and writes D[i] = A B^T + C ([M][N] float32), with
// (M, N, K) = (32, 32, 64), (16, 16, 128), (32, 32, 16), (16, 16, 32) or (32, 32, 16) for the
// forms below.  Operand slot s of a row (s = 0 .. K-1, the index into the caller's row) goes to
// lane group g = s / (bytes per lane), byte s % (bytes per lane) of the lane that supplies the
// row; both operands use the same assignment, so D is the product over the caller's k order
// whatever order the hardware visits the bytes in.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

enum Form {
  kF8_32x32x64 = 0,         // v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, no block scales)
  kF8_32x32x64_scaled = 1,  // v_mfma_scale_f32_32x32x64_f8f6f4 with the caller's E8M0 scales
  kF8_16x16x128 = 2,        // v_mfma_f32_16x16x128_f8f6f4
  kF8_16x16x128_scaled = 3, // v_mfma_scale_f32_16x16x128_f8f6f4
  kF8_32x32x16 = 4,         // v_mfma_f32_32x32x16_fp8_fp8
  kF8_16x16x32 = 5,         // v_mfma_f32_16x16x32_fp8_fp8
  kBF16_32x32x16 = 6,       // v_mfma_f32_32x32x16_bf16 on the bf16 values of the E4M3 codes
};

template <int kM, int kK, int kBytes>
__device__ __forceinline__ void load_operand(const uint8_t* X, int lane, uint8_t (&o)[kBytes]) {
  const int row = lane % kM, g = lane / kM;
#pragma unroll
  for (int b = 0; b < kBytes; ++b) o[b] = X[row * kK + g * kBytes + b];
}

__device__ __forceinline__ v8i pack8(const uint8_t (&o)[32]) {
  v8i r;
#pragma unroll
  for (int w = 0; w < 8; ++w)
    r[w] = (int)((uint32_t)o[4 * w] | ((uint32_t)o[4 * w + 1] << 8) |
                 ((uint32_t)o[4 * w + 2] << 16) | ((uint32_t)o[4 * w + 3] << 24));
  return r;
}
__device__ __forceinline__ long pack2(const uint8_t (&o)[8]) {
  uint64_t r = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) r |= (uint64_t)o[b] << (8 * b);
  return (long)r;
}

// D layouts: 32x32 forms, lane l holds column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4;
// 16x16 forms, column l % 16, rows 4 (l / 16) + i.
template <int kForm>
__global__ void __launch_bounds__(64) probe_kernel(const uint8_t* A, const uint8_t* B,
                                                   const float* C, float* D, int scale_a,
                                                   int scale_b) {
  constexpr bool k32 = kForm == kF8_32x32x64 || kForm == kF8_32x32x64_scaled ||
                       kForm == kF8_32x32x16 || kForm == kBF16_32x32x16;
  constexpr int kM = k32 ? 32 : 16;
  constexpr int kK = (kForm == kF8_32x32x64 || kForm == kF8_32x32x64_scaled) ? 64
                   : (kForm == kF8_16x16x128 || kForm == kF8_16x16x128_scaled) ? 128
                   : (kForm == kF8_16x16x32) ? 32 : 16;
  constexpr int kBytes = kK * kM / 64;
  const int lane = threadIdx.x;
  const int64_t inst = blockIdx.x;
  const uint8_t* a = A + inst * kM * kK;
  const uint8_t* b = B + inst * kM * kK;
  const float* c = C + inst * kM * kM;
  float* d = D + inst * kM * kM;
  uint8_t ao[kBytes], bo[kBytes];
  load_operand<kM, kK, kBytes>(a, lane, ao);
  load_operand<kM, kK, kBytes>(b, lane, bo);
  if constexpr (k32) {
    v16f acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = c[(8 * (i / 4) + 4 * (lane / 32) + i % 4) * kM + lane % 32];
    if constexpr (kForm == kF8_32x32x64) {
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pack8(ao), pack8(bo), acc, 0, 0, 0, 0, 0, 0);
    } else if constexpr (kForm == kF8_32x32x64_scaled) {
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pack8(ao), pack8(bo), acc, 0, 0, 0, scale_a, 0, scale_b);
    } else if constexpr (kForm == kF8_32x32x16) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(pack2(ao), pack2(bo), acc, 0, 0, 0);
    } else {
      v8bf x, y;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t wa = (uint32_t)ao[2 * h] | ((uint32_t)ao[2 * h + 1] << 8);
        const uint32_t wb = (uint32_t)bo[2 * h] | ((uint32_t)bo[2 * h + 1] << 8);
        const v2bf pa = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)wa, 1.0f, false);
        const v2bf pb = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)wb, 1.0f, false);
        x[2 * h] = pa[0]; x[2 * h + 1] = pa[1];
        y[2 * h] = pb[0]; y[2 * h + 1] = pb[1];
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) d[(8 * (i / 4) + 4 * (lane / 32) + i % 4) * kM + lane % 32] = acc[i];
  } else {
    v4f acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = c[(4 * (lane / 16) + i) * kM + lane % 16];
    if constexpr (kForm == kF8_16x16x128) {
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pack8(ao), pack8(bo), acc, 0, 0, 0, 0, 0, 0);
    } else if constexpr (kForm == kF8_16x16x128_scaled) {
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pack8(ao), pack8(bo), acc, 0, 0, 0, scale_a, 0, scale_b);
    } else {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pack2(ao), pack2(bo), acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) d[(4 * (lane / 16) + i) * kM + lane % 16] = acc[i];
  }
}

// Both float32 -> E4M3 conversions the attention kernel could use for P, on every float32 bit
// pattern in [lo, lo + n): v_cvt_pk_fp8_f32 and v_cvt_scalef32_pk_fp8_f32 with scale 1.0, each
// converting the pair (x, x).  Counts the patterns whose two results differ and keeps the
// smallest such pattern (mismatch[0] = count, mismatch[1] = first pattern or 0xFFFFFFFF).
__global__ void __launch_bounds__(256) cvt_probe_kernel(uint32_t lo, uint32_t n,
                                                        unsigned int* mismatch) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  unsigned int count = 0, first = 0xFFFFFFFFu;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) {
    const uint32_t bits = lo + i;
    const float x = __uint_as_float(bits);
    const int plain = __builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false) & 0xFFFF;
    const v2s sc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, x, x, 1.0f, false);
    const int scaled = (int)((uint32_t)(uint16_t)sc[0]);
    if (plain != scaled) {
      ++count;
      first = bits < first ? bits : first;
    }
  }
  if (count) {
    atomicAdd(&mismatch[0], count);
    atomicMin(&mismatch[1], first);
  }
}

// The two conversions of x[i] (as the pair (x, x)): the code bytes of each, for checking their
// behaviour past the E4M3 range.
__global__ void cvt_values_kernel(const float* x, uint8_t* plain, uint8_t* scaled, int n) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  plain[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x[i], x[i], 0, false) & 0xFF);
  const v2s sc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, x[i], x[i], 1.0f, false);
  scaled[i] = (uint8_t)((uint16_t)sc[0] & 0xFF);
}

extern "C" {

int cvt_values_run(const float* x, uint8_t* plain, uint8_t* scaled, int n, hipStream_t stream) {
  if (x == nullptr || plain == nullptr || scaled == nullptr || n < 1) return -1;
  hipLaunchKernelGGL(cvt_values_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, x, plain, scaled, n);
  return (int)hipGetLastError();
}

// Compares the two conversions on the bit patterns [lo, lo + n) (see cvt_probe_kernel);
// mismatch is a device array of 2 words the caller sets to {0, 0xFFFFFFFF}.
int cvt_probe_run(uint32_t lo, uint32_t n, unsigned int* mismatch, hipStream_t stream) {
  if (mismatch == nullptr || n == 0 || (uint64_t)lo + n > (1ull << 32)) return -1;
  hipLaunchKernelGGL(cvt_probe_kernel, dim3(2048), dim3(256), 0, stream, lo, n, mismatch);
  return (int)hipGetLastError();
}

// Shape of a form: *m (= n) and *k; returns 0, or -1 for an unknown form.
int mfma_probe_shape(int form, int* m, int* k) {
  static const int M[7] = {32, 32, 16, 16, 32, 16, 32};
  static const int K[7] = {64, 64, 128, 128, 16, 32, 16};
  if (form < 0 || form > 6 || m == nullptr || k == nullptr) return -1;
  *m = M[form];
  *k = K[form];
  return 0;
}

// Runs `count` instances of `form` (device pointers, sizes as in the file comment); E8M0 scale
// bytes apply to the scaled forms only.  Returns 0, -1 for bad arguments, or the HIP error.
int mfma_probe_run(int form, const uint8_t* a, const uint8_t* b, const float* c, float* d,
                   int count, int scale_a, int scale_b, hipStream_t stream) {
  if (a == nullptr || b == nullptr || c == nullptr || d == nullptr || count < 1) return -1;
  if (scale_a < 0 || scale_a > 255 || scale_b < 0 || scale_b > 255) return -1;
  const dim3 g((unsigned)count), t(64);
  switch (form) {
    case kF8_32x32x64: hipLaunchKernelGGL(probe_kernel<kF8_32x32x64>, g, t, 0, stream, a, b, c, d, scale_a, scale_b); break;
    case kF8_32x32x64_scaled: hipLaunchKernelGGL(probe_kernel<kF8_32x32x64_scaled>, g, t, 0, stream, a, b, c, d, scale_a, scale_b); break;
    case kF8_16x16x128: hipLaunchKernelGGL(probe_kernel<kF8_16x16x128>, g, t, 0, stream, a, b, c, d, scale_a, scale_b); break;
    case kF8_16x16x128_scaled: hipLaunchKernelGGL(probe_kernel<kF8_16x16x128_scaled>, g, t, 0, stream, a, b, c, d, scale_a, scale_b); break;
    case kF8_32x32x16: hipLaunchKernelGGL(probe_kernel<kF8_32x32x16>, g, t, 0, stream, a, b, c, d, scale_a, scale_b); break;
    case kF8_16x16x32: hipLaunchKernelGGL(probe_kernel<kF8_16x16x32>, g, t, 0, stream, a, b, c, d, scale_a, scale_b); break;
    case kBF16_32x32x16: hipLaunchKernelGGL(probe_kernel<kBF16_32x32x16>, g, t, 0, stream, a, b, c, d, scale_a, scale_b); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
