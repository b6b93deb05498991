// Fused quantized attention forward for gfx950: FP8 (E4M3) Q/K/V/P, FP32 softmax, FP32 output —
// the SDPA quantization of the NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with
// Low-Precision Quantization", section "Workflow and Quantization" (bullets 2-4, Fig. 4).
//
// Softmax reading: per query row, an integer offset M = ceil(max of t) with
// t = raw * c1 (c1 = s_q s_k sm_scale log2 e); p = exp2(t - M) lies in (0, 1]; P is quantized
// with the static per-tensor scale 1/448 as E4M3(448 p); the row sum is taken over the
// unquantized float32 p.  Online, each 32-key block of a row is quantized against its own
// integer offset M_kb = ceil(max of t over the block), and BMM2's E8M0 block scale carries
// 2^(M_kb - m_ref) (m_ref: the row's offset on its first tile), so no accumulator is rescaled
// when the maximum grows (a guarded rare path moves m_ref when an offset would pass 2^64).
// Codes then differ from full-row ones by exact powers of two, which E4M3 rounding preserves
// in its normal range: the result equals the full-row definition up to float32 accumulation
// order and the E4M3 subnormal range.
//
// Variants (template arguments): kFP4, BMM1 on the FP4 block-quantized Q and K themselves
// (E2M1 + E8M0 on the scaled MFMA) instead of their FP8 re-quantization; kMode 1, the first
// pass of the literal FakeQuantize of the normalized P (statistics only); kMode 2, its second
// pass (the row's M and l known, every block at the same offset).
// With a bf16 Q (AttnParams::q_bf16, FP8 BMM1), Q's per-tensor FP8 quantization runs here
// instead of in the FP8 tensor quantizer, with its conversion: each Q element is read by one
// lane of one workgroup, so this saves the quantizer's read of Q and the write and re-read of
// its codes, and the codes (hence O) are the quantizer's bit for bit.
//
// Matrix cores.  The page executes QK^T on FP8 (E4M3) inputs (its higher-precision
// accumulation refers to the projection GEMM that produces Q, K, V); the reading taken here
// sums BMM1's E4M3 products exactly up to float32 accumulation, as the oracle does.  gfx950's
// FP8 matrix instructions cannot: every FP8 form (32x32x64 and 16x16x128 f8f6f4, scaled or
// not, and the older fp8_fp8 forms) adds its products in groups of 8 and truncates each one
// toward zero to 2^-13 of the group's largest exponent sum (measured on the hardware), which
// moves scores by ~1e-3 in the exp2 domain; through the E4M3 rounding of P and V's outlier
// channels that misses the output tolerance (max-abs ~2 on the 512x512 Kontext workload, and
// still ~0.14 with the 16 largest channels summed exactly).  So, as a departure from running
// BMM1 on FP8 matrix instructions, BMM1 runs on v_mfma_f32_32x32x16_bf16 fed with the E4M3
// values of Q and K (each exact in bf16; converted on chip, the FP8 codes stay the interface):
// the same products, added in float32.  BMM2 keeps the FP8 instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4): there the truncation only touches products of tiny
// probabilities, far below the output tolerance.
//
// Work decomposition (CDNA4, wave64): workgroup = 8 waves = 256 query rows of one
// (batch, head), one workgroup per CU, two waves per SIMD; wave = 32 query rows; key tiles of
// 64 keys.  Per tile the workgroup stages K (converted to bf16, [64][128]) and V^T (FP8,
// [128][64]) in LDS, double buffered.  Both products are computed transposed so each lane
// owns one query row:
//   S^T (keys x queries) = K · Q^T      A = K rows from LDS, B = Q (registers, loaded once)
//   O^T (d x queries)   += V^T · P^T    A = V^T rows from LDS, B = P (registers)
// so the S accumulator of lane (r, g) holds 32 scores of query r, which is exactly the B
// operand layout P needs for the second product: no cross-lane shuffles of P, and the row
// max / row sum need one exchange between lanes r and r + 32.  The K rows fed to the first
// product are permuted (krow_of_key) so that lane group g ends up holding the 32 consecutive
// keys 32g .. 32g + 31 of the tile; V^T then supplies them as one contiguous 32-byte run.
// LDS rows are padded by 16 bytes, which spreads the operand reads of any 8 (or 16)
// consecutive lanes over distinct 16-byte bank slots.
//
// Schedule (measured on gfx950).  A single wave issues an ordinary VALU instruction only
// about every 8-9 cycles (exp2 and the FP8 conversion about 11), so a tile's softmax costs one
// wave more cycles than its MFMAs.  (Under this load the clock settles where the power budget
// holds it, so the time also follows the energy of the work, mostly the matrix cores'.)
// When both waves of a SIMD mix MFMA and VALU work finely, the older one takes the matrix pipe
// and the other stalls behind its MFMA issues.  So the two waves of each SIMD alternate roles
// (ping-pong): one issues the 20 MFMAs of a tile (matrix-core phase, raised priority) with the
// light VALU work that fits between them — the E4M3 codes and row sums of the previous tile,
// the block maxima of this one, the staging — while the other runs the exp2 part of its
// softmax (VALU phase); workgroup barriers separate the phases.  sched_barrier pins the
// interleaving inside the matrix-core phase.

#include "kq_launch.h"

#include <math.h>

#include <mutex>

// Key-split workspace of kq_attn_quant_fwd_noalloc: one copy per GPU, held until the process
// ends.  Host code never uses this name as an address (it is a host-side stand-in); it uses
// the device address hipGetSymbolAddress returns, once per device, in attn_static_workspace.
static __device__ __align__(256) unsigned char scratch[kq::kAttnStaticWorkspaceBytes];

namespace kq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kWaves = 8;                   // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;            // query rows per workgroup (32 per wave)
static_assert(kBM == kAttnRowsPerBlock, "workspace layout assumes 256-row query blocks");
constexpr int kBN = 64;                     // keys per tile
constexpr int kKPitch = kD * 2 + 16;        // bf16 K row in LDS + 16 bytes of padding
constexpr int kVPitch = kBN + 16;           // FP8 V^T row in LDS + 16 bytes of padding
constexpr int kKStage = kBN * kKPitch;      // 17408 bytes
constexpr int kVStage = kD * kVPitch;       // 10240 bytes
// native MXFP4 BMM1: K rows stay packed E2M1 (64 bytes for d = 128) + an E8M0 scale dword
constexpr int kK4Pitch = kD / 2 + 16;       // packed K row in LDS + 16 bytes of padding
constexpr int kK4Codes = kBN * kK4Pitch;    // 5120 bytes
constexpr int kK4Stage = kK4Codes + kBN * 4;  // + the 4 scale bytes of every key: 5376 bytes
constexpr float kLog2_448 = 8.807354922057604f;

// The exp2 argument (t - M_kb + log2 448, t = fl32(raw c1)) is normally one fma,
// fma(raw, c1, log2 448 - M_kb): exact product, one rounding.  It differs from the definition's
// order by at most half an ulp of t, so it stays within the rounding of E4M3 (p never passes
// 464 / 448) while |t| < 2^20, which the host guarantees from the scales (c1 448^2 128 < 2^20)
// before it launches this form.  Otherwise the kWide instance forms the argument in the
// definition's order, unfused: fl32(raw c1), minus the offset, plus log2 448.
__device__ __forceinline__ float unfused_arg(float s, float c1, float m, float add) {
#pragma clang fp contract(off)
  const float t = s * c1;
  return (t - m) + add;
}

#define KQ_FENCE() __builtin_amdgcn_sched_barrier(0)

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
// The same with the non-temporal cache policy (aux bit 1): for data read once per workgroup
// (Q), which would otherwise take L2 space from the K and V tiles every workgroup of the XCD
// reads.
__device__ __forceinline__ uint2 bload8_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Four float32 -> four E4M3 codes (byte i = value i) after the per-tensor scale: the
// conversion of the FP8 tensor quantizer (product rounded to float32, clamped to +-448 by one
// v_med3, then v_cvt_pk_fp8_f32, nearest even), so Q quantized here has the quantizer's codes.
__device__ __forceinline__ uint32_t e4m3x4_q(float a, float b, float c, float d, float inv) {
  auto sat = [](float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a * inv), sat(b * inv), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c * inv), sat(d * inv), w, true);
  return (uint32_t)w;
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

// E2M1 x E2M1 (format codes 4, 4) with an E8M0 scale per 32-k block on both operands: lane
// (r, g) holds k = 32g .. 32g + 31 of its row as 32 nibbles (low nibble first) in the low 16
// bytes of its operand and supplies the scale byte of that block.
__device__ __forceinline__ v16f mfma_fp4(uint4 a, uint4 b, v16f c, int scale_a, int scale_b) {
  const v8i az = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bz = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(az, bz, c, 4, 4, 0, scale_a, 0, scale_b);
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

// Work assignment over the 8 XCDs (dispatch slot y runs on XCD y mod 8, and each XCD has its
// own L2).  Slots [0, nfull) are whole query blocks; the rem * split slots after them are key
// ranges of the remaining rem blocks, numbered contiguously per XCD, and a block belongs to the
// XCD that runs its first range.  Each XCD takes one contiguous range of logical blocks ((b, h)
// major, query block minor): first the blocks of its whole-block slots, then the blocks it owns
// among the split ones.  So the blocks of a head, and the key ranges of a split block, stay on
// one XCD (exactly so when the counts divide by 8 and by the split) and share its copy of the
// head's K and V.
__device__ __forceinline__ int slots_on_xcd(int n, int x) { return (n - x + 7) >> 3; }

struct XcdSplit {
  int first_part;      // first key-range index of this XCD
  int parts;           // key-range slots on this XCD
  int owned;           // split blocks whose first range runs on this XCD
  int logical0;        // first logical block of this XCD
  int whole;           // whole-block slots on this XCD
};

__device__ __forceinline__ XcdSplit xcd_split(const AttnParams& a, int xcd) {
  const int total = a.rem * a.split;
  XcdSplit r{0, 0, 0, 0, 0};
  for (int x = 0; x <= xcd; ++x) {
    const int whole = slots_on_xcd(a.nfull, x);
    const int parts = slots_on_xcd(a.nfull + total, x) - whole;
    const int owned = a.split > 0 ? (r.first_part + parts + a.split - 1) / a.split -
                                        (r.first_part + a.split - 1) / a.split
                                  : 0;
    if (x == xcd) {
      r.parts = parts;
      r.owned = owned;
      r.whole = whole;
      break;
    }
    r.first_part += parts;
    r.logical0 += whole + owned;
  }
  return r;
}

// Logical block of split block blk (0 .. rem-1): the XCD whose key ranges hold its first one.
__device__ __forceinline__ int split_block_logical(const AttnParams& a, int blk) {
  const int first = blk * a.split, total = a.rem * a.split;
  int first_part = 0, logical0 = 0;
  for (int x = 0;; ++x) {
    const int whole = slots_on_xcd(a.nfull, x);
    const int parts = slots_on_xcd(a.nfull + total, x) - whole;
    const int before = (first_part + a.split - 1) / a.split;   // blocks owned by earlier XCDs
    if (first < first_part + parts || x == 7) return logical0 + whole + blk - before;
    first_part += parts;
    logical0 += whole + (first_part + a.split - 1) / a.split - before;
  }
}

// Per-thread constants of a workgroup.
struct Geo {
  __amdgpu_buffer_rsrc_t krs, vrs;   // K rows [N][128], V^T rows [128][ldv] of this (b, h)
  __amdgpu_buffer_rsrc_t ksr;        // MXFP4: K scale dwords [N][4]
  uint32_t ko, vo;                   // this thread's staging chunk in the first tile
  int kw, vw;                        // its LDS destination within a stage
  int kread, vread;                  // this lane's operand read bases within a stage
  int krole;                         // MXFP4 K staging: 0 codes, 1 scale dword, 2 none
  int n4r;                           // MXFP4: this lane's scale dword index (row r) in a stage
  int n, g;
  int kbase;                         // first key of the workgroup's key range
  float c1;
  float m_fix, lb_fix;               // R1 pass 2: the row's offset M and log2(inv_p / l)
};

// BMM1's Q operand, held in registers for the whole key loop.
template <bool kFP4> struct QOp;
template <> struct QOp<false> {
  v8bf v[8];                         // bf16 values of the E4M3 codes, d = 16m + 8g .. +7
};
template <> struct QOp<true> {
  uint4 c[2];                        // packed E2M1, d = 64h + 32g .. +31
  int s[2];                          // E8M0 byte of block 2h + g
};

// This thread's part of K(tile) (tile counted from the key range's first tile); loads past
// the end of the buffers return zeros.
template <bool kFP4>
__device__ __forceinline__ uint4 kload(const Geo& G, int tile) {
  if constexpr (kFP4) {
    if (G.krole == 0) return bload16(G.krs, (uint32_t)tile * kBN * (kD / 2) + G.ko);
    if (G.krole == 1)
      return make_uint4(__builtin_amdgcn_raw_buffer_load_b32(G.ksr, (uint32_t)tile * kBN * 4 + G.ko, 0, 0), 0u, 0u, 0u);
    return make_uint4(0u, 0u, 0u, 0u);
  } else {
    return bload16(G.krs, (uint32_t)tile * kBN * kD + G.ko);
  }
}

// Stage K(tile) (FP8 codes in kx, converted to bf16) and V^T(tile) (vx) into buffer `buf`.
template <bool kFP4>
__device__ __forceinline__ void stage_k(uint8_t* Ks, int buf, const Geo& G, uint4 kx) {
  if constexpr (kFP4) {
    uint8_t* kb = Ks + buf * kK4Stage + G.kw;
    if (G.krole == 0) *reinterpret_cast<uint4*>(kb) = kx;
    else if (G.krole == 1) *reinterpret_cast<uint32_t*>(kb) = kx.x;
    return;
  }
  uint8_t* kb = Ks + buf * kKStage + G.kw;
  const uint2 a = e4m3x4_to_bf16(kx.x), b = e4m3x4_to_bf16(kx.y);
  const uint2 c = e4m3x4_to_bf16(kx.z), d = e4m3x4_to_bf16(kx.w);
  *reinterpret_cast<uint4*>(kb) = make_uint4(a.x, a.y, b.x, b.y);
  *reinterpret_cast<uint4*>(kb + 16) = make_uint4(c.x, c.y, d.x, d.y);
}
__device__ __forceinline__ void stage_v(uint8_t* Vs, int buf, const Geo& G, uint4 vx) {
  *reinterpret_cast<uint4*>(Vs + buf * kVStage + G.vw) = vx;
}

__device__ __forceinline__ uint4 kread(const uint8_t* kt, int t) {
  return *reinterpret_cast<const uint4*>(kt + (t & 1) * 32 * kKPitch + 32 * (t >> 1));
}

// Sets the scores of keys >= N to -inf; lane (r, g): s[kb][i] = key k0 + 32g + 16kb + i.
// Two float32 values to E4M3 codes (round to nearest even) in the low or high 16 bits of old.
// The scaled conversion with scale 1.0 returns the plain conversion's codes (checked on every
// float32 in [-448, 448]) and issues at a higher rate.
__device__ __forceinline__ int e4m3_pair(float a, float b, int old, bool hi) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s r = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, old), a, b, 1.0f, true)
                   : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, old), a, b, 1.0f, false);
  return __builtin_bit_cast(int, r);
}

// The 32 scores of a lane (s[0], s[1]) become exp2(arg(kb, s)), in place.  Each step issues the
// argument of value t + 2 and the exp2 of value t, so a transcendental always has an
// independent full-rate instruction beside it (a wave alone issues back-to-back exp2 at about
// half the rate it issues them interleaved).
template <class Arg>
__device__ __forceinline__ void exp2_pipeline(v16f (&s)[2], Arg arg) {
  s[0][0] = arg(0, s[0][0]);
  s[0][1] = arg(0, s[0][1]);
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    if (t + 2 < 32) {
      const int u = t + 2;
      s[u >> 4][u & 15] = arg(u >> 4, s[u >> 4][u & 15]);
    }
    s[t >> 4][t & 15] = __builtin_amdgcn_exp2f(s[t >> 4][t & 15]);
    KQ_FENCE();
  }
}

__device__ __forceinline__ void mask_tail(v16f (&s)[2], int k0, const Geo& G) {
  const int nv = G.n - k0 - 32 * G.g;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * kb + i >= nv) s[kb][i] = -INFINITY;
}

// Matrix-core phase j of a wave (see the schedule in the kernel):
//   BMM1(j): sn = S^T of tile j (K(j) in Ks[j&1]), t = 2m + kb;
//   in the slots between those MFMAs the float32 448 p of tile j-1 (pv, written by the
//   previous VALU phase) become the E4M3 codes pop and per-block partial sums, added to lsum
//   with the block offsets d0p, d1p of tile j-1; slot t handles values 2t, 2t+1 (block t/8);
//   BMM2(j-1): O^T += V^T(j-1) · P(j-1)^T with the E8M0 block scale pscale (V^T(j-1) in
//   Vs[(j+1)&1]), with this thread's staging of K(j+1) into Ks[(j+1)&1] and V^T(j) into
//   Vs[j&1] (from kx/vx) and the block maxima of tile j (mx0, mx1 over keys 32g + 16kb ..,
//   both lanes of a row; keys past N masked to -inf first) in its slots, then the fetch of
//   K(j+2) and V^T(j+1).
// The wave runs this phase at raised priority: its few VALU instructions and the MFMA issues
// behind them then win the arbitration against the other wave of the SIMD, which is in its
// VALU phase, and the matrix pipe stays fed.
// With kFP4 (native MXFP4 BMM1), the 4 MFMAs of BMM1 take the packed E2M1 K rows and their
// E8M0 scales from LDS and the packed Q operand from registers; they issue in slots 0, 4, 8
// and 12 of the same 16-slot loop (the P codes of tile j-1 fill every slot).
// With kStats (R1's first pass) there is no P and no BMM2: only BMM1, the row sums and the
// block maxima, and V is never staged.
template <bool kFP4, bool kStats>
__device__ __forceinline__ void mfma_phase(int j, v16f (&sn)[2], const v16f (&pv)[2], v8i& pop,
                                           int pscale, float d0p, float d1p, v16f (&o)[4],
                                           float& lsum, uint4& kx, uint4& vx, float& mx0,
                                           float& mx1, const QOp<kFP4>& qop, uint8_t* Ks,
                                           uint8_t* Vs, const Geo& G) {
  __builtin_amdgcn_s_setprio(1);
  const int cur = j & 1;
  const uint8_t* vt = Vs + (cur ^ 1) * kVStage + G.vread;
  uint4 kv[16], vv[8];
  int ksa[4];
  if constexpr (kFP4) {
    // operand idx = 2h + kb: key block kb (LDS rows 32kb + r), d = 64h + 32g ..
    const uint8_t* kt = Ks + cur * kK4Stage + G.kread;
    const uint32_t* ksc = reinterpret_cast<const uint32_t*>(Ks + cur * kK4Stage + kK4Codes) + G.n4r;
#pragma unroll
    for (int idx = 0; idx < 4; ++idx)
      kv[idx] = *reinterpret_cast<const uint4*>(kt + (idx & 1) * 32 * kK4Pitch + 32 * (idx >> 1));
    const uint32_t s0 = ksc[0], s1 = ksc[32];
#pragma unroll
    for (int idx = 0; idx < 4; ++idx)
      ksa[idx] = (int)(((idx & 1) ? s1 : s0) >> (8 * (2 * (idx >> 1) + G.g))) & 0xFF;
  } else {
    const uint8_t* kt = Ks + cur * kKStage + G.kread;
#pragma unroll
    for (int t = 0; t < 4; ++t) kv[t] = kread(kt, t);
  }
  KQ_FENCE();
  float part0 = 0.0f, part1 = 0.0f, pair = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if constexpr (kFP4) {
      if ((t & 3) == 0) {
        const int idx = t >> 2, kb = idx & 1, h = idx >> 1;
        sn[kb] = mfma_fp4(kv[idx], qop.c[h], h == 0 ? v16f{} : sn[kb], ksa[idx], qop.s[h]);
      }
    } else {
      const int m = t >> 1, kb = t & 1;
      sn[kb] = mfma_bf16(as_bf16x8(kv[t]), qop.v[m], m == 0 ? v16f{} : sn[kb]);
      const uint8_t* kt = Ks + cur * kKStage + G.kread;
      if (t + 4 < 16) kv[t + 4] = kread(kt, t + 4);
    }
    if (!kStats && t >= 8) {
      const int c = (t - 8) >> 1, h = (t - 8) & 1;
      vv[t - 8] = *reinterpret_cast<const uint4*>(vt + c * 32 * kVPitch + 16 * h);
    }
    {
      const int blk = t >> 3, i = 2 * (t & 7), w = 4 * blk + (i >> 2);
      const float p0 = pv[blk][i], p1 = pv[blk][i + 1];
      // the native MXFP4 instance cannot bound |t| from its scales (they are data), and the
      // fused exp2 argument may then put 448 p past 464, where E4M3 conversion gives NaN:
      // its codes saturate at 448 instead
      const float e0 = kFP4 ? fminf(p0, 448.0f) : p0, e1 = kFP4 ? fminf(p1, 448.0f) : p1;
      if ((i & 2) == 0) {
        if (!kStats) pop[w] = e4m3_pair(e0, e1, pop[w], false);
        pair = p0 + p1;
      } else {
        if (!kStats) pop[w] = e4m3_pair(e0, e1, pop[w], true);
        const float q4 = pair + (p0 + p1);
        if (blk) part1 = (i == 2) ? q4 : part1 + q4;
        else part0 = (i == 2) ? q4 : part0 + q4;
      }
    }
    KQ_FENCE();
  }
  lsum += __builtin_amdgcn_ldexpf(part0, (int)d0p) + __builtin_amdgcn_ldexpf(part1, (int)d1p);
  // keep the conversions in the slots above (the compiler would otherwise sink them past the
  // masking branch, next to BMM2)
  asm volatile("" ::"v"(pop), "v"(lsum));
  {
    const int k0 = G.kbase + j * kBN;
    if (k0 + kBN > G.n) mask_tail(sn, k0, G);
  }
  KQ_FENCE();
  uint2 ka, kb2, kc, kd;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (!kStats) o[c] = mfma_f8_scaled(cat8(vv[2 * c], vv[2 * c + 1]), pop, o[c], pscale);
    // block maxima: elements 4c .. 4c + 3 of each block
    if (c == 0) {
      mx0 = fmaxf(fmaxf(sn[0][0], sn[0][1]), fmaxf(sn[0][2], sn[0][3]));
      mx1 = fmaxf(fmaxf(sn[1][0], sn[1][1]), fmaxf(sn[1][2], sn[1][3]));
    } else {
      mx0 = fmaxf(fmaxf(mx0, sn[0][4 * c]), fmaxf(sn[0][4 * c + 1], fmaxf(sn[0][4 * c + 2], sn[0][4 * c + 3])));
      mx1 = fmaxf(fmaxf(mx1, sn[1][4 * c]), fmaxf(sn[1][4 * c + 1], fmaxf(sn[1][4 * c + 2], sn[1][4 * c + 3])));
    }
    if (c == 3) {
      mx0 = max_with_partner(mx0);
      mx1 = max_with_partner(mx1);
    }
    if constexpr (kFP4) {
      if (c == 2) {
        stage_k<true>(Ks, cur ^ 1, G, kx);
        if (!kStats) stage_v(Vs, cur, G, vx);
      }
    } else {
      if (c == 0) {
        ka = e4m3x4_to_bf16(kx.x);
        kb2 = e4m3x4_to_bf16(kx.y);
      } else if (c == 1) {
        kc = e4m3x4_to_bf16(kx.z);
        kd = e4m3x4_to_bf16(kx.w);
      } else if (c == 2) {
        uint8_t* kb = Ks + (cur ^ 1) * kKStage + G.kw;
        *reinterpret_cast<uint4*>(kb) = make_uint4(ka.x, ka.y, kb2.x, kb2.y);
        *reinterpret_cast<uint4*>(kb + 16) = make_uint4(kc.x, kc.y, kd.x, kd.y);
        if (!kStats) stage_v(Vs, cur, G, vx);
      }
    }
    if (c == 3) {
      // past the end the loads return zeros and nothing reads the stages they fill
      kx = kload<kFP4>(G, j + 2);
      if (!kStats) vx = bload16(G.vrs, G.vo + (uint32_t)(j + 1) * kBN);
    }
    KQ_FENCE();
  }
  __builtin_amdgcn_s_setprio(0);
}

// VALU phase j of a wave: softmax of tile j on the scores s (in place: s becomes 448 p), from
// the block maxima mx0, mx1 the matrix-core phase left.
// BMM2's P operand is E4M3 with an E8M0 block scale per 32-key block: block kb holds the s[kb]
// values of both lanes of a row (bytes 0-15 / 16-31 of each lane's operand), and lane group g
// supplies the scale of block g.  Each block is quantized against its own integer offset
// M_kb = ceil(max t over the block) (so p <= 1 and 448 p fits E4M3) and carries
// 2^(M_kb - m_ref) as its scale: no accumulator rescale when the running maximum grows.
// Codes differ from full-row ones by exact powers of two, which E4M3 rounding preserves in its
// normal range.  Outputs the block offsets d0, d1 (relative to m_ref) and the scale byte.
//
// kMode 2 (second pass of the literal FakeQuantize of the normalized P): the row's offset M
// and sum l are known from the first pass, so every block uses M, the scale bytes stay 1.0 and
// the value quantized is p inv_p / l = exp2(t - M + log2(inv_p / l)), saturated at 448.
// kMode 1 (its first pass) also tracks the row's largest raw score.
template <int kMode, bool kWide>
__device__ __forceinline__ void valu_phase(int j, v16f (&s)[2], float mx0, float mx1,
                                           float& m_ref, float& m_top, float& lsum,
                                           v16f (&o)[4], int& pscale, float& d0o, float& d1o,
                                           float& rmax, const Geo& G) {
  const float c1 = G.c1;
  if constexpr (kMode == 2) {
    m_ref = m_top = G.m_fix;
    pscale = 127;
    d0o = d1o = 0.0f;
    const float bias = G.lb_fix - G.m_fix, m_fix = G.m_fix, lb_fix = G.lb_fix;
    exp2_pipeline(s, [&](int, float x) {
      return kWide ? unfused_arg(x, c1, m_fix, lb_fix) : __builtin_fmaf(x, c1, bias);
    });
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = fminf(s[kb][i], 448.0f);
    asm volatile("" ::"v"(s[0]), "v"(s[1]));
    return;
  }
  if constexpr (kMode == 1) rmax = fmaxf(rmax, fmaxf(mx0, mx1));   // the row's largest raw score
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
  pscale = 127 + (int)(G.g ? d1 : d0);
  d0o = d0;
  d1o = d1;
  const float bias0 = kLog2_448 - mb0, bias1 = kLog2_448 - mb1;
  exp2_pipeline(s, [&](int kb, float x) {
    return kWide ? unfused_arg(x, c1, kb ? mb1 : mb0, kLog2_448)
                 : __builtin_fmaf(x, c1, kb ? bias1 : bias0);
  });
  // the values are consumed by the next matrix-core phase; keep them computed here
  asm volatile("" ::"v"(s[0]), "v"(s[1]));
}

// kMode: 0 the one-pass attention; 1 the same plus the (M, l, max p) row statistics of R1's
// first pass; 2 R1's second pass.
template <bool kFP4, int kMode, bool kWide>
__global__ void __launch_bounds__(kThreads, 1) attn_fp8_kernel(AttnParams a, int nqb) {
  constexpr bool kR1 = kMode == 2;
  // bf16 K tiles, or packed E2M1 K tiles + scales (kFP4)
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2 * (kFP4 ? kK4Stage : kKStage)];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[2 * kVStage];   // FP8 V^T tiles

  // Work assignment (see xcd_split): slots below a.nfull are whole query blocks, the slots
  // after them (dispatched last) key ranges of the remaining blocks.
  // (integer divisions run on the vector unit; readfirstlane returns the uniform results to
  // scalar registers so the buffer descriptors below stay scalar)
  const int N = a.n;
  const int ntiles_all = (N + kBN - 1) / kBN;
  const int bid = blockIdx.x;
  int logical, part = -1, t_begin = 0, t_end = ntiles_all;
  const XcdSplit xs = xcd_split(a, bid & 7);
  if (bid < a.nfull) {
    logical = xs.logical0 + (bid >> 3);
  } else {
    part = __builtin_amdgcn_readfirstlane(xs.first_part + (bid >> 3) - xs.whole);
    const int blk = __builtin_amdgcn_readfirstlane(part / a.split);
    const int chunk = part - blk * a.split;
    logical = split_block_logical(a, blk);
    t_begin = __builtin_amdgcn_readfirstlane(chunk * ntiles_all / a.split);
    t_end = __builtin_amdgcn_readfirstlane((chunk + 1) * ntiles_all / a.split);
  }
  const int bh = __builtin_amdgcn_readfirstlane(logical / nqb);
  const int qb = logical - bh * nqb;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 31, g = l >> 5;
  const int q = qb * kBM + w * 32 + r;

  // Q operand (bf16 values of the E4M3 codes): step m covers d = 16m .. 16m + 15; lane (r, g)
  // supplies query q, d = 16m + 8g .. +7.  Rows past N read as zeros.
  // MXFP4: lane (r, g) holds query q's packed d = 64h + 32g .. +31 and the scale of that block.
  QOp<kFP4> qop;
  if constexpr (kFP4) {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + (int64_t)bh * N * (kD / 2), (uint32_t)N * (kD / 2));
    const __amdgpu_buffer_rsrc_t qsr = make_rsrc(a.q_scales + (int64_t)bh * N * 4, (uint32_t)N * 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) qop.c[h] = bload16(qr, (uint32_t)q * (kD / 2) + 32 * h + 16 * g);
    const uint32_t sd = __builtin_amdgcn_raw_buffer_load_b32(qsr, (uint32_t)q * 4, 0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) qop.s[h] = (int)(sd >> (8 * (2 * h + g))) & 0xFF;
  } else if (a.q_bf16 != nullptr) {
    // Q given in bf16: its FP8 codes are formed here, as the FP8 tensor quantizer forms them
    // (each Q element is read by exactly one lane of one workgroup), then widened like the codes
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q_bf16 + (int64_t)bh * N * kD, (uint32_t)N * kD * 2);
    const uint32_t qo = ((uint32_t)q * kD + 8 * g) * 2;
    const float inv = a.q_inv;
    auto lo16 = [](uint32_t w) { return __uint_as_float(w << 16); };
    auto hi16 = [](uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); };
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint4 x = bload16_stream(qr, qo + 32 * m);
      const uint32_t c0 = e4m3x4_q(lo16(x.x), hi16(x.x), lo16(x.y), hi16(x.y), inv);
      const uint32_t c1 = e4m3x4_q(lo16(x.z), hi16(x.z), lo16(x.w), hi16(x.w), inv);
      const uint2 lo = e4m3x4_to_bf16(c0), hi = e4m3x4_to_bf16(c1);
      qop.v[m] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  } else {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + (int64_t)bh * N * kD, (uint32_t)N * kD);
    const uint32_t qo = (uint32_t)q * kD + 8 * g;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint2 c = bload8_stream(qr, qo + 16 * m);
      const uint2 lo = e4m3x4_to_bf16(c.x), hi = e4m3x4_to_bf16(c.y);
      qop.v[m] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  }

  // Tile staging: a K tile is 512 FP8 chunks of 16 bytes (64 keys x 8) and a V^T tile 512
  // chunks (128 d-rows x 4); each thread owns chunk `tid` of both.
  // MXFP4: a K tile is 256 chunks of 16 bytes (64 keys x 4), staged by waves 0-3, plus 64
  // scale dwords, staged by wave 4.
  Geo G;
  {
    const int vd = tid >> 2, vc = tid & 3;                 // d row, 16-byte column
    if constexpr (kFP4) {
      const int kr = (tid >> 2) & 63, kc = tid & 3;        // key row, 16-byte column (waves 0-3)
      G.krole = __builtin_amdgcn_readfirstlane(tid < 256 ? 0 : (tid < 320 ? 1 : 2));
      G.krs = make_rsrc(a.k + (int64_t)bh * N * (kD / 2), (uint32_t)N * (kD / 2));
      G.ksr = make_rsrc(a.k_scales + (int64_t)bh * N * 4, (uint32_t)N * 4);
      if (G.krole == 1) {
        const int ks = tid - 256;                          // key of this scale dword
        G.kw = kK4Codes + krow_of_key(ks) * 4;
        G.ko = (uint32_t)t_begin * kBN * 4 + ks * 4;
      } else {
        G.kw = krow_of_key(kr) * kK4Pitch + 16 * kc;
        G.ko = (uint32_t)t_begin * kBN * (kD / 2) + kr * (kD / 2) + kc * 16;
      }
      G.kread = r * kK4Pitch + 16 * g;
      G.n4r = r;
    } else {
      const int kr = tid >> 3, kc = tid & 7;               // key row, 16-byte column
      G.krole = 0;
      G.kw = krow_of_key(kr) * kKPitch + 32 * kc;
      G.krs = make_rsrc(a.k + (int64_t)bh * N * kD, (uint32_t)N * kD);
      G.ksr = G.krs;
      G.ko = (uint32_t)t_begin * kBN * kD + kr * kD + kc * 16;
      G.kread = r * kKPitch + 16 * g;
      G.n4r = 0;
    }
    G.vw = vd * kVPitch + 16 * vc;
    G.vrs = make_rsrc(a.vt + (int64_t)bh * kD * a.ldv, (uint32_t)(kD * a.ldv));
    G.vo = (uint32_t)(vd * a.ldv + vc * 16 + t_begin * kBN);
    G.vread = r * kVPitch + 32 * g;
    G.n = N;
    G.g = g;
    G.kbase = __builtin_amdgcn_readfirstlane(t_begin * kBN);
    G.c1 = a.c1;
    G.m_fix = 0.0f;
    G.lb_fix = 0.0f;
    if constexpr (kR1) {
      // (M, l) of this row from the first pass; rows past N keep M = 0, l = 1
      const __amdgpu_buffer_rsrc_t sr =
          make_rsrc(a.r1_stats + (int64_t)bh * N * 4, (uint32_t)N * 16);
      const u32x4 st = __builtin_amdgcn_raw_buffer_load_b128(sr, (uint32_t)q * 16, 0, 0);
      const float m = __uint_as_float(st[0]), l = __uint_as_float(st[1]);
      const bool ok = l > 0.0f;
      G.m_fix = ok ? m : 0.0f;
      G.lb_fix = log2f(a.r1_inv_p / (ok ? l : 1.0f));
    }
  }

  v16f o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = 0.0f;
  v16f sA[2], sB[2];                            // scores / 448 p of two consecutive tiles
#pragma unroll
  for (int i = 0; i < 16; ++i) sB[0][i] = sB[1][i] = 0.0f;   // "tile -1": p = 0
  v8i pop = {0, 0, 0, 0, 0, 0, 0, 0};
  int pscale = 127;          // E8M0 scale of this lane group's P block (see valu_phase)
  float d0 = 0.0f, d1 = 0.0f;  // block offsets of the last softmaxed tile, relative to m_ref
  float m_ref = 0.0f;        // per-row reference offset (integer-valued), set on tile 0
  float m_top = -INFINITY;   // largest block offset seen (for the row statistics)
  float rmax = -INFINITY;    // largest raw score of the row (first pass of R1)
  float lsum = 0.0f;         // partial row sum of 448 p * 2^(M_kb - m_ref) over this lane's keys
  const int ntiles = __builtin_amdgcn_readfirstlane(t_end - t_begin);   // tiles of this range
  const int grp = __builtin_amdgcn_readfirstlane(w >> 2);    // 0: waves 0-3, 1: waves 4-7 (one per SIMD each)

  // Ping-pong schedule.  Every wave alternates a matrix-core phase (mfma_phase: BMM1 of tile j,
  // the P codes and row sums of tile j-1, BMM2 of tile j-1, staging) and a VALU phase
  // (valu_phase: softmax of tile j).  Group 1 runs half a period behind group 0, so on every
  // SIMD one wave is in its matrix-core phase while the other is in its VALU phase; workgroup
  // barriers separate the phases.  Phase 2j: group 0 MFMA(j), group 1 VALU(j-1); phase 2j+1:
  // group 0 VALU(j), group 1 MFMA(j).  K(j) and V(j-1) are read in phases 2j and 2j+1; K(j+1)
  // and V(j) are written to the other buffers in the same two phases (half by each group) and
  // are complete before phase 2j+2.  Both groups pass 2 * ntiles + 4 barriers.
  uint4 kx = kload<kFP4>(G, 0), vx;              // K(0)
  stage_k<kFP4>(Ks, 0, G, kx);
  *reinterpret_cast<uint4*>(Vs + kVStage + G.vw) = make_uint4(0, 0, 0, 0);   // "V(-1)" = 0
  kx = kload<kFP4>(G, 1);                          // K(1): this thread's chunk
  vx = bload16(G.vrs, G.vo);                       // V(0)
  __syncthreads();
  if (grp == 1) __syncthreads();
  float mx0, mx1;            // block maxima of the tile just multiplied
  for (int j = 0;; j += 2) {
    mfma_phase<kFP4, kMode == 1>(j, sA, sB, pop, pscale, d0, d1, o, lsum, kx, vx, mx0, mx1, qop, Ks, Vs, G);
    __syncthreads();
    if (j < ntiles) valu_phase<kMode, kWide>(j, sA, mx0, mx1, m_ref, m_top, lsum, o, pscale, d0, d1, rmax, G);
    __syncthreads();
    if (j + 1 > ntiles) break;
    mfma_phase<kFP4, kMode == 1>(j + 1, sB, sA, pop, pscale, d0, d1, o, lsum, kx, vx, mx0, mx1, qop, Ks, Vs, G);
    __syncthreads();
    if (j + 1 < ntiles) valu_phase<kMode, kWide>(j + 1, sB, mx0, mx1, m_ref, m_top, lsum, o, pscale, d0, d1, rmax, G);
    __syncthreads();
    if (j + 2 > ntiles) break;
  }
  if (grp == 0) __syncthreads();

  // ---- epilogue: O = acc * s_v / sum(448 p); lane (r, g) holds d = 32c + 8(i/4) + 4g + i%4
  const float ltot = lsum + __shfl_xor(lsum, 32);      // sum of 448 p relative to m_ref
  const float m_row = fmaxf(m_top, __shfl_xor(m_top, 32));   // the row's M = ceil(max t)
  // A wave's 32 x 128 float tile (o times `scale`) leaves through LDS, so that every store
  // instruction writes whole 128-byte rows of a 32-column chunk, with the non-temporal hint:
  // without it the 4 MB of O a round of blocks writes per XCD pushes the next round's K and V
  // out of the XCD's L2 (the split ranges' partials as well: the merge kernel then reads them
  // from HBM, which costs it less than the K and V fetched again cost here).  Row rr of the
  // tile goes to
  // dst + rr * kD (rows >= rows are skipped).  Each wave uses its own 4 KB of the K stages
  // (callers pass a barrier first, after which no wave reads them): row rr of a chunk at
  // rr * 128 bytes, 16-byte column j at (j ^ (rr & 7)).  The MXFP4 instance's K stages hold
  // less than 32 KB; it stores directly.
  constexpr bool kDirect = kFP4 || 2 * kKStage < kThreads / 64 * 4096;
  auto store_tile = [&](float scale, float* dst, int rows) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    if constexpr (kDirect) {
      if (r < rows) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f4v v = {o[c][4 * i4] * scale, o[c][4 * i4 + 1] * scale,
                           o[c][4 * i4 + 2] * scale, o[c][4 * i4 + 3] * scale};
            *reinterpret_cast<f4v*>(dst + (int64_t)r * kD + 32 * c + 8 * i4 + 4 * g) = v;
          }
      }
    } else {
      float* ws = reinterpret_cast<float*>(Ks + w * 4096);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int j = 2 * i4 + g;
          const f4v v = {o[c][4 * i4] * scale, o[c][4 * i4 + 1] * scale,
                         o[c][4 * i4 + 2] * scale, o[c][4 * i4 + 3] * scale};
          *reinterpret_cast<f4v*>(ws + r * 32 + 4 * (j ^ (r & 7))) = v;
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int rr = 8 * h + (l >> 3), j = l & 7;
          const f4v v = *reinterpret_cast<const f4v*>(ws + rr * 32 + 4 * (j ^ (rr & 7)));
          if (rr < rows)
            __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(dst + (int64_t)rr * kD + 32 * c + 4 * j));
        }
      }
    }
  };
  if (part >= 0) {
    // partial result of a key range: the unnormalized accumulator and (m_ref, l, M, max raw
    // score); R1's first pass has no accumulator
    const int row = w * 32 + r;
    if (kMode != 1) {
      __syncthreads();
      store_tile(1.0f, a.ws + ((int64_t)part * kBM + w * 32) * kD, 32);
    }
    if (g == 0) {
      float* ws = a.ws + (int64_t)a.rem * a.split * kBM * kD + ((int64_t)part * kBM + row) * 4;
      *reinterpret_cast<float4*>(ws) = make_float4(m_ref, ltot, m_row, rmax);
    }
    return;
  }
  // R1 second pass: P was normalized before quantization, O = acc s_P s_V
  const float scale = kR1 ? a.r1_s_p * a.s_v : a.s_v / ltot;
  if (kMode != 1 && a.o != nullptr) {
    __syncthreads();
    const int row0 = qb * kBM + w * 32;
    store_tile(scale, a.o + ((int64_t)bh * N + row0) * kD, N - row0);
  }
  if (!kR1 && q < N && g == 0) {
    // (M, l) with l relative to the row's M
    const float lrel = __builtin_amdgcn_ldexpf(ltot * (1.0f / 448.0f), (int)(m_ref - m_row));
    if (a.stats != nullptr)
      *reinterpret_cast<float2*>(a.stats + ((int64_t)bh * N + q) * 2) = make_float2(m_row, lrel);
    if (kMode == 1) {
      // first pass of R1: also the row's largest p = exp2(max t - M), its argument formed as
      // the loop formed those of its p values (fused, or unfused in the kWide instance)
      const float pmax = exp2f(kWide ? unfused_arg(rmax, a.c1, m_row, 0.0f)
                                     : __builtin_fmaf(rmax, a.c1, -m_row));
      *reinterpret_cast<float4*>(a.stats4 + ((int64_t)bh * N + q) * 4) =
          make_float4(m_row, lrel, pmax, 0.0f);
    }
  }
}

// Merge of the key-range partials of one query block: with R = max m_ref over the parts,
// acc = sum acc_s 2^(m_ref_s - R) and l = sum l_s 2^(m_ref_s - R) (exact power-of-two scaling),
// then O = acc * s_v / l as in the single-pass epilogue.  One thread per (row, 4 columns).
// R1: the second pass's parts share the row's M, and O = acc s_P s_v; the first pass has no
// accumulator and writes the (M, l, max p) statistics.
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnParams a, int nqb) {
  // a workgroup covers 8 rows of one query block (32 threads per row, kBM rows per block), so
  // the block and its logical index are uniform: scalar arithmetic
  static_assert(kBM % 8 == 0, "a combine workgroup must stay inside one query block");
  const int blk = (int)blockIdx.x / (kBM / 8);
  const int row = ((int)blockIdx.x - blk * (kBM / 8)) * 8 + (int)(threadIdx.x >> 5);
  const int d4 = 4 * (threadIdx.x & 31);
  if (blk >= a.rem) return;
  const int logical = split_block_logical(a, blk);
  const int bh = logical / nqb, qb = logical - bh * nqb;
  const int q = qb * kBM + row;
  if (q >= a.n) return;
  const float4* st = reinterpret_cast<const float4*>(a.ws + (int64_t)a.rem * a.split * kBM * kD) +
                     (int64_t)blk * a.split * kBM + row;
  // the partials of up to kBatch ranges are loaded together, the first batch with the
  // statistics, so a typical split (<= kBatch ranges) costs one round trip to memory; the sums
  // still run over the ranges in order
  constexpr int kBatch = 8;
  const bool want_o = a.o != nullptr;
  const float* pb = a.ws + ((int64_t)blk * a.split * kBM + row) * kD + d4;
  const int64_t pstride = (int64_t)kBM * kD;
  float4 x[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u)
    x[u] = (want_o && u < a.split) ? *reinterpret_cast<const float4*>(pb + u * pstride)
                                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float R = -INFINITY, m_row = -INFINITY, rmax = -INFINITY;
  for (int s = 0; s < a.split; ++s) {
    const float4 v = st[(int64_t)s * kBM];
    R = fmaxf(R, v.x);
    m_row = fmaxf(m_row, v.z);
    rmax = fmaxf(rmax, v.w);
  }
  float l = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < a.split; s0 += kBatch) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (want_o && s0 + u < a.split)
          x[u] = *reinterpret_cast<const float4*>(pb + (s0 + u) * pstride);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u < a.split) {
        const float4 v = st[(int64_t)(s0 + u) * kBM];
        const float f = __builtin_amdgcn_ldexpf(1.0f, (int)(v.x - R));
        l += v.y * f;
        acc.x += x[u].x * f;
        acc.y += x[u].y * f;
        acc.z += x[u].z * f;
        acc.w += x[u].w * f;
      }
    }
  }
  if (a.o != nullptr) {
    const float scale = a.r1_stats != nullptr ? a.r1_s_p * a.s_v : a.s_v / l;
    float* op = a.o + ((int64_t)bh * a.n + q) * kD + d4;
    *reinterpret_cast<float4*>(op) = make_float4(acc.x * scale, acc.y * scale, acc.z * scale, acc.w * scale);
  }
  if (d4 != 0 || a.r1_stats != nullptr) return;
  const float lrel = __builtin_amdgcn_ldexpf(l * (1.0f / 448.0f), (int)(R - m_row));
  if (a.stats != nullptr)
    *reinterpret_cast<float2*>(a.stats + ((int64_t)bh * a.n + q) * 2) = make_float2(m_row, lrel);
  if (a.stats4 != nullptr) {
    // the largest p, its exp2 argument formed as the first pass formed those of its p values
    const float pmax = exp2f(a.wide_scores ? unfused_arg(rmax, a.c1, m_row, 0.0f)
                                           : __builtin_fmaf(rmax, a.c1, -m_row));
    *reinterpret_cast<float4*>(a.stats4 + ((int64_t)bh * a.n + q) * 4) =
        make_float4(m_row, lrel, pmax, 0.0f);
  }
}

// amax_P of R1 from first-pass row statistics: amax[0] = max(amax[0], max over rows of
// fl32(pmax / l)), the largest normalized probability.  Grid-stride over the rows, a
// workgroup reduction, then one unsigned atomic max on the float bits per workgroup (every
// value is >= 0, where the unsigned order of the bits is the order of the values).
__global__ void __launch_bounds__(256) r1_amax_kernel(const float* st, int64_t rows, float* amax) {
  __shared__ float red[256];
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows; i += stride) {
    const float4 v = reinterpret_cast<const float4*>(st)[i];
    if (v.y > 0.0f) m = fmaxf(m, v.z / v.y);
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(red[0]));
}

}  // namespace

hipError_t launch_r1_amax(const float* row_stats4, int64_t rows, float* amax, hipStream_t stream) {
  // about four rows per thread, at most 512 workgroups (atomics on the one result word)
  const int64_t g = (rows + 1023) / 1024;
  const unsigned grid = (unsigned)(g < 1 ? 1 : (g > 512 ? 512 : g));
  hipLaunchKernelGGL(r1_amax_kernel, dim3(grid), dim3(256), 0, stream, row_stats4, rows, amax);
  return hipGetLastError();
}

hipError_t attn_static_workspace(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kAttnStaticWorkspaceBytes;
  return hipSuccess;
}

hipError_t launch_attn_fp8(const AttnParams& p, hipStream_t stream) {
  const int nqb = (p.n + kBM - 1) / kBM;
  const int64_t blocks = (int64_t)p.nfull + (int64_t)p.rem * p.split;
  const dim3 g((unsigned)blocks), t(kThreads);
  if (p.q_scales != nullptr)
    hipLaunchKernelGGL((attn_fp8_kernel<true, 0, false>), g, t, 0, stream, p, nqb);
  else if (p.r1_stats != nullptr && p.wide_scores)
    hipLaunchKernelGGL((attn_fp8_kernel<false, 2, true>), g, t, 0, stream, p, nqb);
  else if (p.r1_stats != nullptr)
    hipLaunchKernelGGL((attn_fp8_kernel<false, 2, false>), g, t, 0, stream, p, nqb);
  else if (p.stats4 != nullptr && p.wide_scores)
    hipLaunchKernelGGL((attn_fp8_kernel<false, 1, true>), g, t, 0, stream, p, nqb);
  else if (p.stats4 != nullptr)
    hipLaunchKernelGGL((attn_fp8_kernel<false, 1, false>), g, t, 0, stream, p, nqb);
  else if (p.wide_scores)
    hipLaunchKernelGGL((attn_fp8_kernel<false, 0, true>), g, t, 0, stream, p, nqb);
  else
    hipLaunchKernelGGL((attn_fp8_kernel<false, 0, false>), g, t, 0, stream, p, nqb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.split == 0) return e;
  const int64_t cblocks = ((int64_t)p.rem * kBM * 32 + 255) / 256;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)cblocks), dim3(256), 0, stream, p, nqb);
  return hipGetLastError();
}

}  // namespace kq
