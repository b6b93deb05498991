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
// MFMA (the scaled form for MXFP4, the unscaled one for FP8; 128 accumulator registers).  The
// product is computed transposed, D = B_sub · A_sub^T, so each lane owns one row m of C.  A
// k-step moves 64 bytes of each operand row (64 FP8 or 128 FP4 elements) through LDS: 64-byte
// rows with the 16-byte chunks swizzled (conflict-free operand reads), three stages, each
// step's tile loaded from HBM straight into its stage (buffer_load ... lds) two steps before it
// is multiplied; MXFP4 scales go through a two-slot LDS ring,
// fetched 16 bytes (four k-steps) per row at a time and read once per two steps, the MFMA's
// scale select picking each step's byte.  Ping-pong: the two waves of a SIMD run half a
// step apart, one issuing its step's eight (FP8) or sixteen (FP4) MFMAs while the other
// stages, fetches and reads its six operand sub-tiles, with a workgroup barrier between the
// halves.  C leaves through LDS in whole 256-byte row pieces with the non-temporal hint.
//
// SVD-Quant in FP4 (the same section names it beside PTQ in FP8 and FP4): the weights are
// split offline into bf16 rank-r factors and a residual in MXFP4; per forward,
// lowrank_down_kernel forms T = bf16(A L_down^T) [M][r], and the MXFP4 GEMM of A and the
// residual starts its accumulators from T L_up^T (v_mfma_f32_32x32x16_bf16, whose 32 x 32
// result layout is the f8f6f4 form's), so C = dq(A) dq(R)^T + T L_up^T in one pass.
//
// Operand layouts of the f8f6f4 MFMA (measured): for E4M3, lane (r, g) holds row r with
// k = 16g .. 16g+15 in bytes 0-15 and k = 32+16g .. in bytes 16-31; for E2M1, lane (r, g)
// holds k = 32g .. 32g+31 in 32 nibbles (low first) and supplies the scale of that 32-block.

#include "kq_launch.h"
#include "kq_fp4.h"

namespace kq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kTile = 256;            // workgroup tile of C (M and N)
constexpr int kThreads = 512;         // 8 waves, two per SIMD
constexpr int kRowBytes = 64;         // bytes of one operand row per k-step
// LDS stage rows: chunk c (16 bytes) of row R at 16 * (c ^ ((R >> 2) & 3)).  An operand read
// covers 16 consecutive rows x one chunk per 16-lane group; with the swizzle it touches 16
// distinct 16-byte bank groups.  A wave's share of a stage (16 rows, 1 KB) is contiguous, the
// block a 16-byte LDS-direct load fills (lane l at 16 l).
constexpr int kPitch = kRowBytes;
constexpr int kOpStage = kTile * kPitch;            // 16384 bytes per operand
constexpr int kStage = 2 * kOpStage;                // A, B codes
constexpr int kStages = 3;
// FP4 scales: a ring of two slots, each holding 4 k-steps of the 512 operand rows' E8M0 bytes.
// Dword j = 2p + g of a row holds blocks g and 2 + g of k-step 2p (bytes 0, 1) and of k-step
// 2p + 1 (bytes 2, 3) of the slot's four steps: what lane group g of a 32-row sub-tile needs for
// the step pair p.  A slot stores the dwords of one j contiguously per lane: A row
// m = 64 wm + 32 i + r at ((j * 128 + 32 wm + r) * 2 + i) * 4 (a lane's two A rows in 8 bytes),
// B row n = 128 wn + 32 i + r at 4096 + ((j * 64 + 32 wn + r) * 4 + i) * 4 (its four B rows in
// 16 bytes), so the reads of a step pair are one 8- and one 16-byte read per lane, and a wave's
// reads fall on consecutive addresses (no bank conflicts).
constexpr int kRingSlot = 2 * kTile * 16;
constexpr int kRing = 2 * kRingSlot;
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

// 16 bytes per lane from buffer r at off into LDS at lds_wave + 16 * lane (lds_wave uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave, 16, off,
                                           0, 0, 0);
}

// A wave holds 8 tiles of 32 x 32 (128 accumulator registers) and two waves share each SIMD.
// FP8 takes the unscaled form (zero scale operands select v_mfma_f32_32x32x64_f8f6f4).
__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i cat8(uint4 lo, uint4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// A wave's operands of one k-step, read from LDS in its memory part and consumed by its MFMAs.
template <bool kFP4>
struct KOps {
  uint4 n[4][2], m[2][2];
  uint32_t sn[4], sm[2];
};

// Operand reads of one k-step of a wave's 128 (n) x 64 (m) tile: 4 sub-tiles of B rows (the
// MFMA's A side) and 2 of A rows (its B side), each 32 bytes per lane, from the LDS stage st =
// [A rows][B rows] codes.  FP8: lane (r, g) takes bytes 16g and 32 + 16g of its row
// (k = 16g.., 32+16g..); FP4: k-chunk h = 0, 1 at bytes 32h + 16g (k = 64h + 32g ..).  FP4 with
// kSc (the first step of a pair) also reads the lane's scale dwords of the pair from the ring
// slot sc; the second step keeps them.  The empty asm uses every result, so the reads have
// landed when it returns.
template <bool kFP4, bool kSc>
__device__ __forceinline__ void kread(KOps<kFP4>& o, const uint8_t* st, const uint8_t* sc,
                                      int rbase_n, int rbase_m, int rbase_n2, int rbase_m2,
                                      int sbase_n, int sbase_m) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o.m[i][0] = *reinterpret_cast<const uint4*>(st + rbase_m + i * 32 * kPitch);
    o.m[i][1] = *reinterpret_cast<const uint4*>(st + rbase_m2 + i * 32 * kPitch);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.n[i][0] = *reinterpret_cast<const uint4*>(st + kOpStage + rbase_n + i * 32 * kPitch);
    o.n[i][1] = *reinterpret_cast<const uint4*>(st + kOpStage + rbase_n2 + i * 32 * kPitch);
  }
  if (kFP4 && kSc) {
    const uint2 mv = *reinterpret_cast<const uint2*>(sc + sbase_m);
    const uint4 nv = *reinterpret_cast<const uint4*>(sc + sbase_n);
    o.sm[0] = mv.x; o.sm[1] = mv.y;
    o.sn[0] = nv.x; o.sn[1] = nv.y; o.sn[2] = nv.z; o.sn[3] = nv.w;
  }
#define KQ_V4(X_) (u32x4{(X_).x, (X_).y, (X_).z, (X_).w})
  asm volatile("" ::"v"(KQ_V4(o.n[0][0])), "v"(KQ_V4(o.n[0][1])), "v"(KQ_V4(o.n[1][0])),
               "v"(KQ_V4(o.n[1][1])), "v"(KQ_V4(o.n[2][0])), "v"(KQ_V4(o.n[2][1])),
               "v"(KQ_V4(o.n[3][0])), "v"(KQ_V4(o.n[3][1])), "v"(KQ_V4(o.m[0][0])),
               "v"(KQ_V4(o.m[0][1])), "v"(KQ_V4(o.m[1][0])), "v"(KQ_V4(o.m[1][1])));
  if (kFP4 && kSc) asm volatile("" ::"v"(o.sn[0]), "v"(o.sn[1]), "v"(o.sn[2]), "v"(o.sn[3]), "v"(o.sm[0]), "v"(o.sm[1]));
#undef KQ_V4
}

// E8M0 bytes of four k-steps of a row (dword c = step c, byte i = block i) in the ring's order:
// dword 2p + g = blocks g and 2 + g of step 2p, then of step 2p + 1.
__device__ __forceinline__ uint4 ring_order(uint4 x) {
  auto pick = [](uint32_t a, uint32_t b, int g) -> uint32_t {
    return ((a >> (8 * g)) & 0xFFu) | (((a >> (8 * g + 16)) & 0xFFu) << 8) |
           (((b >> (8 * g)) & 0xFFu) << 16) | (((b >> (8 * g + 16)) & 0xFFu) << 24);
  };
  return make_uint4(pick(x.x, x.y, 0), pick(x.x, x.y, 1), pick(x.z, x.w, 0), pick(x.z, x.w, 1));
}

// A row's four ring dwords (j = 0..3) at p + 1024 j.
__device__ __forceinline__ void ring_put(uint8_t* p, uint4 v) {
  *reinterpret_cast<uint32_t*>(p) = v.x;
  *reinterpret_cast<uint32_t*>(p + 1024) = v.y;
  *reinterpret_cast<uint32_t*>(p + 2048) = v.z;
  *reinterpret_cast<uint32_t*>(p + 3072) = v.w;
}

// FP4 MFMAs of k-chunk h: the scale select kSel picks byte kSel of each scale dword (the block
// of chunk h of this step; see the ring layout), so no instruction extracts it.
template <int kSel>
__device__ __forceinline__ void kmma_fp4_chunk(v16f (&acc)[4][2], const KOps<true>& o, int h) {
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          cat8(o.n[ni][h], z), cat8(o.m[mi][h], z), acc[ni][mi], 4, 4, kSel, (int)o.sn[ni], kSel,
          (int)o.sm[mi]);
}

// The MFMAs of one k-step on operands kread left in registers; kPar is the step's parity.
template <bool kFP4, int kPar>
__device__ __forceinline__ void kmma(v16f (&acc)[4][2], const KOps<kFP4>& o) {
  if constexpr (kFP4) {
    kmma_fp4_chunk<2 * kPar>(acc, o, 0);
    kmma_fp4_chunk<2 * kPar + 1>(acc, o, 1);
  } else {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        acc[ni][mi] = mfma_fp8(cat8(o.n[ni][0], o.n[ni][1]), cat8(o.m[mi][0], o.m[mi][1]), acc[ni][mi]);
  }
}

// Two float32 values -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32) in one dword.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <bool kFP4, bool kBf16, bool kLowRank>
__global__ void __launch_bounds__(kThreads, 1) gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage + (kFP4 ? kRing : 0)];
  uint8_t* const ring = lds + kStages * kStage;
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

  // staging: each operand tile is 256 rows x 4 chunks of 16 bytes, loaded straight into LDS;
  // thread t fills LDS slots t and t + 512 of both (rows t/4 and t/4 + 128, slot t % 4), i.e.
  // it loads the chunk the swizzle puts there, so 4 consecutive lanes still read one row's 64
  // contiguous bytes, and wave w fills the 1 KB blocks of rows 16w .. 16w + 15 (and + 128).
  // FP4 scales: thread t owns the E8M0
  // bytes of operand row t (A rows 0-255, then B rows), fetched 16 bytes (4 k-steps) at a
  // time four steps ahead and written to the ring slot of their block; one dword per row per
  // step would touch a 128-byte line for 4 useful bytes, every step.
  const int crow = tid >> 2, gchunk = (tid & 3) ^ ((crow >> 2) & 3);
  const uint32_t goff_a = (uint32_t)(mt * kTile + crow) * row_bytes + 16 * gchunk;
  const uint32_t goff_b = (uint32_t)(nt * kTile + crow) * row_bytes + 16 * gchunk;
  const uint32_t row128 = 128u * row_bytes;
  const int wlds = __builtin_amdgcn_readfirstlane(w) * 16 * kPitch;    // the wave's 1 KB of a stage
  const bool sc_a = __builtin_amdgcn_readfirstlane(tid) < 256;
  const __amdgpu_buffer_rsrc_t scr =
      make_rsrc(sc_a ? p.a_scales : p.b_scales, (uint32_t)(sc_a ? p.m : p.n) * sc_bytes);
  const uint32_t soff = (uint32_t)((sc_a ? mt : nt) * kTile + (tid & 255)) * sc_bytes;
  // the 16 bytes of scale block c (k-steps 4c .. 4c+3) of this thread's row; rows whose scale
  // bytes are not a multiple of 16 take four dword loads
  const bool sc_al = (sc_bytes & 15) == 0;
  auto sload = [&](int c) -> uint4 {
    const uint32_t o_ = soff + 16u * (uint32_t)c;
    if (sc_al) return bload16(scr, o_);
    return make_uint4(bload4(scr, o_), bload4(scr, o_ + 4), bload4(scr, o_ + 8), bload4(scr, o_ + 12));
  };

  // step s's tile of both operands into LDS stage `stage`
#define KQ_DMA(s, stage)                                                          \
  {                                                                               \
    uint8_t* st_ = lds + (stage) * kStage + wlds;                                 \
    const uint32_t o_ = (uint32_t)(s) * kRowBytes;                                \
    dma16(ar, st_, goff_a + o_);                                                  \
    dma16(ar, st_ + 128 * kPitch, goff_a + row128 + o_);                          \
    dma16(br, st_ + kOpStage, goff_b + o_);                                       \
    dma16(br, st_ + kOpStage + 128 * kPitch, goff_b + row128 + o_);               \
  }
  // a loop barrier without a memory fence: the LDS operations drained, not the loads into LDS
  // (a fence would wait for those too; their visibility comes from each wave's vmcnt(0) at the
  // start of its next memory half, before the next barrier)
#define KQ_BAR() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

  // operand reads of lane (r, g): chunks g and g + 2 of its rows (sub-tile rows are 32 apart,
  // so every row of the lane has the swizzle of r)
  const int cx = g ^ ((r >> 2) & 3);
  const int rbase_n = (wn * 128 + r) * kPitch + 16 * cx, rbase_n2 = (wn * 128 + r) * kPitch + 16 * (cx ^ 2);
  const int rbase_m = (wm * 64 + r) * kPitch + 16 * cx, rbase_m2 = (wm * 64 + r) * kPitch + 16 * (cx ^ 2);
  // ring reads of lane (r, g) (j = 2p + g for step pair p) and this thread's ring row
  const int sbase_n = 4096 + (g * 64 + wn * 32 + r) * 16, sbase_m = (g * 128 + wm * 32 + r) * 8;
  const int wbase = tid < kTile ? (((tid >> 6) * 32 + (tid & 31)) * 2 + ((tid >> 5) & 1)) * 4
                                : 4096 + ((((tid - kTile) >> 7) * 32 + (tid & 31)) * 4 + ((tid >> 5) & 3)) * 4;

  v16f acc[4][2];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ni][mi][i] = 0.0f;
  if constexpr (kLowRank) {
    // SVD-Quant branch: acc = L_up T^T over the rank, 16 ranks per MFMA; lane (r, g) supplies
    // row r (n for L_up, m for T) with ranks 16 s + 8 g .. + 7.  Rows past N or M read zeros.
    const uint32_t rb = (uint32_t)p.rank * 2;
    const __amdgpu_buffer_rsrc_t ur = make_rsrc(p.l_up, (uint32_t)p.n * rb);
    const __amdgpu_buffer_rsrc_t tr = make_rsrc(p.t, (uint32_t)p.m * rb);
    for (int s0 = 0; s0 < p.rank; s0 += 16) {
      v8bf un[4], tm[2];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        un[ni] = __builtin_bit_cast(v8bf, bload16(ur, (uint32_t)(nt * kTile + wn * 128 + 32 * ni + r) * rb + 2 * (s0 + 8 * g)));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        tm[mi] = __builtin_bit_cast(v8bf, bload16(tr, (uint32_t)(mt * kTile + wm * 64 + 32 * mi + r) * rb + 2 * (s0 + 8 * g)));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(un[ni], tm[mi], acc[ni][mi], 0, 0, 0);
    }
  }

  // Step s waits for this wave's loads into LDS (steps s and s + 1, issued in steps s - 2 and
  // s - 1), reads its operands from stage s % 3, then loads step s + 2 into stage (s + 2) % 3
  // (read last in step s - 1) and multiplies.  The load is issued after the operand reads: the
  // compiler cannot tell the stages apart and waits for every outstanding load into LDS before
  // a read from LDS, so a load issued before the reads would be waited for at once.  Past the
  // last step the loads read bytes of the next rows (or zeros past the end) into stages
  // nothing reads.
  uint4 xq = make_uint4(0, 0, 0, 0);     // FP4: scale block of the next ring write
  if constexpr (kFP4) {
    ring_put(ring + wbase, ring_order(sload(0)));
    xq = sload(1);
  }
  KQ_DMA(0, 0);
  KQ_DMA(1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
  __syncthreads();
  // Ping-pong: waves 0-3 (one per SIMD) and waves 4-7 run half a step apart.  Each step of a
  // wave is a memory part (staging, fetch, operand reads) and a matrix part (the MFMAs), each
  // ended by a workgroup barrier, so on every SIMD one wave multiplies while the other moves
  // data.
  const int grp = __builtin_amdgcn_readfirstlane(w >> 2);
  if (grp == 1) __syncthreads();
  KOps<kFP4> ops;
  int st_mul = 0, st_wr = 2;
  // KQ_STEP(s, R, RING): R = s mod 2 (the step's parity within its scale pair),
  // RING = (s mod 4 == 0)
#define KQ_STEP(s_, R_, RING_)                                                     \
  {                                                                               \
    /* scale block (s_)/4 + 1 into its ring slot (read last in step (s_) - 2) */   \
    if (kFP4 && (RING_))                                                          \
      ring_put(ring + ((((s_) >> 2) + 1) & 1) * kRingSlot + wbase, ring_order(xq)); \
    __builtin_amdgcn_s_waitcnt(0x0F70);        /* vmcnt(0) */                     \
    kread<kFP4, (R_) == 0>(ops, lds + st_mul * kStage,                            \
                ring + (((s_) >> 2) & 1) * kRingSlot + 2048 * (((s_) >> 1) & 1),  \
                rbase_n, rbase_m, rbase_n2, rbase_m2, sbase_n, sbase_m);          \
    KQ_DMA((s_) + 2, st_wr);                                                      \
    if (kFP4 && (RING_)) xq = sload(((s_) >> 2) + 2);   /* scale block s/4 + 2 */ \
    KQ_BAR();                                                                     \
    __builtin_amdgcn_s_setprio(1);                                                \
    kmma<kFP4, (R_)>(acc, ops);                                                   \
    __builtin_amdgcn_s_setprio(0);                                                \
    KQ_BAR();                                                                     \
    st_mul = st_mul == 2 ? 0 : st_mul + 1;                                        \
    st_wr = st_wr == 2 ? 0 : st_wr + 1;                                           \
  }
  // blocks of four steps (a ring write at the first), then up to three more
  int s = 0;
  for (; s + 3 < nsteps; s += 4) {
    KQ_STEP(s, 0, true);
    KQ_STEP(s + 1, 1, false);
    KQ_STEP(s + 2, 0, false);
    KQ_STEP(s + 3, 1, false);
  }
  if (s < nsteps) KQ_STEP(s, 0, true);
  if (s + 1 < nsteps) KQ_STEP(s + 1, 1, false);
  if (s + 2 < nsteps) KQ_STEP(s + 2, 0, false);
#undef KQ_STEP
  if (grp == 0) __syncthreads();
#undef KQ_DMA
#undef KQ_BAR

  __builtin_amdgcn_s_waitcnt(0x0F70);          // the last steps' loads into LDS landed
  // epilogue: lane (r, g) owns row m = mt*256 + wm*64 + 32 mi + r and, for each sub-tile ni,
  // columns n = nt*256 + wn*128 + 32 ni + 8q + 4g .. +3 (q = 0..3).  The wave's 64 x 128 tile
  // leaves through the wave's own 8 KB of the (now idle) stages, 32 rows by 256 bytes at a
  // time (float32: 64 columns, sub-tiles 2h and 2h + 1; bf16: all 128), so every store
  // instruction writes whole 256-byte row pieces, with the non-temporal hint: the 64 MB a
  // round of tiles writes would otherwise evict the next round's A and B tiles from the L2.
  // LDS row rr holds its 16-byte granule j at j ^ (rr & 15).
  __syncthreads();
  const float scale = p.scale;
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  uint8_t* wl = lds + w * 8192;
  constexpr int kPieces = kBf16 ? 1 : 2;       // 256-byte pieces of a row of the wave's tile
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int m0 = mt * kTile + wm * 64 + 32 * mi;
#pragma unroll
    for (int h = 0; h < kPieces; ++h) {
#pragma unroll
      for (int nj = 0; nj < 4 / kPieces; ++nj) {
        const int ni = (4 / kPieces) * h + nj;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16f& c = acc[ni][mi];
          const float c0 = c[4 * q] * scale, c1 = c[4 * q + 1] * scale;
          const float c2 = c[4 * q + 2] * scale, c3 = c[4 * q + 3] * scale;
          if constexpr (kBf16) {
            const int j = 4 * ni + q;                 // columns 8j .. 8j + 7
            *reinterpret_cast<uint2*>(wl + r * 256 + 16 * (j ^ (r & 15)) + 8 * g) =
                make_uint2(bf16x2_rne(c0, c1), bf16x2_rne(c2, c3));
          } else {
            const int j = 8 * nj + 2 * q + g;         // columns 64h + 4j .. + 3
            *reinterpret_cast<float4*>(wl + r * 256 + 16 * (j ^ (r & 15))) = make_float4(c0, c1, c2, c3);
          }
        }
      }
      // 4 rows of 16 granules per instruction
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rr = 4 * i + (l >> 4), j = l & 15;
        const u4v v = *reinterpret_cast<const u4v*>(wl + rr * 256 + 16 * (j ^ (rr & 15)));
        const int m = m0 + rr;
        if (m >= p.m) continue;
        if constexpr (kBf16) {
          const int n = nt * kTile + wn * 128 + 8 * j;
          uint16_t* dst = static_cast<uint16_t*>(p.c) + (int64_t)m * p.n + n;
          if (n < p.n) {
            if ((p.n & 7) == 0) {
              __builtin_nontemporal_store(v, reinterpret_cast<u4v*>(dst));
            } else {
              // N % 8 == 4: rows start 8-byte aligned only; 4 columns per store
              typedef unsigned int u2v __attribute__((ext_vector_type(2)));
              __builtin_nontemporal_store(u2v{v[0], v[1]}, reinterpret_cast<u2v*>(dst));
              if (n + 4 < p.n) __builtin_nontemporal_store(u2v{v[2], v[3]}, reinterpret_cast<u2v*>(dst + 4));
            }
          }
        } else {
          const int n = nt * kTile + wn * 128 + 64 * h + 4 * j;
          if (n < p.n)
            __builtin_nontemporal_store(v, reinterpret_cast<u4v*>(static_cast<float*>(p.c) + (int64_t)m * p.n + n));
        }
      }
    }
  }
}

// T = bf16(A L_down^T): A [M][K] bf16, L_down [rank][K] bf16, T [M][rank] bf16 (each value the
// float32 sum rounded once, nearest even).  Workgroup = 8 waves = 32 rows of A (an 8704-row
// activation gives 272 workgroups, two per CU resident at once); the 8 waves split K into
// consecutive ranges of whole 64-k groups and their partial sums meet in LDS at the end.
// Per group a wave loads the 32 rows x 128 bytes of A and the chunks of 32 rows x 128 bytes of
// L_down with whole-line loads (lane l takes row l / 8 + 8 j, 16-byte chunk l % 8), one group
// ahead, writes them to its own LDS stage (rows padded to 144 bytes) and reads them back in the
// MFMA layout: per chunk of 32 ranks, D = L_down_sub A_sub^T on v_mfma_f32_32x32x16_bf16, where
// in MFMA u lane (r, g) supplies row r with k = 32 g + 8 u .. + 7 of the group, the same slots
// for both operands (lane (r, g) owns output row r and ranks 8q + 4g .. + 3 of the chunk).
// Only the wave itself touches its stage, and LDS serves a wave's accesses in order, so no
// barrier is needed until the final sums.  Rows past M and ranks past `rank` read zeros
// (buffer descriptors), are summed as zeros and are not stored.
// kQuant: a lane's 16-byte chunk is a quarter of a 32-element FP4 block, the block's 4 lanes
// are a quad, so the same pass writes A's MXFP4 codes (4 bytes per lane) and E8M0 scales (the
// block quantizer's rule: e = clamp(floor(log2 amax) - 2, -127, 127), amax over the quad by
// DPP, E2M1 of x / 2^e by the hardware conversion).
constexpr int kDownPitch = 144;     // LDS row: 128 bytes of a group + 16 of padding
constexpr int kDownStage = 32 * kDownPitch;

template <bool kQuant, int kNch>
__global__ void __launch_bounds__(512, 2) lowrank_down_kernel(const uint16_t* a, const uint16_t* l_down,
                                                              int m, int k, int rank, uint16_t* t,
                                                              uint32_t* a_codes, uint8_t* a_scales) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 31, g = l >> 5;
  const int lrow = l >> 3, lch = l & 7;                 // load mapping: rows lrow + 8 j, chunk lch
  const int row0 = blockIdx.x * 32;
  const uint32_t kb = (uint32_t)k * 2;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(a, (uint32_t)m * kb);
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(l_down, (uint32_t)rank * kb);
  const int groups = k / 64, per = (groups + 7) / 8;
  const int g0 = min(w * per, groups), g1 = min(g0 + per, groups);
  uint8_t* sa = smem + w * (1 + kNch) * kDownStage;     // this wave's A stage, then its L stages
  uint8_t* sl = sa + kDownStage;
  v16f acc[kNch];
#pragma unroll
  for (int c = 0; c < kNch; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  uint4 xa[4], xl[kNch][4];
  const uint32_t aoff = (uint32_t)(row0 + lrow) * kb + 16 * lch;
  const uint32_t loff = (uint32_t)lrow * kb + 16 * lch;
#define KQ_DOWN_LOAD(G_)                                                                      \
  {                                                                                           \
    const uint32_t k2_ = 128u * (uint32_t)(G_);                                               \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) xa[j] = bload16(ar, aoff + 8 * j * kb + k2_); \
    _Pragma("unroll") for (int c = 0; c < kNch; ++c)                                          \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                           \
        xl[c][j] = bload16(lr, loff + (uint32_t)(32 * c + 8 * j) * kb + k2_);                 \
  }
  // the waves of every workgroup would otherwise read the same L_down slice at the same
  // moment (one L2 channel); each workgroup visits its range from a different group
  const int ng = g1 - g0, rot = ng > 0 ? (int)(blockIdx.x % (unsigned)ng) : 0;
  auto group_at = [&](int s_) { const int q_ = s_ + rot; return g0 + (q_ >= ng ? q_ - ng : q_); };
  if (ng > 0) KQ_DOWN_LOAD(group_at(0));
  for (int step = 0; step < ng; ++step) {
    const int gi = group_at(step);
    uint4 ca[4], cl[kNch][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ca[j] = xa[j];
#pragma unroll
    for (int c = 0; c < kNch; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) cl[c][j] = xl[c][j];
    if (step + 1 < ng) KQ_DOWN_LOAD(group_at(step + 1));
    if constexpr (kQuant) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wv[4] = {ca[j].x, ca[j].y, ca[j].z, ca[j].w};
        u16x2 mx = {0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) mx = mag_max(mx, wv[q]);
        const uint32_t am = quad_max(max((uint32_t)mx[0], (uint32_t)mx[1]));
        const int e = mx_block_exponent(am << 16);
        const int row = row0 + lrow + 8 * j;
        if (row < m) {
          a_codes[(int64_t)row * (k / 8) + 8 * gi + lch] = e2m1x8_bf16(wv, mx_scale_operand(e));
          if ((lch & 3) == 0) a_scales[(int64_t)row * (k / 32) + 2 * gi + (lch >> 2)] = (uint8_t)(e + 127);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint4*>(sa + (lrow + 8 * j) * kDownPitch + 16 * lch) = ca[j];
#pragma unroll
      for (int c = 0; c < kNch; ++c)
        *reinterpret_cast<uint4*>(sl + c * kDownStage + (lrow + 8 * j) * kDownPitch + 16 * lch) = cl[c][j];
    }
    uint4 av[4], lv[kNch][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = *reinterpret_cast<const uint4*>(sa + r * kDownPitch + 16 * (4 * g + u));
#pragma unroll
      for (int c = 0; c < kNch; ++c)
        lv[c][u] = *reinterpret_cast<const uint4*>(sl + c * kDownStage + r * kDownPitch + 16 * (4 * g + u));
    }
#pragma unroll
    for (int c = 0; c < kNch; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lv[c][u]),
                                                         __builtin_bit_cast(v8bf, av[u]), acc[c], 0, 0, 0);
  }
#undef KQ_DOWN_LOAD
  // the 8 waves' partial sums meet in LDS (the stages are no longer read after the barrier);
  // thread tid then sums value (c, i) of lane l for (c, i, l) = its share of the
  // kNch x 16 x 64 results
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);          // [kNch][16][8 waves][64 lanes]
#pragma unroll
  for (int c = 0; c < kNch; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[((c * 16 + i) * 8 + w) * 64 + l] = acc[c][i];
  __syncthreads();
  for (int e = tid; e < kNch * 16 * 64; e += 512) {
    const int ll = e & 63, ci = e >> 6;
    float sum = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) sum += red[(ci * 8 + ww) * 64 + ll];
    red[(ci * 8) * 64 + ll] = sum;             // wave 0's slot holds the total
  }
  __syncthreads();
  const int orow = row0 + (tid & 31), og = (tid >> 5) & 1;
  if (tid >= 64 || orow >= m) return;
  for (int c = 0; c < kNch; ++c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = 32 * c + 8 * q + 4 * og;
      if (j < rank) {
        float v[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) v[x] = red[((c * 16 + 4 * q + x) * 8) * 64 + tid];
        *reinterpret_cast<uint2*>(t + (int64_t)orow * rank + j) =
            make_uint2(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]));
      }
    }
  }
}

}  // namespace

hipError_t launch_lowrank_down(const uint16_t* a, const uint16_t* l_down, int m, int k, int rank,
                               uint16_t* t, uint8_t* a_codes, uint8_t* a_scales,
                               hipStream_t stream) {
  const int blocks = (m + 31) / 32;
  const int nch = (rank + 31) / 32;
  // per wave one A stage and nch L stages; the final sums reuse the same memory
  const size_t stages = (size_t)8 * (1 + nch) * kDownStage;
  const size_t sums = (size_t)nch * 16 * 8 * 64 * sizeof(float);
  const size_t lds = stages > sums ? stages : sums;
  uint32_t* cv = reinterpret_cast<uint32_t*>(a_codes);
#define KQ_DOWN(Q, C)                                                                          \
  hipLaunchKernelGGL((lowrank_down_kernel<Q, C>), dim3(blocks), dim3(512), lds, stream, a,     \
                     l_down, m, k, rank, t, cv, a_scales)
  if (a_codes != nullptr) {
    if (nch == 1) KQ_DOWN(true, 1); else KQ_DOWN(true, 2);
  } else {
    if (nch == 1) KQ_DOWN(false, 1); else KQ_DOWN(false, 2);
  }
#undef KQ_DOWN
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, bool fp4, hipStream_t stream) {
  const int tiles = ((p.m + kTile - 1) / kTile) * ((p.n + kTile - 1) / kTile);
  const bool lr = p.rank > 0;
  if (fp4 && lr && p.out_bf16)
    hipLaunchKernelGGL((gemm_kernel<true, true, true>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else if (fp4 && lr)
    hipLaunchKernelGGL((gemm_kernel<true, false, true>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else if (fp4 && p.out_bf16)
    hipLaunchKernelGGL((gemm_kernel<true, true, false>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else if (fp4)
    hipLaunchKernelGGL((gemm_kernel<true, false, false>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else if (p.out_bf16)
    hipLaunchKernelGGL((gemm_kernel<false, true, false>), dim3(tiles), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<false, false, false>), dim3(tiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kq
