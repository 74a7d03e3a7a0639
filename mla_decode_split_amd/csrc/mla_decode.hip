// mla_decode.hip - MLA decode (DeepSeek-R1 forward_absorb) for gfx950: split-K
// stage 1, LSE-merge stage 2, planner and the C ABI declared in mla_decode.h.
//
// Method (kernelbot-amd-mixed-mla pages): the submission template (675627)
// defines the operation - 16 query heads, one shared latent KV head, scores
// over the 576-wide row with sm_scale = 1/sqrt(576), values = the first 512
// columns of the same row.  Submissions 586148 and 753817 describe the
// two-stage split-K flash decoding this file implements: stage 1 runs an
// online softmax over a slice of a sequence's KV rows and emits a partial
// output with its log-sum-exp; stage 2 merges a sequence's slices with weights
// exp(lse_s - max lse).  Submission 739756's HIP kernel is prior art for the
// LDS-staged MFMA pipeline; the design below is our own for gfx950.
//
// Work decomposition.  The KV rows [0, total_kv) are cut into G equal ranges of
// R rows; workgroup g owns rows [g*R, (g+1)*R).  Because sequences are stored
// back to back (kv_indptr is a CSR offset array), a range covers pieces of one
// or more sequences.  A sequence that lies wholly inside one range is written
// to `out` directly; a piece of a longer sequence goes to partial slot
// 2g + (piece starts before the range ? 0 : 1), and stage 2 merges those.  This
// balances rows, not sequences, so ragged batches keep every CU equally busy.
//
// Stage-1 workgroup: 4 wave64s share an LDS ring of 32-row KV tiles filled by
// 16-byte global->LDS DMA (buffer_load ... lds).  Per tile:
//   QK : wave w computes S^T (16 tokens x 16 heads) for token block (w & 1)
//        over dim half (w >> 1) with MFMA (K rows are the A operand, Q^T the
//        B operand kept in registers); partial scores meet in LDS.
//   softmax: every wave reads the 32 x 16 scores, keeps the running max in
//        base 2 and forms P^T as the B operand of the next product.
//   PV : wave w owns value columns [128w, 128w + 128): O^T += V^T P^T with V^T
//        gathered from the same LDS tile (no second read of the row).
// fp8 / MXFP4 values are widened to bf16 in registers (exact); only fp8 x fp8
// queries/keys use the fp8 matrix instruction directly.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <limits.h>

#include <algorithm>
#include <new>

#include "mla_decode.h"

namespace mla {

constexpr int kHeads = 16;
constexpr int kQK = 576;
constexpr int kV = 512;
constexpr int kTile = 32;  // KV rows per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kScaleRow = kQK / 32;  // MXFP4 scale bytes per row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

enum Dt { DT_BF16 = MLA_DTYPE_BF16, DT_FP8 = MLA_DTYPE_FP8_E4M3FN, DT_MXFP4 = MLA_DTYPE_MXFP4 };

// ---------------------------------------------------------------- geometry

template <int KF>
struct KvGeom;
template <>
struct KvGeom<DT_BF16> {
  static constexpr int kRow = 2 * kQK, kStages = 2, kScaleChunks = 0;
};
template <>
struct KvGeom<DT_FP8> {
  static constexpr int kRow = kQK, kStages = 4, kScaleChunks = 0;
};
template <>
struct KvGeom<DT_MXFP4> {
  static constexpr int kRow = kQK / 2, kStages = 7, kScaleChunks = 1;
};

template <int KF>
struct Geom {
  static constexpr int kRow = KvGeom<KF>::kRow;
  static constexpr int kRowBytes = kTile * kRow;  // row bytes of one tile
  static constexpr int kRowChunks = kRowBytes / 1024;  // one chunk = one wave DMA instruction
  static constexpr int kChunks = kRowChunks + KvGeom<KF>::kScaleChunks;
  static constexpr int kStageBytes = kChunks * 1024;
  static constexpr int kStages = KvGeom<KF>::kStages;
  static constexpr int kRingBytes = kStages * kStageBytes;
  static constexpr int kScoreFloats = kWaves * kHeads * 16;
  static constexpr int kLdsBytes = kRingBytes + kScoreFloats * 4;
  static constexpr int kMaxChunksPerWave = (kChunks + kWaves - 1) / kWaves;
  static_assert(kRowBytes % 1024 == 0, "a tile must fill whole DMA chunks");
  __host__ __device__ static constexpr int chunks_of_wave(int w) { return (kChunks - w + kWaves - 1) / kWaves; }
};

// ------------------------------------------------------------ piece rules
// Shared by the kernels and by the host replay used in tests.

// Slot of the piece of sequence [s, e) inside workgroup range [lo, hi):
// -1 when the whole sequence is inside the range (written to out directly).
__host__ __device__ inline int32_t piece_slot(int64_t s, int64_t e, int64_t lo, int64_t hi, int32_t g) {
  return (s >= lo && e <= hi) ? -1 : 2 * g + (s < lo ? 0 : 1);
}

// Stage-2 view of the same rule: sequence [s, e), e > s, touches workgroups
// g0..g1; the piece in g0 starts inside that range (slot 2*g0 + 1), every
// later piece starts before its range (slot 2*g).
__host__ __device__ inline int32_t merge_slot(int32_t g, int32_t g0) { return 2 * g + (g == g0 ? 1 : 0); }

// ---------------------------------------------------------------- helpers

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline uint32_t bits(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Two fp8 E4M3FN codes (bytes 0,1 or 2,3 of w) -> two bf16, exact.
template <bool HI>
__device__ inline uint32_t fp8x2_bf16(uint32_t w) {
  return bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Eight fp8 codes (little-endian in v) -> eight bf16 in code order.
__device__ inline bf16x8 fp8x8_bf16(u32x2 v) {
  u32x4 r = {fp8x2_bf16<false>(v.x), fp8x2_bf16<true>(v.x), fp8x2_bf16<false>(v.y), fp8x2_bf16<true>(v.y)};
  return __builtin_bit_cast(bf16x8, r);
}

// E8M0 scale byte -> fp32 2^(e-127) (e = 0 is the fp32 subnormal 2^-127, 255 is NaN).
__device__ inline float e8m0_f32(uint32_t e) {
  const uint32_t b = e == 255u ? 0x7fc00000u : (e ? (e << 23) : 0x00400000u);
  return __builtin_bit_cast(float, b);
}

// Byte SEL of w holds two E2M1 codes (low nibble = lower element) -> two bf16 times scale.
template <int SEL>
__device__ inline uint32_t fp4x2_bf16(uint32_t w, float scale) {
  return bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

__device__ inline bf16x8 fp4x8_bf16(uint32_t w, float scale) {
  u32x4 r = {fp4x2_bf16<0>(w, scale), fp4x2_bf16<1>(w, scale), fp4x2_bf16<2>(w, scale), fp4x2_bf16<3>(w, scale)};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

__device__ inline float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// s_waitcnt vmcnt(n) for a runtime n in [0, 31] (the immediate must be constant).
__device__ inline void wait_vmcnt(int n) {
#define MLA_VMCNT_CASE(k) \
  case k:                 \
    asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
  switch (n) {
    MLA_VMCNT_CASE(0) MLA_VMCNT_CASE(1) MLA_VMCNT_CASE(2) MLA_VMCNT_CASE(3) MLA_VMCNT_CASE(4)
    MLA_VMCNT_CASE(5) MLA_VMCNT_CASE(6) MLA_VMCNT_CASE(7) MLA_VMCNT_CASE(8) MLA_VMCNT_CASE(9)
    MLA_VMCNT_CASE(10) MLA_VMCNT_CASE(11) MLA_VMCNT_CASE(12) MLA_VMCNT_CASE(13) MLA_VMCNT_CASE(14)
    MLA_VMCNT_CASE(15) MLA_VMCNT_CASE(16) MLA_VMCNT_CASE(17) MLA_VMCNT_CASE(18) MLA_VMCNT_CASE(19)
    MLA_VMCNT_CASE(20) MLA_VMCNT_CASE(21) MLA_VMCNT_CASE(22) MLA_VMCNT_CASE(23) MLA_VMCNT_CASE(24)
    MLA_VMCNT_CASE(25) MLA_VMCNT_CASE(26) MLA_VMCNT_CASE(27) MLA_VMCNT_CASE(28) MLA_VMCNT_CASE(29)
    MLA_VMCNT_CASE(30)
    default:
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      break;
  }
#undef MLA_VMCNT_CASE
}

// Workgroup barrier that also drains this wave's LDS traffic; the memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: 32-bit data format, raw (unswizzled) addressing.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc+voff into LDS at lds_base + 16*lane.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, const uint8_t* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, (int)voff, 0, 0, 0);
}

// ---------------------------------------------------------------- operands

// K operand (A of S^T = K Q^T): 8 consecutive key dims [dim0, dim0+8) of tile row `row`, as bf16.
template <int KF>
__device__ inline bf16x8 load_k8(const uint8_t* st, int row, int dim0, int sdelta) {
  if constexpr (KF == DT_BF16) {
    return *(const bf16x8*)(st + row * Geom<KF>::kRow + 2 * dim0);
  } else if constexpr (KF == DT_FP8) {
    return fp8x8_bf16(*(const u32x2*)(st + row * Geom<KF>::kRow + dim0));
  } else {
    const uint32_t w = *(const uint32_t*)(st + row * Geom<KF>::kRow + dim0 / 2);
    const uint32_t e = st[Geom<KF>::kRowBytes + sdelta + row * kScaleRow + dim0 / 32];
    return fp4x8_bf16(w, e8m0_f32(e));
  }
}

// V^T operands (A of O^T = V^T P^T) for tile rows 8g+i (i = 0..7) and value
// columns c0 + j (j = 0..7): a[j] element i = V[8g+i][c0+j].  Rows at or past
// `valid` are zeroed when MASK.
template <int KF, bool MASK>
__device__ inline void load_vt(const uint8_t* st, int g, int c0, int sdelta, int valid, bf16x8 a[8]) {
  uint32_t r[8][4];  // r[j][p] = bf16 pair (row 8g+2p, row 8g+2p+1) of column c0+j
  if constexpr (KF == DT_FP8) {
    u32x2 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = *(const u32x2*)(st + (8 * g + i) * Geom<KF>::kRow + c0);
      if (MASK && 8 * g + i >= valid) x[i] = u32x2{0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x2 lo = x[2 * p], hi = x[2 * p + 1];
      // interleave the bytes of two rows: (row0.b0, row1.b0, row0.b1, row1.b1), ...
      const uint32_t l01 = __builtin_amdgcn_perm(hi.x, lo.x, 0x05010400u);
      const uint32_t l23 = __builtin_amdgcn_perm(hi.x, lo.x, 0x07030602u);
      const uint32_t h01 = __builtin_amdgcn_perm(hi.y, lo.y, 0x05010400u);
      const uint32_t h23 = __builtin_amdgcn_perm(hi.y, lo.y, 0x07030602u);
      r[0][p] = fp8x2_bf16<false>(l01);
      r[1][p] = fp8x2_bf16<true>(l01);
      r[2][p] = fp8x2_bf16<false>(l23);
      r[3][p] = fp8x2_bf16<true>(l23);
      r[4][p] = fp8x2_bf16<false>(h01);
      r[5][p] = fp8x2_bf16<true>(h01);
      r[6][p] = fp8x2_bf16<false>(h23);
      r[7][p] = fp8x2_bf16<true>(h23);
    }
  } else {
    u32x4 x[8];  // row-wise bf16 of columns c0..c0+7
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * g + i;
      if constexpr (KF == DT_BF16) {
        x[i] = *(const u32x4*)(st + row * Geom<KF>::kRow + 2 * c0);
      } else {
        const uint32_t w = *(const uint32_t*)(st + row * Geom<KF>::kRow + c0 / 2);
        const uint32_t e = st[Geom<KF>::kRowBytes + sdelta + row * kScaleRow + c0 / 32];
        x[i] = __builtin_bit_cast(u32x4, fp4x8_bf16(w, e8m0_f32(e)));
      }
      if (MASK && row >= valid) x[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4 lo = x[2 * p], hi = x[2 * p + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        r[2 * q][p] = __builtin_amdgcn_perm(hi[q], lo[q], 0x05040100u);
        r[2 * q + 1][p] = __builtin_amdgcn_perm(hi[q], lo[q], 0x07060302u);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = __builtin_bit_cast(bf16x8, u32x4{r[j][0], r[j][1], r[j][2], r[j][3]});
}

// ---------------------------------------------------------------- stage 1

struct SplitParams {
  const uint8_t* q;
  const float* q_scale;
  const uint8_t* kv;
  const uint8_t* kv_scale;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  uint16_t* out;
  float* part_o;
  float* part_lse;
  int64_t total_kv;
  int32_t total_q;
  int32_t batch;
  int32_t rows_per_wg;
  float sm_scale;
};

// Query operand of S^T = K Q^T: lane (head = lane & 15, group = lane >> 4)
// holds Q^T for the dims of its dim half in the same order as the K operand.
template <int QF, int KF>
struct QOperand {
  static constexpr bool kFp8Mfma = (QF == DT_FP8 && KF == DT_FP8);
  bf16x8 b[9];   // bf16 path: dims half*288 + 32c + 8g + [0,8)
  i32x8 b8[2];   // fp8 path: dims half*288 + 128c + 32g + [0,32)
  uint64_t bx;   // fp8 path: dims half*288 + 256 + 8g + [0,8)

  __device__ inline void load(const uint8_t* q, int64_t qrow, int half, int lane) {
    const int h = lane & 15, g = lane >> 4;
    const int64_t base = (qrow * kHeads + h) * kQK + 288 * half;
    if constexpr (kFp8Mfma) {
      b8[0] = *(const i32x8*)(q + base + 32 * g);
      b8[1] = *(const i32x8*)(q + base + 128 + 32 * g);
      bx = *(const uint64_t*)(q + base + 256 + 8 * g);
    } else if constexpr (QF == DT_BF16) {
#pragma unroll
      for (int c = 0; c < 9; ++c) b[c] = *(const bf16x8*)(q + 2 * (base + 32 * c + 8 * g));
    } else {
#pragma unroll
      for (int c = 0; c < 9; ++c) b[c] = fp8x8_bf16(*(const u32x2*)(q + base + 32 * c + 8 * g));
    }
  }
};

template <int QF, int KF>
__device__ inline f32x4 qk_tile(const uint8_t* st, const QOperand<QF, KF>& qo, int row, int half, int g,
                                int sdelta) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (QOperand<QF, KF>::kFp8Mfma) {
    const uint8_t* rp = st + row * Geom<KF>::kRow + 288 * half;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const i32x8 k = *(const i32x8*)(rp + 128 * c + 32 * g);
      // formats 0/0 = fp8 E4M3 for both operands; scale exponents 127 = 2^0
      s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, qo.b8[c], s, 0, 0, 0, 127, 0, 127);
    }
    const uint64_t kx = *(const uint64_t*)(rp + 256 + 8 * g);
    s = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)kx, (long)qo.bx, s, 0, 0, 0);
  } else {
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const bf16x8 k = load_k8<KF>(st, row, 288 * half + 32 * c + 8 * g, sdelta);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, qo.b[c], s, 0, 0, 0);
    }
  }
  return s;
}

template <int QF, int KF>
__device__ void split_piece(const SplitParams& p, uint8_t* ring, float* sx, int64_t qrow, int64_t r0, int n,
                            int32_t slot, float score_scale, float out_scale) {
  using G = Geom<KF>;
  constexpr int NS = G::kStages;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int m = lane & 15;
  const int half = w >> 1;
  const int ntiles = (n + kTile - 1) / kTile;

  // Buffer resources: rows from r0 on (reads past the buffer return zero).
  const uint8_t* kv_base = p.kv + r0 * G::kRow;
  const uint64_t kv_avail = (uint64_t)(p.total_kv - r0) * G::kRow;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kv_base, (uint32_t)std::min<uint64_t>(kv_avail, 0xFFFFF000ull));
  int64_t sbase = 0;
  __amdgpu_buffer_rsrc_t rs = rk;
  if constexpr (KF == DT_MXFP4) {
    sbase = (r0 * kScaleRow) & ~(int64_t)15;
    const uint64_t sbytes = (((uint64_t)p.total_kv * kScaleRow + 15) & ~15ull) - (uint64_t)sbase;
    rs = make_rsrc(p.kv_scale + sbase, (uint32_t)std::min<uint64_t>(sbytes, 0xFFFFF000ull));
  }

  auto issue_tile = [&](int t) {
    uint8_t* stage = ring + (t % NS) * G::kStageBytes;
#pragma unroll
    for (int k = 0; k < G::kMaxChunksPerWave; ++k) {
      const int c = w + kWaves * k;
      if (c < G::kRowChunks) {
        dma16(rk, stage + c * 1024, (uint32_t)(t * G::kRowBytes + c * 1024 + lane * 16));
      } else if (c < G::kChunks) {
        const int64_t a = ((r0 + (int64_t)t * kTile) * kScaleRow) & ~(int64_t)15;
        dma16(rs, stage + G::kRowBytes, (uint32_t)(a - sbase) + lane * 16);
      }
    }
  };

  QOperand<QF, KF> qop;
  qop.load(p.q, qrow, half, lane);

  const int pro = std::min(NS - 1, ntiles);
  for (int t = 0; t < pro; ++t) issue_tile(t);

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int cnt_w = G::chunks_of_wave(w);
  for (int i = 0; i < ntiles; ++i) {
    wait_vmcnt(std::min(NS - 2, ntiles - 1 - i) * cnt_w);
    lds_barrier();  // tile i complete in LDS; every wave is done with tile i-1
    if (i + NS - 1 < ntiles) issue_tile(i + NS - 1);

    const uint8_t* st = ring + (i % NS) * G::kStageBytes;
    const int valid = std::min(kTile, n - i * kTile);
    const int sdelta = (KF == DT_MXFP4) ? (int)(((r0 + (int64_t)i * kTile) * kScaleRow) & 15) : 0;

    // ---- S^T partial for token block (w & 1), dim half (w >> 1)
    const f32x4 s = qk_tile<QF, KF>(st, qop, 16 * (w & 1) + m, half, g, sdelta);
    *(f32x4*)(sx + (w * kHeads + m) * 16 + 4 * g) = s;
    lds_barrier();

    // ---- online softmax (base 2) for tokens 8g..8g+7 of head m
    const int bb = g >> 1, tb = 8 * (g & 1);
    const f32x4 a0 = *(const f32x4*)(sx + (bb * kHeads + m) * 16 + tb);
    const f32x4 a1 = *(const f32x4*)(sx + (bb * kHeads + m) * 16 + tb + 4);
    const f32x4 b0 = *(const f32x4*)(sx + ((bb + 2) * kHeads + m) * 16 + tb);
    const f32x4 b1 = *(const f32x4*)(sx + ((bb + 2) * kHeads + m) * 16 + tb + 4);
    float t[8] = {a0.x + b0.x, a0.y + b0.y, a0.z + b0.z, a0.w + b0.w,
                  a1.x + b1.x, a1.y + b1.y, a1.z + b1.z, a1.w + b1.w};
    const bool tail = valid < kTile;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      t[k] *= score_scale;
      if (tail && 8 * g + k >= valid) t[k] = -INFINITY;
      mx = fmaxf(mx, t[k]);
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float ps = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = __builtin_amdgcn_exp2f(t[2 * k] - m_new);
      const float p1 = __builtin_amdgcn_exp2f(t[2 * k + 1] - m_new);
      ps += p0 + p1;
      pk[k] = pack_bf16x2(p0, p1);
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});

    // ---- O^T += V^T P^T over value columns [128w, 128w+128)
    bf16x8 va[8];
    if (tail)
      load_vt<KF, true>(st, g, 128 * w + 8 * m, sdelta, valid, va);
    else
      load_vt<KF, false>(st, g, 128 * w + 8 * m, sdelta, valid, va);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] *= alpha;
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[j], pb, acc[j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane (head m, group g) holds columns 128w + 32g + 8r + j in acc[j][r]
  float lt = l_run + shfl_xor(l_run, 16);
  lt += shfl_xor(lt, 32);
  const float inv = out_scale / lt;
  const int col0 = 128 * w + 32 * g;
  if (slot < 0) {
    uint16_t* o = p.out + (qrow * kHeads + m) * kV + col0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(acc[2 * q][r] * inv, acc[2 * q + 1][r] * inv);
      *(u32x4*)(o + 8 * r) = v;
    }
  } else {
    float* o = p.part_o + ((int64_t)slot * kHeads + m) * kV + col0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 v0 = {acc[0][r] * inv, acc[1][r] * inv, acc[2][r] * inv, acc[3][r] * inv};
      f32x4 v1 = {acc[4][r] * inv, acc[5][r] * inv, acc[6][r] * inv, acc[7][r] * inv};
      *(f32x4*)(o + 8 * r) = v0;
      *(f32x4*)(o + 8 * r + 4) = v1;
    }
    if (w == 0 && g == 0) p.part_lse[(int64_t)slot * kHeads + m] = (m_run + __builtin_amdgcn_logf(lt)) * kLn2;
  }
}

template <int QF, int KF>
__global__ __launch_bounds__(kThreads, 2) void mla_split_kernel(SplitParams p) {
  using G = Geom<KF>;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[G::kRingBytes];
  __shared__ __attribute__((aligned(16))) float sx[G::kScoreFloats];
  __shared__ int counts[2];

  const int tid = threadIdx.x;
  const int32_t gi = blockIdx.x;
  const int64_t lo = (int64_t)gi * p.rows_per_wg;
  const int64_t hi = std::min<int64_t>(lo + p.rows_per_wg, p.total_kv);
  if (lo >= hi) return;

  // Sequences overlapping [lo, hi): b in [#{j>=1: indptr[j] <= lo}, #{j<bs: indptr[j] < hi}).
  if (tid < 2) counts[tid] = 0;
  __syncthreads();
  int c_first = 0, c_end = 0;
  for (int j = tid; j <= p.batch; j += kThreads) {
    const int64_t v = p.kv_indptr[j];
    c_first += (j >= 1 && v <= lo);
    c_end += (j < p.batch && v < hi);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    c_first += __shfl_xor(c_first, off, 64);
    c_end += __shfl_xor(c_end, off, 64);
  }
  if ((tid & 63) == 0) {
    atomicAdd(&counts[0], c_first);
    atomicAdd(&counts[1], c_end);
  }
  __syncthreads();
  const int b_first = uniform(counts[0]);
  const int b_end = uniform(counts[1]);

  float qs = 1.f, ks = 1.f;
  if (QF == DT_FP8) qs = *p.q_scale;
  if (KF == DT_FP8) ks = *(const float*)p.kv_scale;
  const float score_scale = p.sm_scale * qs * ks * kLog2e;
  const float out_scale = ks;

  for (int b = b_first; b < b_end; ++b) {
    const int64_t s = uniform(p.kv_indptr[b]);
    const int64_t e = uniform(p.kv_indptr[b + 1]);
    const int64_t r0 = std::max(s, lo), r1 = std::min(e, hi);
    if (r0 >= r1) continue;
    const int32_t slot = piece_slot(s, e, lo, hi, gi);
    const int64_t qrow = std::min(std::max(uniform(p.qo_indptr[b]), 0), p.total_q - 1);
    split_piece<QF, KF>(p, ring, sx, qrow, r0, (int)(r1 - r0), slot, score_scale, out_scale);
    lds_barrier();  // the next piece reuses the ring and the score exchange
  }
}

// ---------------------------------------------------------------- stage 2

struct MergeParams {
  const float* part_o;
  const float* part_lse;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  uint16_t* out;
  int64_t total_kv;
  int32_t total_q;
  int32_t rows_per_wg;
  int32_t num_wgs;
};

// One workgroup of 128 threads per (sequence, head); thread t owns columns 4t..4t+3.
__global__ __launch_bounds__(128) void mla_merge_kernel(MergeParams p) {
  const int b = blockIdx.x >> 4, h = blockIdx.x & 15;
  const int t = threadIdx.x;
  const int64_t s = std::max<int64_t>(p.kv_indptr[b], 0);
  const int64_t e = std::min<int64_t>(p.kv_indptr[b + 1], p.total_kv);
  const int64_t qrow = std::min(std::max(p.qo_indptr[b], 0), p.total_q - 1);
  uint16_t* o = p.out + (qrow * kHeads + h) * kV + 4 * t;
  if (e <= s) {  // no KV rows: the softmax is empty, the output is zero
    *(uint2*)o = make_uint2(0u, 0u);
    return;
  }
  const int32_t g0 = (int32_t)std::min<int64_t>(s / p.rows_per_wg, p.num_wgs - 1);
  const int32_t g1 = (int32_t)std::min<int64_t>((e - 1) / p.rows_per_wg, p.num_wgs - 1);
  if (g0 == g1) return;  // written by stage 1
  float mx = -INFINITY;
  for (int32_t g = g0; g <= g1; ++g) mx = fmaxf(mx, p.part_lse[(int64_t)merge_slot(g, g0) * kHeads + h]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int32_t g = g0; g <= g1; ++g) {
    const int64_t slot = merge_slot(g, g0);
    const float lse = p.part_lse[slot * kHeads + h];
    const float wgt = (lse == -INFINITY) ? 0.f : __expf(lse - mx);
    wsum += wgt;
    const f32x4 v = *(const f32x4*)(p.part_o + (slot * kHeads + h) * kV + 4 * t);
    acc += wgt * v;
  }
  const float inv = 1.f / wsum;
  *(uint2*)o = make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
}

// ---------------------------------------------------------------- decode check

__global__ void mla_debug_decode_kernel(int kv_dtype, const uint8_t* codes, const uint8_t* scales, float* out,
                                        int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (kv_dtype == DT_FP8) {
    // 8 codes per thread through the kernel's fp8 -> bf16 path, then the scale.
    if (8 * i >= n) return;
    const float sc = scales ? *(const float*)scales : 1.f;
    uint8_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < 8 && 8 * i + k < n; ++k) c[k] = codes[8 * i + k];
    const u32x2 v = {(uint32_t)c[0] | (uint32_t)c[1] << 8 | (uint32_t)c[2] << 16 | (uint32_t)c[3] << 24,
                     (uint32_t)c[4] | (uint32_t)c[5] << 8 | (uint32_t)c[6] << 16 | (uint32_t)c[7] << 24};
    const bf16x8 d = fp8x8_bf16(v);
    for (int k = 0; k < 8 && 8 * i + k < n; ++k) out[8 * i + k] = (float)d[k] * sc;
  } else if (kv_dtype == DT_MXFP4) {
    // thread i decodes 8 columns of one row: row i / 72, columns 8 * (i % 72) + [0, 8)
    if (i >= n * 72) return;
    const int64_t row = i / 72;
    const int c0 = 8 * (int)(i % 72);
    const uint32_t w = *(const uint32_t*)(codes + row * 288 + c0 / 2);
    const bf16x8 d = fp4x8_bf16(w, e8m0_f32(scales[row * kScaleRow + c0 / 32]));
    for (int k = 0; k < 8; ++k) out[row * kQK + c0 + k] = (float)d[k];
  } else {
    if (i >= n) return;
    out[i] = __builtin_bit_cast(float, (uint32_t)((const uint16_t*)codes)[i] << 16);
  }
}

}  // namespace mla

// ==================================================================== host

using namespace mla;

struct mla_plan {
  mla_problem prob;
  int32_t rows_per_wg;
  int32_t num_wgs;
  int32_t stages;
  int32_t lds_bytes;
  int32_t stage2;
  int32_t num_cus;
  size_t ws_bytes;
  size_t lse_offset;
};

namespace {

thread_local char g_last_error[256] = "";

mla_status hip_fail(hipError_t e, const char* what) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return MLA_ERR_HIP;
}

int tile_stages(int kv_dtype) {
  switch (kv_dtype) {
    case DT_BF16: return Geom<DT_BF16>::kStages;
    case DT_FP8: return Geom<DT_FP8>::kStages;
    default: return Geom<DT_MXFP4>::kStages;
  }
}

int lds_bytes_for(int kv_dtype) {
  switch (kv_dtype) {
    case DT_BF16: return Geom<DT_BF16>::kLdsBytes;
    case DT_FP8: return Geom<DT_FP8>::kLdsBytes;
    default: return Geom<DT_MXFP4>::kLdsBytes;
  }
}

// Smallest row range worth a workgroup: below it the partial write-back and the
// merge cost more than the extra parallelism gains.
int min_rows_for(int kv_dtype) {
  switch (kv_dtype) {
    case DT_BF16: return 64;
    case DT_FP8: return 128;
    default: return 256;
  }
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

template <int QF, int KF>
hipError_t launch_split(const mla_plan* pl, const SplitParams& sp, hipStream_t st) {
  hipLaunchKernelGGL((mla_split_kernel<QF, KF>), dim3(pl->num_wgs), dim3(kThreads), 0, st, sp);
  return hipGetLastError();
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error_string(void) { return g_last_error; }

mla_status mla_decode_plan(const mla_problem* pr, const mla_plan_options* opt, const int32_t* kv_indptr_host,
                           mla_plan** plan_out, size_t* workspace_bytes) {
  if (plan_out) *plan_out = nullptr;
  if (!pr || !plan_out) return MLA_ERR_INVALID_ARG;
  if (pr->batch_size < 1 || pr->total_kv < 0 || pr->total_kv > INT32_MAX || !(pr->sm_scale == pr->sm_scale))
    return MLA_ERR_INVALID_ARG;
  if (pr->num_heads != kHeads || pr->qk_dim != kQK || pr->v_dim != kV) return MLA_ERR_UNSUPPORTED;
  if (pr->total_q != pr->batch_size) return MLA_ERR_UNSUPPORTED;  // one query token per sequence
  if (pr->q_dtype != DT_BF16 && pr->q_dtype != DT_FP8) return MLA_ERR_UNSUPPORTED;
  if (pr->kv_dtype != DT_BF16 && pr->kv_dtype != DT_FP8 && pr->kv_dtype != DT_MXFP4) return MLA_ERR_UNSUPPORTED;
  if (opt && (opt->rows_per_split < 0 || opt->wgs_per_cu < 0)) return MLA_ERR_INVALID_ARG;

  int num_cus = pr->num_cus;
  if (num_cus <= 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "querying the CU count");
  }

  if (kv_indptr_host) {
    if (kv_indptr_host[0] < 0 || kv_indptr_host[pr->batch_size] > pr->total_kv) return MLA_ERR_INVALID_ARG;
    for (int b = 0; b < pr->batch_size; ++b)
      if (kv_indptr_host[b + 1] < kv_indptr_host[b]) return MLA_ERR_INVALID_ARG;
  }

  const int64_t total = pr->total_kv;
  const int wpc = (opt && opt->wgs_per_cu > 0) ? opt->wgs_per_cu : 2;
  int64_t R;
  if (opt && opt->rows_per_split > 0) {
    R = opt->rows_per_split;
  } else {
    const int64_t target = (int64_t)num_cus * wpc;
    R = std::max<int64_t>((total + target - 1) / std::max<int64_t>(target, 1), min_rows_for(pr->kv_dtype));
  }
  R = (R + kTile - 1) / kTile * kTile;
  R = std::min<int64_t>(R, (int64_t)1 << 20);  // keeps per-workgroup byte offsets in 32 bits
  const int64_t G = std::max<int64_t>((total + R - 1) / R, 1);

  bool stage2 = true;
  if (kv_indptr_host) {
    stage2 = false;
    for (int b = 0; b < pr->batch_size && !stage2; ++b) {
      const int64_t s = kv_indptr_host[b], e = kv_indptr_host[b + 1];
      if (e <= s || s / R != (e - 1) / R) stage2 = true;
    }
  }

  mla_plan* pl = new (std::nothrow) mla_plan;
  if (!pl) return MLA_ERR_INVALID_ARG;
  pl->prob = *pr;
  pl->prob.num_cus = num_cus;
  pl->rows_per_wg = (int32_t)R;
  pl->num_wgs = (int32_t)G;
  pl->stages = tile_stages(pr->kv_dtype);
  pl->lds_bytes = lds_bytes_for(pr->kv_dtype);
  pl->stage2 = stage2 ? 1 : 0;
  pl->num_cus = num_cus;
  const size_t slots = 2 * (size_t)G;
  const size_t o_bytes = slots * kHeads * kV * sizeof(float);
  pl->lse_offset = (o_bytes + 255) / 256 * 256;
  pl->ws_bytes = pl->lse_offset + (slots * kHeads * sizeof(float) + 255) / 256 * 256;
  *plan_out = pl;
  if (workspace_bytes) *workspace_bytes = pl->ws_bytes;
  return MLA_OK;
}

void mla_decode_plan_destroy(mla_plan* plan) { delete plan; }

mla_status mla_decode_plan_describe(const mla_plan* pl, mla_plan_desc* d) {
  if (!pl || !d) return MLA_ERR_INVALID_ARG;
  d->num_splits = pl->num_wgs;
  d->rows_per_split = pl->rows_per_wg;
  d->tile_rows = kTile;
  d->stages = pl->stages;
  d->partial_slots = 2 * pl->num_wgs;
  d->stage2 = pl->stage2;
  d->workspace_bytes = (int64_t)pl->ws_bytes;
  d->lds_bytes = pl->lds_bytes;
  d->num_cus = pl->num_cus;
  return MLA_OK;
}

mla_status mla_decode_plan_pieces(const mla_plan* pl, const int32_t* ind, int64_t* rec, int64_t cap, int64_t* count) {
  if (!pl || !ind || !count || cap < 0 || (cap > 0 && !rec)) return MLA_ERR_INVALID_ARG;
  const int bs = pl->prob.batch_size;
  const int64_t R = pl->rows_per_wg, total = pl->prob.total_kv;
  int64_t n = 0;
  for (int32_t g = 0; g < pl->num_wgs; ++g) {
    const int64_t lo = (int64_t)g * R, hi = std::min(lo + R, total);
    if (lo >= hi) continue;
    int b_first = 0, b_end = 0;  // the counting rule the kernel applies
    for (int j = 0; j <= bs; ++j) {
      b_first += (j >= 1 && ind[j] <= lo);
      b_end += (j < bs && ind[j] < hi);
    }
    for (int b = b_first; b < b_end; ++b) {
      const int64_t s = ind[b], e = ind[b + 1];
      const int64_t r0 = std::max(s, lo), r1 = std::min(e, hi);
      if (r0 >= r1) continue;
      if (n < cap) {
        int64_t* r = rec + 5 * n;
        r[0] = g;
        r[1] = b;
        r[2] = r0;
        r[3] = r1;
        r[4] = piece_slot(s, e, lo, hi, g);
      }
      ++n;
    }
  }
  *count = n;
  return MLA_OK;
}

mla_status mla_decode_plan_merge_slots(const mla_plan* pl, const int32_t* ind, int32_t b, int32_t* slots,
                                       int32_t cap, int32_t* count) {
  if (!pl || !ind || !count || b < 0 || b >= pl->prob.batch_size || cap < 0 || (cap > 0 && !slots))
    return MLA_ERR_INVALID_ARG;
  const int64_t s = std::max<int64_t>(ind[b], 0), e = std::min<int64_t>(ind[b + 1], pl->prob.total_kv);
  *count = 0;
  if (e <= s) return MLA_OK;
  const int32_t g0 = (int32_t)std::min<int64_t>(s / pl->rows_per_wg, pl->num_wgs - 1);
  const int32_t g1 = (int32_t)std::min<int64_t>((e - 1) / pl->rows_per_wg, pl->num_wgs - 1);
  if (g0 == g1) return MLA_OK;
  int32_t n = 0;
  for (int32_t g = g0; g <= g1; ++g, ++n)
    if (n < cap) slots[n] = merge_slot(g, g0);
  *count = n;
  return MLA_OK;
}

namespace {

// Validates the run arguments and fills the kernel parameter blocks.
mla_status prepare(const mla_plan* pl, const void* q, const float* q_scale, const void* kv, const void* kv_scale,
                   const int32_t* qo_indptr, const int32_t* kv_indptr, void* out, void* workspace,
                   size_t workspace_bytes, SplitParams* sp, MergeParams* mp) {
  if (!pl || !q || !kv || !qo_indptr || !kv_indptr || !out) return MLA_ERR_INVALID_ARG;
  const mla_problem& pr = pl->prob;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (pr.q_dtype == DT_FP8 && !q_scale) return MLA_ERR_INVALID_ARG;
  if (pr.kv_dtype != DT_BF16 && !kv_scale) return MLA_ERR_INVALID_ARG;
  if (pr.kv_dtype == DT_MXFP4 && !aligned16(kv_scale)) return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < pl->ws_bytes || (pl->ws_bytes && (!workspace || !aligned16(workspace))))
    return MLA_ERR_INVALID_ARG;
  sp->q = (const uint8_t*)q;
  sp->q_scale = q_scale;
  sp->kv = (const uint8_t*)kv;
  sp->kv_scale = (const uint8_t*)kv_scale;
  sp->qo_indptr = qo_indptr;
  sp->kv_indptr = kv_indptr;
  sp->out = (uint16_t*)out;
  sp->part_o = (float*)workspace;
  sp->part_lse = (float*)((uint8_t*)workspace + pl->lse_offset);
  sp->total_kv = pr.total_kv;
  sp->total_q = pr.total_q;
  sp->batch = pr.batch_size;
  sp->rows_per_wg = pl->rows_per_wg;
  sp->sm_scale = pr.sm_scale;
  mp->part_o = sp->part_o;
  mp->part_lse = sp->part_lse;
  mp->qo_indptr = qo_indptr;
  mp->kv_indptr = kv_indptr;
  mp->out = sp->out;
  mp->total_kv = pr.total_kv;
  mp->total_q = pr.total_q;
  mp->rows_per_wg = pl->rows_per_wg;
  mp->num_wgs = pl->num_wgs;
  return MLA_OK;
}

mla_status launch_split_stage(const mla_plan* pl, const SplitParams& sp, hipStream_t st) {
  if (pl->prob.total_kv <= 0) return MLA_OK;
  const int qf = pl->prob.q_dtype, kf = pl->prob.kv_dtype;
  hipError_t e;
  if (qf == DT_BF16 && kf == DT_BF16) e = launch_split<DT_BF16, DT_BF16>(pl, sp, st);
  else if (qf == DT_BF16 && kf == DT_FP8) e = launch_split<DT_BF16, DT_FP8>(pl, sp, st);
  else if (qf == DT_BF16 && kf == DT_MXFP4) e = launch_split<DT_BF16, DT_MXFP4>(pl, sp, st);
  else if (qf == DT_FP8 && kf == DT_FP8) e = launch_split<DT_FP8, DT_FP8>(pl, sp, st);
  else if (qf == DT_FP8 && kf == DT_BF16) e = launch_split<DT_FP8, DT_BF16>(pl, sp, st);
  else e = launch_split<DT_FP8, DT_MXFP4>(pl, sp, st);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "launching the split kernel");
}

mla_status launch_merge_stage(const mla_plan* pl, const MergeParams& mp, hipStream_t st) {
  if (!pl->stage2) return MLA_OK;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(pl->prob.batch_size * kHeads), dim3(128), 0, st, mp);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : hip_fail(e, "launching the merge kernel");
}

}  // namespace

mla_status mla_decode_run(const mla_plan* pl, const void* q, const float* q_scale, const void* kv,
                          const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  SplitParams sp;
  MergeParams mp;
  mla_status s = prepare(pl, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, out, workspace, workspace_bytes, &sp, &mp);
  if (s != MLA_OK) return s;
  s = launch_split_stage(pl, sp, (hipStream_t)stream);
  if (s != MLA_OK) return s;
  return launch_merge_stage(pl, mp, (hipStream_t)stream);
}

mla_status mla_decode_split(const mla_plan* pl, const void* q, const float* q_scale, const void* kv,
                            const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  SplitParams sp;
  MergeParams mp;
  mla_status s = prepare(pl, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, out, workspace, workspace_bytes, &sp, &mp);
  if (s != MLA_OK) return s;
  return launch_split_stage(pl, sp, (hipStream_t)stream);
}

mla_status mla_decode_merge(const mla_plan* pl, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!pl || !qo_indptr || !kv_indptr || !out || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < pl->ws_bytes || (pl->ws_bytes && (!workspace || !aligned16(workspace))))
    return MLA_ERR_INVALID_ARG;
  MergeParams mp;
  mp.part_o = (const float*)workspace;
  mp.part_lse = (const float*)((const uint8_t*)workspace + pl->lse_offset);
  mp.qo_indptr = qo_indptr;
  mp.kv_indptr = kv_indptr;
  mp.out = (uint16_t*)out;
  mp.total_kv = pl->prob.total_kv;
  mp.total_q = pl->prob.total_q;
  mp.rows_per_wg = pl->rows_per_wg;
  mp.num_wgs = pl->num_wgs;
  return launch_merge_stage(pl, mp, (hipStream_t)stream);
}

mla_status mla_debug_decode(int32_t kv_dtype, const void* codes, const void* scales, float* out, int64_t n,
                            void* stream) {
  if (!codes || !out || n < 0) return MLA_ERR_INVALID_ARG;
  if (kv_dtype != DT_BF16 && kv_dtype != DT_FP8 && kv_dtype != DT_MXFP4) return MLA_ERR_UNSUPPORTED;
  if (kv_dtype == DT_MXFP4 && !scales) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  const int64_t threads = kv_dtype == DT_FP8 ? (n + 7) / 8 : (kv_dtype == DT_MXFP4 ? n * 72 : n);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return MLA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mla_debug_decode_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, kv_dtype,
                     (const uint8_t*)codes, (const uint8_t*)scales, out, n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : hip_fail(e, "launching the decode check");
}

}  // extern "C"
