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
// Work decomposition.  The KV rows [0, total_kv) are cut into G ranges in row
// order: equal ranges of R rows, or - with two workgroups per CU - pairs of a
// longer range for the CU's older workgroup and a shorter one for its younger
// (Cut).  Because sequences are stored back to back (kv_indptr is a CSR offset
// array), a range covers pieces of one or more sequences.  With the host
// offsets the plan passes each workgroup's first piece in the kernel
// arguments, so its first KV tile goes out before any other load.  A sequence
// that lies wholly inside one range is written to `out` directly; a piece of a
// longer sequence goes to partial slot 2g + (piece starts before the range ? 0
// : 1), and stage 2 merges those.  This balances rows, not sequences, so
// ragged batches keep every CU equally busy.
//
// Stage-1 workgroup (one query row per sequence): four wave64s (two workgroups
// per CU for bf16 and fp8 KV, three for MXFP4; one wave of each on every SIMD)
// stream the 32-row KV tiles
// of a piece through a shared LDS ring filled by 16-byte global->LDS DMA.  Per
// tile:
//   QK : each wave computes the partial S^T (32 tokens x 16 heads) over its
//        quarter of the 576 dims on MFMA, K from the LDS tile (A operand, fp8
//        and E2M1 codes fed raw to the scaled fp8/fp4 instruction), Q^T held in
//        registers (B operand); the partials meet in LDS;
//   softmax: each wave finishes the scores of a quarter of the tokens (base-2
//        online softmax against a running max that is raised only when a
//        score passes it by more than a slack) and posts the bf16
//        probabilities into the tile's rope bytes, which no wave reads after
//        the score exchange;
//   PV : O^T (the wave's 128 value columns x 16 heads) += V^T P^T on bf16 MFMA,
//        V^T gathered from the same LDS tile, P^T read back from LDS.
// A tile costs two workgroup barriers: tile i's scores, then - after the next
// ring barrier - tile i-1's products.
//
// Variants (template parameters of the stage-1 kernel):
//   QL    query rows per sequence held together (1, 2, 4): every KV tile is
//         multiplied with all of them (multi-token prediction, speculative
//         decoding), one exchange plane and one accumulator set per row; four
//         rows run as two groups of four waves, two rows each, over one ring;
//   CAP   scaled scores soft-capped as cap * tanh(s / cap) before the softmax
//         (the logit_cap argument of the library call on submission 753817's
//         page, which passes 0.0);
//   PAGED paged KV (the kv_indices / page_size arguments of that call): with
//         page size 1 CSR row j is row kv_indices[j] of the buffer; with page
//         size P = 2^k, kv_indices lists pages and row i of sequence b is row
//         i mod P of page kv_indices[kv_page_indptr[b] + i div P].  Wave 3
//         stages each tile's index entries in LDS (with pages it turns them
//         into row numbers there), waves 0-2 gather the rows.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <limits.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <type_traits>

#include "mla_decode.h"

namespace mla {

constexpr int kHeads = 16;
constexpr int kQK = 576;
constexpr int kV = 512;
constexpr int kTile = 32;  // KV rows per LDS tile
constexpr int kScaleRow = kQK / 32;  // MXFP4 scale bytes per row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dt { DT_BF16 = MLA_DTYPE_BF16, DT_FP8 = MLA_DTYPE_FP8_E4M3FN, DT_MXFP4 = MLA_DTYPE_MXFP4 };

// ---------------------------------------------------------------- geometry
//
// A tile is 32 consecutive KV rows.  The four waves of a workgroup stream the
// tiles of a piece through a shared ring of LDS slots; a slot holds the tile's
// rows and, for MXFP4, one 1 KB chunk with the tile's E8M0 scale bytes.

template <int KF>
struct KvGeom;
template <>
struct KvGeom<DT_BF16> {
  static constexpr int kRow = 2 * kQK, kScaleChunks = 0, kDmaWaves = 4;
};
template <>
struct KvGeom<DT_FP8> {
  static constexpr int kRow = kQK, kScaleChunks = 0, kDmaWaves = 4;
};
template <>
struct KvGeom<DT_MXFP4> {
  static constexpr int kRow = kQK / 2, kScaleChunks = 1, kDmaWaves = 3;
};

template <int KF>
struct Geom {
  static constexpr int kRow = KvGeom<KF>::kRow;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRowBytes = kTile * kRow;       // row bytes of one tile
  static constexpr int kRowChunks = kRowBytes / 1024;  // one chunk = one wave DMA instruction
  static constexpr int kChunks = kRowChunks + KvGeom<KF>::kScaleChunks;
  static constexpr int kStageBytes = kChunks * 1024;
  static_assert(kRowBytes % 1024 == 0, "a tile must fill whole DMA chunks");
};

// Which waves move a tile.  DMA wave w issues chunks w, w + kWaves, ...  For the
// 10-chunk MXFP4 tile, leaving wave 3 out of the DMA (4/3/3 chunks) measured
// faster; the 18- and 36-chunk tiles spread over all four waves.  With paged KV
// wave 3 stages the row indices instead and waves 0-2 move the rows.
template <int KF, bool PAGED>
struct Dma {
  static constexpr int kWaves = PAGED ? 3 : KvGeom<KF>::kDmaWaves;
  static constexpr int kMaxChunksPerWave = (Geom<KF>::kChunks + kWaves - 1) / kWaves;
  __host__ __device__ static constexpr int chunks_of_wave(int w) {
    return w < kWaves ? (Geom<KF>::kChunks - w + kWaves - 1) / kWaves : 0;
  }
};

// Paged KV: the physical row indices of tile t sit in slot t % kIdxSlots of a
// ring in LDS (32 int32 per slot), staged kIdxLead tiles ahead of need.
constexpr int kIdxSlots = 8, kIdxLead = 3;

// Partial-score exchange buffer of one query token, one plane per token of a
// lane's f32x4: [wave][block][r][lane] floats, so the wave that finishes the
// scores of component r reads 64 consecutive floats per (wave, block).
constexpr int kXchgBytes = 4 * 2 * 4 * 64 * 4;
// Probability exchange of query token t >= 1 (token 0 uses the tile's rope
// bytes): the bf16 P of every lane (16 bytes each) and the four waves' maxima
// of every head (16 bytes each), per tile parity.
constexpr int kPTokBytes = 64 * 16 + kHeads * 16;

// Query rows per wave and 4-wave groups per workgroup.  With four rows, two
// groups of four waves take two rows each over one shared ring, so each wave
// carries the registers of two rows and each SIMD runs two waves.
template <int QL>
struct RowSplit {
  static constexpr int kGroups = QL == 4 ? 2 : 1;
  static constexpr int kPerWave = QL / kGroups;
};

// Ring depth and residency per (KV format, query tokens per sequence QL).  Each
// query token adds its score-exchange plane, its probability buffers and ~60
// VGPRs (query operand, accumulators, scores).
//   QL = 1: the E2M1 tile is cheap to move and dear to compute, so three
//     workgroups with four-slot rings (measured faster than two with seven);
//     the fp8 and bf16 tiles need their deeper rings to keep HBM busy, which
//     leaves room for two.
//   QL = 2: two workgroups where the registers and LDS allow (fp8 with a
//     three-slot ring - the same speed as four at QL = 1 - and MXFP4), one for
//     bf16, whose 36 KB tiles leave no room for a second ring.
//   QL = 4: one workgroup per CU with the deepest ring that fits.
template <int KF, int QL>
struct RingCfg;
template <> struct RingCfg<DT_BF16, 1> { static constexpr int kStages = 2, kWgsPerCu = 2; };
template <> struct RingCfg<DT_FP8, 1> { static constexpr int kStages = 4, kWgsPerCu = 2; };
template <> struct RingCfg<DT_MXFP4, 1> { static constexpr int kStages = 4, kWgsPerCu = 3; };
template <> struct RingCfg<DT_BF16, 2> { static constexpr int kStages = 3, kWgsPerCu = 1; };
template <> struct RingCfg<DT_FP8, 2> { static constexpr int kStages = 3, kWgsPerCu = 2; };
template <> struct RingCfg<DT_MXFP4, 2> { static constexpr int kStages = 4, kWgsPerCu = 2; };
template <> struct RingCfg<DT_BF16, 4> { static constexpr int kStages = 3, kWgsPerCu = 1; };
template <> struct RingCfg<DT_FP8, 4> { static constexpr int kStages = 6, kWgsPerCu = 1; };
template <> struct RingCfg<DT_MXFP4, 4> { static constexpr int kStages = 8, kWgsPerCu = 1; };

// Paged KV adds the 1 KB index ring: fp8 keeps two workgroups per CU with a
// three-slot ring, bf16 runs one with three slots.  MXFP4 slots grow by 1 KB
// (the gathered scale windows fill the scale chunk, so the rescale path's
// maxima and flags move to an extra chunk); with one query row three
// workgroups with three-slot rings (a few registers spilled) measured faster
// than two with four (119 vs 125 µs on the ragged batch).
template <int KF, int QL>
struct PagedRingCfg {
  static constexpr int kStages = KF == DT_FP8 ? (QL == 4 ? 6 : 3) : KF == DT_MXFP4 ? (QL == 4 ? 6 : QL == 1 ? 3 : 4) : 3;
  static constexpr int kWgsPerCu = KF == DT_BF16 ? 1 : KF == DT_MXFP4 && QL == 1 ? 3 : (QL == 4 ? 1 : 2);
};

template <int KF, int QL, bool PAGED>
struct Ring {
  using Cfg = std::conditional_t<PAGED, PagedRingCfg<KF, QL>, RingCfg<KF, QL>>;
  static constexpr int kStages = Cfg::kStages;
  static constexpr int kWgsPerCu = Cfg::kWgsPerCu;
  // paged MXFP4: one more 1 KB chunk per slot for the rescale maxima and flags
  static constexpr int kAuxBytes = PAGED && KF == DT_MXFP4 ? 1024 : 0;
  static constexpr int kStageBytes = Geom<KF>::kStageBytes + kAuxBytes;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kXchg = QL * kXchgBytes;
  static constexpr int kPBuf = 2 * (QL - 1) * kPTokBytes;
  static constexpr int kIdx = PAGED ? kIdxSlots * kTile * 4 : 0;
  static constexpr int kDtab = PAGED && KF == DT_MXFP4 ? kStages * kTile : 0;  // scale window offsets
  static constexpr int kTotal = kLdsBytes + kXchg + kPBuf + kIdx + kDtab;
  static_assert(kWgsPerCu * kTotal <= 160 * 1024, "resident workgroups per CU must fit the LDS");
  static_assert((kStages - 2) * Dma<KF, PAGED>::kMaxChunksPerWave <= 63, "vmcnt range");
  static_assert(kStages >= 2 && kStages - 3 <= 5, "tiles behind the one needed near the end: 0..5");
  static_assert(!PAGED || kIdxSlots >= kStages - 1 + kIdxLead, "index ring covers the tiles staged ahead");
};

// ------------------------------------------------------------ piece rules
// Shared by the kernels and by the host replay used in tests.

// The cut of the KV rows [0, total_kv) into workgroup ranges, in row order
// ("positions").  Equal ranges (first = 0): position p is workgroup p and owns
// ra rows.  Paired ranges (first = F, G = 2F): a CU's first workgroup, i < F
// (dispatched before the rest), and its second, F + i, own the two halves of
// pair i's 2R rows - ra rows then rb = 2R - ra - at positions 2i and 2i + 1.
// The SIMD arbiter favours the older workgroup on a CU, so a slightly longer
// range for it evens out their finish times, and pair boundaries stay where
// equal ranges would put them.
struct Cut {
  int64_t ra, rb;
  int32_t first, G;
  // Paired ranges, grp > 0: pairs grp * (8a + x) + j (j < grp) go to the CUs
  // of XCD x (workgroup slots 8 (grp a + j) + x: consecutive workgroups go to
  // consecutive XCDs), so grp consecutive pairs - a sequence of grp pairs -
  // share one XCD's L2.  0: pair i is workgroup slot i.
  int32_t grp;
  __host__ __device__ int32_t pos_of(int32_t g) const {
    if (!first) return g;
    const int32_t half = g < first ? 0 : 1;
    int32_t i = g - half * first;
    if (grp) {
      const int32_t k = i / 8, x = i % 8;
      i = grp * (8 * (k / grp) + x) + k % grp;
    }
    return 2 * i + half;
  }
  __host__ __device__ int32_t wg_at(int32_t pos) const {
    if (!first) return pos;
    int32_t i = pos >> 1;
    if (grp) {
      const int32_t r = i % (8 * grp);
      i = 8 * (grp * (i / (8 * grp)) + r % grp) + r / grp;
    }
    return (pos & 1) ? first + i : i;
  }
  __host__ __device__ int64_t lo_at(int32_t pos) const {
    return first ? (int64_t)(pos >> 1) * (ra + rb) + ((pos & 1) ? ra : 0) : (int64_t)pos * ra;
  }
  // position owning `row` (clamped to the last)
  __host__ __device__ int32_t pos_of_row(int64_t row) const {
    int64_t pos;
    if (first) {
      const int64_t i = row / (ra + rb);
      pos = 2 * i + (row - i * (ra + rb) >= ra ? 1 : 0);
    } else {
      pos = row / ra;
    }
    return (int32_t)std::min<int64_t>(pos, G - 1);
  }
};

// Slot of the piece of sequence [s, e) inside workgroup range [lo, hi):
// -1 when the whole sequence is inside the range (written to out directly).
__host__ __device__ inline int32_t piece_slot(int64_t s, int64_t e, int64_t lo, int64_t hi, int32_t g) {
  return (s >= lo && e <= hi) ? -1 : 2 * g + (s < lo ? 0 : 1);
}

// Stage-2 view of the same rule: sequence [s, e), e > s, touches the ranges at
// positions p0..p1; the piece at p0 starts inside its range (slot 2g + 1 of
// that range's workgroup g), every later piece starts before its range (slot 2g).
__host__ __device__ inline int32_t merge_slot(const Cut& cut, int32_t pos, int32_t p0) {
  return 2 * cut.wg_at(pos) + (pos == p0 ? 1 : 0);
}

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

// E8M0 scale byte e -> the fp32 scale operand of the scaled conversions below.
// Those instructions take only the exponent field of their fp32 scale, so the
// float whose exponent field is e scales by 2^(e-127) for every code - e = 0
// (2^-127) and e = 255 (NaN) included: on gfx950 it gives the same bits as the
// fp32 values 2^-127 and NaN for every pair of E2M1 codes (checked over all
// 256 x 256 cases).  One shift, where a table would cost an LDS read.
__device__ inline float e8m0_scale(uint32_t e) { return __builtin_bit_cast(float, e << 23); }

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

__device__ inline float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Four bf16 values (two words) times inv -> E4M3 hi terms and E4M3 lo
// terms of the remainders, four codes per word in element order.
__device__ inline void split4(uint32_t w0, uint32_t w1, float inv, uint32_t& hi, uint32_t& lo) {
  const float x0 = bf_lo(w0) * inv, x1 = bf_hi(w0) * inv, x2 = bf_lo(w1) * inv, x3 = bf_hi(w1) * inv;
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const float r0 = x0 - __builtin_amdgcn_cvt_f32_fp8(h, 0), r1 = x1 - __builtin_amdgcn_cvt_f32_fp8(h, 1);
  const float r2 = x2 - __builtin_amdgcn_cvt_f32_fp8(h, 2), r3 = x3 - __builtin_amdgcn_cvt_f32_fp8(h, 3);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, l, true);
  hi = (uint32_t)h;
  lo = (uint32_t)l;
}

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int N>
__device__ inline void wait_vmcnt_clamped() {
  wait_vmcnt<(N < 63 ? N : 63)>();
}

// Wait until at most k * CHUNKS DMA instructions of this wave are in flight,
// k in [0, 5] (the tiles issued after the one needed may stay in flight).
template <int CHUNKS>
__device__ inline void wait_tiles_behind_n(int k) {
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt_clamped<CHUNKS>(); break;
    case 2: wait_vmcnt_clamped<2 * CHUNKS>(); break;
    case 3: wait_vmcnt_clamped<3 * CHUNKS>(); break;
    case 4: wait_vmcnt_clamped<4 * CHUNKS>(); break;
    default: wait_vmcnt_clamped<5 * CHUNKS>(); break;
  }
}

// Same for a wave that issues `chunks` DMA instructions per tile, where
// chunks is MAXC or MAXC - 1 (the tile's 1 KB chunks are dealt round robin).
template <int MAXC>
__device__ inline void wait_tiles_behind(int chunks, int k) {
  if (chunks == MAXC)
    wait_tiles_behind_n<MAXC>(k);
  else
    wait_tiles_behind_n<(MAXC > 1 ? MAXC - 1 : 1)>(k);
}

// The same with k fixed at compile time (one branch on the chunk count).
template <int MAXC, int K>
__device__ inline void wait_tiles_behind_fixed(int chunks) {
  if (chunks == MAXC)
    wait_vmcnt_clamped<K * MAXC>();
  else
    wait_vmcnt_clamped<K * (MAXC > 1 ? MAXC - 1 : 1)>();
}

// Workgroup barrier that also drains this wave's LDS traffic; the memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource: base, no stride, `bytes` records, dword3 0x00020000
// (32-bit data format, unswizzled).  Reads at or past `bytes` return zero.
__device__ inline i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

typedef const __attribute__((address_space(3))) uint8_t* lds_cbytes;

// 16- and 8-byte loads through a global (flat) or an LDS pointer; the LDS
// forms compile to ds_read, which the LDS counter tracks, not the memory one.
__device__ inline u32x4 ld16(const uint8_t* p) { return *(const u32x4*)p; }
__device__ inline u32x2 ld8(const uint8_t* p) { return *(const u32x2*)p; }
__device__ inline u32x4 ld16(lds_cbytes p) { return *(const __attribute__((address_space(3))) u32x4*)p; }
__device__ inline u32x2 ld8(lds_cbytes p) { return *(const __attribute__((address_space(3))) u32x2*)p; }
typedef const __attribute__((address_space(3))) uint16_t* lds_chalves;
__device__ inline u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }
__device__ inline u32x4 ld16(lds_chalves p) { return *(const __attribute__((address_space(3))) u32x4*)p; }
// The 16-bit element pointer of the same address space as a byte pointer.
template <typename BP>
struct Elem16;
template <>
struct Elem16<const uint8_t*> {
  using type = const uint16_t*;
};
template <>
struct Elem16<lds_cbytes> {
  using type = lds_chalves;
};

// 16 bytes per lane from rsrc + voff into LDS at lds_base + 16 * lane
// (lds_base wave-uniform).  Issued through inline asm on purpose: the compiler
// would otherwise treat every later LDS read as dependent on this write and
// wait for all DMA in flight, which serialises the tile ring.  Completion is
// tracked explicitly with s_waitcnt vmcnt before a tile is read.  m0 is not
// used for anything else in these kernels.  The loads are non-temporal (nt):
// every KV byte is read once, and with the streaming cache policy the same
// ring moves 302 MB in 44 us instead of 50 (6.9 against 6.0 TB/s).
__device__ inline void dma16(i32x4 r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(lds_base), "v"(voff), "s"(r)
               : "memory", "m0");
}

// The same DMA with the default cache policy, for E2M1 rows and scale windows
// gathered one by one (pages of one row: 288-byte rows and 32-byte windows at
// scattered places, where the non-temporal policy measured 8 us slower on the
// ragged MXFP4 batch; with pages of 16 rows it is 4 us faster).
__device__ inline void dma16_cached(i32x4 r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_base), "v"(voff), "s"(r)
               : "memory", "m0");
}

// The same DMA without a memory clobber, for the loads a workgroup issues
// before anything else (no LDS access precedes the wait that consumes them),
// so that the scalar loads the compiler places after them stay scalar.
__device__ inline void dma16_first(i32x4 r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(lds_base), "v"(voff), "s"(r) : "m0");
}
// The same with the default cache policy, for the query row: every workgroup
// of a sequence reads it, and the later ones find it in L2 (bs 32 stage 1
// 11.1 -> 10.3 us against the non-temporal form).
__device__ inline void dma16_first_cached(i32x4 r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_base), "v"(voff), "s"(r) : "m0");
}

// 4 bytes per active lane from rsrc + voff into LDS at lds_base + 4 * lane (the
// paged-KV index staging; tracked with vmcnt like dma16).
__device__ inline void dma4(i32x4 r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_base), "v"(voff), "s"(r)
               : "memory", "m0");
}

// ---------------------------------------------------------------- LDS layout
//
// A tile row of kRow bytes is stored as kRow / 16 units of 16 bytes, with unit
// u of row r placed at unit u ^ swz(r).  The XOR moves rows that would fall on
// the same LDS banks (576-byte rows repeat the bank pattern every 4 rows,
// 1152-byte rows every 2, 288-byte rows every 8) onto different banks for the
// access patterns below, and costs nothing at read time: every read offset is
// a per-lane constant plus an immediate.  The DMA realises the layout by
// choosing, for each LDS slot, which global 16-byte unit it loads.

template <int KF>
struct Layout;
template <>
struct Layout<DT_FP8> {
  static constexpr int kUnits = 36;
  __host__ __device__ static constexpr int swz(int row) { return (row >> 2) & 3; }
};
template <>
struct Layout<DT_BF16> {
  static constexpr int kUnits = 72;
  __host__ __device__ static constexpr int swz(int row) { return (row >> 1) & 3; }
};
template <>
struct Layout<DT_MXFP4> {
  static constexpr int kUnits = 18;
  __host__ __device__ static constexpr int swz(int row) { return (row >> 3) & 1; }
};

// Global byte offset (within a tile) of the 16-byte unit the DMA puts in LDS slot s.
template <int KF>
__device__ inline uint32_t dma_src_offset(int s) {
  constexpr int U = Layout<KF>::kUnits;
  const int r = s / U, u = s - r * U;
  return (uint32_t)(16 * (r * U + (u ^ Layout<KF>::swz(r))));
}

// ---------------------------------------------------------------- operands
//
// MFMA 16x16x32 (bf16) operand layouts: lane l holds, for the A operand, row
// l & 15 and the eight reduction indices of group l >> 4; for the B operand,
// column l & 15 and the same eight reduction indices; the result puts rows
// 4 * (l >> 4) + r, r = 0..3, of column l & 15 in lane l.  Only the pairing of
// A and B reduction indices matters, so the dims of a chunk can be laid out
// freely as long as K and Q use the same layout.

// Tile row of the i-th token a lane of group g feeds to the PV product: the
// tokens whose scores the same lane holds after S^T = K Q^T (rows 4g..4g+3 of
// each 16-row block), so P^T needs no data movement.
__device__ inline int pv_row(int g, int i) { return (i < 4) ? 4 * g + i : 12 + 4 * g + i; }
constexpr int pv_row_base(int i) { return (i < 4) ? i : 12 + i; }  // pv_row(g, i) - 4g

// Per-lane LDS byte offsets (within a tile) of the reads a lane (m, g) of
// wave w makes:
//   x[blk][e]  : fp8 keys, 16-byte half e of the 32 key bytes of chunk c of
//                token block blk is at x[blk][e] + 128 c;
//   v[h]       : V rows; row pv_row(g, i) column group q starts at
//                v[(i & 3) >> 1] + vrow(i) + vstep * q (E2M1: q = w folded in);
// and with this wave's share of the dims folded in:
//   xw[blk][e] : fp8 keys, x[blk][e] + 128 w (main chunk w); E2M1 keys, the
//                unit of the 32 codes of main chunk w (e = 0);
//   kr[blk]    : rope chunk w (waves 0, 1) of the fp8 and E2M1 keys;
//   kb[blk]    : bf16 keys, chunk w + 4k is at kb[blk] + 256 k.
template <int KF>
struct LaneOffs {
  int x[2][2];
  int v[2];
  int xw[2][2];
  int kr[2];
  int kb[2];

  __device__ inline void init(int m, int g, int w) {
    constexpr int R = Geom<KF>::kRow;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int row = 16 * blk + m;
      const int f = Layout<KF>::swz(row);
      if constexpr (KF == DT_FP8) {
        // fp8 keys, dims 128c + 32g + [0, 32): units 8c + 2g + e
        const int base = row * R + 16 * (4 * (g >> 1));
        x[blk][0] = base + 16 * ((2 * (g & 1)) ^ f);
        x[blk][1] = base + 16 * ((2 * (g & 1) + 1) ^ f);
      } else {
        x[blk][0] = x[blk][1] = 0;
      }
    }
    // fp8 rope: dims 32c + 8g + [0, 8) are unit 2c + (g >> 1), byte 8 (g & 1),
    // for chunk c = 16 + w with par = w & 1 (computed, not selected, so that the
    // offsets stay in registers)
    const int par = w & 1;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int row = 16 * blk + m;
      const int f = Layout<KF>::swz(row);
      xw[blk][0] = x[blk][0] + 128 * w;
      xw[blk][1] = x[blk][1] + 128 * w;
      if constexpr (KF == DT_FP8) {
        kr[blk] = row * R + 16 * ((2 * par + (g >> 1)) ^ f) + 8 * (g & 1) + 512;
        kb[blk] = 0;
      } else if constexpr (KF == DT_BF16) {
        kr[blk] = 0;
        kb[blk] = row * R + 16 * (g ^ f) + 64 * w;
      } else {
        // main chunk w: the 32 E2M1 codes of dims 128w + 32g + [0, 32) are unit 4w + g;
        // rope (waves 0, 1): dims 512 + 32w + 8g + [0, 8) are unit 16 + w, byte 4g
        xw[blk][0] = row * R + 16 * ((4 * w + g) ^ f);
        xw[blk][1] = 0;
        kr[blk] = row * R + 16 * ((16 + (w & 1)) ^ f) + 4 * g;
        kb[blk] = 0;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = pv_row(g, 2 * h);  // any row with the same (i & 3) >> 1 has the same swizzle
      const int f = Layout<KF>::swz(row);
      if constexpr (KF == DT_FP8) {
        // columns 128q + 8m + [0, 8): unit 8q + (m >> 1), byte 8 (m & 1)
        v[h] = 4 * g * R + 16 * ((m >> 1) ^ f) + 8 * (m & 1);
      } else if constexpr (KF == DT_BF16) {
        // unit 16q + m
        v[h] = 4 * g * R + 16 * (m ^ f);
      } else {
        // unit 4q + (m >> 2), byte 4 (m & 3)
        v[h] = 4 * g * R + 16 * ((m >> 2) ^ f) + 4 * (m & 3);
      }
    }
  }
};

// K operand of the bf16 path: key dims [32c + 8g, 32c + 8g + 8) of token
// block blk for this wave's chunk c = w + 4k.
template <int KF>
__device__ inline bf16x8 load_kw(const uint8_t* st, const LaneOffs<KF>& lo, int blk, int k) {
  static_assert(KF == DT_BF16, "fp8 and E2M1 keys use the matrix unit's own formats");
  return *(const bf16x8*)(st + lo.kb[blk] + 256 * k);
}

// Where a tile's E8M0 scale bytes sit in its LDS slot: row r's 18 bytes start
// at at(r).  Contiguous KV: the DMA copies the 16-byte-aligned span holding the
// tile's 576 bytes, so at(r) = kRowBytes + d + 18 r with d the span's lead.
// Paged KV: each row's 18 bytes are gathered as the aligned 32-byte window
// holding them, window r at kRowBytes + 32 r, and dt[r] (LDS) is the row's
// offset in it.
template <bool PAGED>
struct ScaleRows;
// at(rl, rc): tile offset of row rl + rc's scale bytes, rl per lane, rc a
// compile-time constant.
template <>
struct ScaleRows<false> {
  int sdelta;  // the span's lead d
  __device__ inline int at(int rl, int rc) const { return Geom<DT_MXFP4>::kRowBytes + sdelta + (rl + rc) * kScaleRow; }
};
template <>
struct ScaleRows<true> {
  const uint8_t* dt;
  // The empty asm keeps rc's part out of the per-lane sum, so that it ends in
  // the LDS read's immediate offset: otherwise the compiler keeps one register
  // per row (32 (rl + rc) with the bits of rl and rc merged), which at three
  // workgroups per CU spills.
  __device__ inline int at(int rl, int rc) const {
    int a = 32 * rl + (int)dt[rl + rc];
    asm("" : "+v"(a));
    return a + Geom<DT_MXFP4>::kRowBytes + 32 * rc;
  }
};

// V^T operands (A of O^T = V^T P^T) for value columns 128q + 8m + j (j = 0..7):
// a[j] element i = V[pv_row(g, i)][128q + 8m + j].  Rows at or past `valid`
// are zero when MASK.
template <int KF, bool PAGED, bool MASK>
__device__ inline void load_vt(const uint8_t* st, const LaneOffs<KF>& lo, int q, int m, int g, const ScaleRows<PAGED>& sc,
                               int valid,
                               bf16x8 a[8]) {
  constexpr int R = Geom<KF>::kRow;
  uint32_t r[8][4];  // r[j][p] = bf16 pair (token 2p, token 2p+1) of column j
  if constexpr (KF == DT_FP8) {
    u32x2 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = *(const u32x2*)(st + lo.v[(i & 3) >> 1] + pv_row_base(i) * R + 128 * q);
      if (MASK && pv_row(g, i) >= valid) x[i] = u32x2{0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x2 lo2 = x[2 * p], hi2 = x[2 * p + 1];
      // interleave the bytes of two rows: (row0.b0, row1.b0, row0.b1, row1.b1), ...
      const uint32_t l01 = __builtin_amdgcn_perm(hi2.x, lo2.x, 0x05010400u);
      const uint32_t l23 = __builtin_amdgcn_perm(hi2.x, lo2.x, 0x07030602u);
      const uint32_t h01 = __builtin_amdgcn_perm(hi2.y, lo2.y, 0x05010400u);
      const uint32_t h23 = __builtin_amdgcn_perm(hi2.y, lo2.y, 0x07030602u);
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
    u32x4 x[8];  // row-wise bf16 of the 8 columns
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KF == DT_BF16) {
        x[i] = *(const u32x4*)(st + lo.v[(i & 3) >> 1] + pv_row_base(i) * R + 256 * q);
      } else {
        const uint32_t w = *(const uint32_t*)(st + lo.v[(i & 3) >> 1] + pv_row_base(i) * R + 64 * q);
        const uint32_t e = st[sc.at(4 * g, pv_row_base(i)) + 4 * q + (m >> 2)];
        x[i] = __builtin_bit_cast(u32x4, fp4x8_bf16(w, e8m0_scale(e)));
      }
      if (MASK && pv_row(g, i) >= valid) x[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4 lo2 = x[2 * p], hi2 = x[2 * p + 1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[2 * k][p] = __builtin_amdgcn_perm(hi2[k], lo2[k], 0x05040100u);
        r[2 * k + 1][p] = __builtin_amdgcn_perm(hi2[k], lo2[k], 0x07060302u);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = __builtin_bit_cast(bf16x8, u32x4{r[j][0], r[j][1], r[j][2], r[j][3]});
}

// ---------------------------------------------------------------- stage 1

#ifdef MLA_WG_TRACE
// Measurement build only (-DMLA_WG_TRACE; the product build has none of it):
// the timeline of each stage-1 workgroup of the last launch, read back with
// mla_debug_wg_trace.  Entry g: [0] start (after the range check), [1] its
// first tile complete in LDS, [2] end, all on the 100 MHz real-time counter,
// and [3] the XCC_ID register | the HW_ID register << 8.
constexpr int kWgTraceMax = 8192;
__device__ uint64_t g_wg_trace[kWgTraceMax * 4];
struct WgTraceEnd {
  int32_t g;
  __device__ ~WgTraceEnd() {
    if (threadIdx.x == 0 && g < kWgTraceMax) g_wg_trace[4 * g + 2] = __builtin_amdgcn_s_memrealtime();
  }
};
#endif

struct SplitParams {
  const uint8_t* q;
  const float* q_scale;
  const uint8_t* kv;
  const uint8_t* kv_scale;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  uint16_t* out;
  uint16_t* part_o;
  float* part_lse;
  int64_t total_kv;
  int32_t total_q;
  int32_t batch;
  Cut cut;
  float sm_scale;
  float logit_cap;  // > 0: scaled scores soft-capped as cap * tanh(s / cap)
  const int32_t* kv_indices;      // paged KV: row or page indices
  int64_t kv_rows;                // paged KV: rows of the kv buffer
  const int32_t* kv_page_indptr;  // pages (page_shift > 0): sequence b's page list starts
                                  // at kv_indices[kv_page_indptr[b]]
  int32_t page_shift;             // paged KV: log2 of the page size
};

// Where a piece's index entries start in kv_indices (base), how many may be
// read from there (count), and the piece's first row within its sequence
// (jj0; 0 with page size 1, where the entries follow the CSR rows).
struct PageSpan {
  int64_t base;
  int64_t count;
  int32_t jj0;
};

// Query operand of S^T = K Q^T for the dims this wave multiplies.  The four
// waves of a workgroup split the 576 dims (each computes a partial S^T over
// its share for all tokens of the tile; the partials are summed through LDS),
// so every product is computed once.  Lane (head = lane & 15, group = lane >> 4)
// holds:
//   fp8 keys      : dims 128w + 32g + [0, 32) (one 16x16x128 chunk, laid out like
//                   K) and, for waves 0 and 1, rope dims 512 + 32w + 8g + [0, 8);
//   E2M1 keys     : dims 128w + 16g + [0, 16) and 128w + 64 + 16g + [0, 16) - the
//                   16x16x128 instruction pairs these with the A lane group that
//                   holds key dims 128w + 32g' + [0, 32) (one E8M0 block per lane,
//                   which is what the per-lane A scale applies to) - and, for
//                   waves 0 and 1, the bf16 rope dims 512 + 32w + 8g + [0, 8);
//   bf16 keys     : dims 32c + 8g + [0, 8) of chunks c = w + 4k, k < 5, c < 18.
// The operand kinds:
//   fp8 q with fp8 / E2M1 keys : the fp8 codes, on the matrix unit's own formats;
//   bf16 q with fp8 / E2M1 keys: q / s split into two fp8 terms hi + lo with one
//                    power-of-two s per head (hi = E4M3(q / s), lo = E4M3(q / s - hi)).
//                    A bf16 value has 8 significant bits and hi, lo carry 4 each,
//                    so the split is exact except for elements far below the
//                    head's maximum; keys feed the matrix unit unconverted;
//   bf16 keys      : bf16 (fp8 q widened exactly).
template <int QF, int KF>
struct QOperand {
  static constexpr bool kByteK = (KF == DT_FP8);    // K fed as raw fp8 bytes
  static constexpr bool kFp4K = (KF == DT_MXFP4);   // K fed as raw E2M1 codes with their E8M0 scales
  static constexpr bool kFp8Codes = (QF == DT_FP8 && (kByteK || kFp4K));  // q's fp8 codes as the B operand
  static constexpr bool kHiLo = (QF == DT_BF16 && (kByteK || kFp4K));     // bf16 q split into two fp8 terms
  static constexpr int kBfChunks = 5;
  bf16x8 b[kBfChunks];  // bf16 form (bf16 KV)
  i32x8 b8;             // fp8 forms (hi term): main chunk
  uint64_t bx;          //                      rope chunk (waves 0, 1), fp8 KV
  i32x8 l8;             // split form, lo term
  uint64_t lx;
  bf16x8 br;            // rope chunk (waves 0, 1) of the E2M1 path, bf16 (divided by the split scale)
  float scale;          // factor of the scores (s for the split form, else 1)

  // Raw query words as loaded (hi/lo form: 32 + 8 bf16; bf16 form with fp8 q: codes).
  u32x4 raw[4];
  u32x4 rx;
  u32x2 r8[kBfChunks];

  // Issues this wave's query loads (phase 1 of 3), from global memory or (q an
  // LDS pointer) from a copy of the query rows staged in LDS.
  template <typename BP>
  __device__ inline void fetch(BP q, int64_t qrow, int lane, int w) {
    const int h = lane & 15, g = lane >> 4;
    const int64_t base = (qrow * kHeads + h) * kQK;
    bx = lx = 0;
    rx = u32x4{0u, 0u, 0u, 0u};
    r8[0] = u32x2{0u, 0u};
    // For E2M1 keys the matrix unit pairs the 32 K values of B lane group g with
    // A values that, given A lane group g' = dims 32g' + [0, 32) of the chunk (one
    // E8M0 block per lane, as the per-lane A scale requires), are dims
    // 16g + [0, 16) and 64 + 16g + [0, 16); for fp8 keys B lane group g holds
    // dims 32g + [0, 32).
    const int m0 = kFp4K ? 128 * w + 16 * g : 128 * w + 32 * g;  // first 16 dims of this lane's B part
    const int m1 = kFp4K ? m0 + 64 : m0 + 16;                     // second 16
    if constexpr (kFp8Codes) {
      b8 = __builtin_bit_cast(i32x8, __builtin_shufflevector(ld16(q + base + m0), ld16(q + base + m1), 0, 1, 2, 3, 4,
                                                             5, 6, 7));
      if (w < 2) {
        if constexpr (kByteK)
          bx = __builtin_bit_cast(uint64_t, ld8(q + base + 512 + 32 * w + 8 * g));
        else
          r8[0] = ld8(q + base + 512 + 32 * w + 8 * g);
      }
    } else if constexpr (kHiLo) {
      const typename Elem16<BP>::type qb = (typename Elem16<BP>::type)q + base;  // bf16 elements
      raw[0] = ld16(qb + m0);
      raw[1] = ld16(qb + m0 + 8);
      raw[2] = ld16(qb + m1);
      raw[3] = ld16(qb + m1 + 8);
      if (w < 2) rx = ld16(qb + 512 + 32 * w + 8 * g);
    } else {
#pragma unroll
      for (int k = 0; k < kBfChunks; ++k) {
        const int c = w + 4 * k;
        if (c < kQK / 32) {
          if constexpr (QF == DT_BF16)
            b[k] = __builtin_bit_cast(bf16x8, ld16(q + 2 * (base + 32 * c + 8 * g)));
          else
            r8[k] = ld8(q + base + 32 * c + 8 * g);
        } else {
          b[k] = bf16x8{};
          r8[k] = u32x2{0u, 0u};
        }
      }
    }
  }

  // Makes the compiler complete the query loads here (phase 2), before any
  // KV DMA is issued: the compiler's wait for them would otherwise also wait
  // for every DMA issued in between.
  __device__ inline void arrive() {
    if constexpr (kFp8Codes) {
      asm volatile("" ::"v"(b8), "v"(bx), "v"(r8[0]));
    } else if constexpr (kHiLo) {
      asm volatile("" ::"v"(raw[0]), "v"(raw[1]), "v"(raw[2]), "v"(raw[3]), "v"(rx));
    } else if constexpr (QF == DT_BF16) {
#pragma unroll
      for (int k = 0; k < kBfChunks; ++k) asm volatile("" ::"v"(b[k]));
    } else {
#pragma unroll
      for (int k = 0; k < kBfChunks; ++k) asm volatile("" ::"v"(r8[k]));
    }
  }

  // Builds the operand from the raw words (phase 3).  The empty asm keeps this
  // arithmetic after the DMA issued between arrive() and here.  For the split
  // form the four waves agree on one scale per head (through `amax_lds`, 64
  // floats of LDS, with a workgroup barrier), so their partial scores add
  // without rescaling.  Every wave of the workgroup must call it.
  __device__ inline void prepare(float* amax_lds, int w, int lane) {
    scale = 1.f;
    if constexpr (kHiLo) {
      asm volatile("" : "+v"(raw[0]), "+v"(raw[1]), "+v"(raw[2]), "+v"(raw[3]), "+v"(rx));
      // max |q| over this wave's dims of the head (4 lanes per head), then over the waves
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(raw[k][e])), fabsf(bf_hi(raw[k][e]))));
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(rx[e])), fabsf(bf_hi(rx[e]))));
      amax = fmaxf(amax, shfl_xor(amax, 16));
      amax = fmaxf(amax, shfl_xor(amax, 32));
      if (lane < 16) amax_lds[16 * w + lane] = amax;
      lds_barrier();
      const int h = lane & 15;
      amax = fmaxf(fmaxf(amax_lds[h], amax_lds[16 + h]), fmaxf(amax_lds[32 + h], amax_lds[48 + h]));
      // s = smallest power of two with amax / s <= 448
      const uint32_t tb = __builtin_bit_cast(uint32_t, amax * (1.0f / 448.0f));
      int ex = (int)((tb >> 23) & 255u) + ((tb & 0x7fffffu) ? 1 : 0);
      ex = amax > 0.f ? std::min(std::max(ex, 1), 253) : 127;
      scale = __builtin_bit_cast(float, (uint32_t)ex << 23);
      const float inv = __builtin_bit_cast(float, (uint32_t)(254 - ex) << 23);
      u32x4 hw[2], lw[2];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          uint32_t hv, lv;
          split4(raw[k][e], raw[k][e + 1], inv, hv, lv);
          hw[k >> 1][2 * (k & 1) + (e >> 1)] = hv;
          lw[k >> 1][2 * (k & 1) + (e >> 1)] = lv;
        }
      b8 = __builtin_bit_cast(i32x8, __builtin_shufflevector(hw[0], hw[1], 0, 1, 2, 3, 4, 5, 6, 7));
      l8 = __builtin_bit_cast(i32x8, __builtin_shufflevector(lw[0], lw[1], 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (kByteK) {
        uint32_t h0, l0, h1, l1;
        split4(rx[0], rx[1], inv, h0, l0);
        split4(rx[2], rx[3], inv, h1, l1);
        bx = (uint64_t)h0 | ((uint64_t)h1 << 32);
        lx = (uint64_t)l0 | ((uint64_t)l1 << 32);
      } else {
        // rope stays bf16; dividing by the power of two s is exact
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(bf_lo(rx[e]) * inv, bf_hi(rx[e]) * inv);
        br = __builtin_bit_cast(bf16x8, r);
      }
    } else if constexpr (kFp8Codes && kFp4K) {
      asm volatile("" : "+v"(r8[0]));
      br = fp8x8_bf16(r8[0]);
    } else if constexpr (!kFp8Codes && QF == DT_FP8) {
#pragma unroll
      for (int k = 0; k < kBfChunks; ++k) {
        asm volatile("" : "+v"(r8[k]));
        b[k] = fp8x8_bf16(r8[k]);
      }
    }
  }

  // Keeps the finished operand in registers from here on (the compiler would
  // otherwise be free to re-derive parts of it inside the tile loop).
  __device__ inline void settle() {
    if constexpr (kByteK || kFp4K) {
      asm volatile("" ::"v"(b8), "v"(bx));
      if constexpr (kHiLo) asm volatile("" ::"v"(l8), "v"(lx));
      if constexpr (kFp4K) asm volatile("" ::"v"(br));
    } else {
#pragma unroll
      for (int k = 0; k < kBfChunks; ++k) asm volatile("" ::"v"(b[k]));
    }
  }
};

// This wave's partial S^T for the two 16-token blocks of a tile and each query
// token t: s[t][blk][r] = partial score of KV row 16 * blk + 4g + r for head
// lane & 15 of query token t (before any scaling).  The K operand is read once
// per block and multiplied with every token's query; two independent chains
// (the blocks) keep the matrix pipe busy.
template <int QF, int KF, int QL, bool PAGED>
__device__ inline void qk_tile(const uint8_t* st, const QOperand<QF, KF> (&qo)[QL], const LaneOffs<KF>& lo, int w,
                               int m, const ScaleRows<PAGED>& sc, f32x4 (&s)[QL][2]) {
  using QO = QOperand<QF, KF>;
#pragma unroll
  for (int t = 0; t < QL; ++t) {
    s[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[t][1] = s[t][0];
  }
  if constexpr (QO::kByteK) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const u32x4 k0 = *(const u32x4*)(st + lo.xw[blk][0]);
      const u32x4 k1 = *(const u32x4*)(st + lo.xw[blk][1]);
      const i32x8 k = __builtin_bit_cast(i32x8, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int t = 0; t < QL; ++t) {
        // formats 0/0 = fp8 E4M3 for both operands; scale exponents 127 = 2^0
        s[t][blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, qo[t].b8, s[t][blk], 0, 0, 0, 127, 0, 127);
        if constexpr (QO::kHiLo)
          s[t][blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, qo[t].l8, s[t][blk], 0, 0, 0, 127, 0, 127);
      }
    }
    if (w < 2) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        // rope dims 512 + 32w + 8g + [0, 8) sit where the bf16 path's chunk 16 + w does
        const uint64_t k = *(const uint64_t*)(st + lo.kr[blk]);
#pragma unroll
        for (int t = 0; t < QL; ++t) {
          s[t][blk] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k, (long)qo[t].bx, s[t][blk], 0, 0, 0);
          if constexpr (QO::kHiLo)
            s[t][blk] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k, (long)qo[t].lx, s[t][blk], 0, 0, 0);
        }
      }
    }
  } else if constexpr (QO::kFp4K) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // A lane group g: the 32 E2M1 codes of dims 128w + 32g + [0, 32), one E8M0
      // block, in natural order (the upper half of the operand is unused for
      // 4-bit data); the query operand holds the dims they pair with
      const u32x4 k4 = *(const u32x4*)(st + lo.xw[blk][0]);
      const i32x8 k = __builtin_bit_cast(i32x8, __builtin_shufflevector(k4, u32x4{0u, 0u, 0u, 0u}, 0, 1, 2, 3, 4, 5, 6, 7));
      const int e = st[sc.at(m, 16 * blk) + 4 * w + (threadIdx.x & 63) / 16];
#pragma unroll
      for (int t = 0; t < QL; ++t) {
        // formats: A = 4 (E2M1), B = 0 (fp8 E4M3); B scale exponent 127 = 2^0
        s[t][blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, qo[t].b8, s[t][blk], 4, 0, 0, e, 0, 127);
        if constexpr (QO::kHiLo)
          s[t][blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, qo[t].l8, s[t][blk], 4, 0, 0, e, 0, 127);
      }
    }
    if (w < 2) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        // rope dims 512 + 32w + 8g + [0, 8), widened to bf16 with their block scale
        const uint32_t word = *(const uint32_t*)(st + lo.kr[blk]);
        const uint32_t e = st[sc.at(m, 16 * blk) + 16 + w];
        const bf16x8 kb = fp4x8_bf16(word, e8m0_scale(e));
#pragma unroll
        for (int t = 0; t < QL; ++t)
          s[t][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qo[t].br, s[t][blk], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < QO::kBfChunks; ++k) {
      const int c = w + 4 * k;
      if (k == QO::kBfChunks - 1 && c >= kQK / 32) break;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const bf16x8 kk = load_kw<KF>(st, lo, blk, k);
#pragma unroll
        for (int t = 0; t < QL; ++t) s[t][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qo[t].b[k], s[t][blk], 0, 0, 0);
      }
    }
  }
}

// Softmax state of one piece.  m_run (the running maximum, base 2, per head)
// is identical in the four waves; l_run is the lane's part of the running sum
// over the tokens this wave takes the softmax of; acc is O^T for the wave's
// 128 value columns: acc[j][r] = column 128w + 32g + 8r + j of head lane & 15.
struct WaveState {
  float m_run;
  float l_run;
  f32x4 acc[8];
};

// 16-byte units of a tile row that hold the rope dims (used only by S = Q K^T):
// once every wave has its partial scores, the current tile's rope units carry
// the probability exchange.
template <int KF>
struct RopeUnits;
template <>
struct RopeUnits<DT_FP8> {
  static constexpr int kFirst = 32, kCount = 4;
};
template <>
struct RopeUnits<DT_BF16> {
  static constexpr int kFirst = 64, kCount = 8;
};
template <>
struct RopeUnits<DT_MXFP4> {
  static constexpr int kFirst = 16, kCount = 2;
};

// LDS byte offsets (within a tile slot) of the probability exchange of query
// row 0 (later rows: p_ptr / max_ptr below):
//   P slot of lane l (16 bytes): bf16 P of the eight tokens lane l feeds to the
//     PV product, [block][wave] - row l >> 1, rope unit (l & 1);
//   max slot of head h (16 bytes): the four waves' maxima of the head's scores;
//   flag slots (16 bytes per four waves): per wave a word whose bit r says a
//     score of query row r passed the rescale slack.
template <int KF>
__device__ inline int p_slot(int lane) {
  constexpr int R = Geom<KF>::kRow;
  const int row = lane >> 1;
  return row * R + 16 * ((RopeUnits<KF>::kFirst + (lane & 1)) ^ Layout<KF>::swz(row));
}
// E2M1 rows have two rope units: the maxima and flags go to the unused tail of
// the tile's scale chunk, or (paged KV, where gathered scale windows fill that
// chunk) to the same offsets of the slot's extra chunk after it.
template <int KF, bool PAGED>
__device__ inline int max_slot(int h) {
  constexpr int R = Geom<KF>::kRow;
  if constexpr (RopeUnits<KF>::kCount >= 4)
    return h * R + 16 * ((RopeUnits<KF>::kFirst + 2) ^ Layout<KF>::swz(h));
  else
    return Geom<KF>::kRowBytes + (PAGED ? 1024 : 0) + 768 + 16 * h;
}
// flag words of waves 4 * half .. 4 * half + 3 (half 1 only with two row groups)
template <int KF, bool PAGED>
__device__ inline int flag_slot(int half) {
  if constexpr (RopeUnits<KF>::kCount >= 4)
    return half * Geom<KF>::kRow + 16 * ((RopeUnits<KF>::kFirst + 3) ^ Layout<KF>::swz(half));
  else
    return Geom<KF>::kRowBytes + (PAGED ? 1024 : 0) + 704 + 16 * half;
}

// P slot and max slot of query row t: row 0 in the tile's rope bytes, later
// rows in `pb`, the tile parity's kPTokBytes-sized records (t is a
// compile-time index after unrolling when there is one row group).
template <int KF>
__device__ inline uint8_t* p_ptr(uint8_t* st, uint8_t* pb, int t, int lane) {
  return t == 0 ? st + p_slot<KF>(lane) : pb + (t - 1) * kPTokBytes + 16 * lane;
}
template <int KF, bool PAGED>
__device__ inline uint8_t* max_ptr(uint8_t* st, uint8_t* pb, int t, int h) {
  return t == 0 ? st + max_slot<KF, PAGED>(h) : pb + (t - 1) * kPTokBytes + 64 * 16 + 16 * h;
}

// A tile goes through two steps, one ring barrier apart, so that every tile
// costs two workgroup barriers and the products of consecutive tiles overlap:
//
// score_tile: S^T partials (this wave's share of the 576 dims, every query
//   token) -> LDS; after the exchange barrier, for each query token the full
//   scores of this wave's KV rows 4g + w and 16 + 4g + w (head m) and their
//   probabilities relative to the token's running maximum -> the token's P
//   slots, with a per-wave flag word: bit t set when some probability of token
//   t would exceed 2^kRescaleSlack.
// finish_tile (after the next barrier): for each flagged token the maximum is
//   raised to the tile's, the accumulators rescaled and the probabilities
//   recomputed and exchanged again (rare: the first tile, and a score well above
//   all before it); then every wave reads V^T once and, for each token, takes
//   the eight probabilities its PV lanes need and multiplies them into its 128
//   value columns.
// Below the slack bf16 P and the fp32 sums hold p = 2^(t - m_run) without loss,
// and the final normalisation by the running sum is unchanged.
// Logit soft-cap in the units the scores are summed in: a raw score v (sum of
// products, before the base-2 factor c) becomes U tanh(v / U) with U = cap *
// log2(e) / c, so that c times it is cap * tanh(s / cap) in base 2 for the
// natural score s = c v / log2(e).  tanh(y) = 1 - 2 / (e^(2y) + 1), with e^(2y)
// = 2^(v * k), k = 2 c / cap; it saturates to +-1 where the exponential
// overflows or underflows.
template <int QL, bool ON>
struct SoftCap {
  static constexpr bool on = ON;
  float u[QL], k[QL];
  __device__ inline float apply(float v, int t) const {
    const float e = __builtin_amdgcn_exp2f(v * k[t]);
    return u[t] * fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f);
  }
};

struct TileScores {
  float sv[2];  // raw scores of KV rows 4g + w and 16 + 4g + w, head m (-inf when masked)
  float p[2];   // their probabilities against m_run as it was when they were posted
};

// tb: the first query row of this wave's group; w8: the wave in the workgroup
// (w = w8 & 3 its share of dims and value columns).
template <int QF, int KF, int QW, int NG, bool CAP, bool PAGED, bool MASK>
__device__ inline void score_tile(uint8_t* st, uint8_t* pb, float* xchg, const QOperand<QF, KF> (&qo)[QW],
                                  const LaneOffs<KF>& lo, const WaveState (&ws)[QW], int w, int w8, int tb, int m, int g,
                                  const ScaleRows<PAGED>& sc, int valid, const float (&c)[QW], const SoftCap<QW, CAP>& cap,
                                  TileScores (&ts)[QW]) {
  const int lane = threadIdx.x & 63;
  {
    f32x4 part[QW][2];
    qk_tile<QF, KF, QW, PAGED>(st, qo, lo, w, m, sc, part);
#pragma unroll
    for (int t = 0; t < QW; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          xchg[(tb + t) * (kXchgBytes / 4) + ((2 * w + blk) * 4 + r) * 64 + lane] = part[t][blk][r];
  }
  lds_barrier();  // every wave's partial scores are in LDS and every wave is done with the rope dims
  int flags = 0;
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    const float* xt = xchg + (tb + t) * (kXchgBytes / 4);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // summed in wave order
      float v = xt[((0 + blk) * 4 + w) * 64 + lane];
      v += xt[((2 + blk) * 4 + w) * 64 + lane];
      v += xt[((4 + blk) * 4 + w) * 64 + lane];
      v += xt[((6 + blk) * 4 + w) * 64 + lane];
      if constexpr (CAP) v = cap.apply(v, t);
      ts[t].sv[blk] = (MASK && 16 * blk + 4 * g + w >= valid) ? -INFINITY : v;
    }
    // the base-2 score is sv * c with c >= 0; a masked row's probability is 0
    // by selection (with c = 0, a zero q or KV scale, -inf * c would be NaN)
    const float t0 = fmaf(ts[t].sv[0], c[t], -ws[t].m_run), t1 = fmaf(ts[t].sv[1], c[t], -ws[t].m_run);
    ts[t].p[0] = (MASK && 4 * g + w >= valid) ? 0.f : __builtin_amdgcn_exp2f(t0);
    ts[t].p[1] = (MASK && 16 + 4 * g + w >= valid) ? 0.f : __builtin_amdgcn_exp2f(t1);
    uint8_t* ps = p_ptr<KF>(st, pb, tb + t, lane);
    *(__bf16*)(ps + 2 * w) = (__bf16)ts[t].p[0];
    *(__bf16*)(ps + 8 + 2 * w) = (__bf16)ts[t].p[1];
    if (__builtin_amdgcn_ballot_w64(t0 > kRescaleSlack || t1 > kRescaleSlack) != 0) flags |= 1 << (tb + t);
  }
  if (lane == 0) {
    if constexpr (NG == 1)
      ((int*)(st + flag_slot<KF, PAGED>(0)))[w] = flags;
    else
      ((int*)(st + flag_slot<KF, PAGED>(w8 >> 2)))[w8 & 3] = flags;
  }
}

template <int QF, int KF, int QW, int NG, bool PAGED, bool MASK>
__device__ inline void finish_tile(uint8_t* st, uint8_t* pb, const LaneOffs<KF>& lo, WaveState (&ws)[QW], int w, int tb,
                                   int m, int g, const ScaleRows<PAGED>& sc, int valid, const float (&c)[QW],
                                   TileScores (&ts)[QW]) {
  const int lane = threadIdx.x & 63;
  bf16x8 va[8];
  load_vt<KF, PAGED, MASK>(st, lo, w, m, g, sc, valid, va);
  // bit r: some wave flagged query row r (the same value in every wave)
  const u32x4 fl = *(const u32x4*)(st + flag_slot<KF, PAGED>(0));
  uint32_t any = fl[0] | fl[1] | fl[2] | fl[3];
  if constexpr (NG == 2) {
    const u32x4 f1 = *(const u32x4*)(st + flag_slot<KF, PAGED>(1));
    any |= f1[0] | f1[1] | f1[2] | f1[3];
  }
  if (any != 0u) {
#pragma unroll
    for (int t = 0; t < QW; ++t) {
      if (!((any >> (tb + t)) & 1u)) continue;
      // tile maximum per head: this wave's rows (over the lane groups), then the waves
      float mx = fmaxf(ts[t].sv[0], ts[t].sv[1]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      // a wave whose rows are all masked posts -inf (not -inf * c, NaN when c = 0)
      if (g == 0) *(float*)(max_ptr<KF, PAGED>(st, pb, tb + t, m) + 4 * w) = mx == -INFINITY ? -INFINITY : mx * c[t];
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < QW; ++t) {
      if (!((any >> (tb + t)) & 1u)) continue;
      const f32x4 mw = *(const f32x4*)max_ptr<KF, PAGED>(st, pb, tb + t, m);
      const float tmax = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
      const float m_new = fmaxf(ws[t].m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(ws[t].m_run - m_new);
      ws[t].m_run = m_new;
      ws[t].l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) ws[t].acc[j] *= alpha;
      ts[t].p[0] = (MASK && 4 * g + w >= valid) ? 0.f : __builtin_amdgcn_exp2f(fmaf(ts[t].sv[0], c[t], -ws[t].m_run));
      ts[t].p[1] = (MASK && 16 + 4 * g + w >= valid) ? 0.f : __builtin_amdgcn_exp2f(fmaf(ts[t].sv[1], c[t], -ws[t].m_run));
      uint8_t* ps = p_ptr<KF>(st, pb, tb + t, lane);
      *(__bf16*)(ps + 2 * w) = (__bf16)ts[t].p[0];
      *(__bf16*)(ps + 8 + 2 * w) = (__bf16)ts[t].p[1];
    }
    lds_barrier();  // the probabilities against the new maxima are in LDS
  }
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    ws[t].l_run += ts[t].p[0] + ts[t].p[1];
    const bf16x8 pv = __builtin_bit_cast(bf16x8, *(const u32x4*)p_ptr<KF>(st, pb, tb + t, lane));
#pragma unroll
    for (int j = 0; j < 8; ++j) ws[t].acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[j], pv, ws[t].acc[j], 0, 0, 0);
  }
}

// Workgroups share each CU, and the SIMD arbiter favours older waves, so with
// equal priorities the workgroups dispatched later fall behind and the kernel
// waits for them.  Each wave's priority instead follows how much of its
// workgroup's row range is left (3 above one half, 2 above a quarter, 1 above
// an eighth, else 0): whichever workgroup lags is favoured until it catches up.
__device__ inline void set_priority(int prio) {
  switch (prio) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// One piece: rows [r0, r0 + n) of a sequence whose query rows are qrow0 ..
// qrow0 + nq - 1 (nq in [1, QL]; the operands of tokens past nq repeat the
// last row and their results are dropped).
// G1: E2M1 KV in pages of one row (its gathers take the default cache policy).
template <int QF, int KF, int QL, bool CAP, bool PAGED, bool G1 = false>
__device__ void split_piece(const SplitParams& p, uint8_t* ring, float* xchg, uint8_t* pbuf, int32_t* idxring,
                            uint8_t* dtab,
                            int64_t qrow0, int nq, int64_t r0,
                            int n, int32_t slot, float score_scale, float out_scale, int64_t wg_hi, int32_t wg_rows,
                            PageSpan ps, bool staged) {
  using G = Geom<KF>;
  using DM = Dma<KF, PAGED>;
  constexpr int NS = Ring<KF, QL, PAGED>::kStages;
  constexpr int NG = RowSplit<QL>::kGroups, QW = RowSplit<QL>::kPerWave;
  const int lane = threadIdx.x & 63;
  const int w8 = uniform(threadIdx.x >> 6);
  const int w = NG == 1 ? w8 : (w8 & 3);      // share of dims and value columns
  const int grp = NG == 1 ? 0 : (w8 >> 2);    // row group: query rows tb .. tb + QW - 1
  const int tb = grp * QW;
  const int wd = grp == 0 ? w : Geom<KF>::kWaves;  // DMA wave index (group 0 moves the tiles)
  const int g = lane >> 4;
  const int m = lane & 15;
  const int ntiles = (n + kTile - 1) / kTile;

  // Buffer resources: rows from r0 on (reads past the buffer return zero); with
  // paged KV the whole buffer (its size checked on the host) and the piece's
  // indices.
  const uint8_t* kv_base = PAGED ? p.kv : p.kv + r0 * G::kRow;
  const uint64_t kv_avail = PAGED ? (uint64_t)p.kv_rows * G::kRow : (uint64_t)(p.total_kv - r0) * G::kRow;
  const i32x4 rk = make_rsrc(kv_base, (uint32_t)std::min<uint64_t>(kv_avail, 0xFFFFF000ull));
  i32x4 ri = rk;
  if constexpr (PAGED)
    ri = make_rsrc(p.kv_indices + ps.base, (uint32_t)std::min<uint64_t>((uint64_t)ps.count * 4, 0xFFFFF000ull));
  int64_t sbase = 0;
  i32x4 rs = rk;
  if constexpr (KF == DT_MXFP4) {
    // E8M0 rows are read in 16-byte units: the allocation is readable up to the
    // next multiple of 16 bytes past its rows (reads past it return zero)
    const uint64_t rows = PAGED ? (uint64_t)p.kv_rows : (uint64_t)p.total_kv;
    sbase = PAGED ? 0 : (r0 * kScaleRow) & ~(int64_t)15;
    const uint64_t sbytes = ((rows * kScaleRow + 15) & ~15ull) - (uint64_t)sbase;
    rs = make_rsrc(p.kv_scale + sbase, (uint32_t)std::min<uint64_t>(sbytes, 0xFFFFF000ull));
  }

  // Tile t goes to slot t % NS; DMA wave w issues the chunks c = w, w + DM::kWaves, ...
  // Lane offsets of its row chunks follow the swizzled layout: tile row prow[k],
  // byte src[k] of the tile (of the row when paged).
  uint32_t src[DM::kMaxChunksPerWave];
  int prow[DM::kMaxChunksPerWave];
#pragma unroll
  for (int k = 0; k < DM::kMaxChunksPerWave; ++k) {
    const int c = wd + DM::kWaves * k;
    src[k] = c < G::kRowChunks ? dma_src_offset<KF>(64 * c + lane) : 0u;
    prow[k] = (int)(src[k] / G::kRow);
    if (PAGED) src[k] -= (uint32_t)(prow[k] * G::kRow);
  }
  auto issue_tile = [&](int t) {
    if (wd >= DM::kWaves) return;
    const uint8_t* stage = ring + (t % NS) * Ring<KF, QL, PAGED>::kStageBytes;
    const int32_t* ix = idxring + (t % kIdxSlots) * kTile;
#pragma unroll
    for (int k = 0; k < DM::kMaxChunksPerWave; ++k) {
      const int c = wd + DM::kWaves * k;
      if (c >= G::kChunks) break;
      if (PAGED && c < G::kRowChunks) {
        // physical row of this lane's tile row (an index outside the buffer
        // wraps or lands past its end, where the read returns zero)
        const uint32_t off = (uint32_t)ix[prow[k]] * (uint32_t)G::kRow + src[k];
        if constexpr (G1)
          dma16_cached(rk, uniform(lds_addr(stage + c * 1024)), off);
        else
          dma16(rk, uniform(lds_addr(stage + c * 1024)), off);
      } else if (PAGED) {
        // E8M0 bytes of tile row lane >> 1: the aligned 32-byte window holding
        // its 18 (two 16-byte halves), and the row's offset in it
        const uint32_t sb = (uint32_t)ix[lane >> 1] * (uint32_t)kScaleRow;
        const uint32_t soff = (sb & ~15u) + 16u * (uint32_t)(lane & 1);
        if constexpr (G1)
          dma16_cached(rs, uniform(lds_addr(stage + G::kRowBytes)), soff);
        else
          dma16(rs, uniform(lds_addr(stage + G::kRowBytes)), soff);
        if ((lane & 1) == 0) dtab[(t % NS) * kTile + (lane >> 1)] = (uint8_t)(sb & 15u);
      } else if (c < G::kRowChunks) {
        dma16(rk, uniform(lds_addr(stage + c * 1024)), (uint32_t)(t * G::kRowBytes) + src[k]);
      } else {
        const int64_t a = ((r0 + (int64_t)t * kTile) * kScaleRow) & ~(int64_t)15;
        dma16(rs, uniform(lds_addr(stage + G::kRowBytes)), (uint32_t)(a - sbase) + lane * 16);
      }
    }
  };

  LaneOffs<KF> lo;
  lo.init(m, g, w);

  // Paged KV: wave 3 stages the physical row indices of tile t (32 lanes, 4
  // bytes each) into index slot t % kIdxSlots, kIdxLead tiles ahead of the
  // tile whose DMA needs them; waves 0-2 read them when they issue that DMA.
  // With pages the entry of tile row r is that of the row's page.
  auto stage_idx = [&](int t) {
    const uint32_t base = uniform(lds_addr(idxring + (t % kIdxSlots) * kTile));
    if (lane < kTile) dma4(ri, base, 4u * ((uint32_t)(ps.jj0 + t * kTile + lane) >> p.page_shift));
  };
  // Pages: once tile t's entries are in LDS, wave 3 replaces each page number
  // by its row's number (page * P + the row's place in the page) before the
  // barrier that publishes them.
  auto pages_to_rows = [&](int t) {
    if (PAGED && p.page_shift && wd == 3 && lane < kTile) {
      int32_t* e = idxring + (t % kIdxSlots) * kTile + lane;
      const uint32_t in_page = (uint32_t)(ps.jj0 + t * kTile + lane) & ((1u << p.page_shift) - 1u);
      *e = (int32_t)(((uint32_t)*e << p.page_shift) | in_page);
    }
  };
  if (PAGED && wd == 3)
    for (int t = 0; t <= NS - 2 + kIdxLead; ++t) stage_idx(t);

  const int my_chunks = DM::chunks_of_wave(wd);
  QOperand<QF, KF> qop[QW];
  if (staged) {
    // The kernel issued tile 0, then this sequence's query row (into slot NS - 1),
    // then tiles 1 .. NS - 2: wait for the first two and read the query from LDS.
    if (my_chunks > 0) wait_tiles_behind<DM::kMaxChunksPerWave>(my_chunks, NS - 2);
    lds_barrier();
    qop[0].fetch((lds_cbytes)(ring + (NS - 1) * Ring<KF, QL, PAGED>::kStageBytes), 0, lane, w);
    qop[0].arrive();
  } else {
#pragma unroll
    for (int t = 0; t < QW; ++t) qop[t].fetch(p.q, qrow0 + std::min(tb + t, nq - 1), lane, w);
#pragma unroll
    for (int t = 0; t < QW; ++t) qop[t].arrive();
  }
  const int pro = std::min(NS - 1, ntiles);
  if constexpr (PAGED) {
    if (wd == 3) {
      wait_vmcnt<0>();  // the staged indices are in LDS
      for (int t = 0; t < pro; ++t) pages_to_rows(t);
    }
    lds_barrier();
  }
  if (!staged)
    for (int t = 0; t < pro; ++t) issue_tile(t);
  // per-token head maxima past the sequence counts at the start of xchg
#pragma unroll
  for (int t = 0; t < QW; ++t) qop[t].prepare(xchg + 256 + 64 * (tb + t), w, lane);
#pragma unroll
  for (int t = 0; t < QW; ++t) qop[t].settle();

  WaveState ws[QW];
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    ws[t].m_run = -INFINITY;
    ws[t].l_run = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ws[t].acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // tile i is complete in LDS and every wave is done with tile i - 1
  auto advance = [&](int i) {
    if (my_chunks > 0) {
      if (i + NS - 2 < ntiles)  // the usual case: the NS - 2 tiles after tile i stay in flight
        wait_tiles_behind_fixed<DM::kMaxChunksPerWave, NS - 2>(my_chunks);
      else
        wait_tiles_behind<DM::kMaxChunksPerWave>(my_chunks, ntiles - 1 - i);
    }
    lds_barrier();
  };
  // Paged KV, after advance(i) of every tile with a refill: the indices of tile
  // i + NS - 1 (staged kIdxLead steps earlier, or in the prologue) are complete
  // for wave 3, and the score exchange barrier publishes them before refill(i)
  // reads them; then the indices kIdxLead tiles further on go out.  Wave 3 has
  // no other loads in flight, so vmcnt counts index loads only.
  auto idx_step = [&](int i) {
    if (PAGED && wd == 3) {
      wait_vmcnt<kIdxLead - 1>();
      pages_to_rows(i + NS - 1);
      stage_idx(i + NS - 1 + kIdxLead);
    }
  };
  // The DMA of tile i + NS - 1 (into the slot tile i - 1 left) goes out after
  // tile i's products are issued: when the memory pipeline is full the issue
  // waits for room, and there it waits while the matrix cores work.
  auto refill = [&](int i) {
    if (i + NS - 1 < ntiles) issue_tile(i + NS - 1);
  };
  auto scales_of = [&](int i) -> ScaleRows<PAGED> {
    if constexpr (PAGED)
      return ScaleRows<true>{dtab + (i % NS) * kTile};
    else
      return ScaleRows<false>{(KF == DT_MXFP4) ? (int)(((r0 + (int64_t)i * kTile) * kScaleRow) & 15) : 0};
  };
  // full tiles in the loop (one code path, so the accumulators stay in place);
  // a partial last tile after it
  const int nfull = n / kTile;
  // priority 3 while more than half the range is left, 2 above a quarter, 1
  // above an eighth: with rows_left(i) = wg_hi - (r0 + 32 i), 8 rows_left(i) > x
  // exactly when i < below(x)
  const int64_t d8 = 8 * (wg_hi - r0);
  auto below = [&](int64_t x) -> int { return d8 > x ? (int)std::min<int64_t>((d8 - x + 255) / 256, INT_MAX) : 0; };
  const int f4 = below(4 * (int64_t)wg_rows), f2 = below(2 * (int64_t)wg_rows), f1 = below(wg_rows);
  // tile at which the priority changes next (it only falls, at f4, f2 and f1;
  // the calls come for consecutive tiles from 0)
  int next_prio = 0;
  auto priority = [&](int i) {
    if (i == next_prio) {
      const int want = (i < f4) + (i < f2) + (i < f1);
      set_priority(want);
      next_prio = want == 3 ? f4 : want == 2 ? f2 : want == 1 ? f1 : INT_MAX;
    }
  };
  float cs[QW];
#pragma unroll
  for (int t = 0; t < QW; ++t) cs[t] = score_scale * qop[t].scale;
  SoftCap<QW, CAP> cap;
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    // c = 0 (a zero q or KV scale): every score is 0 and stays 0
    const bool live = CAP && cs[t] > 0.f;
    cap.u[t] = live ? p.logit_cap * kLog2e / cs[t] : 0.f;
    cap.k[t] = live ? 2.f * cs[t] / p.logit_cap : 0.f;
  }
  const int last_valid = n - (ntiles - 1) * kTile;
  auto stage = [&](int i) { return ring + (i % NS) * Ring<KF, QL, PAGED>::kStageBytes; };
  // probability records of tokens >= 1: one set per tile parity
  auto pbuf_of = [&](int i) { return pbuf + (i & 1) * ((QL - 1) * kPTokBytes); };
  TileScores ts[QW];
  // tile 0, then for each later tile: its scores and the previous tile's products
  priority(0);
  advance(0);
#ifdef MLA_WG_TRACE
  if (threadIdx.x == 0 && blockIdx.x < kWgTraceMax && g_wg_trace[4 * blockIdx.x + 1] == 0)
    g_wg_trace[4 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
#endif
  idx_step(0);
  if (nfull > 0)
    score_tile<QF, KF, QW, NG, CAP, PAGED, false>(stage(0), pbuf_of(0), xchg, qop, lo, ws, w, w8, tb, m, g, scales_of(0), kTile, cs, cap, ts);
  else
    score_tile<QF, KF, QW, NG, CAP, PAGED, true>(stage(0), pbuf_of(0), xchg, qop, lo, ws, w, w8, tb, m, g, scales_of(0), last_valid, cs, cap,
                                 ts);
  refill(0);
  for (int i = 1; i < nfull; ++i) {
    priority(i);
    advance(i);
    idx_step(i);
    finish_tile<QF, KF, QW, NG, PAGED, false>(stage(i - 1), pbuf_of(i - 1), lo, ws, w, tb, m, g, scales_of(i - 1), kTile, cs, ts);
    score_tile<QF, KF, QW, NG, CAP, PAGED, false>(stage(i), pbuf_of(i), xchg, qop, lo, ws, w, w8, tb, m, g, scales_of(i), kTile, cs, cap, ts);
    refill(i);
  }
  if (nfull > 0 && nfull < ntiles) {  // the partial last tile
    advance(nfull);
    finish_tile<QF, KF, QW, NG, PAGED, false>(stage(nfull - 1), pbuf_of(nfull - 1), lo, ws, w, tb, m, g, scales_of(nfull - 1), kTile,
                                   cs, ts);
    score_tile<QF, KF, QW, NG, CAP, PAGED, true>(stage(nfull), pbuf_of(nfull), xchg, qop, lo, ws, w, w8, tb, m, g, scales_of(nfull),
                                 last_valid, cs, cap, ts);
  }
  lds_barrier();  // the last tile's probabilities are in LDS
  if (nfull < ntiles)
    finish_tile<QF, KF, QW, NG, PAGED, true>(stage(ntiles - 1), pbuf_of(ntiles - 1), lo, ws, w, tb, m, g, scales_of(ntiles - 1),
                                  last_valid, cs, ts);
  else
    finish_tile<QF, KF, QW, NG, PAGED, false>(stage(ntiles - 1), pbuf_of(ntiles - 1), lo, ws, w, tb, m, g, scales_of(ntiles - 1),
                                   kTile, cs, ts);

  if (PAGED && wd == 3) wait_vmcnt<0>();  // no index load outlives the piece

  // ---- epilogue: lane (head m, group g) holds columns 128w + 32g + 8r + j in acc[j][r]
  // running sums: this wave's rows (over the lane groups), then over the waves
  // (every wave is past its last read of the score planes)
  float lt[QW];
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    lt[t] = ws[t].l_run + shfl_xor(ws[t].l_run, 16);
    lt[t] += shfl_xor(lt[t], 32);
    if (g == 0) xchg[64 * (tb + t) + 16 * w + m] = lt[t];
  }
  lds_barrier();
  const int col0 = 128 * w + 32 * g;
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    const int r = tb + t;  // query row of the sequence
    if (r >= nq) break;
    lt[t] = xchg[64 * r + m] + xchg[64 * r + 16 + m] + xchg[64 * r + 32 + m] + xchg[64 * r + 48 + m];
    const float inv = out_scale / lt[t];
    // whole sequence: the output; piece of a split one: its partial O, also bf16 (the
    // merge adds at most one bf16 rounding of the weighted terms to the output's own)
    uint16_t* o = (slot < 0 ? p.out + ((qrow0 + r) * kHeads + m) * kV
                            : p.part_o + (((int64_t)slot * QL + r) * kHeads + m) * kV) +
                  col0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      u32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = pack_bf16x2(ws[t].acc[2 * k][r] * inv, ws[t].acc[2 * k + 1][r] * inv);
      *(u32x4*)(o + 8 * r) = v;
    }
    if (slot >= 0 && w == 0 && g == 0)
      p.part_lse[((int64_t)slot * QL + r) * kHeads + m] = (ws[t].m_run + __builtin_amdgcn_logf(lt[t])) * kLn2;
  }
}

// Each workgroup's first piece, derived by the planner from the host kv_indptr
// and passed with the kernel arguments (read with scalar loads), where the
// kernel would otherwise search kv_indptr and load the sequence bounds before
// its first KV load.  Entry g: the piece's rows (bits 0-15; 0 = the range holds
// no rows of any sequence), its sequence (bits 16-29), whether the sequence
// starts at the range's first row (bit 30) and whether it ends inside the
// range (bit 31).  The piece always starts at the range's first row.  Used with
// one query row per sequence, when the plan
// knows the offsets, kv_indptr[0] = 0, G <= kSplitTable, batch <= 2^14 and
// R < 2^16.
constexpr int kSplitTable = 768;
struct SplitTable {
  static constexpr bool kHas = true;
  uint32_t first[kSplitTable];
};
struct NoSplitTable {
  static constexpr bool kHas = false;
};
static_assert(sizeof(SplitParams) + sizeof(SplitTable) <= 4096, "kernel arguments within 4 KB");

template <int QF, int KF, int QL, bool CAP, bool PAGED, typename Tab, bool G1>
__global__ __launch_bounds__(Geom<KF>::kThreads * RowSplit<QL>::kGroups) __attribute__((amdgpu_waves_per_eu(
    Ring<KF, QL, PAGED>::kWgsPerCu * RowSplit<QL>::kGroups,
    Ring<KF, QL, PAGED>::kWgsPerCu * RowSplit<QL>::kGroups))) void mla_split_kernel(SplitParams p, Tab tab) {
  using RG = Ring<KF, QL, PAGED>;
  constexpr int kThreads = Geom<KF>::kThreads * RowSplit<QL>::kGroups;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[RG::kLdsBytes];
  __shared__ float xchg[RG::kXchg / 4];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[QL > 1 ? RG::kPBuf : 16];
  __shared__ __attribute__((aligned(16))) int32_t idxring[PAGED ? kIdxSlots * kTile : 1];
  __shared__ __attribute__((aligned(16))) uint8_t dtab[RG::kDtab ? RG::kDtab : 1];
  int* counts = (int*)xchg;  // the sequence search runs before any exchange

  const int tid = threadIdx.x;
  const int32_t gi = blockIdx.x;
  const int32_t pos = p.cut.pos_of(gi);
  const int64_t lo = p.cut.lo_at(pos);
  const int64_t hi = std::min<int64_t>(p.cut.lo_at(pos + 1), p.total_kv);
  if (lo >= hi) return;
#ifdef MLA_WG_TRACE
  if (tid == 0 && gi < kWgTraceMax) {
    g_wg_trace[4 * gi + 0] = __builtin_amdgcn_s_memrealtime();
    g_wg_trace[4 * gi + 3] = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)) |
                             ((uint64_t)__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11)) << 8);
  }
  const WgTraceEnd trace_end{gi};
#endif

  float qs = 1.f, ks = 1.f;
  if (QF == DT_FP8) qs = *p.q_scale;
  if (KF == DT_FP8) ks = *(const float*)p.kv_scale;
  const float score_scale = p.sm_scale * qs * ks * kLog2e;
  const float out_scale = ks;

  int b_first, b_end;
  if constexpr (Tab::kHas && (PAGED || KF == DT_MXFP4)) {
    // Paged KV and MXFP4 KV: the first piece from the table, so its loads
    // (indices, query) go out without the kv_indptr search first.  With pages
    // of one row a piece's CSR rows are its kv_indices entries; with larger
    // pages the sequence's page list and first row come in one round trip.
    // MXFP4 tiles are not issued before the query: there the first tiles of
    // every workgroup together, not the search, bound the start.
    static_assert(QL == 1, "first-piece table: one query row");
    const uint32_t v = tab.first[gi];
    const int n_first = (int)(v & 0xffffu);
    const int b0 = (int)((v >> 16) & 0x3fffu);
    if (n_first > 0) {
      const int64_t s0 = (v >> 30) & 1u ? lo : lo - 1;  // only "before lo" matters below lo
      const int64_t e0 = (v >> 31) ? lo + n_first : hi + 1;
      PageSpan ps{lo, p.total_kv - lo, 0};
      if (PAGED && p.page_shift) {
        const int32_t s_raw = p.kv_indptr[b0], pb_raw = p.kv_page_indptr[b0], pe_raw = p.kv_page_indptr[b0 + 1];
        const int64_t s = uniform(s_raw), pb = uniform(pb_raw), pe = uniform(pe_raw);
        // a page list that cannot be read is read as empty (all pages 0)
        const bool ok = pb >= 0 && pe >= pb;
        ps = PageSpan{ok ? pb : 0, ok ? pe - pb : 0, (int32_t)(lo - s)};
      }
      split_piece<QF, KF, QL, CAP, PAGED, G1>(p, ring, xchg, pbuf, idxring, dtab,
                                          b0, 1, lo, n_first,
                                          piece_slot(s0, e0, lo, hi, gi), score_scale, out_scale, hi, (int32_t)(hi - lo),
                                          ps, false);
      lds_barrier();  // the next piece refills the ring
    }
    if (n_first == 0 || lo + n_first >= hi) return;
    b_first = b0 + 1;
    b_end = p.batch;  // pieces until one starts at or past hi
  } else if constexpr (Tab::kHas) {
    // Staged start: tile 0 of the first piece (which starts at lo) goes out at
    // once, then - with the piece's sequence from the table - that sequence's
    // query row into the ring's last slot, then tiles 1 .. NS - 2; the piece
    // waits for tile 0 and the query only.
    static_assert(!PAGED && QL == 1 && KF != DT_MXFP4, "staged start: one query row, contiguous bf16 / fp8 KV");
    using G = Geom<KF>;
    using DM = Dma<KF, PAGED>;
    constexpr int NS = RG::kStages;
    const int wd = uniform(tid >> 6), lane = tid & 63;
    const i32x4 rk = make_rsrc(p.kv + lo * G::kRow,
                               (uint32_t)std::min<uint64_t>((uint64_t)(p.total_kv - lo) * G::kRow, 0xFFFFF000ull));
    auto issue = [&](int t) {
#pragma unroll
      for (int k = 0; k < DM::kMaxChunksPerWave; ++k) {
        const int c = wd + DM::kWaves * k;
        if (c >= G::kRowChunks) break;
        dma16_first(rk, uniform(lds_addr(ring + (t % NS) * RG::kStageBytes + c * 1024)),
                    (uint32_t)(t * G::kRowBytes) + dma_src_offset<KF>(64 * c + lane));
      }
    };
    issue(0);
    const uint32_t v = tab.first[gi];
    const int n_first = (int)(v & 0xffffu);
    const int b0 = (int)((v >> 16) & 0x3fffu);
    if (n_first > 0) {
      constexpr uint32_t kQBytes = kHeads * kQK * (QF == DT_BF16 ? 2 : 1);
      const i32x4 rq = make_rsrc(p.q + (int64_t)b0 * kQBytes, kQBytes);
      for (int c = wd; c < (int)(kQBytes / 1024); c += DM::kWaves)
        dma16_first_cached(rq, uniform(lds_addr(ring + (NS - 1) * RG::kStageBytes + c * 1024)), (uint32_t)(c * 1024 + 16 * lane));
      for (int t = 1; t < NS - 1; ++t) issue(t);
      const int64_t s0 = (v >> 30) & 1u ? lo : lo - 1;  // only "before lo" matters below lo
      const int64_t e0 = (v >> 31) ? lo + n_first : hi + 1;
      split_piece<QF, KF, QL, CAP, PAGED, G1>(p, ring, xchg, pbuf, idxring, dtab,
                                          b0, 1, lo, n_first,
                                          piece_slot(s0, e0, lo, hi, gi), score_scale, out_scale, hi, (int32_t)(hi - lo),
                                          PageSpan{lo, p.total_kv - lo, 0}, true);
      lds_barrier();  // the next piece refills the ring
    }
    wait_vmcnt<0>();  // nothing staged is still landing in LDS (a piece shorter than the ring)
    if (n_first == 0 || lo + n_first >= hi) return;
    b_first = b0 + 1;
    b_end = p.batch;  // pieces until one starts at or past hi
  } else {
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
    b_first = uniform(counts[0]);
    b_end = uniform(counts[1]);
  }

  for (int b = b_first; b < b_end; ++b) {
    // the loads are independent; issue them together
    const int32_t s_raw = p.kv_indptr[b], e_raw = p.kv_indptr[b + 1], q_raw = p.qo_indptr[b];
    int32_t qe_raw = 0;
    if constexpr (QL > 1) qe_raw = p.qo_indptr[b + 1];
    const int64_t s = uniform(s_raw);
    const int64_t e = uniform(e_raw);
    if (Tab::kHas && s >= hi) break;
    const int64_t qrow0 = std::min(std::max(uniform(q_raw), 0), p.total_q - 1);
    int nq = 1;
    if constexpr (QL > 1) {
      // query rows of the sequence, at most QL and inside the q buffer
      nq = (int)std::min<int64_t>(std::min<int64_t>(std::max<int64_t>((int64_t)uniform(qe_raw) - uniform(q_raw), 0), QL),
                                  p.total_q - qrow0);
      if (nq <= 0) continue;
    }
    const int64_t r0 = std::max(s, lo), r1 = std::min(e, hi);
    if (r0 >= r1) continue;
    const int32_t slot = piece_slot(s, e, lo, hi, gi);
    PageSpan ps{r0, p.total_kv - r0, 0};
    if (PAGED && p.page_shift) {
      const int32_t pb_raw = p.kv_page_indptr[b], pe_raw = p.kv_page_indptr[b + 1];
      const int64_t pb = uniform(pb_raw), pe = uniform(pe_raw);
      // a page list that cannot be read is read as empty (all pages 0)
      const bool ok = pb >= 0 && pe >= pb;
      ps = PageSpan{ok ? pb : 0, ok ? pe - pb : 0, (int32_t)(r0 - s)};
    }
    split_piece<QF, KF, QL, CAP, PAGED, G1>(p, ring, xchg, pbuf, idxring, dtab, qrow0, nq,
                            r0, (int)(r1 - r0), slot, score_scale, out_scale, hi, (int32_t)(hi - lo), ps, false);
    lds_barrier();  // the next piece refills the ring
  }
}

// ---------------------------------------------------------------- stage 2

struct MergeParams {
  const uint16_t* part_o;
  const float* part_lse;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  uint16_t* out;
  int64_t total_kv;
  int32_t total_q;
  Cut cut;
};

// One workgroup of two waves per (sequence, query token, pair of heads); wave w
// takes head 2j + w and its lane i columns 8i..8i+7 (16-byte loads).  The
// log-sum-exps and partial outputs of up to NB slots are loaded together (none
// depends on another), then combined with a running maximum, so a sequence of
// up to NB pieces costs one round trip to memory after the index loads.  With
// the host offsets the plan knows the most pieces any sequence has and picks
// the smallest NB of 2, 4, 8 and 16 that holds them (a batch issues a load for
// every one of its NB slots, and the wide batch holds twice the registers);
// otherwise NB is kMergeBatch.  Partial slot s holds QL query tokens: O at
// ((s * QL + t) * 16 + h) * 512, LSE at (s * QL + t) * 16 + h.
constexpr int kMergeBatch = 8;

// Range positions g0..g1 of every sequence, derived by the planner from the
// host kv_indptr and passed with the kernel arguments (read in parallel with
// them, where the offsets would be one more dependent load); g1 < g0 marks a
// sequence with no rows.  Used when the plan knows the offsets, the batch
// fits and G < 2^16.
constexpr int kMergeTable = 512;
struct MergeTable {
  static constexpr bool kHas = true;
  uint32_t g01[kMergeTable];  // g0 | g1 << 16: one scalar load per sequence
};
struct NoMergeTable {
  static constexpr bool kHas = false;
};

template <typename Tab, int QL, int NB>
__global__ __launch_bounds__(128) void mla_merge_kernel(MergeParams p, Tab tab) {
  // two heads per workgroup: wave w of head 2 (blockIdx & 7) + w, 8 columns per lane
  const int bt = blockIdx.x >> 3, h = 2 * (blockIdx.x & 7) + (threadIdx.x >> 6);
  const int b = bt / QL, tq = bt % QL;
  const int t = threadIdx.x & 63;
  int64_t qrow;
  if constexpr (QL == 1) {
    qrow = std::min(std::max(p.qo_indptr[b], 0), p.total_q - 1);
  } else {
    const int32_t q0 = p.qo_indptr[b], q1 = p.qo_indptr[b + 1];
    qrow = (int64_t)q0 + tq;
    // the same query rows stage 1 takes: at most QL, inside the q buffer
    if (tq >= (int64_t)q1 - q0 || q0 < 0 || qrow >= p.total_q) return;
  }
  uint16_t* o = p.out + (qrow * kHeads + h) * kV + 8 * t;
  int32_t g0, g1;
  if constexpr (Tab::kHas) {
    const uint32_t v = tab.g01[b];
    // the output row is needed only by the final store: have its load complete
    // together with the table read rather than after the merge
    if constexpr (QL == 1) asm volatile("" ::"s"((int32_t)qrow), "s"(v));
    g0 = (int32_t)(v & 0xffffu);
    g1 = (int32_t)(v >> 16);
  } else {
    const int64_t s = std::max<int64_t>(p.kv_indptr[b], 0);
    const int64_t e = std::min<int64_t>(p.kv_indptr[b + 1], p.total_kv);
    g0 = p.cut.pos_of_row(s);
    g1 = e > s ? p.cut.pos_of_row(e - 1) : g0 - 1;
  }
  if (g1 < g0) {  // no KV rows: the softmax is empty, the output is zero
    *(u32x4*)o = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  if (g0 == g1) return;  // written by stage 1
  // Every weight is taken against the largest LSE of the sequence: a sequence
  // of more than NB slots first reads every LSE for it, one of at most NB
  // slots finds it in its only batch.  With the products added by explicit
  // fused multiply-adds in slot order, the output does not depend on the batch
  // size (slots past g1 add exact zeros).
  float m_run = -INFINITY, wsum = 0.f;
  if (g1 - g0 >= NB)
    for (int32_t base = g0; base <= g1; base += NB) {
      float lse[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k)
        lse[k] = p.part_lse[((int64_t)merge_slot(p.cut, std::min(base + k, g1), g0) * QL + tq) * kHeads + h];
#pragma unroll
      for (int k = 0; k < NB; ++k) m_run = fmaxf(m_run, lse[k]);
    }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = acc;
  for (int32_t base = g0; base <= g1; base += NB) {
    // straight-line loads (slots past g1 re-read slot g1 and get weight 0), so
    // that they are all in flight before the first is used; the partials are
    // read once, non-temporal (0.2-1 us faster per call than cached loads)
    float lse[NB];
    u32x4 u[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int64_t slot = (int64_t)merge_slot(p.cut, std::min(base + k, g1), g0) * QL + tq;
      lse[k] = p.part_lse[slot * kHeads + h];
      u[k] = __builtin_nontemporal_load((const u32x4*)(p.part_o + (slot * kHeads + h) * kV + 8 * t));
    }
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (base + k > g1) lse[k] = -INFINITY;
    f32x4 v[NB], v2[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      v[k] = f32x4{bf_lo(u[k][0]), bf_hi(u[k][0]), bf_lo(u[k][1]), bf_hi(u[k][1])};
      v2[k] = f32x4{bf_lo(u[k][2]), bf_hi(u[k][2]), bf_lo(u[k][3]), bf_hi(u[k][3])};
    }
    float mx = m_run;
#pragma unroll
    for (int k = 0; k < NB; ++k) mx = fmaxf(mx, lse[k]);
    // only empty slices (mx = -inf): every weight is 0, with no branch (a
    // branch here lets the compiler hold the partial loads back until the
    // maxima are known)
    const float mref = mx == -INFINITY ? 0.f : mx;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float wgt = (lse[k] == -INFINITY) ? 0.f : __expf(lse[k] - mref);
      wsum += wgt;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] = __builtin_fmaf(wgt, v[k][c], acc[c]);
        acc2[c] = __builtin_fmaf(wgt, v2[k][c], acc2[c]);
      }
    }
    m_run = mx;
  }
  const float inv = 1.f / wsum;
  *(u32x4*)o = u32x4{pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv),
                     pack_bf16x2(acc2.x * inv, acc2.y * inv), pack_bf16x2(acc2.z * inv, acc2.w * inv)};
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
    const bf16x8 d = fp4x8_bf16(w, e8m0_scale(scales[row * kScaleRow + c0 / 32]));
    for (int k = 0; k < 8; ++k) out[row * kQK + c0 + k] = (float)d[k];
  } else {
    if (i >= n) return;
    out[i] = __builtin_bit_cast(float, (uint32_t)((const uint16_t*)codes)[i] << 16);
  }
}

// ---------------------------------------------------------------- read ceiling

// Streams a buffer with 16-byte non-temporal loads: each workgroup reads its
// own contiguous share, 4 KB per load instruction of its 256 threads and four
// in flight (measured 6.8-7.1 TB/s over 1 GiB, against 5.9 TB/s for a grid
// stride, where consecutive workgroups read adjacent 4 KB blocks).  It folds
// what it reads into one word that is stored only if it equals a value no
// sane input produces (so the loads cannot be removed).
__global__ __launch_bounds__(256) void mla_debug_stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                                    uint32_t* sink) {
  const int64_t share = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * share, hi = std::min<int64_t>(lo + share, n16);
  u32x4 acc = {0, 0, 0, 0};
  int64_t i = lo + threadIdx.x;
  for (; i + 3 * 256 < hi; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + 256);
    const u32x4 c = __builtin_nontemporal_load(p + i + 512), d = __builtin_nontemporal_load(p + i + 768);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < hi; i += 256) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = acc.x;
}

// The read that stage 1's memory side does, with no arithmetic: each workgroup
// streams its contiguous share of whole 18 KB tiles (fp8 geometry) through the
// same four-slot LDS ring by the same 16-byte LDS DMA, chunks dealt round robin
// to the four waves, NS - 2 tiles kept in flight, two workgroup barriers per
// tile and the refill issued after the second; two workgroups per CU, like the
// fp8 kernel.  Each tile is touched once in LDS.
__global__ __launch_bounds__(Geom<DT_FP8>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_debug_stream_ring_kernel(const uint8_t* buf, int64_t tiles, uint32_t* sink) {
  using G = Geom<DT_FP8>;
  using DM = Dma<DT_FP8, false>;
  constexpr int NS = RingCfg<DT_FP8, 1>::kStages;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * G::kStageBytes];
  const int wd = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t t0 = tiles * blockIdx.x / gridDim.x, t1 = tiles * (blockIdx.x + 1) / gridDim.x;
  const int n = (int)(t1 - t0);
  if (n <= 0) return;
  const i32x4 r = make_rsrc(buf + t0 * G::kStageBytes, (uint32_t)((int64_t)n * G::kStageBytes));
  auto issue = [&](int t) {
#pragma unroll
    for (int k = 0; k < DM::kMaxChunksPerWave; ++k) {
      const int c = wd + DM::kWaves * k;
      if (c >= G::kRowChunks) break;
      dma16(r, uniform(lds_addr(ring + (t % NS) * G::kStageBytes + c * 1024)),
            (uint32_t)(t * G::kRowBytes) + dma_src_offset<DT_FP8>(64 * c + lane));
    }
  };
  const int my_chunks = DM::chunks_of_wave(wd);
  for (int t = 0; t < NS - 1 && t < n; ++t) issue(t);
  uint32_t acc = 0;
  for (int i = 0; i < n; ++i) {
    if (i + NS - 2 < n)
      wait_tiles_behind_fixed<DM::kMaxChunksPerWave, NS - 2>(my_chunks);
    else
      wait_tiles_behind<DM::kMaxChunksPerWave>(my_chunks, n - 1 - i);
    lds_barrier();
    acc ^= *(const uint32_t*)(ring + (i % NS) * G::kStageBytes + 1024 * wd + 16 * lane);
    lds_barrier();
    if (i + NS - 1 < n) issue(i + NS - 1);
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace mla

// ==================================================================== host

using namespace mla;

// Workspace of mla_decode_run_noalloc: one static array per device, allocated
// when the code object loads and held until the process ends.  34 MiB covers
// the partial slots of every plan the planner makes by default on a 256-CU
// part (at most 2 * 768 slots of one query row, or 2 * 512 of two, or 2 * 256
// of four, plus their log-sum-exps) unless total_kv passes about 2.7e8 rows.
// Host code never names it except to look up its device address.
constexpr size_t kScratchBytes = size_t(34) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct mla_plan {
  mla_problem prob;
  Cut cut;  // workgroup ranges: G = cut.G workgroups
  int32_t num_wgs;
  int32_t stages;
  int32_t lds_bytes;
  int32_t stage2;
  int32_t num_cus;
  int32_t wgs_per_cu;
  int32_t ql;  // query tokens per sequence a stage-1 workgroup holds (1, 2 or 4)
  size_t ws_bytes;
  size_t lse_offset;
  bool has_table;  // merge ranges known at plan time (host kv_indptr, batch and G small enough)
  MergeTable table;
  int32_t merge_batch;  // slots stage 2 loads at once (see mla_merge_kernel)
  bool has_split_table;  // each workgroup's first piece known at plan time (staged start)
  SplitTable split_table;
};

namespace {

thread_local char g_last_error[256] = "";

mla_status hip_fail(hipError_t e, const char* what) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return MLA_ERR_HIP;
}

struct RingInfo {
  int stages, lds_bytes, wgs_per_cu;
};

template <int KF, int QL, bool PAGED>
constexpr RingInfo ring_info() {
  return RingInfo{Ring<KF, QL, PAGED>::kStages, Ring<KF, QL, PAGED>::kTotal, Ring<KF, QL, PAGED>::kWgsPerCu};
}

template <int QL>
RingInfo ring_info_for(int kv_dtype, bool paged) {
  switch (kv_dtype) {
    case DT_BF16: return paged ? ring_info<DT_BF16, QL, true>() : ring_info<DT_BF16, QL, false>();
    case DT_FP8: return paged ? ring_info<DT_FP8, QL, true>() : ring_info<DT_FP8, QL, false>();
    default: return paged ? ring_info<DT_MXFP4, QL, true>() : ring_info<DT_MXFP4, QL, false>();
  }
}

RingInfo ring_info_for(int kv_dtype, int ql, bool paged) {
  return ql == 1 ? ring_info_for<1>(kv_dtype, paged)
                 : ql == 2 ? ring_info_for<2>(kv_dtype, paged) : ring_info_for<4>(kv_dtype, paged);
}

// Per mille of R moved to the first workgroup on each CU when there are more
// workgroups than CUs (see Cut).  Swept with the non-temporal KV loads: 120
// against 80 / 100 / 150 ran bs 256 in 183.9 against 187.5 / 184.6 / 188.0 us
// per call, bs 64 within 0.3 us.
constexpr int kDefaultAgeSkew = 120;

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

template <int QF, int KF, bool CAP, bool PAGED, bool G1>
void launch_split_v(const mla_plan* pl, const SplitParams& sp, hipStream_t st) {
  const dim3 grid(pl->num_wgs), block(Geom<KF>::kThreads * (pl->ql == 4 ? RowSplit<4>::kGroups : 1));
  {
    if (pl->ql == 1 && pl->has_split_table) {
      hipLaunchKernelGGL((mla_split_kernel<QF, KF, 1, CAP, PAGED, SplitTable, G1>), grid, block, 0, st, sp,
                         pl->split_table);
      return;
    }
  }
  if (pl->ql == 1)
    hipLaunchKernelGGL((mla_split_kernel<QF, KF, 1, CAP, PAGED, NoSplitTable, G1>), grid, block, 0, st, sp, NoSplitTable{});
  else if (pl->ql == 2)
    hipLaunchKernelGGL((mla_split_kernel<QF, KF, 2, CAP, PAGED, NoSplitTable, G1>), grid, block, 0, st, sp, NoSplitTable{});
  else
    hipLaunchKernelGGL((mla_split_kernel<QF, KF, 4, CAP, PAGED, NoSplitTable, G1>), grid, block, 0, st, sp, NoSplitTable{});
}

template <int QF, int KF, bool PAGED, bool G1>
void launch_split_c(const mla_plan* pl, const SplitParams& sp, hipStream_t st) {
  if (pl->prob.logit_cap > 0.f)
    launch_split_v<QF, KF, true, PAGED, G1>(pl, sp, st);
  else
    launch_split_v<QF, KF, false, PAGED, G1>(pl, sp, st);
}

template <int QF, int KF, bool PAGED>
void launch_split_p(const mla_plan* pl, const SplitParams& sp, hipStream_t st) {
  if constexpr (PAGED && KF == DT_MXFP4) {
    if (pl->prob.kv_paged == 1) {
      launch_split_c<QF, KF, PAGED, true>(pl, sp, st);
      return;
    }
  }
  launch_split_c<QF, KF, PAGED, false>(pl, sp, st);
}

template <int QF, int KF>
hipError_t launch_split(const mla_plan* pl, const SplitParams& sp, hipStream_t st) {
  if (pl->prob.kv_paged)
    launch_split_p<QF, KF, true>(pl, sp, st);
  else
    launch_split_p<QF, KF, false>(pl, sp, st);
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
  // sm_scale must be finite and positive (the kernel takes the maximum score as
  // sm_scale times the maximum dot product)
  if (pr->batch_size < 1 || pr->total_kv < 0 || pr->total_kv > INT32_MAX || !(pr->sm_scale > 0.f) ||
      !(pr->sm_scale < INFINITY))
    return MLA_ERR_INVALID_ARG;
  if (pr->num_heads != kHeads || pr->qk_dim != kQK || pr->v_dim != kV) return MLA_ERR_UNSUPPORTED;
  // query rows per sequence: one, or up to max_q_len (2 or 4 kernels; 3 runs on the 4-token one)
  if (pr->max_q_len < 0 || pr->max_q_len > 4) return MLA_ERR_UNSUPPORTED;
  if (!(pr->logit_cap >= 0.f) || !(pr->logit_cap < INFINITY)) return MLA_ERR_INVALID_ARG;
  // 0: contiguous; P = 2^k in [1, 65536]: paged with pages of P rows
  if (pr->kv_paged < 0 || pr->kv_paged > 65536 || (pr->kv_paged & (pr->kv_paged - 1))) return MLA_ERR_INVALID_ARG;
  const int ql = pr->max_q_len <= 1 ? 1 : pr->max_q_len == 2 ? 2 : 4;
  if (ql == 1 && pr->total_q != pr->batch_size) return MLA_ERR_UNSUPPORTED;  // one query token per sequence
  if (ql > 1 && (pr->total_q < 1 || (int64_t)pr->total_q > (int64_t)pr->batch_size * pr->max_q_len))
    return MLA_ERR_INVALID_ARG;
  if (pr->q_dtype != DT_BF16 && pr->q_dtype != DT_FP8) return MLA_ERR_UNSUPPORTED;
  if (pr->kv_dtype != DT_BF16 && pr->kv_dtype != DT_FP8 && pr->kv_dtype != DT_MXFP4) return MLA_ERR_UNSUPPORTED;
  if (opt && (opt->rows_per_split < 0 || opt->wgs_per_cu < 0 || opt->age_skew < -1 || opt->age_skew > 500 ||
              opt->xcd_group < -1 || opt->xcd_group > 64))
    return MLA_ERR_INVALID_ARG;

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
  const RingInfo ri = ring_info_for(pr->kv_dtype, ql, pr->kv_paged != 0);
  const int wpc = (opt && opt->wgs_per_cu > 0) ? opt->wgs_per_cu : ri.wgs_per_cu;
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
  // With more workgroups than CUs, the first one on each CU (the first num_cus
  // dispatched) takes `skew` per mille of R more rows and the later ones fewer,
  // in whole tiles, so that the later ones - which the SIMD arbiter serves
  // second - finish with it.
  Cut cut{R, R, 0, (int32_t)G, 0};
  const int skew = opt && opt->age_skew != 0 ? opt->age_skew : kDefaultAgeSkew;
  if (skew > 0 && G == 2 * (int64_t)num_cus) {
    const int64_t d = (R * skew / 1000 + kTile / 2) / kTile * kTile;
    if (d > 0 && d < R) {
      const int grp = opt && opt->xcd_group > 0 ? opt->xcd_group : 0;
      cut = Cut{R + d, R - d, num_cus, (int32_t)G, grp > 0 && num_cus % (8 * grp) == 0 ? grp : 0};
    }
  }

  bool stage2 = true;
  if (kv_indptr_host) {
    stage2 = false;
    for (int b = 0; b < pr->batch_size && !stage2; ++b) {
      const int64_t s = kv_indptr_host[b], e = kv_indptr_host[b + 1];
      if (e <= s || cut.pos_of_row(s) != cut.pos_of_row(e - 1)) stage2 = true;
    }
  }

  mla_plan* pl = new (std::nothrow) mla_plan;
  if (!pl) return MLA_ERR_INVALID_ARG;
  pl->prob = *pr;
  pl->prob.num_cus = num_cus;
  pl->cut = cut;
  pl->num_wgs = (int32_t)G;
  pl->stages = ri.stages;
  pl->lds_bytes = ri.lds_bytes;
  pl->ql = ql;
  pl->stage2 = stage2 ? 1 : 0;
  pl->num_cus = num_cus;
  pl->wgs_per_cu = wpc;
  const size_t slots = 2 * (size_t)G;
  const size_t o_bytes = slots * ql * kHeads * kV * sizeof(uint16_t);
  pl->lse_offset = (o_bytes + 255) / 256 * 256;
  pl->has_table = kv_indptr_host && pr->batch_size <= kMergeTable && G < 65536;
  int64_t max_pieces = 0;  // the most pieces of one sequence (with the table)
  if (pl->has_table) {
    for (int b = 0; b < pr->batch_size; ++b) {
      const int64_t s = std::max<int64_t>(kv_indptr_host[b], 0);
      const int64_t e = std::min<int64_t>(kv_indptr_host[b + 1], total);
      const int64_t g0 = cut.pos_of_row(s);
      const int64_t g1 = e > s ? cut.pos_of_row(e - 1) : g0 - 1;
      // empty: g0 = 1 > g1 = 0
      pl->table.g01[b] = g1 < g0 ? 1u : (uint32_t)g0 | ((uint32_t)g1 << 16);
      max_pieces = std::max<int64_t>(max_pieces, g1 - g0 + 1);
    }
  }
  pl->merge_batch = !pl->has_table ? kMergeBatch : max_pieces <= 2 ? 2 : max_pieces <= 4 ? 4 : max_pieces <= 8 ? 8 : 16;
  pl->ws_bytes = pl->lse_offset + (slots * ql * kHeads * sizeof(float) + 255) / 256 * 256;
  // First-piece table (one query row): each workgroup's
  // first piece from the host offsets, found by the kernel's own counting rule.
  pl->has_split_table = kv_indptr_host && ql == 1 &&
                        kv_indptr_host[0] == 0 && G <= kSplitTable && pr->batch_size <= (1 << 14) && cut.ra < (1 << 16);
  if (pl->has_split_table) {
    const int32_t* ind = kv_indptr_host;
    for (int64_t g = 0; g < G; ++g) {
      const int32_t pos = cut.pos_of((int32_t)g);
      const int64_t lo = cut.lo_at(pos), hi = std::min(cut.lo_at(pos + 1), total);
      int b = 0;  // first sequence with ind[b + 1] > lo
      for (int lo_b = 0, hi_b = pr->batch_size; lo_b < hi_b;) {
        const int mid = (lo_b + hi_b) / 2;
        if (ind[mid + 1] <= lo) lo_b = b = mid + 1; else hi_b = mid;
      }
      uint32_t v = 0;  // no rows of any sequence
      if (b < pr->batch_size && lo < ind[pr->batch_size]) {
        const int64_t s = ind[b], e = ind[b + 1];  // s <= lo < e
        v = (uint32_t)(std::min(e, hi) - lo) | ((uint32_t)b << 16) | ((s == lo ? 1u : 0u) << 30) |
            ((e <= hi ? 1u : 0u) << 31);
      }
      pl->split_table.first[g] = v;
    }
  }
  *plan_out = pl;
  if (workspace_bytes) *workspace_bytes = pl->ws_bytes;
  return MLA_OK;
}

void mla_decode_plan_destroy(mla_plan* plan) { delete plan; }

mla_status mla_decode_plan_describe(const mla_plan* pl, mla_plan_desc* d) {
  if (!pl || !d) return MLA_ERR_INVALID_ARG;
  d->num_splits = pl->num_wgs;
  d->rows_per_split = (int32_t)pl->cut.ra;
  d->paired_splits = pl->cut.first;
  d->second_rows_per_split = (int32_t)pl->cut.rb;
  d->xcd_group = pl->cut.grp;
  d->merge_batch = pl->merge_batch;
  d->first_piece_table = pl->has_split_table ? 1 : 0;
  d->tile_rows = kTile;
  d->stages = pl->stages;
  d->partial_slots = 2 * pl->num_wgs;
  d->stage2 = pl->stage2;
  d->workspace_bytes = (int64_t)pl->ws_bytes;
  d->lds_bytes = pl->lds_bytes;
  d->num_cus = pl->num_cus;
  d->wgs_per_cu = pl->wgs_per_cu;
  d->query_tokens = pl->ql;
  return MLA_OK;
}

mla_status mla_decode_plan_pieces(const mla_plan* pl, const int32_t* ind, int64_t* rec, int64_t cap, int64_t* count) {
  if (!pl || !ind || !count || cap < 0 || (cap > 0 && !rec)) return MLA_ERR_INVALID_ARG;
  const int bs = pl->prob.batch_size;
  const int64_t total = pl->prob.total_kv;
  int64_t n = 0;
  for (int32_t g = 0; g < pl->num_wgs; ++g) {
    const int32_t pos = pl->cut.pos_of(g);
    const int64_t lo = pl->cut.lo_at(pos), hi = std::min(pl->cut.lo_at(pos + 1), total);
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
  const int32_t g0 = pl->cut.pos_of_row(s);
  const int32_t g1 = pl->cut.pos_of_row(e - 1);
  if (g0 == g1) return MLA_OK;
  int32_t n = 0;
  for (int32_t pos = g0; pos <= g1; ++pos, ++n)
    if (n < cap) slots[n] = merge_slot(pl->cut, pos, g0);
  *count = n;
  return MLA_OK;
}

namespace {

// Validates the run arguments and fills the kernel parameter blocks.
// kv_indices / kv_rows / kv_page_indptr: the paged entry points (kv_indices
// != NULL) with a paged plan, the others (NULL) with a contiguous one; the page
// lists (kv_page_indptr) with pages of more than one row only.
mla_status prepare(const mla_plan* pl, const void* q, const float* q_scale, const void* kv, const void* kv_scale,
                   const int32_t* kv_indices, int64_t kv_rows, const int32_t* kv_page_indptr,
                   const int32_t* qo_indptr, const int32_t* kv_indptr, void* out, void* workspace,
                   size_t workspace_bytes, SplitParams* sp, MergeParams* mp) {
  if (!pl || !q || !kv || !qo_indptr || !kv_indptr || !out) return MLA_ERR_INVALID_ARG;
  const mla_problem& pr = pl->prob;
  if ((kv_indices != nullptr) != (pr.kv_paged != 0)) return MLA_ERR_INVALID_ARG;
  if ((kv_page_indptr != nullptr) != (pr.kv_paged > 1)) return MLA_ERR_INVALID_ARG;
  if (kv_page_indptr && ((uintptr_t)kv_page_indptr & 3u)) return MLA_ERR_INVALID_ARG;
  if (kv_indices) {
    const int64_t row_bytes = pr.kv_dtype == DT_BF16 ? 2 * kQK : pr.kv_dtype == DT_FP8 ? kQK : kQK / 2;
    if (((uintptr_t)kv_indices & 3u) || kv_rows < 1) return MLA_ERR_INVALID_ARG;
    if (kv_rows > (int64_t)0xFFFFF000 / row_bytes) return MLA_ERR_UNSUPPORTED;  // 32-bit row offsets
  }
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
  sp->part_o = (uint16_t*)workspace;
  sp->part_lse = (float*)((uint8_t*)workspace + pl->lse_offset);
  sp->total_kv = pr.total_kv;
  sp->total_q = pr.total_q;
  sp->batch = pr.batch_size;
  sp->cut = pl->cut;
  sp->sm_scale = pr.sm_scale;
  sp->logit_cap = pr.logit_cap;
  sp->kv_indices = kv_indices;
  sp->kv_rows = kv_rows;
  sp->kv_page_indptr = kv_page_indptr;
  sp->page_shift = pr.kv_paged > 1 ? __builtin_ctz((unsigned)pr.kv_paged) : 0;
  mp->part_o = sp->part_o;
  mp->part_lse = sp->part_lse;
  mp->qo_indptr = qo_indptr;
  mp->kv_indptr = kv_indptr;
  mp->out = sp->out;
  mp->total_kv = pr.total_kv;
  mp->total_q = pr.total_q;
  mp->cut = pl->cut;
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

extern "C++" {
template <int QL>
void launch_merge_nb(const mla_plan* pl, const MergeParams& mp, hipStream_t st) {
  const dim3 grid(pl->prob.batch_size * pl->ql * kHeads / 2), block(128);
  switch (pl->merge_batch) {
    case 2: hipLaunchKernelGGL((mla_merge_kernel<MergeTable, QL, 2>), grid, block, 0, st, mp, pl->table); break;
    case 4: hipLaunchKernelGGL((mla_merge_kernel<MergeTable, QL, 4>), grid, block, 0, st, mp, pl->table); break;
    case 16: hipLaunchKernelGGL((mla_merge_kernel<MergeTable, QL, 16>), grid, block, 0, st, mp, pl->table); break;
    default: hipLaunchKernelGGL((mla_merge_kernel<MergeTable, QL, kMergeBatch>), grid, block, 0, st, mp, pl->table); break;
  }
}
}  // extern "C++"

mla_status launch_merge_stage(const mla_plan* pl, const MergeParams& mp, hipStream_t st) {
  if (!pl->stage2) return MLA_OK;
  if (pl->has_table) {
    if (pl->ql == 1)
      launch_merge_nb<1>(pl, mp, st);
    else if (pl->ql == 2)
      launch_merge_nb<2>(pl, mp, st);
    else
      launch_merge_nb<4>(pl, mp, st);
  } else {
    const dim3 grid(pl->prob.batch_size * pl->ql * kHeads / 2), block(128);
    if (pl->ql == 1)
      hipLaunchKernelGGL((mla_merge_kernel<NoMergeTable, 1, kMergeBatch>), grid, block, 0, st, mp, NoMergeTable{});
    else if (pl->ql == 2)
      hipLaunchKernelGGL((mla_merge_kernel<NoMergeTable, 2, kMergeBatch>), grid, block, 0, st, mp, NoMergeTable{});
    else
      hipLaunchKernelGGL((mla_merge_kernel<NoMergeTable, 4, kMergeBatch>), grid, block, 0, st, mp, NoMergeTable{});
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : hip_fail(e, "launching the merge kernel");
}

}  // namespace

mla_status mla_decode_run(const mla_plan* pl, const void* q, const float* q_scale, const void* kv,
                          const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  SplitParams sp;
  MergeParams mp;
  mla_status s = prepare(pl, q, q_scale, kv, kv_scale, nullptr, 0, nullptr, qo_indptr, kv_indptr, out, workspace,
                         workspace_bytes, &sp, &mp);
  if (s != MLA_OK) return s;
  s = launch_split_stage(pl, sp, (hipStream_t)stream);
  if (s != MLA_OK) return s;
  return launch_merge_stage(pl, mp, (hipStream_t)stream);
}

mla_status mla_decode_run_paged(const mla_plan* pl, const void* q, const float* q_scale, const void* kv,
                                const void* kv_scale, int64_t kv_rows, const int32_t* kv_indices,
                                const int32_t* kv_page_indptr, const int32_t* qo_indptr, const int32_t* kv_indptr,
                                void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv_indices) return MLA_ERR_INVALID_ARG;
  SplitParams sp;
  MergeParams mp;
  mla_status s = prepare(pl, q, q_scale, kv, kv_scale, kv_indices, kv_rows, kv_page_indptr, qo_indptr, kv_indptr,
                         out, workspace, workspace_bytes, &sp, &mp);
  if (s != MLA_OK) return s;
  s = launch_split_stage(pl, sp, (hipStream_t)stream);
  if (s != MLA_OK) return s;
  return launch_merge_stage(pl, mp, (hipStream_t)stream);
}

mla_status mla_decode_split_paged(const mla_plan* pl, const void* q, const float* q_scale, const void* kv,
                                  const void* kv_scale, int64_t kv_rows, const int32_t* kv_indices,
                                  const int32_t* kv_page_indptr, const int32_t* qo_indptr, const int32_t* kv_indptr,
                                  void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv_indices) return MLA_ERR_INVALID_ARG;
  SplitParams sp;
  MergeParams mp;
  mla_status s = prepare(pl, q, q_scale, kv, kv_scale, kv_indices, kv_rows, kv_page_indptr, qo_indptr, kv_indptr,
                         out, workspace, workspace_bytes, &sp, &mp);
  if (s != MLA_OK) return s;
  return launch_split_stage(pl, sp, (hipStream_t)stream);
}

mla_status mla_decode_split(const mla_plan* pl, const void* q, const float* q_scale, const void* kv,
                            const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  SplitParams sp;
  MergeParams mp;
  mla_status s = prepare(pl, q, q_scale, kv, kv_scale, nullptr, 0, nullptr, qo_indptr, kv_indptr, out, workspace,
                         workspace_bytes, &sp, &mp);
  if (s != MLA_OK) return s;
  return launch_split_stage(pl, sp, (hipStream_t)stream);
}

mla_status mla_decode_merge(const mla_plan* pl, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!pl || !qo_indptr || !kv_indptr || !out || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < pl->ws_bytes || (pl->ws_bytes && (!workspace || !aligned16(workspace))))
    return MLA_ERR_INVALID_ARG;
  MergeParams mp;
  mp.part_o = (const uint16_t*)workspace;
  mp.part_lse = (const float*)((const uint8_t*)workspace + pl->lse_offset);
  mp.qo_indptr = qo_indptr;
  mp.kv_indptr = kv_indptr;
  mp.out = (uint16_t*)out;
  mp.total_kv = pl->prob.total_kv;
  mp.total_q = pl->prob.total_q;
  mp.cut = pl->cut;
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

namespace {

// Device address of `scratch` per device, looked up once per device (with that
// device current) on the first mla_decode_run_noalloc call there.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mla_status scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "querying the current device");
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_last_error, sizeof g_last_error, "device %d: at most %d devices are supported", dev, kMaxDevices);
    return MLA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "looking up the static workspace");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_run_noalloc(const mla_plan* pl, const void* q, const float* q_scale, const void* kv,
                                  const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                                  void* stream) {
  if (!pl) return MLA_ERR_INVALID_ARG;
  if (pl->ws_bytes > kScratchBytes) {
    snprintf(g_last_error, sizeof g_last_error,
             "the plan needs %zu bytes of workspace; mla_decode_run_noalloc has %zu (use mla_decode_run)",
             pl->ws_bytes, kScratchBytes);
    return MLA_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  mla_status s = scratch_address(&ws);
  if (s != MLA_OK) return s;
  return mla_decode_run(pl, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, out, ws, kScratchBytes, stream);
}

mla_status mla_debug_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 0 || (bytes & 15) || ((uintptr_t)buf & 15)) return MLA_ERR_INVALID_ARG;
  if (bytes == 0) return MLA_OK;
  hipLaunchKernelGGL(mla_debug_stream_read_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf,
                     bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : hip_fail(e, "launching the read-ceiling kernel");
}

mla_status mla_debug_stream_ring(const void* buf, int64_t bytes, int32_t wgs, uint32_t* sink, void* stream) {
  constexpr int64_t kTileBytes = Geom<DT_FP8>::kStageBytes;
  if (!buf || !sink || bytes < 0 || bytes % kTileBytes || ((uintptr_t)buf & 15) || wgs < 1 ||
      bytes / kTileBytes / wgs > (0xFFFFF000ll / kTileBytes))
    return MLA_ERR_INVALID_ARG;
  if (bytes == 0) return MLA_OK;
  hipLaunchKernelGGL(mla_debug_stream_ring_kernel, dim3(wgs), dim3(Geom<DT_FP8>::kThreads), 0, (hipStream_t)stream,
                     (const uint8_t*)buf, bytes / kTileBytes, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : hip_fail(e, "launching the ring-read kernel");
}

mla_status mla_debug_wg_trace(uint64_t* host, int64_t n, int32_t clear) {
#ifdef MLA_WG_TRACE
  if (n < 0 || n > (int64_t)kWgTraceMax * 4 || (n > 0 && !host)) return MLA_ERR_INVALID_ARG;
  hipError_t e = hipSuccess;
  if (clear) {
    static uint64_t zeros[kWgTraceMax * 4];
    e = hipMemcpyToSymbol(HIP_SYMBOL(mla::g_wg_trace), zeros, sizeof zeros);
  }
  if (e == hipSuccess && n > 0) e = hipMemcpyFromSymbol(host, HIP_SYMBOL(mla::g_wg_trace), (size_t)n * 8);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "copying the workgroup timeline");
#else
  (void)host;
  (void)n;
  (void)clear;
  snprintf(g_last_error, sizeof g_last_error, "built without MLA_WG_TRACE (see mla_decode_split_amd/build.py)");
  return MLA_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
