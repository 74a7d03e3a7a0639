/*
 * mla_decode.h - C ABI of the MLA decode library for AMD Instinct MI355X (gfx950).
 *
 * The operation is DeepSeek-R1 forward_absorb Multi-head Latent Attention
 * decode as the kernelbot-amd-mixed-mla submission template (submission 675627)
 * defines it in its docstring ("DeepSeek R1 forward_absorb MLA config", "KV
 * buffer format", "Input tuple", "Output"): 16 query heads share one latent KV
 * head; for sequence b, query row t and head h
 *
 *     s_j      = sm_scale * sum_{d<576} q[t,h,d] * kv[j,d]
 *     out[t,h,v] = sum_j softmax_j(s) * kv[j,v]          (v < 512)
 *
 * over the KV rows j in [kv_indptr[b], kv_indptr[b+1]).  Keys are the full
 * 576-wide row (512 latent + 64 rope), values the first 512 columns of the same
 * row.  The work is split along the KV rows ("split-K" flash decoding, the
 * two-stage scheme of submissions 586148 and 753817): stage 1 turns each
 * workgroup's slice into a partial output plus its log-sum-exp, stage 2 merges
 * the slices of a sequence with LSE weights.
 *
 * Conventions shared by every entry point:
 *   - Device pointers are HIP device addresses; host pointers are plain host
 *     memory.  Every device buffer is owned by the caller and must stay valid
 *     until the work queued on `stream` has finished.  `stream` is a
 *     hipStream_t passed as void* (NULL = the null stream).
 *   - Entry points return a status and never throw.  MLA_ERR_HIP keeps the last
 *     HIP error, which mla_last_error_string() describes.
 *   - Thread safety: plans are immutable after creation and may be shared;
 *     runs on different streams need separate workspaces.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size, workspace too small, bad indptr */
  MLA_ERR_UNSUPPORTED = 2, /* shape or dtype combination the library does not implement */
  MLA_ERR_HIP = 3          /* a HIP call or kernel launch failed */
} mla_status;

typedef enum mla_dtype {
  MLA_DTYPE_BF16 = 0,       /* bfloat16, 2 bytes per element */
  MLA_DTYPE_FP8_E4M3FN = 1, /* OCP fp8 E4M3FN code, 1 byte, with one fp32 scale per tensor */
  MLA_DTYPE_MXFP4 = 2       /* OCP MXFP4: E2M1 pairs (element 2i in the low nibble) + one
                               E8M0 scale byte per 32 elements; KV only */
} mla_dtype;

/* The decode problem a plan is made for. */
typedef struct mla_problem {
  int32_t batch_size; /* sequences; >= 1 */
  int32_t total_q;    /* rows of q and out: batch_size when max_q_len <= 1, else in
                         [1, batch_size * max_q_len] */
  int64_t total_kv;   /* rows in the KV buffer; kv_indptr[batch_size] <= total_kv < 2^31 */
  int32_t num_heads;  /* query heads; must be 16 */
  int32_t qk_dim;     /* key width; must be 576 (512 latent + 64 rope) */
  int32_t v_dim;      /* value width; must be 512 (first columns of the KV row) */
  int32_t q_dtype;    /* MLA_DTYPE_BF16 or MLA_DTYPE_FP8_E4M3FN */
  int32_t kv_dtype;   /* any mla_dtype, with either q dtype */
  float sm_scale;     /* softmax scale, 1/sqrt(576) for DeepSeek-R1; finite and > 0 */
  int32_t num_cus;    /* compute units to plan for; 0 = ask the current HIP device */
  int32_t max_q_len;  /* query rows per sequence at most (0 or 1: exactly one each; 2..4:
                         qo_indptr[b+1] - qo_indptr[b] in [0, max_q_len], every row attending
                         to all KV rows of its sequence with no mask - multi-token prediction
                         or speculative decoding).  Larger values: MLA_ERR_UNSUPPORTED */
  float logit_cap;    /* 0: none; > 0 (finite): every scaled score s is soft-capped to
                         logit_cap * tanh(s / logit_cap) before the softmax - the logit_cap
                         argument of the library decode call on submission 753817's page,
                         read as the usual soft-cap (the page passes 0.0) */
  int32_t kv_paged;   /* 0: sequence b's KV rows are rows [kv_indptr[b], kv_indptr[b+1]) of kv.
                         P >= 1, a power of two up to 65536: paged KV with pages of P rows
                         (the kv_indices / page_size arguments of the library decode call on
                         submission 753817's page, which passes page_size 1); runs go
                         through the _paged entry points.  P = 1: CSR row j is row
                         kv_indices[j] of kv.  P > 1: kv_indices lists pages, sequence b's
                         from entry kv_page_indptr[b] on, and row i of sequence b (i from
                         0) is row kv_indices[kv_page_indptr[b] + i / P] * P + i % P of kv.
                         Any KV format (MXFP4 scale rows are indexed like their rows).
                         Other values: MLA_ERR_INVALID_ARG */
} mla_problem;

/* Optional planner overrides (NULL = planner's choice for every field). */
typedef struct mla_plan_options {
  int32_t rows_per_split; /* > 0: KV rows each stage-1 workgroup takes (rounded up to 32) */
  int32_t wgs_per_cu;     /* > 0: stage-1 workgroups per CU the planner sizes the split for
                             (default: as many as are resident together - with one query row
                             per sequence 2 for bf16 and fp8 KV, 3 for MXFP4 KV; see
                             mla_plan_desc.wgs_per_cu for others) */
  int32_t age_skew;       /* with two stage-1 workgroups per CU (G = 2 * num_cus), per mille of
                             R moved from each CU's second workgroup to its first (dispatched
                             first, and favoured by the hardware), whose ranges are then
                             adjacent (see mla_plan_desc.num_splits): 0 = planner's choice,
                             -1 = equal ranges, 1..500 = that much */
  int32_t xcd_group;      /* paired ranges: J > 0 puts J consecutive pairs on the CUs of one XCD
                             (used when the CU count is a multiple of 8 J); 0 = planner's
                             choice, -1 = pair i on workgroups i and F + i */
} mla_plan_options;

/* What a plan decided (for tests, benchmarks and logs). */
typedef struct mla_plan_desc {
  int32_t num_splits;      /* stage-1 workgroups G.  F = paired_splits = 0: workgroup g owns KV rows
                              [g*R, (g+1)*R).  F > 0 (then G = 2F): workgroups s and F + s - a
                              CU's first and second - hold pair i (i = s, or see xcd_group) and
                              own the rows [i*P, i*P + R) and [i*P + R, (i+1)*P) with
                              P = R + R2.  Ranges are clipped to total_kv */
  int32_t rows_per_split;  /* R, a multiple of tile_rows */
  int32_t tile_rows;       /* KV rows per LDS tile */
  int32_t stages;          /* depth of the LDS tile ring */
  int32_t partial_slots;   /* 2*G partial (O, LSE) slots in the workspace, each for query_tokens
                              rows: O as bf16 [query_tokens][16][512] (normalised by its own
                              running sum), LSE as fp32 [query_tokens][16] */
  int32_t stage2;          /* 1 if mla_decode_run launches the LSE-merge kernel */
  int64_t workspace_bytes; /* bytes mla_decode_run needs */
  int32_t lds_bytes;       /* LDS per stage-1 workgroup */
  int32_t num_cus;         /* compute units planned for */
  int32_t wgs_per_cu;      /* stage-1 workgroups per CU the plan is sized for (resident together) */
  int32_t query_tokens;    /* query rows of a sequence each stage-1 workgroup multiplies every KV
                              tile with: 1, 2 or 4 (max_q_len rounded up) */
  int32_t paired_splits;   /* F: 0 for equal ranges, else the CU count (see num_splits) */
  int32_t second_rows_per_split; /* R2 <= R, a multiple of tile_rows: rows of workgroups g >= F when paired */
  int32_t xcd_group;       /* paired ranges: J > 0 - workgroups s and F + s hold pair
                              J * (8 * (k / J) + s % 8) + k % J with k = s / 8 (J consecutive
                              pairs on one XCD); 0 - they hold pair s */
  int32_t merge_batch;     /* partial slots stage 2 loads at once: with kv_indptr_host the
                              smallest of 2, 4, 8, 16 that holds the most slots one sequence
                              has (16 when more), else 8 */
  int32_t first_piece_table; /* 1: each stage-1 workgroup's first piece was derived from
                              kv_indptr_host and travels with the kernel arguments, so its first
                              loads go out without a kv_indptr search: with contiguous bf16 or
                              fp8 KV its first KV tile and its query row, before any other load;
                              with MXFP4 KV or paged KV its query row and its first KV tiles (or
                              their kv_indices entries; with pages of more than one row after one
                              round trip for the sequence's page list).
                              Planned with kv_indptr_host, one query row per sequence (then
                              qo_indptr[b] = b, which the run's contract implies, and the first
                              piece's query row is taken to be row b), kv_indptr_host[0] = 0, at
                              most 768 workgroups, batch <= 2^14 and rows per workgroup < 2^16;
                              else 0 (the kernel searches kv_indptr) */
} mla_plan_desc;

typedef struct mla_plan mla_plan;

/*
 * Plan a decode: how many stage-1 workgroups, and which KV rows each takes.
 * This is the split-count choice of page kernelbot-amd-mixed-mla-586148 (its
 * docstring's "Adaptive num_splits" and the host code that aims at a fixed
 * number of programs for the GPU) and of page kernelbot-amd-mixed-mla-753817
 * ("Entry point": the split count picked from batch size and KV length before
 * stage 1 launches).  Here the rows of the whole batch are cut into ranges
 * sized to the CU count, so that one sequence may span several ranges and one
 * range several sequences.
 * Host-only: no device memory is touched and no HIP call is
 * made unless problem->num_cus == 0.
 *   problem         shape and dtypes (see mla_problem).
 *   options         NULL or overrides.
 *   kv_indptr_host  NULL, or the host copy of kv_indptr (batch_size + 1 int32,
 *                   non-decreasing, kv_indptr[0] >= 0, last <= total_kv).  With it the
 *                   planner checks the offsets and skips stage 2 when every
 *                   sequence is non-empty and lies inside one workgroup's rows;
 *                   the plan is then valid only for runs with those offsets.
 *                   Without it the plan is valid for any offsets with the same
 *                   batch_size and total_kv.
 *   plan_out        receives a library-owned plan; free with mla_decode_plan_destroy.
 *   workspace_bytes receives the size of the device workspace run needs.
 * Returns MLA_ERR_UNSUPPORTED for shapes/dtypes the library does not implement and
 * MLA_ERR_INVALID_ARG for bad arguments; *plan_out is NULL on failure.
 */
mla_status mla_decode_plan(const mla_problem* problem, const mla_plan_options* options,
                           const int32_t* kv_indptr_host, mla_plan** plan_out, size_t* workspace_bytes);

/*
 * Run a planned decode asynchronously on `stream` (stage 1, then stage 2 when
 * the plan needs it): the custom_kernel call of page kernelbot-amd-mixed-mla-753817
 * ("Entry point": stage 1 over the splits, stage 2 only when a sequence has
 * more than one), computing the output the template page
 * kernelbot-amd-mixed-mla-675627 defines ("Input tuple", "Output";
 * custom_kernel_bf16 is its plain form).  The argument shapes below are that
 * input tuple's.  No allocation, no host<->device copy, no synchronisation.
 * All device pointers must be 16-byte aligned.
 *   q          device, [total_q][16][576]: bf16, or fp8 E4M3FN codes when q_dtype is fp8.
 *   q_scale    device fp32[1] (fp8 q: q = code * q_scale, q_scale >= 0); ignored for bf16 q (may be NULL).
 *   kv         device, [total_kv][576] bf16 | [total_kv][576] fp8 codes | [total_kv][288] MXFP4 bytes.
 *   kv_scale   fp8 KV: device fp32[1] (kv = code * kv_scale, kv_scale >= 0).
 *              MXFP4 KV: device uint8 [total_kv][18] E8M0 bytes, one per 32 columns,
 *              read in 16-byte units: the allocation must be readable up to the next
 *              multiple of 16 bytes past total_kv*18.
 *              bf16 KV: ignored (may be NULL).
 *   qo_indptr  device int32[batch_size + 1]; sequence b's query rows are
 *              [qo_indptr[b], qo_indptr[b+1]) - exactly one when the plan's max_q_len
 *              is 0 or 1, else at most max_q_len (rows of a sequence with none are
 *              not written).  Every row attends to all KV rows of its sequence.
 *   kv_indptr  device int32[batch_size + 1]; sequence b owns KV rows
 *              [kv_indptr[b], kv_indptr[b+1]).  Values inconsistent with the plan
 *              (or decreasing) give undefined output, but every access stays inside
 *              [0, total_kv) rows.
 *   out        device bf16 [total_q][16][512]; the rows of a sequence with no KV rows
 *              get zeros.
 *   workspace  device scratch of at least the planned workspace_bytes (contents
 *              need not be initialised; they are overwritten).
 */
mla_status mla_decode_run(const mla_plan* plan, const void* q, const float* q_scale, const void* kv,
                          const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_run for a plan made with kv_paged = P >= 1.  The arguments are
 * those of mla_decode_run, with total_kv counting CSR rows, plus:
 *   kv_rows    rows of the kv buffer ([kv_rows][576] bf16 or fp8 codes, [kv_rows][288]
 *              MXFP4 bytes with kv_scale [kv_rows][18]); at most 0xFFFFF000 bytes of
 *              rows (larger buffers: MLA_ERR_UNSUPPORTED).
 *   kv_indices device int32, 4-byte aligned.  P = 1: [total_kv] entries, CSR row j
 *              of the plan is row kv_indices[j] of kv.  P > 1: page numbers, at
 *              least kv_page_indptr[batch_size] entries; page p is rows
 *              [p * P, p * P + P) of kv.  An index outside the buffer gives
 *              undefined output for its sequence, but every KV read stays inside
 *              the kv buffer (reads past it return zero).
 *   kv_page_indptr  P > 1: device int32 [batch_size + 1], 4-byte aligned: sequence
 *              b's pages are kv_indices[kv_page_indptr[b] ..], ceil(len_b / P) of
 *              them (len_b = kv_indptr[b+1] - kv_indptr[b]).  The caller keeps
 *              every listed entry inside kv_indices; a decreasing pair reads its
 *              sequence as page 0.  P = 1: NULL.
 * A contiguous plan, a NULL kv_indices, or a kv_page_indptr that does not match
 * P is MLA_ERR_INVALID_ARG (and a paged plan passed to mla_decode_run or
 * mla_decode_split is too).
 */
mla_status mla_decode_run_paged(const mla_plan* plan, const void* q, const float* q_scale, const void* kv,
                                const void* kv_scale, int64_t kv_rows, const int32_t* kv_indices,
                                const int32_t* kv_page_indptr, const int32_t* qo_indptr, const int32_t* kv_indptr,
                                void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Stage 1 alone of mla_decode_run_paged (stage 2 is mla_decode_merge, unchanged). */
mla_status mla_decode_split_paged(const mla_plan* plan, const void* q, const float* q_scale, const void* kv,
                                  const void* kv_scale, int64_t kv_rows, const int32_t* kv_indices,
                                  const int32_t* kv_page_indptr, const int32_t* qo_indptr, const int32_t* kv_indptr,
                                  void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages of mla_decode_run as separate calls, for callers that put
 * work or an exchange between them (for example merging partials produced on
 * several devices) and for per-stage timing.  mla_decode_split with the same
 * arguments as mla_decode_run launches stage 1 only: each workgroup's online
 * softmax over its KV rows, writing whole sequences to `out` and the
 * partial (O, LSE) of split sequences to the workspace (the split-K stage 1 of
 * submissions 586148 / 753817).  mla_decode_merge launches stage 2 only: for
 * each sequence split across workgroups, out = sum_s w_s O_s / sum_s w_s with
 * w_s = exp(LSE_s - max LSE), and zeros for sequences with no KV rows; it
 * does nothing when the plan needs no stage 2.  Calling split then merge on
 * one stream equals mla_decode_run.
 */
mla_status mla_decode_split(const mla_plan* plan, const void* q, const float* q_scale, const void* kv,
                            const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);
mla_status mla_decode_merge(const mla_plan* plan, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_run for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, which is instead a static device
 * array of 34 MiB (35,651,584 bytes) that the library holds on every device it
 * runs on until the process ends.  Allocates nothing and frees nothing; the
 * first call on a device looks the array's address up once.
 *   Plans whose workspace_bytes exceed 34 MiB get MLA_ERR_UNSUPPORTED (with
 *   mla_last_error_string() saying so); every plan the planner makes by
 *   default for up to ~2.7e8 KV rows on a 256-CU device fits.
 *   All calls on one device share the array, and nothing in it needs to start
 *   at zero: calls that overlap on one device (concurrent streams, or threads)
 *   race on it and give undefined output.  Calls ordered on one stream are safe.
 */
mla_status mla_decode_run_noalloc(const mla_plan* plan, const void* q, const float* q_scale, const void* kv,
                                  const void* kv_scale, const int32_t* qo_indptr, const int32_t* kv_indptr,
                                  void* out, void* stream);

/* Free a plan (NULL is accepted). */
void mla_decode_plan_destroy(mla_plan* plan);

/* Copy what the plan decided into *desc. */
mla_status mla_decode_plan_describe(const mla_plan* plan, mla_plan_desc* desc);

/*
 * Host replay of how stage 1 cuts the batch (the same piece rule the kernel
 * uses), for tests and tooling: which KV rows of which sequence each program
 * takes (page kernelbot-amd-mixed-mla-586148, docstring: each program takes
 * its share of the KV tokens and writes a partial).  Writes up to `capacity` records of 5 int64
 * each: {workgroup g, sequence b, first row, end row, slot (-1 = written to out
 * directly)} in workgroup order, and the total number of records to *count.
 * kv_indptr_host as in mla_decode_plan (required here).
 */
mla_status mla_decode_plan_pieces(const mla_plan* plan, const int32_t* kv_indptr_host, int64_t* records,
                                  int64_t capacity, int64_t* count);

/*
 * Partial slots stage 2 merges for sequence b (host replay of the stage-2
 * rule; page kernelbot-amd-mixed-mla-753817, "Stage 2: LSE-weighted
 * reduction of split partial outputs").  Writes up to `capacity` slot indices to `slots` and the number of
 * slots to *count (0 when the sequence was written directly or is empty).
 */
mla_status mla_decode_plan_merge_slots(const mla_plan* plan, const int32_t* kv_indptr_host, int32_t b,
                                       int32_t* slots, int32_t capacity, int32_t* count);

/*
 * Decode stored KV codes to fp32 with the device functions the decode kernel
 * uses (for bit-exactness tests of the dequantisation).  The formats are the
 * template page's (kernelbot-amd-mixed-mla-675627, "Input tuple": fp8 codes
 * with one scalar scale, fp4x2 bytes with fp8_e8m0 scales), read as the OCP
 * fp8 and MX definitions give them.
 *   MLA_DTYPE_FP8_E4M3FN: codes = n bytes, scales = device fp32[1] or NULL (1.0);
 *                         out[i] = fp32(value(code_i)) * scale, one fp32 rounding.
 *   MLA_DTYPE_MXFP4:      codes = n rows of 288 bytes, scales = n rows of 18 bytes;
 *                         out = n x 576 values, each the bf16 the kernel feeds to its
 *                         matrix instructions, widened to fp32.
 *   MLA_DTYPE_BF16:       codes = n bf16 values; out[i] = fp32(code_i).
 * Device pointers, asynchronous on `stream`.
 */
mla_status mla_debug_decode(int32_t kv_dtype, const void* codes, const void* scales, float* out, int64_t n,
                            void* stream);

/*
 * Read-bandwidth reference for reports (not part of the decode, and defined by
 * none of the pages; a measurement aid): one launch
 * that reads `bytes` of device memory at `buf` with 16-byte non-temporal loads
 * (4096 workgroups, each streaming its own contiguous share) and nothing else,
 * so that timing it gives the HBM read rate this device sustains, against
 * which the decode's rate can be set.
 *   buf    device, 16-byte aligned; bytes a multiple of 16 (MLA_ERR_INVALID_ARG otherwise).
 *   sink   device uint32[1]; written only in the (practically impossible) case that
 *          the XOR of everything read equals 0x9E3779B9.
 * Asynchronous on `stream`.
 */
mla_status mla_debug_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Read-bandwidth reference with stage 1's own access pattern (a measurement
 * aid, defined by none of the pages): `wgs` workgroups, two per CU, each stream
 * a contiguous share of `bytes` in 18 KB tiles through the four-slot LDS ring
 * of the fp8 stage-1 kernel (the same 16-byte LDS DMA, waits and two barriers
 * per tile), with no arithmetic.  Timing it over the bytes of a call gives the
 * rate the decode's memory side reaches when nothing else runs.
 *   buf    device, 16-byte aligned; bytes a multiple of 18432, at most about
 *          4 GB per workgroup share (MLA_ERR_INVALID_ARG otherwise); wgs >= 1.
 *   sink   device uint32[1]; written only in the (practically impossible) case
 *          that the XOR of the words it samples equals 0x9E3779B9.
 * Asynchronous on `stream`.
 */
mla_status mla_debug_stream_ring(const void* buf, int64_t bytes, int32_t wgs, uint32_t* sink, void* stream);

/*
 * Per-workgroup timeline of the last stage-1 launch (a measurement aid, defined
 * by none of the pages; for finding where a call's time goes).  Only the
 * library built with -DMLA_WG_TRACE records it (mla_decode_split_amd/build.py,
 * build_trace); the product build returns MLA_ERR_UNSUPPORTED and its kernels
 * carry no part of it.  Entry g of the host array (4 uint64 per stage-1
 * workgroup g < 8192): start, first KV tile complete in LDS, end, all on the
 * device's 100 MHz real-time counter, and the XCC_ID | HW_ID << 8 register
 * values of the CU it ran on.  Workgroups that own no rows write nothing.
 *   host   receives the first n uint64 entries (n <= 4 * 8192); may be NULL when n = 0.
 *   clear  nonzero: zero the record first (before a launch to be traced).
 * Synchronous (device-wide copies).
 */
mla_status mla_debug_wg_trace(uint64_t* host, int64_t n, int32_t clear);

/* Human-readable status name. */
const char* mla_status_string(mla_status status);

/* Description of the last HIP error seen by this thread ("" if none). */
const char* mla_last_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
