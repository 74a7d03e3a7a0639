/*
 * synth.c - seeded synthetic inputs for MLA decode workloads.
 *
 * This module only draws random numbers and encodes them into the storage
 * formats the decode path reads (bf16, OCP fp8 E4M3FN with a per-tensor scale,
 * OCP MXFP4 = E2M1 elements with one E8M0 scale per 32 elements).  It holds
 * none of the attention arithmetic and none of the decoders: both the CPU
 * oracle and the GPU library consume the bytes written here.
 *
 * Random numbers: the ctr-th output of a SplitMix64 generator (Steele, Lea,
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
 * 64-bit finaliser constants of Vigna's public reference version) whose state
 * starts at a key derived from (seed, stream).  Being counter based, any
 * element can be produced independently, which lets the generator run on many
 * threads and be re-run for a second pass without storing the first.
 * Standard normals use the Box-Muller transform on two consecutive outputs.
 *
 * The template page of the kernelbot-amd-mixed-mla pages ("Input tuple" in the
 * docstring, and its quantize_fp8 helper) fixes the formats and the per-tensor
 * fp8 recipe amax / finfo.max; the MXFP4 recipe follows the OCP Microscaling
 * Formats (MX) v1.0 specification, section 6.3 (shared exponent =
 * floor(log2(amax)) - emax_elem, emax_elem = 2 for E2M1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of the stream (seed, stream): the first output of a SplitMix64 seeded
 * with a linear combination of the two. */
uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GAMMA + stream * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL);
}

/* ctr-th output (ctr = 0, 1, ...) of SplitMix64 whose state starts at key. */
uint64_t synth_u64(uint64_t key, uint64_t ctr) { return mix64(key + (ctr + 1) * GAMMA); }

/* Element i of a standard normal stream: Box-Muller on the outputs 2*(i/2) and
 * 2*(i/2)+1; even i takes the cosine branch, odd i the sine branch.  The
 * double result is rounded once to fp32. */
static inline float normal_at(uint64_t key, uint64_t i) {
  const uint64_t j = i >> 1;
  const uint64_t a = synth_u64(key, 2 * j), b = synth_u64(key, 2 * j + 1);
  const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
  const double r = sqrt(-2.0 * log(u1));
  const double th = 2.0 * M_PI * u2;
  return (float)((i & 1) ? r * sin(th) : r * cos(th));
}

/* fp32 -> bf16 bits, round to nearest even; NaN stays NaN. */
static inline uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* bf16-rounded standard normal: the source every tensor is drawn from. */
static inline float normal_bf16_at(uint64_t key, uint64_t i) { return bf16_to_f32(bf16_rne(normal_at(key, i))); }

/* Round a finite fp32 to the nearest OCP E4M3FN code (ties to even), saturating
 * at +-448.  E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent
 * field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN and there is no inf. */
uint8_t synth_encode_e4m3fn(float x) {
  if (x != x) return 0x7f;
  uint8_t sign = 0;
  if (x < 0 || (x == 0 && signbit(x))) { sign = 0x80; x = -x; }
  if (x >= 448.0f) return sign | 0x7e;
  /* Work in units of the smallest subnormal, 2^-9: exact in double. */
  double v = (double)x;
  int e;
  frexp(v, &e); /* v = f * 2^e, f in [0.5, 1) -> unbiased exponent of v is e-1 */
  int ue = e - 1;
  if (ue < -6) ue = -6; /* subnormal range shares the quantum of exponent -6 */
  const double quantum = ldexp(1.0, ue - 3);
  double q = v / quantum; /* exact: power-of-two division */
  double fl = floor(q);
  double rem = q - fl;
  double n = fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
  /* n * quantum is the rounded magnitude; n may reach 16 (carry into next exponent). */
  double r = n * quantum;
  if (r >= 448.0) return sign | 0x7e;
  if (r == 0.0) return sign;
  int re;
  frexp(r, &re);
  int uexp = re - 1;
  if (uexp < -6) { /* subnormal: field 0, mantissa r / 2^-9 */
    return sign | (uint8_t)(r / ldexp(1.0, -9));
  }
  int mant = (int)(ldexp(r, -uexp) * 8.0) - 8;
  return sign | (uint8_t)(((uexp + 7) << 3) | mant);
}

/* Round a finite value to the nearest OCP E2M1 code (ties to the even code),
 * saturating at +-6.  Magnitudes by code: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
uint8_t synth_encode_e2m1(float x) {
  static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  uint8_t sign = 0;
  if (x < 0 || (x == 0 && signbit(x))) { sign = 8; x = -x; }
  if (x >= 6.0f) return sign | 7;
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    float dc = fabsf(x - mag[c]), db = fabsf(x - mag[best]);
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return sign | (uint8_t)best;
}

/* One MXFP4 block of 32 values -> 16 packed bytes (element 2i in the low
 * nibble, 2i+1 in the high nibble) and one E8M0 scale byte.  Shared exponent
 * floor(log2(amax)) - 2; an all-zero block gets scale 2^0 (byte 127). */
void synth_encode_mxfp4_block(const float* x, uint8_t* packed16, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  int se = 0;
  if (amax > 0.0f) {
    int e;
    frexp(amax, &e);
    se = (e - 1) - 2;
  }
  if (se < -127) se = -127;
  if (se > 127) se = 127;
  *scale = (uint8_t)(se + 127);
  for (int i = 0; i < 16; ++i) {
    uint8_t lo = synth_encode_e2m1((float)ldexp((double)x[2 * i], -se));
    uint8_t hi = synth_encode_e2m1((float)ldexp((double)x[2 * i + 1], -se));
    packed16[i] = (uint8_t)(lo | (hi << 4));
  }
}

/* ---------------------------------------------------------------- threading */

typedef struct {
  int kind;
  uint64_t key;
  uint64_t begin, end; /* element (or row) range of this worker */
  void* out;
  void* out2;
  float scale;
  int row_elems;
  float amax;
} job_t;

enum { JOB_BF16 = 0, JOB_AMAX = 1, JOB_FP8 = 2, JOB_MXFP4 = 3 };

static void* run_job(void* arg) {
  job_t* j = (job_t*)arg;
  switch (j->kind) {
    case JOB_BF16: {
      uint16_t* o = (uint16_t*)j->out;
      for (uint64_t i = j->begin; i < j->end; ++i) o[i] = bf16_rne(normal_at(j->key, i));
      break;
    }
    case JOB_AMAX: {
      float m = 0.0f;
      for (uint64_t i = j->begin; i < j->end; ++i) m = fmaxf(m, fabsf(normal_bf16_at(j->key, i)));
      j->amax = m;
      break;
    }
    case JOB_FP8: {
      uint8_t* o = (uint8_t*)j->out;
      const float s = j->scale;
      for (uint64_t i = j->begin; i < j->end; ++i) {
        float v = normal_bf16_at(j->key, i) / s; /* fp32 division, round to nearest */
        if (v > 448.0f) v = 448.0f;
        if (v < -448.0f) v = -448.0f;
        o[i] = synth_encode_e4m3fn(v);
      }
      break;
    }
    case JOB_MXFP4: {
      uint8_t* packed = (uint8_t*)j->out;
      uint8_t* scales = (uint8_t*)j->out2;
      const int d = j->row_elems, nb = d / 32;
      float blk[32];
      for (uint64_t r = j->begin; r < j->end; ++r) {
        for (int b = 0; b < nb; ++b) {
          for (int i = 0; i < 32; ++i) blk[i] = normal_bf16_at(j->key, r * (uint64_t)d + (uint64_t)(b * 32 + i));
          synth_encode_mxfp4_block(blk, packed + r * (uint64_t)(d / 2) + (uint64_t)b * 16, scales + r * (uint64_t)nb + b);
        }
      }
      break;
    }
  }
  return NULL;
}

static float run_parallel(int kind, uint64_t key, uint64_t n, void* out, void* out2, float scale, int row_elems,
                          int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((uint64_t)nthreads > n) nthreads = n ? (int)n : 1;
  job_t jobs[256];
  pthread_t th[256];
  const uint64_t per = (n + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].kind = kind;
    jobs[t].key = key;
    jobs[t].begin = per * (uint64_t)t < n ? per * (uint64_t)t : n;
    jobs[t].end = per * (uint64_t)(t + 1) < n ? per * (uint64_t)(t + 1) : n;
    jobs[t].out = out;
    jobs[t].out2 = out2;
    jobs[t].scale = scale;
    jobs[t].row_elems = row_elems;
    jobs[t].amax = 0.0f;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
  run_job(&jobs[0]);
  float amax = jobs[0].amax;
  for (int t = 1; t < nthreads; ++t) {
    pthread_join(th[t], NULL);
    amax = fmaxf(amax, jobs[t].amax);
  }
  return amax;
}

/* --------------------------------------------------------------- public API */

/* n bf16 standard normals of stream (seed, stream). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t n, uint16_t* out, int nthreads) {
  run_parallel(JOB_BF16, synth_stream_key(seed, stream), n, out, NULL, 0.0f, 0, nthreads);
}

/* max |x| over the first n bf16 normals of the stream. */
float synth_amax_bf16(uint64_t seed, uint64_t stream, uint64_t n, int nthreads) {
  return run_parallel(JOB_AMAX, synth_stream_key(seed, stream), n, NULL, NULL, 0.0f, 0, nthreads);
}

/* Per-tensor fp8: scale = amax / 448 (fp32), codes = E4M3FN(clamp(x / scale)).
 * Writes n codes; returns the scale. */
float synth_fp8_tensor(uint64_t seed, uint64_t stream, uint64_t n, uint8_t* codes, int nthreads) {
  const uint64_t key = synth_stream_key(seed, stream);
  float amax = run_parallel(JOB_AMAX, key, n, NULL, NULL, 0.0f, 0, nthreads);
  if (amax < 1e-12f) amax = 1e-12f;
  const float scale = amax / 448.0f;
  run_parallel(JOB_FP8, key, n, codes, NULL, scale, 0, nthreads);
  return scale;
}

/* MXFP4 rows: rows x row_elems normals -> packed [rows][row_elems/2] and
 * scales [rows][row_elems/32].  row_elems must be a multiple of 32. */
int synth_mxfp4_rows(uint64_t seed, uint64_t stream, uint64_t rows, int row_elems, uint8_t* packed, uint8_t* scales,
                     int nthreads) {
  if (row_elems <= 0 || row_elems % 32) return -1;
  run_parallel(JOB_MXFP4, synth_stream_key(seed, stream), rows, packed, scales, 0.0f, row_elems, nthreads);
  return 0;
}

/* bs lengths uniform on [lo, hi] (hi - lo + 1 need not be a power of two:
 * rejection sampling keeps the draw exactly uniform). */
void synth_uniform_lengths(uint64_t seed, uint64_t stream, int bs, int lo, int hi, int32_t* out) {
  const uint64_t key = synth_stream_key(seed, stream);
  const uint64_t span = (uint64_t)(hi - lo) + 1;
  const uint64_t limit = UINT64_MAX - (UINT64_MAX % span);
  uint64_t ctr = 0;
  for (int b = 0; b < bs; ++b) {
    uint64_t r;
    do r = synth_u64(key, ctr++);
    while (r >= limit);
    out[b] = lo + (int32_t)(r % span);
  }
}

/* Encoders exposed for tests that build specific inputs by hand. */
void synth_encode_e4m3fn_array(const float* x, uint64_t n, uint8_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = synth_encode_e4m3fn(x[i]);
}
void synth_encode_mxfp4_array(const float* x, uint64_t rows, int row_elems, uint8_t* packed, uint8_t* scales) {
  const int nb = row_elems / 32;
  for (uint64_t r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b)
      synth_encode_mxfp4_block(x + r * (uint64_t)row_elems + b * 32, packed + r * (uint64_t)(row_elems / 2) + b * 16,
                               scales + r * (uint64_t)nb + b);
}
void synth_bf16_from_f32(const float* x, uint64_t n, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = bf16_rne(x[i]);
}
