/*
 * Seeded synthetic inputs for the W4A16 skinny matmul.
 *
 * This module only draws random numbers and encodes them in the storage
 * formats of the inputs (packed bytes, bf16 bit patterns, int32 ids).  It
 * holds none of the matmul's arithmetic: no dequantisation, no dot product,
 * no argmax.  Both the CPU oracle's tests and the GPU path's tests and bench
 * take their inputs from here, so the two read exactly the same bits.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Its n-th output is the 64-bit mixing
 * function applied to  state0 + (n+1)*gamma,  so any element can be produced
 * from its index alone; generation is deterministic under any threading.
 * A stream is keyed by (seed, stream_id).
 *
 * Value recipes (the pages name no distributions of their own; these are the
 * recipes of the synthetic workloads):
 *   codes  : every byte is 8 uniform bits, i.e. two uniform 4-bit codes.
 *   normal : z ~ N(0,1) by Box-Muller from two 53-bit uniforms in (0,1].
 *   scales : bf16( 0.02*|z| + 1e-3 ).
 *   x      : bf16( z ).
 *   ids    : Floyd's sampling of distinct ids from [0, n_rows), kept in the
 *            order they were drawn.
 * bf16 encoding is round-to-nearest-even from double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Initial state of the stream (seed, stream_id). */
static inline uint64_t stream_state(uint64_t seed, uint64_t stream_id) {
  return mix64(seed + GAMMA) ^ mix64(stream_id * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL);
}

/* n-th output of the stream. */
static inline uint64_t draw(uint64_t state, uint64_t n) { return mix64(state + (n + 1) * GAMMA); }

/* Uniform in (0, 1] with 53 random bits. */
static inline double unit_open0(uint64_t r) { return (double)((r >> 11) + 1) * (1.0 / 9007199254740992.0); }

static inline double normal_at(uint64_t state, uint64_t i) {
  double u1 = unit_open0(draw(state, 2 * i));
  double u2 = unit_open0(draw(state, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* double -> bf16 bits, round to nearest, ties to even.  Finite inputs whose
 * magnitude is a normal float are handled exactly; that covers every value
 * the recipes above produce. */
uint16_t synth_bf16_from_double(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  double m = frexp(fabs(v), &e);   /* |v| = m * 2^e, m in [0.5, 1) */
  double r = nearbyint(m * 256.0); /* 8 significant bits, ties to even (default mode) */
  double q = ldexp(r, e - 8);
  float f = (float)q; /* exact: q has 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t b = (uint16_t)(u >> 16);
  return signbit(v) ? (uint16_t)(b | 0x8000) : b;
}

/* ---- parallel fill over element ranges ---- */
typedef struct {
  int kind;
  uint64_t state;
  void* out;       /* element i of the stream goes to out[i - base] */
  uint64_t begin, end, base;
} job_t;

enum { KIND_BYTES = 0, KIND_SCALES = 1, KIND_NORMAL_BF16 = 2 };

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  if (j->kind == KIND_BYTES) {
    uint8_t* o = (uint8_t*)j->out - j->base;
    /* byte i comes from bits 8*(i%8).. of draw i/8 */
    uint64_t i = j->begin;
    while (i < j->end) {
      uint64_t r = draw(j->state, i >> 3);
      for (unsigned b = (unsigned)(i & 7); b < 8 && i < j->end; ++b, ++i) o[i] = (uint8_t)(r >> (8 * b));
    }
  } else if (j->kind == KIND_SCALES) {
    uint16_t* o = (uint16_t*)j->out;
    for (uint64_t i = j->begin; i < j->end; ++i)
      o[i - j->base] = synth_bf16_from_double(0.02 * fabs(normal_at(j->state, i)) + 1e-3);
  } else {
    uint16_t* o = (uint16_t*)j->out;
    for (uint64_t i = j->begin; i < j->end; ++i) o[i - j->base] = synth_bf16_from_double(normal_at(j->state, i));
  }
  return NULL;
}

/* Elements [start, start + count) of a stream into out[0 .. count). */
static void fill(int kind, uint64_t seed, uint64_t stream_id, void* out, uint64_t start, uint64_t count,
                 int nthreads) {
  uint64_t state = stream_state(seed, stream_id);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (count < (uint64_t)nthreads * 65536) nthreads = 1;
  job_t jobs[256];
  pthread_t th[256];
  uint64_t per = (count + nthreads - 1) / nthreads;
  per = (per + 7) & ~7ULL;
  int launched = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t b = per * t, e = b + per;
    if (b >= count) break;
    if (e > count) e = count;
    jobs[t] = (job_t){kind, state, out, start + b, start + e, start};
    if (t == 0) continue;
    if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) { run_job(&jobs[t]); th[t] = 0; }
    launched = t + 1;
  }
  run_job(&jobs[0]);
  for (int t = 1; t < launched; ++t)
    if (th[t]) pthread_join(th[t], NULL);
}

/* Uniform bytes (two 4-bit codes per byte). */
void synth_codes(uint64_t seed, uint64_t stream_id, uint8_t* out, uint64_t n_bytes, int nthreads) {
  fill(KIND_BYTES, seed, stream_id, out, 0, n_bytes, nthreads);
}

/* bf16 scales 0.02*|z| + 1e-3. */
void synth_scales(uint64_t seed, uint64_t stream_id, uint16_t* out, uint64_t n, int nthreads) {
  fill(KIND_SCALES, seed, stream_id, out, 0, n, nthreads);
}

/* bf16 standard normals. */
void synth_normal_bf16(uint64_t seed, uint64_t stream_id, uint16_t* out, uint64_t n, int nthreads) {
  fill(KIND_NORMAL_BF16, seed, stream_id, out, 0, n, nthreads);
}

/* Bytes [start, start + n_bytes) and scales [start, start + n) of the same
 * streams: any rows of a weight without generating the rest. */
void synth_codes_range(uint64_t seed, uint64_t stream_id, uint8_t* out, uint64_t start, uint64_t n_bytes) {
  fill(KIND_BYTES, seed, stream_id, out, start, n_bytes, 1);
}

void synth_scales_range(uint64_t seed, uint64_t stream_id, uint16_t* out, uint64_t start, uint64_t n) {
  fill(KIND_SCALES, seed, stream_id, out, start, n, 1);
}

/* Floyd's algorithm: n_ids distinct values from [0, n_rows), in draw order.
 * Returns 0 on success, -1 on bad arguments or allocation failure. */
int synth_distinct_ids(uint64_t seed, uint64_t stream_id, int32_t* out, int64_t n_ids, int64_t n_rows) {
  if (n_ids < 0 || n_rows < 0 || n_ids > n_rows || n_rows > 0x7fffffffLL) return -1;
  uint64_t state = stream_state(seed, stream_id);
  uint8_t* seen = (uint8_t*)calloc((size_t)((n_rows + 7) / 8 + 1), 1);
  if (!seen) return -1;
  int64_t c = 0;
  for (int64_t j = n_rows - n_ids; j < n_rows; ++j, ++c) {
    uint64_t r = draw(state, (uint64_t)c) >> 32;                 /* 32 uniform bits */
    int64_t t = (int64_t)((r * (uint64_t)(j + 1)) >> 32);        /* in [0, j] */
    int64_t pick = (seen[t >> 3] >> (t & 7)) & 1 ? j : t;
    seen[pick >> 3] |= (uint8_t)(1u << (pick & 7));
    out[c] = (int32_t)pick;
  }
  free(seen);
  return 0;
}
