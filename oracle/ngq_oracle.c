/*
 * ngq_oracle.c -- CPU oracle for the small-T groupwise-int projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file.  Its only users are the tests, the smoke check and
 * the CPU-baseline leg of the bench.  It shares no code, header, table or
 * constant with the HIP library: every rule below is written out here again
 * from the definition of the operation.
 *
 * What it computes (the plain definition, no blocking, no reordering):
 *
 *   y[t][n] = sum_{k=0}^{K-1} x[t][k] * c[k][n] * s[k/64][n]      (fp64, k ascending)
 *   out     = bf16 round-to-nearest-even of y, rounded directly from fp64
 *
 * Source of the operation: the NInfer-4090 V3 topic (lcz.me/topic/2047),
 * section "What V3 did", names T=8 routing of small-batch Q4/Q5 projections
 * (GDN projection, attention Q5 projection, SwiGLU path); the ninfer-ext
 * README, section "Comparison with upstream NInfer", names the groupwise-int
 * Q5 K-split path for speculative-verify rounds; the single-4090 notes
 * (yudady blog), section "VRAM and multimodal space", give ~17.0 GB of
 * groupwise-int weights.  The pages print no formula, bit layout or shape;
 * the symmetric dequantisation w = c * s with one scale per 64 consecutive
 * k and column, int4 codes stored offset-binary 8 per 32-bit word along K,
 * int5 stored as a low-nibble plane plus a one-bit high plane, fp32
 * accumulation and bf16 output are therefore readings, not quotations, and
 * are restated below as the layout this oracle reads.
 *
 * Packed layout (all words little-endian, row-major, column index fastest):
 *   int4: P0 = u32[K/8][N];  bits 4i..4i+3 of word (kb,n) hold u = c+8
 *         for k = 8*kb + i, i = 0..7.
 *   int5: P0 as int4 but holding u & 15 with u = c+16; then immediately
 *         after P0, P1 = u32[K/32][N]; bit i of word (kb,n) holds u >> 4
 *         for k = 32*kb + i, i = 0..31.
 *   int8: P0 = u32[K/4][N];  byte i of word (kb,n) holds u = c+128 for
 *         k = 4*kb + i, i = 0..3.
 *   scales: [K/64][N] raw 16-bit values, fp16 or bf16.
 *   x:      [T][K] raw bf16 bits.
 * Readings taken where the pages are silent (offset-binary int5/int8, LSB
 * first field order, row-major orientation, RNE from fp64) are listed in
 * the design notes of the repository.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP 64

/* ---- 16-bit float decoding (IEEE binary16 and bfloat16), exact in fp64 ---- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xFF;
  int f = b & 0x7F;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133); /* subnormal: f * 2^-126 * 2^-7 */
  } else if (e == 255) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(128 + f), e - 134); /* (1 + f/128) * 2^(e-127) */
  }
  return sign ? -v : v;
}

/* Round a double to the nearest bfloat16, ties to even, directly from fp64
 * (no intermediate fp32 rounding).  Overflow gives +-inf, NaN stays NaN. */
uint16_t oracle_round_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1, so a lies in [2^(e-1), 2^e) */
  int exp_unb = e - 1;              /* a in [2^exp_unb, 2^(exp_unb+1)) */
  if (exp_unb < -126) exp_unb = -126; /* subnormal range has a fixed quantum */
  double quantum = ldexp(1.0, exp_unb - 7); /* 8 significant bits */
  double q = a / quantum;                   /* exact: power-of-two division */
  double r = floor(q);
  double frac = q - r;                      /* exact */
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double rounded = r * quantum; /* exact */
  if (rounded >= ldexp(1.0, 128)) return sign | 0x7F80;
  /* Encode: rounded has at most 8 significant bits and lies in bf16 range. */
  if (rounded < ldexp(1.0, -126)) {
    int frac_bits = (int)(rounded / ldexp(1.0, -133)); /* 0..128 */
    if (frac_bits == 128) return sign | 0x0080; /* rounded up to min normal */
    return sign | (uint16_t)frac_bits;
  }
  int e2;
  double m2 = frexp(rounded, &e2); /* rounded = m2 * 2^e2, m2 in [0.5, 1) */
  int biased = (e2 - 1) + 127;
  int mant = (int)(m2 * 256.0) - 128; /* 7 fraction bits */
  return sign | (uint16_t)(biased << 7) | (uint16_t)mant;
}

/* ---- packed layout: read and write one code --------------------------- */

static uint32_t rd_u32(const uint8_t* p, size_t word_index) {
  const uint8_t* b = p + 4 * word_index;
  return (uint32_t)b[0] | ((uint32_t)b[1] << 8) | ((uint32_t)b[2] << 16) | ((uint32_t)b[3] << 24);
}

static void wr_u32(uint8_t* p, size_t word_index, uint32_t w) {
  uint8_t* b = p + 4 * word_index;
  b[0] = (uint8_t)(w & 0xFF);
  b[1] = (uint8_t)((w >> 8) & 0xFF);
  b[2] = (uint8_t)((w >> 16) & 0xFF);
  b[3] = (uint8_t)((w >> 24) & 0xFF);
}

static int valid_shape(int K, int N, int bits) {
  if (K < 0 || N < 0) return 0;
  if (bits != 4 && bits != 5 && bits != 8) return 0;
  if (K % ORACLE_GROUP) return 0;
  return 1;
}

/* Bytes of the packed weight buffer: P0 (+ P1 for int5). */
size_t oracle_packed_bytes(int K, int N, int bits) {
  if (!valid_shape(K, N, bits)) return 0;
  size_t kn = (size_t)K * (size_t)N;
  if (bits == 4) return kn / 2;
  if (bits == 5) return kn / 2 + kn / 8;
  return kn;
}

/* The signed code c[k][n] read from the packed buffer, per the layout above. */
int oracle_code_at(const uint8_t* packed, int K, int N, int bits, int k, int n) {
  if (bits == 4) {
    uint32_t w = rd_u32(packed, (size_t)(k / 8) * N + n);
    int u = (int)((w >> (4 * (k % 8))) & 0xFu);
    return u - 8;
  }
  if (bits == 5) {
    uint32_t w0 = rd_u32(packed, (size_t)(k / 8) * N + n);
    size_t p1_first_word = (size_t)(K / 8) * N; /* P1 follows P0 */
    uint32_t w1 = rd_u32(packed, p1_first_word + (size_t)(k / 32) * N + n);
    int lo = (int)((w0 >> (4 * (k % 8))) & 0xFu);
    int hi = (int)((w1 >> (k % 32)) & 1u);
    return lo + 16 * hi - 16;
  }
  /* bits == 8 */
  uint32_t w = rd_u32(packed, (size_t)(k / 4) * N + n);
  int u = (int)((w >> (8 * (k % 4))) & 0xFFu);
  return u - 128;
}

/* Codes int8 [K][N] -> packed buffer.  Returns 0, or -1 on bad arguments or
 * a code outside [-2^(bits-1), 2^(bits-1)-1]. */
int oracle_pack(int K, int N, int bits, const int8_t* codes, uint8_t* out) {
  if (!valid_shape(K, N, bits)) return -1;
  int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
  for (size_t i = 0; i < (size_t)K * N; ++i)
    if (codes[i] < lo || codes[i] > hi) return -1;
  memset(out, 0, oracle_packed_bytes(K, N, bits));
  for (int k = 0; k < K; ++k) {
    for (int n = 0; n < N; ++n) {
      int c = codes[(size_t)k * N + n];
      if (bits == 4) {
        size_t wi = (size_t)(k / 8) * N + n;
        uint32_t u = (uint32_t)(c + 8);
        wr_u32(out, wi, rd_u32(out, wi) | (u << (4 * (k % 8))));
      } else if (bits == 5) {
        uint32_t u = (uint32_t)(c + 16);
        size_t wi0 = (size_t)(k / 8) * N + n;
        wr_u32(out, wi0, rd_u32(out, wi0) | ((u & 0xFu) << (4 * (k % 8))));
        size_t wi1 = (size_t)(K / 8) * N + (size_t)(k / 32) * N + n;
        wr_u32(out, wi1, rd_u32(out, wi1) | (((u >> 4) & 1u) << (k % 32)));
      } else {
        size_t wi = (size_t)(k / 4) * N + n;
        uint32_t u = (uint32_t)(c + 128);
        wr_u32(out, wi, rd_u32(out, wi) | (u << (8 * (k % 4))));
      }
    }
  }
  return 0;
}

/* Packed buffer -> codes int8 [K][N]. */
int oracle_unpack(int K, int N, int bits, const uint8_t* packed, int8_t* codes) {
  if (!valid_shape(K, N, bits)) return -1;
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n)
      codes[(size_t)k * N + n] = (int8_t)oracle_code_at(packed, K, N, bits, k, n);
  return 0;
}

static double scale_at(const uint16_t* scales, int N, int scale_bf16, int k, int n) {
  uint16_t raw = scales[(size_t)(k / ORACLE_GROUP) * N + n];
  return scale_bf16 ? oracle_bf16_to_f64(raw) : oracle_f16_to_f64(raw);
}

/* Dequantised weight w[k][n] = c * s in fp64 (exact: |c| <= 128 needs at most
 * 8 significant bits and a 16-bit scale at most 11). */
int oracle_dequant_f64(int K, int N, int bits, const uint8_t* packed, const uint16_t* scales,
                       int scale_bf16, double* w) {
  if (!valid_shape(K, N, bits)) return -1;
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n)
      w[(size_t)k * N + n] =
          (double)oracle_code_at(packed, K, N, bits, k, n) * scale_at(scales, N, scale_bf16, k, n);
  return 0;
}

/* ---- the projection ------------------------------------------------------ */

typedef struct {
  int T, K, N, bits, scale_bf16;
  const uint16_t* x;
  const uint8_t* packed;
  const uint16_t* scales;
  const int32_t* cols; /* column list, or NULL for 0..ncols-1 */
  int c_begin, c_end;  /* slice of the column list handled by one thread */
  int ncols;
  double* y64;     /* [T][ncols] */
  double* abs_xw;  /* [T][ncols] sum_k |x * w|, or NULL */
  double* abs_xs;  /* [T][ncols] sum_k |x| * s, or NULL */
} gemm_job;

static void* gemm_worker(void* arg) {
  gemm_job* j = (gemm_job*)arg;
  double* wcol = (double*)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
  double* scol = (double*)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
  for (int ci = j->c_begin; ci < j->c_end; ++ci) {
    int n = j->cols ? j->cols[ci] : ci;
    for (int k = 0; k < j->K; ++k) {
      scol[k] = scale_at(j->scales, j->N, j->scale_bf16, k, n);
      wcol[k] = (double)oracle_code_at(j->packed, j->K, j->N, j->bits, k, n) * scol[k];
    }
    for (int t = 0; t < j->T; ++t) {
      double acc = 0.0, axw = 0.0, axs = 0.0;
      for (int k = 0; k < j->K; ++k) {
        double xv = oracle_bf16_to_f64(j->x[(size_t)t * j->K + k]);
        acc += xv * wcol[k];
        axw += fabs(xv * wcol[k]);
        axs += fabs(xv) * scol[k];
      }
      size_t o = (size_t)t * j->ncols + ci;
      j->y64[o] = acc;
      if (j->abs_xw) j->abs_xw[o] = axw;
      if (j->abs_xs) j->abs_xs[o] = axs;
    }
  }
  free(wcol);
  free(scol);
  return NULL;
}

/* y64[t][i] = sum_k x[t][k] * c[k][n_i] * s[k/64][n_i] for the columns n_i in
 * `cols` (all N columns when cols is NULL and ncols == N).  Accumulates in fp64
 * with k ascending.  Also returns the magnitudes sum_k |x w| and sum_k |x| s
 * (either may be NULL), which bound the rounding error of any fp32 evaluation.
 * `nthreads` splits the column list over POSIX threads; the sum for each output
 * is computed by exactly one thread in the same order, so the result does not
 * depend on the thread count. */
int oracle_gemm_f64(int T, int K, int N, int bits, int scale_bf16, const uint16_t* x,
                    const uint8_t* packed, const uint16_t* scales, const int32_t* cols, int ncols,
                    double* y64, double* abs_xw, double* abs_xs, int nthreads) {
  if (!valid_shape(K, N, bits) || T < 0 || ncols < 0) return -1;
  if (!cols && ncols != N) return -1;
  if (cols)
    for (int i = 0; i < ncols; ++i)
      if (cols[i] < 0 || cols[i] >= N) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > ncols) nthreads = ncols > 0 ? ncols : 1;
  gemm_job* jobs = (gemm_job*)calloc((size_t)nthreads, sizeof(gemm_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    gemm_job* j = &jobs[i];
    j->T = T; j->K = K; j->N = N; j->bits = bits; j->scale_bf16 = scale_bf16;
    j->x = x; j->packed = packed; j->scales = scales; j->cols = cols; j->ncols = ncols;
    j->c_begin = (int)((long long)ncols * i / nthreads);
    j->c_end = (int)((long long)ncols * (i + 1) / nthreads);
    j->y64 = y64; j->abs_xw = abs_xw; j->abs_xs = abs_xs;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, gemm_worker, &jobs[i]);
  gemm_worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(jobs);
  free(th);
  return 0;
}

/* SwiGLU on exact projections: h = SiLU(g) * u = g * u / (1 + e^-g), fp64.
 * The SwiGLU path of the NInfer-4090 V3 topic ("What V3 did") multiplies the
 * gate projection's SiLU by the up projection; neither is rounded first. */
int oracle_swiglu_f64(int count, const double* g, const double* u, double* h) {
  for (int i = 0; i < count; ++i) h[i] = g[i] * u[i] / (1.0 + exp(-g[i]));
  return 0;
}

/* Round an array of doubles to bf16 bits (RNE from fp64). */
int oracle_round_bf16_array(int count, const double* v, uint16_t* out) {
  for (int i = 0; i < count; ++i) out[i] = oracle_round_bf16(v[i]);
  return 0;
}

/* Per-row RMS rescale used to chain layers of the stack sweep:
 * x'[t][:] = bf16( z[t][:] / sqrt(mean_k z[t][k]^2) ), no epsilon, fp64.
 * The pages describe no such step (it is harness, not method).  A row whose
 * mean square is zero has no scale to divide by; without an epsilon the
 * plainest result is the row itself, i.e. zeros. */
int oracle_rms_rescale(int T, int N, const uint16_t* z, uint16_t* out) {
  for (int t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int n = 0; n < N; ++n) {
      double v = oracle_bf16_to_f64(z[(size_t)t * N + n]);
      ss += v * v;
    }
    double r = sqrt(ss / (double)N);
    for (int n = 0; n < N; ++n)
      out[(size_t)t * N + n] = r > 0.0 ? oracle_round_bf16(oracle_bf16_to_f64(z[(size_t)t * N + n]) / r) : 0;
  }
  return 0;
}
