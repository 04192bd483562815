/*
 * oracle.c -- the CPU oracle for the QLoRA NF4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Plain C11 + pthreads, built with
 * -O2 -fno-fast-math -ffp-contract=off so that every float operation written
 * here is one IEEE operation in the precision written (x86-64 SSE: float is
 * fp32, double is fp64, no excess precision).  Each output element is
 * produced by one thread in a fixed order, so results never depend on the
 * thread count.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* a tiny parallel-for over [0, n)                                           */
/* ------------------------------------------------------------------------ */
typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void* ctx; int64_t lo, hi; } range_job;

static void* range_thread(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) { fn(ctx, 0, n); return; }
  pthread_t tid[256];
  range_job job[256];
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    job[t].fn = fn; job[t].ctx = ctx;
    job[t].lo = n * t / nthreads; job[t].hi = n * (t + 1) / nthreads;
    if (pthread_create(&tid[t], NULL, range_thread, &job[t]) != 0) {
      fn(ctx, job[t].lo, job[t].hi);   /* could not start a thread: do it here */
      tid[t] = 0;
    } else {
      started++;
    }
  }
  for (int t = 0; t < nthreads; ++t)
    if (tid[t]) pthread_join(tid[t], NULL);
  (void)started;
}

/* ------------------------------------------------------------------------ */
/* O1: the NF4 level table.                                                  */
/* Ultralytics "QLoRA", "How QLoRA works", the snippet that builds the       */
/* levels: 8 positive quantiles at probabilities evenly spaced from          */
/* 0.9677083 down to (but excluding) 0.5, 7 negated quantiles at             */
/* probabilities evenly spaced the same way with one step fewer, an exact    */
/* zero, sorted, then divided by the largest value so that the ends are      */
/* -1 and +1.  Evaluated in double and rounded once to fp32.                 */
/* ------------------------------------------------------------------------ */
static double normal_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

double oracle_normal_quantile(double p) {
  /* Phi is strictly increasing: bisect until the bracket cannot shrink. */
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 400; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

static int cmp_double(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x > y) - (x < y);
}

void oracle_nf4_levels(float out[16]) {
  const double offset = 0.9677083;
  double v[16];
  int n = 0;
  for (int i = 0; i < 8; ++i)                      /* 9 points, last (0.5) dropped */
    v[n++] = oracle_normal_quantile(offset + (0.5 - offset) * (double)i / 8.0);
  for (int i = 0; i < 7; ++i)                      /* 8 points, last (0.5) dropped */
    v[n++] = -oracle_normal_quantile(offset + (0.5 - offset) * (double)i / 7.0);
  v[n++] = 0.0;
  qsort(v, 16, sizeof(double), cmp_double);
  double vmax = v[15];
  for (int i = 0; i < 16; ++i) out[i] = (float)(v[i] / vmax);
}

/* ------------------------------------------------------------------------ */
/* O4: nearest level.  "code = argmin |w/absmax - level|" with the first     */
/* index winning a tie (what argmin returns).  The distances are fp32.       */
/* ------------------------------------------------------------------------ */
int oracle_nearest_level(float v, const float levels[16]) {
  int best = 0;
  float bd = fabsf(v - levels[0]);
  for (int i = 1; i < 16; ++i) {
    float d = fabsf(v - levels[i]);
    if (d < bd) { bd = d; best = i; }
  }
  return best;
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN (sign, 4 exponent bits with bias 7, 3 mantissa bits;       */
/* exponent 0 is subnormal m/8 * 2^-6; S.1111.111 is NaN; max 448).          */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Nearest non-negative finite E4M3 value to v >= 0, ties to the even code
 * (codes are ordered like their values, and the code's low bit is the
 * mantissa's low bit).  Values above 448 give 448.  Exactness: every
 * distance compared near a tie is a difference of an fp32 value and an
 * E4M3 value at most 41 bits apart, which double holds exactly. */
uint8_t oracle_e4m3_encode(float v) {
  double x = (double)v;
  int best = 0;
  double bd = fabs(x - oracle_e4m3_value(0));
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(x - oracle_e4m3_value((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) { bd = d; best = c; }
  }
  return (uint8_t)best;
}

/* ------------------------------------------------------------------------ */
/* fp32 -> bf16, round to nearest, ties to even: pick the nearer of the two  */
/* bf16 neighbours (truncation and the next value away from zero).           */
/* ------------------------------------------------------------------------ */
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

uint16_t oracle_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040);
  uint32_t lo = u & 0xFFFF0000u;             /* toward zero */
  uint32_t hi = lo + 0x00010000u;            /* away from zero (may become inf) */
  if (isinf(u2f(lo))) return (uint16_t)(lo >> 16);
  /* past the largest finite bf16 the next step is 2^128 (IEEE overflow rule) */
  double vhi = isinf(u2f(hi)) ? copysign(ldexp(1.0, 128), (double)f) : (double)u2f(hi);
  double dlo = fabs((double)f - (double)u2f(lo));
  double dhi = fabs(vhi - (double)f);
  if (dlo < dhi) return (uint16_t)(lo >> 16);
  if (dhi < dlo) return (uint16_t)(hi >> 16);
  return ((lo >> 16) & 1) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

static double bf16_to_double(uint16_t h) { return (double)u2f((uint32_t)h << 16); }

/* ------------------------------------------------------------------------ */
/* O2-O5: blockwise absmax, nearest-level encode, pack two codes per byte.   */
/* Ultralytics "QLoRA", "How QLoRA works": one absmax scale per block of 64  */
/* weights; each weight divided by its block's absmax and mapped to the      */
/* nearest level.  An all-zero block has no defined quotient: it gets the    */
/* code that v = 0 would get (the exact zero level of NF4; for a codebook    */
/* without zero, the nearer of the two levels around it, the lower on a tie). */
/* ------------------------------------------------------------------------ */
typedef struct {
  const float* W; int64_t cols; const float* levels; uint8_t* codes; float* absmax;
} enc_ctx;

static void enc_range(void* p, int64_t b0, int64_t b1) {
  enc_ctx* c = (enc_ctx*)p;
  const int zero_code = oracle_nearest_level(0.0f, c->levels);
  for (int64_t b = b0; b < b1; ++b) {
    const float* x = c->W + b * 64;
    float a = 0.0f;
    for (int e = 0; e < 64; ++e) { float ax = fabsf(x[e]); if (ax > a) a = ax; }
    if (c->absmax) c->absmax[b] = a;
    uint8_t q[64];
    for (int e = 0; e < 64; ++e) {
      if (a == 0.0f) { q[e] = (uint8_t)zero_code; continue; }
      float v = x[e] / a;                       /* one IEEE fp32 division */
      q[e] = (uint8_t)oracle_nearest_level(v, c->levels);
    }
    for (int e = 0; e < 64; e += 2)
      c->codes[b * 32 + e / 2] = (uint8_t)(q[e] | (q[e + 1] << 4));
  }
}

int oracle_encode_blocks(const float* W, int64_t rows, int64_t cols,
                         const float levels[16], uint8_t* codes, float* absmax_out,
                         int nthreads) {
  if (!W || !levels || !codes || rows <= 0 || cols <= 0 || cols % 64) return -1;
  enc_ctx c = { W, cols, levels, codes, absmax_out };
  parallel_for(rows * cols / 64, nthreads, enc_range, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O6: double quantization of the block scales.                              */
/* Ultralytics "QLoRA" (double quantization bullet): block scales are        */
/* themselves quantized to 8 bits in blocks of 256; vnread "Grokking QLoRA", */
/* "Double Quantization": the 8-bit format is FP8.  Reading taken: OCP E4M3, */
/* each group's largest scale maps to the format's max 448, so the group     */
/* constant is d = max / 448 and each scale is stored as E4M3(absmax / d).   */
/* The NF4 codes use the exact fp32 absmax.  The Ultralytics bullet alone     */
/* ("8 bits") also reads as a plain 8-bit integer grid; that reading is the  */
/* second-level format 2 (uint8-linear, below).                              */
/* ------------------------------------------------------------------------ */
int oracle_quantize(const float* W, int64_t rows, int64_t cols, const float levels[16],
                    int double_quant, uint8_t* codes, uint8_t* qscale, float* dscale,
                    float* absmax_out, int nthreads) {
  if (!W || !levels || !codes || !dscale || (double_quant && !qscale) || rows <= 0 || cols <= 0 ||
      cols % 64 || double_quant < 0 || double_quant > 2)
    return -1;
  int64_t nb = rows * cols / 64;
  float* a = (float*)malloc((size_t)nb * sizeof(float));
  if (!a) return -1;
  int rc = oracle_encode_blocks(W, rows, cols, levels, codes, a, nthreads);
  if (rc) { free(a); return rc; }
  if (!double_quant) {                            /* the block scales kept as fp32 */
    memcpy(dscale, a, (size_t)nb * sizeof(float));
    if (absmax_out) memcpy(absmax_out, a, (size_t)nb * sizeof(float));
    free(a);
    return 0;
  }
  int64_t ng = (nb + 255) / 256;
  for (int64_t g = 0; g < ng; ++g) {
    int64_t b0 = g * 256, b1 = b0 + 256 < nb ? b0 + 256 : nb;
    float c = 0.0f;
    for (int64_t b = b0; b < b1; ++b) if (a[b] > c) c = a[b];
    if (double_quant == 2) {
      /* uint8-linear reading: 256 evenly spaced values 0, d, ..., 255 d with
       * d = max / 255; each scale goes to the nearest multiple of d (the
       * fp32 quotient rounded half to even, at most 255) */
      float d = c / 255.0f;                       /* fp32 division */
      dscale[g] = d;
      for (int64_t b = b0; b < b1; ++b) {
        if (d == 0.0f) { qscale[b] = 0; continue; }
        float t = rintf(a[b] / d);                /* fp32 division, round half to even */
        qscale[b] = (uint8_t)(t > 255.0f ? 255.0f : t);
      }
      continue;
    }
    float d = c / 448.0f;                         /* fp32 division */
    dscale[g] = d;
    for (int64_t b = b0; b < b1; ++b)
      qscale[b] = (d == 0.0f) ? 0 : oracle_e4m3_encode(a[b] / d);
  }
  if (absmax_out) memcpy(absmax_out, a, (size_t)nb * sizeof(float));
  free(a);
  return 0;
}

int oracle_nf4_quantize(const float* W, int64_t rows, int64_t cols, int block, int dq_block,
                        uint8_t* codes, uint8_t* qscale, float* dscale, float* absmax_out,
                        int nthreads) {
  if (block != 64 || dq_block != 256) return -3;
  if (!qscale) return -1;
  float L[16];
  oracle_nf4_levels(L);
  return oracle_quantize(W, rows, cols, L, 1, codes, qscale, dscale, absmax_out, nthreads);
}

/* INT4, the comparison codebook of the Ultralytics "QLoRA" encoding snippet:
 * 16 evenly spaced levels on [-1, 1], L[i] = -1 + 2 i / 15, each rounded once
 * to fp32 (the quotient (2 i - 15) / 15 is formed in double; no value lies
 * near enough to an fp32 midpoint for the double step to matter). */
void oracle_int4_levels(float out[16]) {
  for (int i = 0; i < 16; ++i) out[i] = (float)((double)(2 * i - 15) / 15.0);
}

/* ------------------------------------------------------------------------ */
/* O7: dequantize.  Ultralytics "QLoRA", "How QLoRA works": a weight is      */
/* restored as level[code] times its block scale, and the forward pass uses  */
/* the bfloat16 result.  The block scale is first restored from its E4M3     */
/* code and the group constant.                                              */
/* ------------------------------------------------------------------------ */
typedef struct {
  const uint8_t* codes; const uint8_t* qscale; const float* dscale; int64_t cols;
  uint16_t* out; float L[16]; int double_quant;
} deq_ctx;

static void deq_range(void* p, int64_t b0, int64_t b1) {
  deq_ctx* c = (deq_ctx*)p;
  for (int64_t b = b0; b < b1; ++b) {
    /* E4M3 value (4 significant bits) or an 8-bit integer times an fp32:
     * exact in double, then rounded once; without double quantization the
     * fp32 scale itself */
    float s = c->double_quant == 1 ? (float)(oracle_e4m3_value(c->qscale[b]) * (double)c->dscale[b / 256])
            : c->double_quant == 2 ? (float)((double)c->qscale[b] * (double)c->dscale[b / 256])
                                   : c->dscale[b];
    for (int e = 0; e < 64; ++e) {
      uint8_t byte = c->codes[b * 32 + e / 2];
      int code = (e & 1) ? (byte >> 4) : (byte & 15);
      float w = c->L[code] * s;                  /* fp32 multiply */
      c->out[b * 64 + e] = oracle_bf16_rne(w);
    }
  }
}

int oracle_dequantize(const uint8_t* codes, const uint8_t* qscale, const float* dscale,
                      int64_t rows, int64_t cols, const float levels[16], int double_quant,
                      uint16_t* out_bf16, int nthreads) {
  if (!codes || (double_quant && !qscale) || !dscale || !levels || !out_bf16 || rows <= 0 ||
      cols <= 0 || cols % 64 || double_quant < 0 || double_quant > 2)
    return -1;
  deq_ctx c;
  c.codes = codes; c.qscale = qscale; c.dscale = dscale; c.cols = cols; c.out = out_bf16;
  c.double_quant = double_quant;
  memcpy(c.L, levels, sizeof(c.L));
  parallel_for(rows * cols / 64, nthreads, deq_range, &c);
  return 0;
}

int oracle_nf4_dequantize(const uint8_t* codes, const uint8_t* qscale, const float* dscale,
                          int64_t rows, int64_t cols, uint16_t* out_bf16, int nthreads) {
  if (!qscale) return -1;
  float L[16];
  oracle_nf4_levels(L);
  return oracle_dequantize(codes, qscale, dscale, rows, cols, L, 1, out_bf16, nthreads);
}

/* ------------------------------------------------------------------------ */
/* O8: forward.  Ultralytics "QLoRA", "How QLoRA works": each frozen layer    */
/* dequantizes to bfloat16 just before the matrix product and then adds the  */
/* LoRA path; ezsol "Mastering model fine-tuning" (LoRA): Delta W = B A;     */
/* IBM "What is LoRA?": lora_alpha is the scaling factor (applied as         */
/* alpha / r).  bf16 inputs are exact in double; sums run over the index in  */
/* increasing order in double.                                               */
/* ------------------------------------------------------------------------ */
typedef struct {
  const uint16_t* Wdq; int64_t N, K; const uint16_t* X; const uint16_t* A; const uint16_t* B;
  int r; double s; const int64_t* row_idx; double* Y; double* T;
} fwd_ctx;

static void fwd_range(void* p, int64_t i0, int64_t i1) {
  fwd_ctx* c = (fwd_ctx*)p;
  double* t = (double*)malloc((size_t)c->r * sizeof(double));
  for (int64_t i = i0; i < i1; ++i) {
    int64_t m = c->row_idx ? c->row_idx[i] : i;
    const uint16_t* x = c->X + m * c->K;
    for (int j = 0; j < c->r; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < c->K; ++k)
        acc += bf16_to_double(x[k]) * bf16_to_double(c->A[(int64_t)j * c->K + k]);
      t[j] = acc;
      if (c->T) c->T[i * c->r + j] = acc;
    }
    for (int64_t n = 0; n < c->N; ++n) {
      const uint16_t* w = c->Wdq + n * c->K;
      double base = 0.0;
      for (int64_t k = 0; k < c->K; ++k) base += bf16_to_double(x[k]) * bf16_to_double(w[k]);
      double lora = 0.0;
      for (int j = 0; j < c->r; ++j) lora += t[j] * bf16_to_double(c->B[n * c->r + j]);
      c->Y[i * c->N + n] = base + c->s * lora;
    }
  }
  free(t);
}

int oracle_qlora_fwd(const uint16_t* Wdq, int64_t N, int64_t K,
                     const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                     int r, double alpha, const int64_t* row_idx, int64_t n_rows,
                     double* Y_out, double* T_out, int nthreads) {
  if (!Wdq || !X || !A || !B || !Y_out || N <= 0 || K <= 0 || M <= 0 || r <= 0) return -1;
  if (!row_idx) n_rows = M;
  for (int64_t i = 0; row_idx && i < n_rows; ++i)
    if (row_idx[i] < 0 || row_idx[i] >= M) return -2;
  fwd_ctx c = { Wdq, N, K, X, A, B, r, alpha / (double)r, row_idx, Y_out, T_out };
  parallel_for(n_rows, nthreads, fwd_range, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O9: backward.  Ultralytics "QLoRA", "How QLoRA works": gradients flow     */
/* through the dequantized weights, and only the two LoRA matrices are       */
/* updated (the frozen base gets no gradient).  With Y = X W'^T + s X A^T B^T */
/* and upstream gradient dY:                                                  */
/*   dX = dY W' + s (dY B) A,  dA = s (dY B)^T X,  dB = s dY^T (X A^T).       */
/* ------------------------------------------------------------------------ */
typedef struct {
  const uint16_t* Wdq; int64_t N, K; const uint16_t* dY; const uint16_t* A; const uint16_t* B;
  int r; double s; const int64_t* row_idx; double* dX;
} dx_ctx;

static void dx_range(void* p, int64_t i0, int64_t i1) {
  dx_ctx* c = (dx_ctx*)p;
  double* u = (double*)malloc((size_t)c->r * sizeof(double));
  double* row = (double*)malloc((size_t)c->K * sizeof(double));
  for (int64_t i = i0; i < i1; ++i) {
    int64_t m = c->row_idx ? c->row_idx[i] : i;
    const uint16_t* g = c->dY + m * c->N;
    for (int j = 0; j < c->r; ++j) {
      double acc = 0.0;
      for (int64_t n = 0; n < c->N; ++n)
        acc += bf16_to_double(g[n]) * bf16_to_double(c->B[n * c->r + j]);
      u[j] = acc;
    }
    /* base term: for each k, sum over n in increasing order (row by row of W') */
    for (int64_t k = 0; k < c->K; ++k) row[k] = 0.0;
    for (int64_t n = 0; n < c->N; ++n) {
      double gn = bf16_to_double(g[n]);
      const uint16_t* w = c->Wdq + n * c->K;
      for (int64_t k = 0; k < c->K; ++k) row[k] += gn * bf16_to_double(w[k]);
    }
    for (int64_t k = 0; k < c->K; ++k) {
      double lora = 0.0;
      for (int j = 0; j < c->r; ++j) lora += u[j] * bf16_to_double(c->A[(int64_t)j * c->K + k]);
      c->dX[i * c->K + k] = row[k] + c->s * lora;
    }
  }
  free(row);
  free(u);
}

int oracle_qlora_bwd_dx(const uint16_t* Wdq, int64_t N, int64_t K,
                        const uint16_t* dY, int64_t M, const uint16_t* A, const uint16_t* B,
                        int r, double alpha, const int64_t* row_idx, int64_t n_rows,
                        double* dX_out, int nthreads) {
  if (!Wdq || !dY || !A || !B || !dX_out || N <= 0 || K <= 0 || M <= 0 || r <= 0) return -1;
  if (!row_idx) n_rows = M;
  for (int64_t i = 0; row_idx && i < n_rows; ++i)
    if (row_idx[i] < 0 || row_idx[i] >= M) return -2;
  dx_ctx c = { Wdq, N, K, dY, A, B, r, alpha / (double)r, row_idx, dX_out };
  parallel_for(n_rows, nthreads, dx_range, &c);
  return 0;
}

/* T = X A^T and U = dY B in double, one row of M per task.  Every element  */
/* is one sum in increasing contraction order (k for T, n for U); U keeps a  */
/* running sum per rank and walks dY and B row by row.                       */
typedef struct {
  int64_t N, K; const uint16_t* X; const uint16_t* dY; const uint16_t* A; const uint16_t* B;
  int r; double* T; double* U;
} tu_ctx;

static void tu_range(void* p, int64_t m0, int64_t m1) {
  tu_ctx* c = (tu_ctx*)p;
  for (int64_t m = m0; m < m1; ++m) {
    for (int j = 0; j < c->r; ++j) {
      double t = 0.0;
      for (int64_t k = 0; k < c->K; ++k)
        t += bf16_to_double(c->X[m * c->K + k]) * bf16_to_double(c->A[(int64_t)j * c->K + k]);
      c->T[m * c->r + j] = t;
    }
    double* u = c->U + m * c->r;
    for (int j = 0; j < c->r; ++j) u[j] = 0.0;
    for (int64_t n = 0; n < c->N; ++n) {
      const double g = bf16_to_double(c->dY[m * c->N + n]);
      const uint16_t* b = c->B + n * c->r;
      for (int j = 0; j < c->r; ++j) u[j] += g * bf16_to_double(b[j]);
    }
  }
}

typedef struct {
  int64_t M, N, K; const uint16_t* X; const uint16_t* dY; int r; double s;
  const double* T; const double* U; double* dA; double* dB;
} ad_ctx;

/* Columns of dA and rows of dB in chunks of AD_CHUNK: tasks [0, ka) take    */
/* columns [AD_CHUNK t, AD_CHUNK t + AD_CHUNK) of dA, tasks [ka, ka + nb)    */
/* rows of dB.  Each element is one sum over m in increasing order;          */
/* walking m in the outer loop keeps the reads of X, dY, U and T sequential. */
#define AD_CHUNK 32
static void ad_range(void* p, int64_t t0, int64_t t1) {
  ad_ctx* c = (ad_ctx*)p;
  const int64_t ka = (c->K + AD_CHUNK - 1) / AD_CHUNK;
  double* acc = (double*)malloc((size_t)c->r * AD_CHUNK * sizeof(double));
  if (!acc) abort();   /* no result is better than a wrong one */
  for (int64_t t = t0; t < t1; ++t) {
    if (t < ka) {
      if (!c->dA) continue;
      const int64_t k0 = t * AD_CHUNK, kn = (c->K - k0 < AD_CHUNK) ? c->K - k0 : AD_CHUNK;
      for (int64_t i = 0; i < (int64_t)c->r * AD_CHUNK; ++i) acc[i] = 0.0;
      for (int64_t m = 0; m < c->M; ++m) {
        const uint16_t* x = c->X + m * c->K + k0;
        const double* u = c->U + m * c->r;
        for (int j = 0; j < c->r; ++j) {
          double* a = acc + (int64_t)j * AD_CHUNK;
          for (int64_t kk = 0; kk < kn; ++kk) a[kk] += u[j] * bf16_to_double(x[kk]);
        }
      }
      for (int j = 0; j < c->r; ++j)
        for (int64_t kk = 0; kk < kn; ++kk)
          c->dA[(int64_t)j * c->K + k0 + kk] = c->s * acc[(int64_t)j * AD_CHUNK + kk];
    } else {
      if (!c->dB) continue;
      const int64_t n0 = (t - ka) * AD_CHUNK, nn = (c->N - n0 < AD_CHUNK) ? c->N - n0 : AD_CHUNK;
      for (int64_t i = 0; i < (int64_t)c->r * AD_CHUNK; ++i) acc[i] = 0.0;
      for (int64_t m = 0; m < c->M; ++m) {
        const uint16_t* g = c->dY + m * c->N + n0;
        const double* tm = c->T + m * c->r;
        for (int64_t i = 0; i < nn; ++i) {
          const double gv = bf16_to_double(g[i]);
          double* a = acc + i * c->r;
          for (int j = 0; j < c->r; ++j) a[j] += gv * tm[j];
        }
      }
      for (int64_t i = 0; i < nn; ++i)
        for (int j = 0; j < c->r; ++j) c->dB[(n0 + i) * c->r + j] = c->s * acc[i * c->r + j];
    }
  }
  free(acc);
}

int oracle_qlora_bwd_adapters(int64_t N, int64_t K, const uint16_t* X, const uint16_t* dY,
                              int64_t M, const uint16_t* A, const uint16_t* B, int r,
                              double alpha, double* dA_out, double* dB_out, int nthreads) {
  if (!X || !dY || !A || !B || N <= 0 || K <= 0 || M <= 0 || r <= 0) return -1;
  double* T = (double*)malloc((size_t)(M * r) * sizeof(double));
  double* U = (double*)malloc((size_t)(M * r) * sizeof(double));
  if (!T || !U) { free(T); free(U); return -1; }
  tu_ctx tc = { N, K, X, dY, A, B, r, T, U };
  parallel_for(M, nthreads, tu_range, &tc);
  ad_ctx ac = { M, N, K, X, dY, r, alpha / (double)r, T, U, dA_out, dB_out };
  parallel_for((K + AD_CHUNK - 1) / AD_CHUNK + (N + AD_CHUNK - 1) / AD_CHUNK, nthreads, ad_range, &ac);
  free(T);
  free(U);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Selected dA / dB entries.  Same definitions as above: columns of U and T  */
/* in double for the ranks the entries use, then one sum over m per entry.   */
/* ------------------------------------------------------------------------ */
typedef struct {
  int64_t N, K, M; const uint16_t* X; const uint16_t* dY; const uint16_t* A; const uint16_t* B;
  int r; const int* need_u; const int* need_t; double* Ucol; double* Tcol;
} col_ctx;

static void col_range(void* p, int64_t m0, int64_t m1) {
  col_ctx* c = (col_ctx*)p;
  for (int64_t m = m0; m < m1; ++m) {
    for (int j = 0; j < c->r; ++j) {
      if (c->need_u[j]) {
        double u = 0.0;
        for (int64_t n = 0; n < c->N; ++n)
          u += bf16_to_double(c->dY[m * c->N + n]) * bf16_to_double(c->B[n * c->r + j]);
        c->Ucol[(int64_t)j * c->M + m] = u;
      }
      if (c->need_t[j]) {
        double t = 0.0;
        for (int64_t k = 0; k < c->K; ++k)
          t += bf16_to_double(c->X[m * c->K + k]) * bf16_to_double(c->A[(int64_t)j * c->K + k]);
        c->Tcol[(int64_t)j * c->M + m] = t;
      }
    }
  }
}

int oracle_qlora_adapter_entries(int64_t N, int64_t K, const uint16_t* X, const uint16_t* dY,
                                 int64_t M, const uint16_t* A, const uint16_t* B, int r,
                                 double alpha, int64_t n_dA, const int64_t* dA_j,
                                 const int64_t* dA_k, double* dA_out, int64_t n_dB,
                                 const int64_t* dB_n, const int64_t* dB_j, double* dB_out,
                                 int nthreads) {
  if (!X || !dY || !A || !B || N <= 0 || K <= 0 || M <= 0 || r <= 0) return -1;
  int* need_u = (int*)calloc((size_t)r, sizeof(int));
  int* need_t = (int*)calloc((size_t)r, sizeof(int));
  if (!need_u || !need_t) { free(need_u); free(need_t); return -1; }
  for (int64_t i = 0; i < n_dA; ++i) {
    if (dA_j[i] < 0 || dA_j[i] >= r || dA_k[i] < 0 || dA_k[i] >= K) { free(need_u); free(need_t); return -2; }
    need_u[dA_j[i]] = 1;
  }
  for (int64_t i = 0; i < n_dB; ++i) {
    if (dB_j[i] < 0 || dB_j[i] >= r || dB_n[i] < 0 || dB_n[i] >= N) { free(need_u); free(need_t); return -2; }
    need_t[dB_j[i]] = 1;
  }
  double* Ucol = (double*)malloc((size_t)(M * r) * sizeof(double));
  double* Tcol = (double*)malloc((size_t)(M * r) * sizeof(double));
  if (!Ucol || !Tcol) { free(Ucol); free(Tcol); free(need_u); free(need_t); return -1; }
  col_ctx cc = { N, K, M, X, dY, A, B, r, need_u, need_t, Ucol, Tcol };
  parallel_for(M, nthreads, col_range, &cc);
  const double s = alpha / (double)r;
  for (int64_t i = 0; i < n_dA; ++i) {
    double acc = 0.0;
    for (int64_t m = 0; m < M; ++m)
      acc += Ucol[dA_j[i] * M + m] * bf16_to_double(X[m * K + dA_k[i]]);
    dA_out[i] = s * acc;
  }
  for (int64_t i = 0; i < n_dB; ++i) {
    double acc = 0.0;
    for (int64_t m = 0; m < M; ++m)
      acc += bf16_to_double(dY[m * N + dB_n[i]]) * Tcol[dB_j[i] * M + m];
    dB_out[i] = s * acc;
  }
  free(Ucol); free(Tcol); free(need_u); free(need_t);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* bf16 RNE of a double.  The candidates are the bf16 value whose pattern is  */
/* the top half of the nearest float and its two neighbours of the same sign */
/* (the exact value lies within one float step of that float, so it is       */
/* bracketed by two of them); the nearest wins, ties go to the even pattern. */
/* Past the largest finite bf16 the next step is 2^128 (IEEE overflow rule). */
/* ------------------------------------------------------------------------ */
static double bf16_value_for_rounding(uint16_t h) {
  if ((h & 0x7FFF) == 0x7F80) return (h & 0x8000) ? -ldexp(1.0, 128) : ldexp(1.0, 128);
  return bf16_to_double(h);
}

uint16_t oracle_bf16_rne_double(double x) {
  if (isnan(x)) return 0x7FC0;
  const uint16_t c = (uint16_t)(f2u((float)x) >> 16);
  const uint16_t sign = c & 0x8000, mag = c & 0x7FFF;
  uint16_t cand[3];
  int n = 0;
  if (mag > 0) cand[n++] = (uint16_t)(sign | (mag - 1));
  cand[n++] = c;
  if (mag < 0x7F80) cand[n++] = (uint16_t)(sign | (mag + 1));
  uint16_t best = cand[0];
  double bd = fabs(bf16_value_for_rounding(cand[0]) - x);
  for (int i = 1; i < n; ++i) {
    const double d = fabs(bf16_value_for_rounding(cand[i]) - x);
    if (d < bd || (d == bd && (cand[i] & 1) == 0)) { best = cand[i]; bd = d; }
  }
  /* a finite x never rounds to a value of the other sign, and zero keeps x's sign */
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  return best;
}

/* ------------------------------------------------------------------------ */
/* Merge / unmerge (IBM "What is LoRA?"; Ultralytics "QLoRA", "Trade-offs"):  */
/* W_out = bf16(W_base + sign (alpha/r) B A), one rounding per element.       */
/* ------------------------------------------------------------------------ */
typedef struct {
  const uint16_t* W; int64_t N, K; const uint16_t* A; const uint16_t* B; int r; double s;
  uint16_t* out;
} merge_ctx;

static void merge_range(void* p, int64_t n0, int64_t n1) {
  merge_ctx* c = (merge_ctx*)p;
  double* row = (double*)malloc((size_t)c->K * sizeof(double));
  for (int64_t n = n0; n < n1; ++n) {
    for (int64_t k = 0; k < c->K; ++k) row[k] = 0.0;
    for (int j = 0; j < c->r; ++j) {
      const double b = bf16_to_double(c->B[n * c->r + j]);
      const uint16_t* a = c->A + (int64_t)j * c->K;
      for (int64_t k = 0; k < c->K; ++k) row[k] += b * bf16_to_double(a[k]);
    }
    for (int64_t k = 0; k < c->K; ++k)
      c->out[n * c->K + k] = oracle_bf16_rne_double(bf16_to_double(c->W[n * c->K + k]) + c->s * row[k]);
  }
  free(row);
}

int oracle_lora_merge(const uint16_t* W_base, int64_t N, int64_t K, const uint16_t* A,
                      const uint16_t* B, int r, double alpha, int sign, uint16_t* W_out,
                      int nthreads) {
  if (!W_base || !A || !B || !W_out || N <= 0 || K <= 0 || r <= 0 || (sign != 1 && sign != -1)) return -1;
  merge_ctx c = { W_base, N, K, A, B, r, (double)sign * alpha / (double)r, W_out };
  parallel_for(N, nthreads, merge_range, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Gated activation of the gate and up projections: H = silu(G) * U.        */
/* ------------------------------------------------------------------------ */
void oracle_swiglu(const double* G, const double* U, int64_t n, double* H) {
  for (int64_t i = 0; i < n; ++i) {
    const double g = G[i];
    H[i] = g / (1.0 + exp(-g)) * U[i];
  }
}

/* ------------------------------------------------------------------------ */
/* Adapter optimizer step: Adam with bias correction and decoupled weight   */
/* decay (the state that the paged optimizers of the pages hold).            */
/* ------------------------------------------------------------------------ */
void oracle_adamw_step(double* theta, double* m, double* v, const double* g, int64_t n, double lr,
                       double b1, double b2, double eps, double wd, int t) {
  const double bc1 = 1.0 - pow(b1, (double)t);
  const double bc2 = 1.0 - pow(b2, (double)t);
  for (int64_t i = 0; i < n; ++i) {
    double th = theta[i] * (1.0 - lr * wd);
    m[i] = b1 * m[i] + (1.0 - b1) * g[i];
    v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
    th -= lr * (m[i] / bc1) / (sqrt(v[i] / bc2) + eps);
    theta[i] = th;
  }
}
