/*
 * lin_attn_oracle.c -- slow, plain fp64 CPU oracle for causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Its only users are the tests under tests/, the
 * smoke check in __graft_entry__.smoke() and the CPU baseline leg of bench.py.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What it computes (the plain definition, nothing reordered or blocked):
 *
 *   "MiniMax-M1で理解する：大規模言語モデルのコンテキスト長限界を突破する
 *   革新的アーキテクチャ" (zenn.dev/liushuzhi), section
 *   "線形アテンションの数学的基礎": linear attention with a feature map phi,
 *   computed through its recurrent form
 *        S_t = S_{t-1} + phi(k_t) v_t^T,       o_t = phi(q_t) S_t ,
 *   with a state S in R^{D x d} whose update costs O(Dd) per token.
 *
 *   Readings taken where the page is silent: phi is the identity (D = d), no
 *   decay, no normaliser, no 1/sqrt(d) scale; o_t reads the state AFTER the
 *   token's own k_t v_t^T was added (so the causal mask includes the
 *   diagonal); S[i][j] has row i = key feature, column j = value feature.
 *
 * The tiled ("Lightning") form is an exact re-association of the same sums
 * ("Почему M2 в итоге стала моделью с полным вниманием?" (ai.flicky.cc),
 * section 1, glossary entry "Lightning Attention": a masked matrix inside a
 * block and a K^T V state between blocks), so this token-by-token loop is
 * the oracle for every block size.
 *
 * Inputs arrive as float32 arrays: fp32 and bf16 values are both exactly
 * representable in fp32, and every value is widened to double exactly before
 * use.  All arithmetic is IEEE double; build without -ffast-math and with
 * -ffp-contract=off.
 *
 * The bf16-stored-state variant (lao_decode_bf16_state) models a state that
 * is kept in bfloat16 between steps -- the low-precision storage hazard that
 * "ノーフリーランチ：MiniMax M2が高効率アテンション機構を解体"
 * (winzheng.jp), section "推論システム統合の課題", and section 4 of the
 * ai.flicky.cc digest describe: the state is widened to double, updated,
 * read out, then rounded to bf16 (round to nearest, ties to even) once.
 *
 * lao_recurrence_stored_state generalises it: the state is stored every
 * `block` tokens in bf16 or in OCP FP8 E4M3 (the format those pages name as
 * the extreme case), with a per-head scale, and the tokens in between run
 * through the exact recurrence above from the widened store.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { LAO_OK = 0, LAO_EINVAL = -1, LAO_ENOMEM = -2 };

/* ---------------------------------------------------------------------- */
/* One (batch, head) recurrence.                                           */
/* q, k, v : [N][d] float32 ; o : [N][d] double (out) ;                    */
/* S : [d][d] double (in: S_0, out: S_N).                                  */
/* ---------------------------------------------------------------------- */
static void recurrence_one_head(const float *q, const float *k,
                                const float *v, double *o, double *S,
                                int64_t N, int64_t d) {
  for (int64_t t = 0; t < N; ++t) {
    const float *qt = q + t * d;
    const float *kt = k + t * d;
    const float *vt = v + t * d;
    double *ot = o + t * d;
    /* S_t = S_{t-1} + k_t v_t^T */
    for (int64_t i = 0; i < d; ++i) {
      const double ki = (double)kt[i];
      double *Si = S + i * d;
      for (int64_t j = 0; j < d; ++j) Si[j] += ki * (double)vt[j];
    }
    /* o_t[j] = sum_i q_t[i] S_t[i][j] */
    for (int64_t j = 0; j < d; ++j) ot[j] = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      const double qi = (double)qt[i];
      const double *Si = S + i * d;
      for (int64_t j = 0; j < d; ++j) ot[j] += qi * Si[j];
    }
  }
}

/* Round a double to the nearest bfloat16, ties to even; returns the bf16 bit
 * pattern.  Written from the format's definition: 1 sign bit, 8 exponent
 * bits (same as binary32), 7 stored fraction bits.  The value is scaled so
 * that the bf16 grid of its binade becomes the integers, rounded once with
 * rint() (nearest, ties to even, in the default rounding mode), and scaled
 * back; there is no intermediate rounding to binary32. */
static uint16_t double_to_bf16_rne(double x) {
  if (isnan(x)) return (uint16_t)0x7fc0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  /* bf16 largest finite = (2 - 2^-7) * 2^127; halfway to 2^128 rounds up */
  const double max_finite = ldexp(2.0 - ldexp(1.0, -7), 127);
  const double overflow_edge = ldexp(2.0 - ldexp(1.0, -8), 127);
  if (a >= overflow_edge) return (uint16_t)(sign | 0x7f80); /* inf */
  int e;
  frexp(a, &e);           /* a = m * 2^e, m in [0.5, 1) */
  int unb = e - 1;        /* a in [2^unb, 2^(unb+1)) */
  if (unb < -126) unb = -126; /* subnormal range uses the smallest exponent */
  /* spacing of bf16 values in this binade: 2^(unb-7) */
  double scaled = ldexp(a, 7 - unb); /* in [128, 256) for normals */
  double r = rint(scaled);           /* nearest, ties to even */
  double y = ldexp(r, unb - 7);
  if (y > max_finite) return (uint16_t)(sign | 0x7f80);
  /* encode y exactly */
  float f = (float)y; /* exact: y has <= 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | ((bits >> 16) & 0x7fff));
}

static double bf16_to_double(uint16_t b) {
  uint32_t bits = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Round a double to the nearest OCP FP8 E4M3 value ("e4m3fn"), ties to
 * even, saturating; returns the 8-bit code.  Written from the format's
 * definition: 1 sign bit, 4 exponent bits with bias 7, 3 stored fraction
 * bits; exponent field 0 holds the subnormals f * 2^-9 (f = 0..7); the code
 * S.1111.111 is NaN and there is no infinity, so the largest finite value is
 * 1.75 * 2^8 = 448.  Reading taken for values beyond the range: they are
 * clamped to +-448 (a stored state must stay finite; the conversion that the
 * pages' FP8 storage implies is not specified further).  As for bf16, the
 * value is scaled so that the grid of its binade becomes the integers and
 * rounded once with rint(). */
static uint8_t double_to_e4m3_rne_sat(double x) {
  uint8_t sign = signbit(x) ? 0x80 : 0;
  if (isnan(x)) return (uint8_t)(sign | 0x7f);
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (a >= 448.0) return (uint8_t)(sign | 0x7e);
  int e;
  frexp(a, &e);
  int unb = e - 1;            /* a in [2^unb, 2^(unb+1)) */
  if (unb < -6) unb = -6;     /* subnormals share the smallest exponent */
  double r = rint(ldexp(a, 3 - unb)); /* grid step 2^(unb-3) */
  double y = ldexp(r, unb - 3);
  if (y > 448.0) y = 448.0;   /* rounded past the largest finite value */
  if (y < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)r); /* subnormal, r in 0..7 */
  frexp(y, &e);
  unb = e - 1;                                 /* may have moved up a binade */
  int mant = (int)ldexp(y, 3 - unb);           /* 8 .. 15 */
  return (uint8_t)(sign | ((unb + 7) << 3) | (mant - 8));
}

static double e4m3_to_double(uint8_t c) {
  const int e = (c >> 3) & 15, f = c & 7;
  double y;
  if (e == 15 && f == 7) y = NAN;
  else if (e == 0) y = ldexp((double)f, -9);
  else y = ldexp((double)(8 + f), e - 10);
  return (c & 0x80) ? -y : y;
}

/* A state kept in a narrow format between uses: entry x is stored as the
 * code of x / scale and read back as value(code) * scale. */
enum { LAO_FMT_BF16 = 1, LAO_FMT_E4M3 = 2 };

static double stored_to_double(const void *codes, int64_t i, int fmt, double scale) {
  if (fmt == LAO_FMT_BF16) return bf16_to_double(((const uint16_t *)codes)[i]) * scale;
  return e4m3_to_double(((const uint8_t *)codes)[i]) * scale;
}

static void double_to_stored(void *codes, int64_t i, int fmt, double x, double scale) {
  if (fmt == LAO_FMT_BF16) ((uint16_t *)codes)[i] = double_to_bf16_rne(x / scale);
  else ((uint8_t *)codes)[i] = double_to_e4m3_rne_sat(x / scale);
}

/* The recurrence over N tokens with the state stored in a narrow format every
 * `block` tokens ("ノーフリーランチ" (winzheng.jp), section
 * "推論システム統合の課題": FP8 or other low-precision storage of a state that
 * is rewritten again and again).  The stored state is widened, the tokens of
 * one block run through the exact recurrence from it (so every output of the
 * block reads the widened carry plus its block's own exact terms), and the
 * result is rounded back into the store.  block = 1 is the decode step of a
 * low-precision state; block = N stores only the final state. */
static void stored_state_one_head(const float *q, const float *k, const float *v,
                                  double *o, void *codes, int fmt, double scale,
                                  double *work, int64_t N, int64_t d, int64_t block) {
  const int64_t dd = d * d;
  for (int64_t i = 0; i < dd; ++i) work[i] = stored_to_double(codes, i, fmt, scale);
  for (int64_t t0 = 0; t0 < N; t0 += block) {
    const int64_t n = (N - t0 < block) ? N - t0 : block;
    recurrence_one_head(q + t0 * d, k + t0 * d, v + t0 * d, o + t0 * d, work, n, d);
    for (int64_t i = 0; i < dd; ++i) {
      double_to_stored(codes, i, fmt, work[i], scale);
      work[i] = stored_to_double(codes, i, fmt, scale);
    }
  }
}

/* One decode token step per head with the state stored as bf16. */
static void decode_bf16_state_one_head(const float *q, const float *k,
                                       const float *v, double *o,
                                       uint16_t *Sb, double *work,
                                       int64_t d) {
  for (int64_t i = 0; i < d; ++i)
    for (int64_t j = 0; j < d; ++j) work[i * d + j] = bf16_to_double(Sb[i * d + j]);
  recurrence_one_head(q, k, v, o, work, 1, d);
  for (int64_t i = 0; i < d; ++i)
    for (int64_t j = 0; j < d; ++j) Sb[i * d + j] = double_to_bf16_rne(work[i * d + j]);
}

/* ---------------------------------------------------------------------- */
/* Thread fan-out over heads.                                              */
/* ---------------------------------------------------------------------- */
typedef struct {
  const float *q, *k, *v;
  double *o;
  double *S;
  uint16_t *Sb;
  int64_t nheads, N, d;
  int64_t next_head; /* guarded by mu */
  pthread_mutex_t mu;
  int bf16_state;
  int fmt;              /* stored-state recurrence: LAO_FMT_*, else 0 */
  void *codes;          /* [nheads][d][d] codes of the stored state */
  const float *scale;   /* [nheads] or NULL (1.0) */
  int64_t block;        /* tokens between stores */
} job_t;

static void *worker(void *arg) {
  job_t *jb = (job_t *)arg;
  double *work = NULL;
  if (jb->bf16_state || jb->fmt) {
    work = (double *)malloc(sizeof(double) * (size_t)(jb->d * jb->d));
    if (!work) return (void *)1;
  }
  for (;;) {
    pthread_mutex_lock(&jb->mu);
    int64_t h = jb->next_head++;
    pthread_mutex_unlock(&jb->mu);
    if (h >= jb->nheads) break;
    const int64_t td = jb->N * jb->d;
    if (jb->fmt) {
      const size_t es = jb->fmt == LAO_FMT_BF16 ? 2 : 1;
      stored_state_one_head(jb->q + h * td, jb->k + h * td, jb->v + h * td, jb->o + h * td,
                            (char *)jb->codes + (size_t)(h * jb->d * jb->d) * es, jb->fmt,
                            jb->scale ? (double)jb->scale[h] : 1.0, work, jb->N, jb->d,
                            jb->block);
    } else if (jb->bf16_state)
      decode_bf16_state_one_head(jb->q + h * td, jb->k + h * td, jb->v + h * td,
                                 jb->o + h * td, jb->Sb + h * jb->d * jb->d, work,
                                 jb->d);
    else
      recurrence_one_head(jb->q + h * td, jb->k + h * td, jb->v + h * td,
                          jb->o + h * td, jb->S + h * jb->d * jb->d, jb->N, jb->d);
  }
  free(work);
  return NULL;
}

static int run_job(job_t *jb, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > jb->nheads) nthreads = (int)(jb->nheads > 0 ? jb->nheads : 1);
  pthread_mutex_init(&jb->mu, NULL);
  jb->next_head = 0;
  int rc = LAO_OK;
  if (nthreads == 1) {
    if (worker(jb) != NULL) rc = LAO_ENOMEM;
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) {
      pthread_mutex_destroy(&jb->mu);
      return LAO_ENOMEM;
    }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
      if (pthread_create(&th[i], NULL, worker, jb) != 0) break;
      ++started;
    }
    if (started == 0) { /* no threads at all: run inline */
      if (worker(jb) != NULL) rc = LAO_ENOMEM;
    }
    for (int i = 0; i < started; ++i) {
      void *ret = NULL;
      pthread_join(th[i], &ret);
      if (ret != NULL) rc = LAO_ENOMEM;
    }
    free(th);
  }
  pthread_mutex_destroy(&jb->mu);
  return rc;
}

/* ---------------------------------------------------------------------- */
/* Exported entry points (called from oracle/oracle.py through ctypes).    */
/* ---------------------------------------------------------------------- */

/* Token-by-token recurrence over `nheads` independent (batch, head) pairs.
 * q, k, v : [nheads][N][d] float32 ; o : [nheads][N][d] double (out) ;
 * state : [nheads][d][d] double, in: S_0, out: S_N.
 * A decode step is the same call with N = 1. */
int lao_recurrence(const float *q, const float *k, const float *v, double *o,
                   double *state, int64_t nheads, int64_t N, int64_t d,
                   int nthreads) {
  if (nheads < 0 || N < 0 || d <= 0) return LAO_EINVAL;
  if (nheads == 0 || N == 0) return LAO_OK;
  if (!q || !k || !v || !o || !state) return LAO_EINVAL;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.q = q; jb.k = k; jb.v = v; jb.o = o; jb.S = state;
  jb.nheads = nheads; jb.N = N; jb.d = d; jb.bf16_state = 0;
  return run_job(&jb, nthreads);
}

/* One decode step per head with a bf16-stored state (in place).
 * q, k, v : [nheads][d] float32 ; o : [nheads][d] double (out) ;
 * state_bf16 : [nheads][d][d] bf16 bit patterns, in and out. */
int lao_decode_bf16_state(const float *q, const float *k, const float *v,
                          double *o, uint16_t *state_bf16, int64_t nheads,
                          int64_t d, int nthreads) {
  if (nheads < 0 || d <= 0) return LAO_EINVAL;
  if (nheads == 0) return LAO_OK;
  if (!q || !k || !v || !o || !state_bf16) return LAO_EINVAL;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.q = q; jb.k = k; jb.v = v; jb.o = o; jb.Sb = state_bf16;
  jb.nheads = nheads; jb.N = 1; jb.d = d; jb.bf16_state = 1;
  return run_job(&jb, nthreads);
}

/* Exposed so the tests can pin the rounding against an independent library
 * conversion. */
void lao_round_bf16(const double *x, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = double_to_bf16_rne(x[i]);
}

/* Recurrence with a state stored in a narrow format every `block` tokens
 * (and after the last token).
 * q, k, v : [nheads][N][d] float32 ; o : [nheads][N][d] double (out) ;
 * codes   : [nheads][d][d] uint16 bf16 patterns (fmt 1) or uint8 OCP E4M3
 *           codes (fmt 2), in: S_0, out: S_N ;
 * scale   : [nheads] positive finite, or NULL for 1.0. */
int lao_recurrence_stored_state(const float *q, const float *k, const float *v, double *o,
                                void *codes, int fmt, const float *scale, int64_t nheads,
                                int64_t N, int64_t d, int64_t block, int nthreads) {
  if (nheads < 0 || N < 0 || d <= 0 || block < 1) return LAO_EINVAL;
  if (fmt != LAO_FMT_BF16 && fmt != LAO_FMT_E4M3) return LAO_EINVAL;
  if (nheads == 0 || N == 0) return LAO_OK;
  if (!q || !k || !v || !o || !codes) return LAO_EINVAL;
  if (scale)
    for (int64_t h = 0; h < nheads; ++h)
      if (!(scale[h] > 0.0f) || isinf(scale[h])) return LAO_EINVAL;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.q = q; jb.k = k; jb.v = v; jb.o = o;
  jb.nheads = nheads; jb.N = N; jb.d = d;
  jb.fmt = fmt; jb.codes = codes; jb.scale = scale; jb.block = block;
  return run_job(&jb, nthreads);
}

void lao_round_e4m3(const double *x, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = double_to_e4m3_rne_sat(x[i]);
}

void lao_widen_e4m3(const uint8_t *c, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_double(c[i]);
}

/* ---------------------------------------------------------------------- */
/* Gradients of the recurrence (training), per head.                       */
/* ---------------------------------------------------------------------- */
/* For the scalar L = sum_t <o_t, do_t> + <S_N, dS_N>, with o_t = q_t^T S_t
 * and S_t = S_{t-1} + k_t v_t^T ([ZENN], section "線形アテンションの数学的
 * 基礎", recurrence equations), the chain rule through the recurrence gives:
 *   dq_t = S_t do_t                        (S_t: the forward state at t)
 *   G_t  = dS_N + sum_{r >= t} q_r do_r^T  (gradient reaching S_t)
 *   dk_t = G_t v_t,   dv_t = G_t^T k_t,   dS_0 = G_0.
 * The forward loop recomputes S_t; the backward loop carries G from the end.
 * q, k, v, dout : [N][d] float32 ; dS_N : [d][d] double or NULL (zero) ;
 * dq, dk, dv : [N][d] double (out) ; dS0 : [d][d] double (out) ;
 * S : [d][d] double (in: S_0; clobbered) ; work : [d][d] double scratch. */
static void backward_one_head(const float *q, const float *k, const float *v,
                              const float *dout, const double *dSN, double *dq,
                              double *dk, double *dv, double *dS0, double *S,
                              int64_t N, int64_t d) {
  for (int64_t t = 0; t < N; ++t) {
    const float *kt = k + t * d, *vt = v + t * d, *dot = dout + t * d;
    for (int64_t i = 0; i < d; ++i) {
      const double kfi = (double)kt[i];
      for (int64_t j = 0; j < d; ++j) S[i * d + j] += kfi * (double)vt[j];
    }
    for (int64_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int64_t j = 0; j < d; ++j) acc += S[i * d + j] * (double)dot[j];
      dq[t * d + i] = acc;
    }
  }
  double *G = dS0; /* carried in place: ends as G_0 = dS_0 */
  for (int64_t i = 0; i < d * d; ++i) G[i] = dSN ? dSN[i] : 0.0;
  for (int64_t t = N - 1; t >= 0; --t) {
    const float *qt = q + t * d, *kt = k + t * d, *vt = v + t * d, *dot = dout + t * d;
    for (int64_t i = 0; i < d; ++i) {
      const double qri = (double)qt[i];
      for (int64_t j = 0; j < d; ++j) G[i * d + j] += qri * (double)dot[j];
    }
    for (int64_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int64_t j = 0; j < d; ++j) acc += G[i * d + j] * (double)vt[j];
      dk[t * d + i] = acc;
    }
    for (int64_t j = 0; j < d; ++j) dv[t * d + j] = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      const double kbi = (double)kt[i];
      for (int64_t j = 0; j < d; ++j) dv[t * d + j] += G[i * d + j] * kbi;
    }
  }
}

typedef struct {
  const float *q, *k, *v, *dout;
  const double *S0, *dSN;
  double *dq, *dk, *dv, *dS0;
  int64_t nheads, N, d;
  int64_t next_head;
  pthread_mutex_t mu;
} bwd_job_t;

static void *bwd_worker(void *arg) {
  bwd_job_t *jb = (bwd_job_t *)arg;
  const int64_t dd = jb->d * jb->d, td = jb->N * jb->d;
  double *S = (double *)malloc(sizeof(double) * (size_t)dd);
  if (!S) return (void *)1;
  for (;;) {
    pthread_mutex_lock(&jb->mu);
    int64_t h = jb->next_head++;
    pthread_mutex_unlock(&jb->mu);
    if (h >= jb->nheads) break;
    for (int64_t i = 0; i < dd; ++i) S[i] = jb->S0 ? jb->S0[h * dd + i] : 0.0;
    backward_one_head(jb->q + h * td, jb->k + h * td, jb->v + h * td, jb->dout + h * td,
                      jb->dSN ? jb->dSN + h * dd : NULL, jb->dq + h * td, jb->dk + h * td,
                      jb->dv + h * td, jb->dS0 + h * dd, S, jb->N, jb->d);
  }
  free(S);
  return NULL;
}

/* Gradients of L = sum <o, dout> + <S_N, dS_N> for `nheads` heads.
 * q, k, v, dout : [nheads][N][d] float32 ; S0, dSN : [nheads][d][d] double
 * or NULL (zero) ; dq, dk, dv : [nheads][N][d] double (out) ;
 * dS0 : [nheads][d][d] double (out). */
int lao_backward(const float *q, const float *k, const float *v, const float *dout,
                 const double *S0, const double *dSN, double *dq, double *dk, double *dv,
                 double *dS0, int64_t nheads, int64_t N, int64_t d, int nthreads) {
  if (nheads < 0 || N < 0 || d <= 0) return LAO_EINVAL;
  if (nheads == 0) return LAO_OK;
  if (!dS0 || (N > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))) return LAO_EINVAL;
  bwd_job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.q = q; jb.k = k; jb.v = v; jb.dout = dout; jb.S0 = S0; jb.dSN = dSN;
  jb.dq = dq; jb.dk = dk; jb.dv = dv; jb.dS0 = dS0;
  jb.nheads = nheads; jb.N = N; jb.d = d;
  pthread_mutex_init(&jb.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nheads) nthreads = (int)nheads;
  int rc = LAO_OK;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  if (th)
    for (int i = 0; i < nthreads; ++i) {
      if (pthread_create(&th[i], NULL, bwd_worker, &jb) != 0) break;
      ++started;
    }
  if (started == 0 && bwd_worker(&jb) != NULL) rc = LAO_ENOMEM;
  for (int i = 0; i < started; ++i) {
    void *ret = NULL;
    pthread_join(th[i], &ret);
    if (ret != NULL) rc = LAO_ENOMEM;
  }
  free(th);
  pthread_mutex_destroy(&jb.mu);
  return rc;
}
