/*
 * oracle.c -- plain FP64 CPU oracle for BF16 softmax attention with the
 * duplicate-max ("stabilised") safe-softmax shift.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load this
 * library: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py do.  It shares no code, header, table or helper with the HIP
 * library; the only thing the two sides share is the seeded input generator,
 * which holds none of the method's arithmetic.
 *
 * Sources (web pages on Qiu & Yao, "Why Low-Precision Transformer Training
 * Fails: An Analysis on Flash Attention", arXiv 2510.04212):
 *   [ITS] itsolotime.com/archives/23922 -- Chinese summary of the paper.
 *   [HM]  91haoming.cn/news/show-608006 -- Chinese retelling of the paper.
 *   [TH]  itsolotime.com/th/archives/23923 -- Thai translation of [ITS].
 *
 * What is computed, row by row, with every row materialised in full (no
 * tiling, no online rescaling):
 *   - raw_ij = q_i . k_j exactly (bf16 inputs), S_ij = scale * raw_ij;
 *   - rm_i = max_j S_ij over the visible keys and rs_i = how many visible keys
 *     reach it (the duplicate-max count of [ITS] "极简修复方案", the minimal
 *     fix; [TH] same section);
 *   - the plain softmax result P = exp(S - rm) / rowsum, O = P V, the
 *     natural-log LSE ([ITS] "机制解释二", the forward formulas for P_bar, P
 *     and O);
 *   - the fix's shift m* (beta * rm when the max repeats and is positive,
 *     0 when it repeats and is negative, rm otherwise; same section of
 *     [ITS]) and from it P_bar = exp(S - m*), the literal stabilised
 *     output O_stab, max(P_bar) and whether its bf16 rounding equals 1;
 *   - the backward: delta_i = sum_c dO_ic O_ic ([HM] section 三, a row-sum
 *     of an elementwise product), dP = dO V^T, dS = P o (dP - delta),
 *     dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO (the standard
 *     softmax-attention gradient; the pages name dP and delta, the rest is
 *     the chain rule of the forward above);
 *   - element-wise error tolerances for a bf16 kernel with fp32 accumulation.
 *
 * A bf16 soft-float (decode, correctly rounded conversion from an exact
 * double-double value in five rounding modes, exact-sum addition) backs the
 * worked addition example of [HM] section 四 and the P_bar == 1 predicate.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* bf16 soft-float                                                     */
/* ------------------------------------------------------------------ */

enum { ORC_RNE = 0, ORC_RNA = 1, ORC_RTZ = 2, ORC_RD = 3, ORC_RU = 4 };

#define BF16_ONE 0x3F80u
#define TWO128 0x1p128

/* bf16 = 1 sign bit, 8 exponent bits (bias 127), 7 stored fraction bits. */
double orc_bf16_decode(uint16_t b) {
  int s = b >> 15, e = (b >> 7) & 0xFF, f = b & 0x7F;
  double v;
  if (e == 0xFF) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -133);          /* subnormal: f * 2^-133 */
  else v = ldexp((double)(f | 0x80), e - 127 - 7);      /* 1.f * 2^(e-127)      */
  return s ? -v : v;
}

/* spacing of the bf16 grid in the binade holding magnitude a > 0 */
static double bf16_spacing(double a) {
  int E;
  frexp(a, &E);                       /* a = f 2^E, f in [0.5, 1) */
  int e = E - 1;                      /* a in [2^e, 2^(e+1))      */
  return e < -126 ? 0x1p-133 : ldexp(1.0, e - 7);
}

/* encode a non-negative bf16-representable magnitude (2^128 means inf) */
static uint16_t bf16_encode_mag(double m) {
  if (m == 0.0) return 0;
  if (m >= TWO128) return 0x7F80;
  int E;
  double f = frexp(m, &E);
  int e = E - 1;
  if (e < -126) return (uint16_t)ldexp(m, 133);       /* subnormal code */
  int frac = (int)ldexp(2.0 * f, 7) & 0x7F;
  return (uint16_t)(((e + 127) << 7) | frac);
}

static double bf16_next_up_mag(double t) {  /* t >= 0 representable */
  if (t == 0.0) return 0x1p-133;
  return t + bf16_spacing(t);                /* reaches 2^128 == "inf" at the top */
}

static double bf16_next_down_mag(double t) {  /* t > 0 representable */
  double sp = bf16_spacing(t);
  int E;
  double f = frexp(t, &E);
  /* just below a normal power of two the grid is twice as fine */
  if (f == 0.5 && t > 0x1p-126) sp *= 0.5;
  return t - sp;
}

/*
 * Round the exact value hi + lo (|lo| <= ulp(hi)/2, as left by TwoSum) to
 * bf16 in the given mode.  Returns the bf16 bit pattern.
 */
uint16_t orc_bf16_round2(double hi, double lo, int mode) {
  if (isnan(hi)) return 0x7FC0;
  if (hi == 0.0 && lo != 0.0) { hi = lo; lo = 0.0; }
  int neg = signbit(hi) ? 1 : 0;
  uint16_t sbit = neg ? 0x8000 : 0;
  if (isinf(hi)) return sbit | 0x7F80;
  double a = fabs(hi), l = neg ? -lo : lo;   /* magnitude is a + l exactly */
  if (a == 0.0) return sbit;
  if (a >= TWO128) {                          /* beyond the largest finite value */
    int to_inf = mode == ORC_RNE || mode == ORC_RNA || (mode == ORC_RD && neg) ||
                 (mode == ORC_RU && !neg);
    return sbit | (to_inf ? 0x7F80 : 0x7F7F);
  }
  double sp = bf16_spacing(a);
  double t = floor(a / sp) * sp;             /* truncation toward zero */
  double L, U;
  if (a > t) { L = t; U = bf16_next_up_mag(t); }
  else if (l > 0) { L = t; U = bf16_next_up_mag(t); }
  else if (l < 0) { L = bf16_next_down_mag(t); U = t; }
  else return sbit | bf16_encode_mag(t);     /* exactly representable */
  /* strictly between L and U: compare with the midpoint, exactly */
  double M = 0.5 * (L + U);
  double dm = a - M;                          /* exact (Sterbenz / common grid) */
  double side = dm + l;                       /* sign of this sum is exact */
  int cmp = side > 0 ? 1 : (side < 0 ? -1 : 0);
  double R;
  switch (mode) {
    case ORC_RNE:
      if (cmp < 0) R = L;
      else if (cmp > 0) R = U;
      else R = (bf16_encode_mag(L) & 1) ? U : L;
      break;
    case ORC_RNA: R = cmp < 0 ? L : U; break;
    case ORC_RTZ: R = L; break;
    case ORC_RD: R = neg ? U : L; break;
    case ORC_RU: R = neg ? L : U; break;
    default: return 0xFFFF;
  }
  return sbit | bf16_encode_mag(R);
}

uint16_t orc_bf16_from_double(double x, int mode) { return orc_bf16_round2(x, 0.0, mode); }

/* bf16 addition: one rounding of the exact sum (TwoSum keeps it exact). */
uint16_t orc_bf16_add(uint16_t a, uint16_t b, int mode) {
  double x = orc_bf16_decode(a), y = orc_bf16_decode(b);
  double s = x + y;
  double bb = s - x;
  double err = (x - (s - bb)) + (y - bb);
  if (isinf(s) || isnan(s)) err = 0.0;
  return orc_bf16_round2(s, err, mode);
}

void orc_bf16_round_array(const double* x, int64_t n, int mode, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(x[i], mode);
}

/* ------------------------------------------------------------------ */
/* exact dot products of bf16 vectors                                  */
/* ------------------------------------------------------------------ */

/* value = m * 2^x with m a signed integer of at most 8 bits */
static void bf16_split(uint16_t b, int* m, int* x) {
  int s = b >> 15, e = (b >> 7) & 0xFF, f = b & 0x7F;
  if (e == 0) { *m = f; *x = -133; }
  else { *m = f | 0x80; *x = e - 134; }
  if (s) *m = -*m;
}

/* exponent of the lowest set bit over the non-zero entries of a vector */
static int lsb_exponent(const uint16_t* v, int d) {
  int best = 1 << 20;
  for (int c = 0; c < d; ++c) {
    int m, x;
    bf16_split(v[c], &m, &x);
    if (m == 0) continue;
    int am = m < 0 ? -m : m;
    while ((am & 1) == 0) { am >>= 1; ++x; }
    if (x < best) best = x;
  }
  return best;
}

/*
 * Kulisch accumulator: sum of limb[t] * 2^(32 t + KBASE).  Every product of two
 * finite bf16 values is an integer below 2^16 times 2^(>= -266), and its top
 * bit is below 2^(256+16), so 20 limbs above 2^-300 hold any sum exactly.
 */
#define KL 20
#define KBASE (-300)
typedef struct { int64_t w[KL]; } kacc;

static void kacc_dot(const uint16_t* a, const uint16_t* b, int d, kacc* acc) {
  memset(acc, 0, sizeof(*acc));
  for (int c = 0; c < d; ++c) {
    int ma, xa, mb, xb;
    bf16_split(a[c], &ma, &xa);
    bf16_split(b[c], &mb, &xb);
    int64_t p = (int64_t)ma * mb;
    if (p == 0) continue;
    int pos = xa + xb - KBASE;
    acc->w[pos / 32] += p * ((int64_t)1 << (pos % 32));
  }
  for (int t = 0; t < KL - 1; ++t) {        /* carries: limbs into [0, 2^32) */
    int64_t carry = acc->w[t] >> 32;        /* arithmetic shift = floor */
    acc->w[t] -= carry * ((int64_t)1 << 32);
    acc->w[t + 1] += carry;
  }
}

static int kacc_cmp(const kacc* x, const kacc* y) {
  for (int t = KL - 1; t >= 0; --t) {
    if (x->w[t] != y->w[t]) return x->w[t] < y->w[t] ? -1 : 1;
  }
  return 0;
}

static double kacc_to_double(const kacc* x) {
  long double s = 0.0L;
  for (int t = KL - 1; t >= 0; --t) s += ldexpl((long double)x->w[t], 32 * t + KBASE);
  return (double)s;
}

/*
 * Exact dot product of two bf16 vectors.  The double sum is certified exact
 * when every partial sum is a multiple of 2^L (L = sum of the two lowest set
 * bits) below 2^(L+52); otherwise the Kulisch accumulator decides.
 * Returns 1 when the fast double path was certified.
 */
int orc_exact_dot(const uint16_t* a, const uint16_t* b, int d, double* value) {
  double s = 0.0, sa = 0.0;
  for (int c = 0; c < d; ++c) {
    double p = orc_bf16_decode(a[c]) * orc_bf16_decode(b[c]);
    s += p;
    sa += fabs(p);
  }
  int L = lsb_exponent(a, d) + lsb_exponent(b, d);
  if (sa == 0.0 || sa <= ldexp(1.0, L + 52)) { *value = s; return 1; }
  kacc k;
  kacc_dot(a, b, d, &k);
  *value = kacc_to_double(&k);
  return 0;
}

/* ------------------------------------------------------------------ */
/* problem description and outputs                                     */
/* ------------------------------------------------------------------ */

typedef struct {
  const uint16_t* q;   /* bf16 [B][H][N][D] */
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;  /* may be NULL for the forward */
  int B, H, N, D;
  double scale;
  int causal, stabilise;
  double beta;
} orc_problem;

typedef struct {
  double* O;          /* [B][H][N][D] plain softmax attention            */
  double* O_stab;     /* [B][H][N][D] through the literal shifted P_bar   */
  double* tol_O;      /* [B][H][N][D]                                    */
  double* lse;        /* [B][H][N] natural log                           */
  double* tol_lse;    /* [B][H][N]                                       */
  double* rowmax;     /* [B][H][N] rm in scaled units                     */
  double* shift;      /* [B][H][N] m* in scaled units                     */
  double* pbar_max;   /* [B][H][N] exp(rm - m*)                           */
  int32_t* ties;      /* [B][H][N] rs                                     */
  int32_t* pbar_one;  /* [B][H][N] bf16_RNE(exp(rm - m*)) == 1            */
  int32_t* near_ones; /* [B][H][N] #keys with bf16_RNE(exp(S - m*)) == 1  */
  int32_t* amb_tie;   /* [B][H][N] tie count not decidable in fp32        */
  int32_t* amb_pbar;  /* [B][H][N] exp(rm - m*) at the bf16 1.0 boundary  */
  int32_t* amb_near;  /* [B][H][N] some exp(S - m*) at the bf16 1.0 boundary */
  int32_t* flags;     /* [B][H][N] bit0 rm==0 tie, bit1 underflow, bit2 slow dots */
} orc_fwd_out;

typedef struct {
  double* delta;      /* [B][H][N] */
  double* tol_delta;
  double* dQ;         /* [B][H][N][D] */
  double* dK;
  double* dV;
  double* tol_dQ;
  double* tol_dK;
  double* tol_dV;
} orc_bwd_out;

#define U_BF16 0x1p-8   /* bf16 unit roundoff */
#define U_F32 0x1p-24

typedef struct {
  double *q, *k, *v, *dO;  /* decoded copies */
  int *lq, *lk;            /* lowest-set-bit exponent per row */
} decoded;

static double* decode_all(const uint16_t* x, int64_t n) {
  double* r = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) r[i] = orc_bf16_decode(x[i]);
  return r;
}

static int decode_problem(const orc_problem* p, decoded* dc) {
  int64_t rows = (int64_t)p->B * p->H * p->N, n = rows * p->D;
  memset(dc, 0, sizeof(*dc));
  dc->q = decode_all(p->q, n);
  dc->k = decode_all(p->k, n);
  dc->v = p->v ? decode_all(p->v, n) : NULL;
  dc->dO = p->dO ? decode_all(p->dO, n) : NULL;
  dc->lq = (int*)malloc(sizeof(int) * (size_t)(rows > 0 ? rows : 1));
  dc->lk = (int*)malloc(sizeof(int) * (size_t)(rows > 0 ? rows : 1));
  for (int64_t r = 0; r < rows; ++r) {
    dc->lq[r] = lsb_exponent(p->q + r * p->D, p->D);
    dc->lk[r] = lsb_exponent(p->k + r * p->D, p->D);
  }
  for (int64_t i = 0; i < n; ++i) {
    if (!isfinite(dc->q[i]) || !isfinite(dc->k[i])) return -1;
    if (dc->v && !isfinite(dc->v[i])) return -1;
    if (dc->dO && !isfinite(dc->dO[i])) return -1;
  }
  return 0;
}

static void free_decoded(decoded* dc) {
  free(dc->q); free(dc->k); free(dc->v); free(dc->dO); free(dc->lq); free(dc->lk);
}

/* the fix's shift rule ([ITS] "极简修复方案"), in scaled units */
double orc_shift_rule(double rm, int rs, int stabilise, double beta) {
  if (stabilise && rs > 1 && rm > 0) return beta * rm;
  if (stabilise && rs > 1 && rm < 0) return 0.0;
  return rm;
}

/* visible keys of query row i: j <= i when causal, else all j < N */
static inline int last_key(const orc_problem* p, int i) { return p->causal ? i : p->N - 1; }

typedef struct {
  double* raw;    /* [N] exact q.k */
  double* sabs;   /* [N] sum |q_c k_c| */
  double* err;    /* [N] relative error bound of the kernel's P_bar_j beyond its bf16 rounding */
  int* f32exact;  /* [N] every fp32 partial sum exact */
  char* ismax;    /* [N] raw_j equals the row max exactly */
  kacc* ka;       /* [N] exact accumulators (only when needed) */
} row_scratch;

static void scratch_init(row_scratch* s, int N) {
  s->raw = (double*)malloc(sizeof(double) * (size_t)N);
  s->sabs = (double*)malloc(sizeof(double) * (size_t)N);
  s->err = (double*)malloc(sizeof(double) * (size_t)N);
  s->f32exact = (int*)malloc(sizeof(int) * (size_t)N);
  s->ismax = (char*)malloc((size_t)N);
  s->ka = NULL;
}
static void scratch_free(row_scratch* s) {
  free(s->raw); free(s->sabs); free(s->err); free(s->f32exact); free(s->ismax); free(s->ka);
}

/*
 * Exact scores of row (bh, i) over keys 0..jl.  Returns the exact max and its
 * count (rs) and whether the slow exact path was needed.
 */
static int row_scores(const orc_problem* p, const decoded* dc, int64_t bh, int i, int jl,
                      row_scratch* s, double* rm_raw, int* rs) {
  const int D = p->D, N = p->N;
  const int64_t qrow = bh * N + i;
  const double* q = dc->q + qrow * D;
  int certified = 1;
  for (int j = 0; j <= jl; ++j) {
    const int64_t krow = bh * N + j;
    const double* k = dc->k + krow * D;
    double acc = 0.0, sa = 0.0;
    for (int c = 0; c < D; ++c) {
      double t = q[c] * k[c];
      acc += t;
      sa += fabs(t);
    }
    int L = dc->lq[qrow] + dc->lk[krow];
    s->raw[j] = acc;
    s->sabs[j] = sa;
    if (!(sa == 0.0 || sa <= ldexp(1.0, L + 52))) certified = 0;
    s->f32exact[j] = (sa == 0.0) || (L >= -126 && sa < ldexp(1.0, L + 23));
  }
  if (certified) {
    double m = -INFINITY;
    int c = 0;
    for (int j = 0; j <= jl; ++j) {
      if (s->raw[j] > m) { m = s->raw[j]; c = 1; }
      else if (s->raw[j] == m) ++c;
    }
    for (int j = 0; j <= jl; ++j) s->ismax[j] = s->raw[j] == m;
    *rm_raw = m;
    *rs = c;
    return 0;
  }
  /* slow exact path: Kulisch accumulators decide the max and its count */
  if (!s->ka) s->ka = (kacc*)malloc(sizeof(kacc) * (size_t)N);
  const uint16_t* qb = p->q + qrow * D;
  int best = 0, c = 0;
  for (int j = 0; j <= jl; ++j) {
    kacc_dot(qb, p->k + (bh * N + j) * D, D, &s->ka[j]);
    s->raw[j] = kacc_to_double(&s->ka[j]);
    int cmp = j == 0 ? 1 : kacc_cmp(&s->ka[j], &s->ka[best]);
    if (cmp > 0) { best = j; c = 1; }
    else if (cmp == 0) ++c;
  }
  /* make raw[] equal exactly where the exact values are equal */
  for (int j = 0; j <= jl; ++j) {
    s->ismax[j] = kacc_cmp(&s->ka[j], &s->ka[best]) == 0;
    if (s->ismax[j]) s->raw[j] = s->raw[best];
  }
  *rm_raw = s->raw[best];
  *rs = c;
  return 1;
}

/*
 * Whether a bf16 kernel that forms q.k in fp32 could count the max of this
 * row differently: some other key lies within the fp32 accumulation error of
 * the max, or the tied keys are different vectors whose fp32 sums need not
 * round alike.  Keys whose fp32 partial sums are all exact carry no error;
 * bitwise-equal key vectors always give equal fp32 sums.
 */
static int tie_ambiguous(const orc_problem* p, int64_t bh, int jl, const row_scratch* s,
                         double rm_raw, int rs) {
  const int D = p->D, N = p->N;
  const double gamma = 2.0 * D * U_F32;
  int first = -1;
  double E = 0.0;
  for (int j = 0; j <= jl; ++j) {
    if (!s->ismax[j]) continue;
    if (first < 0) first = j;
    double e = s->f32exact[j] ? 0.0 : gamma * s->sabs[j];
    if (e > E) E = e;
  }
  int nnear = 0;
  for (int j = 0; j <= jl; ++j) {
    double e = s->f32exact[j] ? 0.0 : gamma * s->sabs[j];
    if (rm_raw - s->raw[j] <= e + E) ++nnear;
  }
  if (nnear > rs) return 1;  /* a key off the max lies within reach of it */
  if (rs > 1 && E > 0.0) {
    const uint16_t* kf = p->k + (bh * N + first) * D;
    for (int j = first + 1; j <= jl; ++j) {
      if (!s->ismax[j]) continue;
      if (memcmp(kf, p->k + (bh * N + j) * D, sizeof(uint16_t) * (size_t)D) != 0) return 1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* forward                                                             */
/* ------------------------------------------------------------------ */

static void forward_row(const orc_problem* p, const decoded* dc, int64_t row, row_scratch* s,
                        const orc_fwd_out* out) {
  const int N = p->N, D = p->D;
  const int64_t bh = row / N;
  const int i = (int)(row % N);
  const int jl = last_key(p, i);
  const int nvis = jl + 1;
  double rm_raw;
  int rs;
  int slow = row_scores(p, dc, bh, i, jl, s, &rm_raw, &rs);

  const double rm = p->scale * rm_raw;
  /* plain softmax: P = exp(S - rm) / sum */
  double ell = 0.0;
  for (int j = 0; j <= jl; ++j) ell += exp(p->scale * s->raw[j] - rm);
  const double lse = rm + log(ell);
  /* the fix's shift and the literal stabilised P_bar */
  const double mstar = orc_shift_rule(rm, rs, p->stabilise, p->beta);
  double ell_stab = 0.0;
  int near = 0, near_amb = 0;
  for (int j = 0; j <= jl; ++j) {
    double pb = exp(p->scale * s->raw[j] - mstar);
    ell_stab += pb;
    if (orc_bf16_from_double(pb, ORC_RNE) == BF16_ONE) ++near;
    if (fabs(pb - (1.0 - 0x1p-9)) <= 0x1p-14) near_amb = 1;
  }
  const double pmax = exp(rm - mstar);
  const double nfac = (double)nvis * U_F32;

  /*
   * Error of the kernel's P_bar_j beyond its bf16 rounding, as a relative
   * error (natural-log units of its exponent): the fp32 dot product (at most
   * D fp32 additions of exact bf16 products), the rounding of scale * log2(e)
   * and of the exponent (at most |S_j| + |shift| in size, for any shift the
   * online rule passes through), and exp2 itself.
   */
  const double shift_mag = fabs(rm) * (1.0 + (p->stabilise ? p->beta : 0.0));
  double lse_score = 0.0;  /* sum_j P_j * that error: its effect on LSE */
  for (int j = 0; j <= jl; ++j) {
    const double sj = p->scale * s->raw[j];
    const double ej = p->scale * D * U_F32 * s->sabs[j] + 0x1p-22 * (2.0 * fabs(sj) + shift_mag + 1.0);
    s->err[j] = ej;
    lse_score += exp(sj - rm) / ell * ej;
  }

  if (out->O || out->tol_O || out->O_stab) {
    double* o = (double*)calloc((size_t)D, sizeof(double));
    double* oa = (double*)calloc((size_t)D, sizeof(double));
    double* os = (double*)calloc((size_t)D, sizeof(double));
    double* dev = (double*)calloc((size_t)D, sizeof(double));
    for (int j = 0; j <= jl; ++j) {
      double sj = p->scale * s->raw[j];
      double pj = exp(sj - rm) / ell;
      double pbj = exp(sj - mstar) / ell_stab;
      const double* vj = dc->v + (bh * N + j) * D;
      for (int c = 0; c < D; ++c) {
        o[c] += pj * vj[c];
        oa[c] += pj * fabs(vj[c]);
        os[c] += pbj * vj[c];
      }
    }
    if (out->tol_O) {
      /*
       * O = sum_j w_j v_j with w_j = p_j / sum_k p_k, p_j = P_bar_j (1 + e_j):
       * normalising by the sum of the very values that multiply V gives
       * O' - O = sum_j P_j e_j (v_j - O) / (1 + sum_k P_k e_k), so a relative
       * error e_j of each weight (u from the bf16 rounding of P_bar, plus the
       * score error above) is bounded by sum_j P_j |e_j| |v_j - O|.
       */
      for (int j = 0; j <= jl; ++j) {
        const double w = exp(p->scale * s->raw[j] - rm) / ell * (U_BF16 + s->err[j]);
        const double* vj = dc->v + (bh * N + j) * D;
        for (int c = 0; c < D; ++c) dev[c] += w * fabs(vj[c] - o[c]);
      }
    }
    const int64_t base = row * D;
    for (int c = 0; c < D; ++c) {
      if (out->O) out->O[base + c] = o[c];
      if (out->O_stab) out->O_stab[base + c] = ell_stab > 0.0 ? os[c] : NAN;
      /* the weights' errors, the bf16 output (u), fp32 sums over the row; x2 */
      if (out->tol_O)
        out->tol_O[base + c] = 2.0 * (dev[c] + U_BF16 * fabs(o[c])) + 2.0 * nfac * (oa[c] + fabs(o[c]));
    }
    free(o); free(oa); free(os); free(dev);
  }
  if (out->lse) out->lse[row] = lse;
  /*
   * LSE = (shift + log2 l) ln 2 with l the fp32 sum of the row's P_bar: each
   * lane adds half the row's keys one by one and rescales once per 64-key
   * tile (relative error (n/2 + n/64 + 2) 2^-24 of a sum of positive terms);
   * the weights' score errors move LSE by sum_j P_j e_j; log2 and the final
   * sum and product round once each.  x2.
   */
  if (out->tol_lse)
    out->tol_lse[row] = 2.0 * (lse_score + ((double)nvis / 2.0 + (double)nvis / 64.0 + 2.0) * U_F32 +
                               0x1p-22 * log(2.0) * fmax(1.0, fabs(lse - mstar) / log(2.0)) +
                               0x1p-23 * fabs(lse));
  if (out->rowmax) out->rowmax[row] = rm;
  if (out->shift) out->shift[row] = mstar;
  if (out->pbar_max) out->pbar_max[row] = pmax;
  if (out->ties) out->ties[row] = rs;
  if (out->pbar_one) out->pbar_one[row] = orc_bf16_from_double(pmax, ORC_RNE) == BF16_ONE;
  if (out->near_ones) out->near_ones[row] = near;
  if (out->amb_tie) out->amb_tie[row] = tie_ambiguous(p, bh, jl, s, rm_raw, rs);
  if (out->amb_pbar) out->amb_pbar[row] = fabs(pmax - (1.0 - 0x1p-9)) <= 0x1p-14;
  if (out->amb_near) out->amb_near[row] = near_amb;
  if (out->flags) {
    int f = 0;
    if (rs > 1 && rm == 0.0) f |= 1;
    if (!(ell_stab > 0.0) || pmax < 0x1p-126) f |= 2;
    if (slow) f |= 4;
    out->flags[row] = f;
  }
}

static int nthreads_used = 1;

int orc_threads(void) { return nthreads_used; }

/* rows: flattened (b*H + h)*N + i, or NULL for every row. Returns 0, or -1 on bad input. */
int orc_forward(const orc_problem* p, const int64_t* rows, int64_t nrows, const orc_fwd_out* out) {
  if (p->N <= 0 || p->B <= 0 || p->H <= 0) return 0;
  decoded dc;
  if (decode_problem(p, &dc) != 0) { free_decoded(&dc); return -1; }
  const int64_t total = rows ? nrows : (int64_t)p->B * p->H * p->N;
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    nthreads_used = omp_get_num_threads();
#endif
    row_scratch s;
    scratch_init(&s, p->N);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < total; ++t) forward_row(p, &dc, rows ? rows[t] : t, &s, out);
    scratch_free(&s);
  }
  free_decoded(&dc);
  return 0;
}

/* ------------------------------------------------------------------ */
/* the online rule, tile by tile                                       */
/* ------------------------------------------------------------------ */

/*
 * [ITS] section "极简修复方案" states the rule on a whole row; a tiled kernel
 * applies it to the running (max, count) pair, merged tile by tile in key
 * order (larger max keeps its count, equal maxima add counts), and forms
 * P_bar_j = exp(S_j - m*) for the keys of each tile with the shift m* of
 * the pair as it stands after that tile.  This counts, for one row, the keys
 * whose P_bar so formed rounds (bf16 nearest-even) to exactly 1, tiles of
 * `tile` keys starting at key 0.  *amb is set when a running maximum could be
 * counted differently from fp32 dot products (another key within their
 * error of it, or tied keys that are different vectors with inexact sums),
 * when some P_bar lies within 2^-14 of the bf16 1.0 boundary, or when the
 * exact scores needed the slow path.
 */
static void online_row(const orc_problem* p, const decoded* dc, int64_t row, row_scratch* s, int tile,
                       int32_t* ones, int32_t* amb) {
  const int N = p->N, D = p->D;
  const int64_t bh = row / N;
  const int i = (int)(row % N);
  const int jl = last_key(p, i);
  double rm_raw;
  int rs;
  int ambig = row_scores(p, dc, bh, i, jl, s, &rm_raw, &rs);
  const double gamma = 2.0 * D * U_F32;
  double m = -INFINITY;
  int c = 0, count = 0;
  for (int t0 = 0; t0 <= jl; t0 += tile) {
    const int t1 = t0 + tile - 1 < jl ? t0 + tile - 1 : jl;
    double tm = -INFINITY;
    int tc = 0;
    for (int j = t0; j <= t1; ++j) {
      if (s->raw[j] > tm) { tm = s->raw[j]; tc = 1; }
      else if (s->raw[j] == tm) ++tc;
    }
    if (tm > m) { m = tm; c = tc; }
    else if (tm == m) c += tc;
    /* could fp32 sums decide this running pair differently? */
    double E = 0.0;
    int first = -1;
    for (int j = 0; j <= t1; ++j) {
      if (s->raw[j] != m) continue;
      if (first < 0) first = j;
      double e = s->f32exact[j] ? 0.0 : gamma * s->sabs[j];
      if (e > E) E = e;
    }
    int nnear = 0;
    for (int j = 0; j <= t1; ++j) {
      double e = s->f32exact[j] ? 0.0 : gamma * s->sabs[j];
      if (m - s->raw[j] <= e + E) ++nnear;
    }
    if (nnear > c) ambig = 1;
    if (c > 1 && E > 0.0) {
      const uint16_t* kf = p->k + (bh * N + first) * D;
      for (int j = first + 1; j <= t1; ++j)
        if (s->raw[j] == m && memcmp(kf, p->k + (bh * N + j) * D, sizeof(uint16_t) * (size_t)D) != 0) ambig = 1;
    }
    const double mstar = orc_shift_rule(p->scale * m, c, p->stabilise, p->beta);
    for (int j = t0; j <= t1; ++j) {
      const double pb = exp(p->scale * s->raw[j] - mstar);
      if (orc_bf16_from_double(pb, ORC_RNE) == BF16_ONE) ++count;
      if (fabs(pb - (1.0 - 0x1p-9)) <= 0x1p-14) ambig = 1;
    }
  }
  ones[row] = count;
  if (amb) amb[row] = ambig;
}

/* rows: flattened rows or NULL for all; ones / amb: [B][H][N]. Returns 0, or -1. */
int orc_online_ones(const orc_problem* p, int tile, const int64_t* rows, int64_t nrows, int32_t* ones,
                    int32_t* amb) {
  if (p->N <= 0 || p->B <= 0 || p->H <= 0) return 0;
  if (tile < 1 || !ones) return -1;
  decoded dc;
  if (decode_problem(p, &dc) != 0) { free_decoded(&dc); return -1; }
  const int64_t total = rows ? nrows : (int64_t)p->B * p->H * p->N;
#pragma omp parallel
  {
    row_scratch s;
    scratch_init(&s, p->N);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < total; ++t) online_row(p, &dc, rows ? rows[t] : t, &s, tile, ones, amb);
    scratch_free(&s);
  }
  free_decoded(&dc);
  return 0;
}

/* ------------------------------------------------------------------ */
/* emulation of a bf16-accumulated P_bar V                             */
/* ------------------------------------------------------------------ */

/*
 * [ITS] section "机制解释二" and [HM] section 四: with several P_bar entries
 * exactly 1 (a repeated row max) the products P_bar V are the V values
 * themselves, and adding mostly negative bf16 numbers in bf16 (significand
 * overflow, a right shift, the shifted-out and sticky bits deciding the
 * rounding) errs to one side.  This emulates that arithmetic for one row,
 * in key order:
 *   P_bar_j = exp(S_j - m*) (FP64, m* from the duplicate-max rule when
 *             p->stabilise), rounded to bf16 nearest-even when pbar_round;
 *   term_j  = P_bar_j * v_jc, exact, then rounded to bf16 in acc_mode;
 *   acc     = acc (+) term_j, the exact sum rounded to bf16 in acc_mode;
 *   O_c     = acc / l, l = sum_j P_bar_j in FP64.
 * acc_mode < 0 accumulates the exact terms in FP64 instead (no bf16 step).
 * events = how many P_bar_j equal 1 after the rounding.
 */
static void emulate_row(const orc_problem* p, const decoded* dc, int64_t row, row_scratch* s, int pbar_round,
                        int acc_mode, double* O, int32_t* events) {
  const int N = p->N, D = p->D;
  const int64_t bh = row / N;
  const int i = (int)(row % N);
  const int jl = last_key(p, i);
  double rm_raw;
  int rs;
  row_scores(p, dc, bh, i, jl, s, &rm_raw, &rs);
  const double m = orc_shift_rule(p->scale * rm_raw, rs, p->stabilise, p->beta);
  double* pb = s->sabs;  /* reuse: P_bar per key */
  double l = 0.0;
  int ev = 0;
  for (int j = 0; j <= jl; ++j) {
    double x = exp(p->scale * s->raw[j] - m);
    if (pbar_round) x = orc_bf16_decode(orc_bf16_from_double(x, ORC_RNE));
    pb[j] = x;
    l += x;
    if (x == 1.0) ++ev;
  }
  for (int c = 0; c < D; ++c) {
    if (acc_mode < 0) {
      double acc = 0.0;
      for (int j = 0; j <= jl; ++j) acc += pb[j] * dc->v[(bh * N + j) * D + c];
      O[row * D + c] = acc / l;
    } else {
      uint16_t acc = 0;
      for (int j = 0; j <= jl; ++j) {
        const uint16_t term = orc_bf16_from_double(pb[j] * dc->v[(bh * N + j) * D + c], acc_mode);
        acc = orc_bf16_add(acc, term, acc_mode);
      }
      O[row * D + c] = orc_bf16_decode(acc) / l;
    }
  }
  if (events) events[row] = ev;
}

/* rows: flattened row indices or NULL for all; O [B][H][N][D], events [B][H][N] (nullable). */
int orc_emulate_pv(const orc_problem* p, const int64_t* rows, int64_t nrows, int pbar_round, int acc_mode,
                   double* O, int32_t* events) {
  if (p->N <= 0 || p->B <= 0 || p->H <= 0) return 0;
  if (!p->v) return -1;
  decoded dc;
  if (decode_problem(p, &dc) != 0) { free_decoded(&dc); return -1; }
  const int64_t total = rows ? nrows : (int64_t)p->B * p->H * p->N;
#pragma omp parallel
  {
    row_scratch s;
    scratch_init(&s, p->N);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < total; ++t) emulate_row(p, &dc, rows ? rows[t] : t, &s, pbar_round, acc_mode, O, events);
    scratch_free(&s);
  }
  free_decoded(&dc);
  return 0;
}

/* ------------------------------------------------------------------ */
/* backward                                                            */
/* ------------------------------------------------------------------ */

/*
 * heads: flattened b*H + h indices (NULL = all).  O, lse and tol_O, tol_lse
 * must hold the oracle forward for every row of those heads.
 */
int orc_backward(const orc_problem* p, const int64_t* heads, int64_t nheads, const double* O,
                 const double* lse, const double* tol_O, const double* tol_lse,
                 const orc_bwd_out* out) {
  if (p->N <= 0 || p->B <= 0 || p->H <= 0) return 0;
  if (!p->dO || !O || !lse || !tol_O || !tol_lse) return -1;
  (void)tol_O; /* delta's bound follows the forward's error model directly (below) */
  decoded dc;
  if (decode_problem(p, &dc) != 0) { free_decoded(&dc); return -1; }
  const int N = p->N, D = p->D;
  const int64_t nh = heads ? nheads : (int64_t)p->B * p->H;
  const int64_t total = nh * N;
  const double sc = p->scale;
  const double gamma = 2.0 * D * U_F32;
  double* delta = (double*)malloc(sizeof(double) * (size_t)p->B * p->H * N);
  double* tdel = (double*)malloc(sizeof(double) * (size_t)p->B * p->H * N);

  /*
   * Error model of a bf16 kernel with fp32 accumulation (x2 in every
   * tolerance).  e_b(i, j): relative error of the kernel's P_ij = exp(S_ij -
   * LSE_i) beyond the LSE's own error: the fp32 dot product (D additions of
   * exact bf16 products), the rounding of scale * log2(e), of the exponent and
   * of LSE * log2(e), and exp2.  The forward's O reaches delta through
   * delta_i = sum_c dO_ic O_ic: with O' - O = sum_j P_ij e_j (v_j - O) plus
   * the rounding r_c of each bf16 output, the error of delta is
   * sum_j P_ij e_j (dP_ij - delta_i) + sum_c dO_ic r_c, so it is bounded by
   * sum_j P_ij |e_j| |dP_ij - delta_i| + u sum_c |dO_ic O_ic| (e_j: u for the
   * bf16 P_bar plus the forward's score error), plus the fp32 sums of the
   * forward (n 2^-24 per term) and of delta itself (D 2^-24).
   */
  /* pass 1, per query row: delta, then dQ = scale * sum_j dS_ij k_j */
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    double* tac = (double*)malloc(sizeof(double) * (size_t)D);
    double* pk = (double*)malloc(sizeof(double) * (size_t)D);
    double* Pj = (double*)malloc(sizeof(double) * (size_t)N);
    double* dpj = (double*)malloc(sizeof(double) * (size_t)N);
    double* dpaj = (double*)malloc(sizeof(double) * (size_t)N);
    double* sj = (double*)malloc(sizeof(double) * (size_t)N);
    double* saj = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < total; ++t) {
      const int64_t bh = heads ? heads[t / N] : t / N;
      const int i = (int)(t % N);
      const int64_t row = bh * N + i;
      const double* o = O + row * D;
      const double* g = dc.dO + row * D;
      const double* q = dc.q + row * D;
      double dl = 0.0, dla = 0.0;
      for (int c = 0; c < D; ++c) {
        dl += g[c] * o[c];
        dla += fabs(g[c] * o[c]);
      }
      const int jl = last_key(p, i);
      const int nvis = jl + 1;
      double rm = -INFINITY;
      for (int j = 0; j <= jl; ++j) {
        const int64_t kr = bh * N + j;
        const double* k = dc.k + kr * D;
        const double* v = dc.v + kr * D;
        double raw = 0.0, sa = 0.0, dp = 0.0, dpa = 0.0;
        for (int c = 0; c < D; ++c) {
          raw += q[c] * k[c];
          sa += fabs(q[c] * k[c]);
          dp += g[c] * v[c];
          dpa += fabs(g[c] * v[c]);
        }
        sj[j] = sc * raw;
        saj[j] = sa;
        dpj[j] = dp;
        dpaj[j] = dpa;
        Pj[j] = exp(sc * raw - lse[row]);
        if (sj[j] > rm) rm = sj[j];
      }
      /* the forward's shift is at most |rm| (1 + beta) in size, whichever mode */
      const double shift_mag = fabs(rm) * (1.0 + (p->stabilise ? p->beta : 0.0));
      double dev = 0.0, pdpa = 0.0;
      for (int j = 0; j <= jl; ++j) {
        const double ef = sc * D * U_F32 * saj[j] + 0x1p-22 * (2.0 * fabs(sj[j]) + shift_mag + 1.0);
        dev += Pj[j] * (U_BF16 + ef) * fabs(dpj[j] - dl);
        pdpa += Pj[j] * dpaj[j];
      }
      const double nfac = (double)nvis * U_F32;
      const double td = 2.0 * (dev + U_BF16 * dla + nfac * (pdpa + dla)) + gamma * dla;
      delta[row] = dl;
      tdel[row] = td;
      for (int c = 0; c < D; ++c) { acc[c] = 0.0; tac[c] = 0.0; pk[c] = 0.0; }
      for (int j = 0; j <= jl; ++j) {
        const double* k = dc.k + (bh * N + j) * D;
        const double P = Pj[j];
        const double dS = P * (dpj[j] - dl);
        const double eb = tol_lse[row] + sc * D * U_F32 * saj[j] + 0x1p-22 * (2.0 * fabs(sj[j]) + fabs(lse[row]) + 1.0);
        /* per-entry errors of dS; delta's error, common to the row, is added below */
        const double eds = U_BF16 * fabs(dS) + P * gamma * dpaj[j] + (fabs(dS) + P * td) * eb;
        for (int c = 0; c < D; ++c) {
          acc[c] += dS * k[c];
          tac[c] += eds * fabs(k[c]);
          pk[c] += P * k[c];
        }
      }
      for (int c = 0; c < D; ++c) {
        const double dq = sc * acc[c];
        if (out->dQ) out->dQ[row * D + c] = dq;
        /* delta's error d enters dQ_i as -scale d sum_j P_ij k_j */
        if (out->tol_dQ) out->tol_dQ[row * D + c] = 2.0 * (sc * (tac[c] + td * fabs(pk[c])) + U_BF16 * fabs(dq));
      }
      if (out->delta) out->delta[row] = dl;
      if (out->tol_delta) out->tol_delta[row] = td;
    }
    free(acc); free(tac); free(pk); free(Pj); free(dpj); free(dpaj); free(sj); free(saj);
  }

  /* pass 2, per key row: dK = scale * sum_i dS_ij q_i, dV = sum_i P_ij dO_i */
#pragma omp parallel
  {
    double* ak = (double*)malloc(sizeof(double) * (size_t)D);
    double* tk = (double*)malloc(sizeof(double) * (size_t)D);
    double* av = (double*)malloc(sizeof(double) * (size_t)D);
    double* tv = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < total; ++t) {
      const int64_t bh = heads ? heads[t / N] : t / N;
      const int j = (int)(t % N);
      const int64_t kr = bh * N + j;
      const double* k = dc.k + kr * D;
      const double* v = dc.v + kr * D;
      for (int c = 0; c < D; ++c) { ak[c] = tk[c] = av[c] = tv[c] = 0.0; }
      const int i0 = p->causal ? j : 0;
      for (int i = i0; i < N; ++i) {
        const int64_t row = bh * N + i;
        const double* q = dc.q + row * D;
        const double* g = dc.dO + row * D;
        double raw = 0.0, sa = 0.0, dp = 0.0, dpa = 0.0;
        for (int c = 0; c < D; ++c) {
          raw += q[c] * k[c];
          sa += fabs(q[c] * k[c]);
          dp += g[c] * v[c];
          dpa += fabs(g[c] * v[c]);
        }
        const double P = exp(sc * raw - lse[row]);
        const double dS = P * (dp - delta[row]);
        const double eb = tol_lse[row] + sc * D * U_F32 * sa + 0x1p-22 * (2.0 * fabs(sc * raw) + fabs(lse[row]) + 1.0);
        /* delta's error differs from row to row here: bounded term by term */
        const double eds = U_BF16 * fabs(dS) + P * (tdel[row] + gamma * dpa) + (fabs(dS) + P * tdel[row]) * eb;
        const double ep = P * eb;
        for (int c = 0; c < D; ++c) {
          ak[c] += dS * q[c];
          tk[c] += eds * fabs(q[c]);
          av[c] += P * g[c];
          tv[c] += (2.0 * U_BF16 * P + ep) * fabs(g[c]);
        }
      }
      for (int c = 0; c < D; ++c) {
        const double dk = sc * ak[c];
        if (out->dK) out->dK[kr * D + c] = dk;
        if (out->tol_dK) out->tol_dK[kr * D + c] = 2.0 * (sc * tk[c] + U_BF16 * fabs(dk));
        if (out->dV) out->dV[kr * D + c] = av[c];
        if (out->tol_dV) out->tol_dV[kr * D + c] = 2.0 * (tv[c] + U_BF16 * fabs(av[c]));
      }
    }
    free(ak); free(tk); free(av); free(tv);
  }
  free(delta);
  free(tdel);
  free_decoded(&dc);
  return 0;
}
