/*
 * CPU oracle for the batched GEMM with fused epilogue, D = act(alpha * A x B + beta * C).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this code. The GPU library never links, includes or calls it,
 * and it includes nothing from the GPU library.
 *
 * Everything here is the plain definition, evaluated slowly:
 *   - inputs are decoded exactly to double from their stored codes;
 *   - every output element is a k-ascending fp64 dot product;
 *   - the epilogue follows the order of the pages' accumulator visit (quack-kernels
 *     0.1.10 -> 0.2.0 diff, page 5, quack/dense_gemm_sm90.py, GemmSm90.epi_visit_acc_subtile;
 *     page 6, quack/gemm_act_sm90.py, GemmActSm90.epi_visit_acc_subtile): scale by alpha,
 *     add beta * C, then the activation on that unrounded fp32-domain value;
 *   - outputs are rounded to nearest-even from double straight to the output type;
 *   - the tile map uses '/' and '%' only.
 * The page's FastDivmod (page 6, quack/fast_math.py) is restated here in 64-bit arithmetic
 * only so that its quotient/remainder can be checked against true division.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Element types (oracle-local numbering; the Python wrapper maps names to these). */
enum { ORC_NONE = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_F32 = 3, ORC_E4M3 = 4, ORC_E5M2 = 5 };
/* Activations: page 6, quack/gemm_act_sm90.py, act_fn_map (none, relu, relu_sq,
 * gelu_tanh_approx). SiLU, x * sigmoid(x) by its standard definition, is not in that map:
 * the grouped MoE workload's epilogue uses it. */
enum { ORC_ACT_NONE = 0, ORC_ACT_RELU = 1, ORC_ACT_RELU_SQ = 2, ORC_ACT_GELU_TANH = 3, ORC_ACT_SILU = 4 };

/* ------------------------------------------------------------------------------------ */
/* Exact decoding of stored codes.                                                      */
/* ------------------------------------------------------------------------------------ */

/* Binary interchange format with `ebits` exponent bits, `mbits` mantissa bits and bias
 * 2^(ebits-1)-1. `ieee_special`: the all-ones exponent means inf/NaN (fp16, bf16, e5m2).
 * e4m3fn instead has no infinities and only S.1111.111 as NaN (OCP 8-bit float spec). */
static double decode_generic(uint32_t code, int ebits, int mbits, int ieee_special) {
  uint32_t sign = (code >> (ebits + mbits)) & 1u;
  uint32_t e = (code >> mbits) & ((1u << ebits) - 1u);
  uint32_t m = code & ((1u << mbits) - 1u);
  int bias = (1 << (ebits - 1)) - 1;
  double v;
  if (ieee_special && e == (1u << ebits) - 1u) {
    v = m ? NAN : INFINITY;
  } else if (!ieee_special && e == (1u << ebits) - 1u && m == (1u << mbits) - 1u) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, 1 - bias - mbits); /* subnormal: m * 2^(1-bias-mbits) */
  } else {
    v = ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
  }
  return sign ? -v : v;
}

double orc_decode(int dt, uint32_t code) {
  switch (dt) {
    case ORC_F16: return decode_generic(code & 0xFFFFu, 5, 10, 1);
    case ORC_BF16: return decode_generic(code & 0xFFFFu, 8, 7, 1);
    case ORC_E4M3: return decode_generic(code & 0xFFu, 4, 3, 0);
    case ORC_E5M2: return decode_generic(code & 0xFFu, 5, 2, 1);
    case ORC_F32: {
      float f;
      memcpy(&f, &code, 4);
      return (double)f;
    }
    default: return NAN;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Round-to-nearest-even from double straight to fp16 / bf16 / fp32 codes.             */
/* ------------------------------------------------------------------------------------ */

/* Round x to the grid of a binary format with `mbits` stored mantissa bits and minimum
 * normal exponent `emin`; returns the rounded value (may be 2^(emax+1) on overflow). */
static double round_to_format(double x, int mbits, int emin) {
  int e;
  frexp(x, &e); /* x = f * 2^e with 0.5 <= |f| < 1, so |x| in [2^(e-1), 2^e) */
  int ex = e - 1;
  if (ex < emin) ex = emin;
  double ulp = ldexp(1.0, ex - mbits);
  double q = x / ulp;            /* exact: ulp is a power of two */
  double r = nearbyint(q);       /* default rounding mode: nearest, ties to even */
  return r * ulp;
}

static uint32_t encode_binary16like(double x, int ebits, int mbits) {
  int bias = (1 << (ebits - 1)) - 1;
  int emin = 1 - bias;
  uint32_t sign = signbit(x) ? 1u : 0u;
  uint32_t inf = ((1u << ebits) - 1u) << mbits;
  if (isnan(x)) return (sign << (ebits + mbits)) | inf | (1u << (mbits - 1));
  double a = fabs(x);
  if (isinf(a)) return (sign << (ebits + mbits)) | inf;
  double r = a == 0.0 ? 0.0 : round_to_format(a, mbits, emin);
  double maxfin = ldexp(2.0 - ldexp(1.0, -mbits), bias);
  if (r > maxfin) return (sign << (ebits + mbits)) | inf;
  if (r == 0.0) return sign << (ebits + mbits);
  int e;
  frexp(r, &e);
  int ex = e - 1;
  uint32_t efield, mfield;
  if (ex < emin) { /* subnormal */
    efield = 0;
    mfield = (uint32_t)ldexp(r, -(emin - mbits));
  } else {
    efield = (uint32_t)(ex + bias);
    mfield = (uint32_t)(ldexp(r, -(ex - mbits)) - ldexp(1.0, mbits));
  }
  return (sign << (ebits + mbits)) | (efield << mbits) | mfield;
}

/* OCP fp8 with round-to-nearest-even and saturation to the largest finite value
 * ("satfinite": what a D / PostAct output in an fp8 type receives; page 5's is_valid_dtypes
 * admits Float8E4M3FN and Float8E5M2 for D). Magnitudes above the largest finite value,
 * infinities included, become it; NaN stays NaN (e4m3fn: S.1111.111; e5m2: S.11111.10).
 * e4m3fn has no infinity, so its top exponent holds normal numbers up to 448. */
static uint32_t encode_fp8_satfinite(double x, int ebits, int mbits) {
  int fn = ebits == 4; /* e4m3fn */
  int bias = (1 << (ebits - 1)) - 1;
  int emin = 1 - bias;
  uint32_t sign = signbit(x) ? 1u : 0u;
  uint32_t top = (1u << ebits) - 1u;
  if (isnan(x)) return (sign << 7) | (fn ? 0x7Fu : ((top << mbits) | (1u << (mbits - 1))));
  double maxfin = fn ? 448.0 : 57344.0;
  double a = fabs(x);
  double r = isinf(a) ? maxfin : (a == 0.0 ? 0.0 : round_to_format(a, mbits, emin));
  if (r > maxfin) r = maxfin;
  if (r == 0.0) return sign << 7;
  int e;
  frexp(r, &e);
  int ex = e - 1;
  uint32_t efield, mfield;
  if (ex < emin) {
    efield = 0;
    mfield = (uint32_t)ldexp(r, -(emin - mbits));
  } else {
    efield = (uint32_t)(ex + bias);
    mfield = (uint32_t)(ldexp(r, -(ex - mbits)) - ldexp(1.0, mbits));
  }
  return (sign << 7) | (efield << mbits) | mfield;
}

uint32_t orc_encode(int dt, double x) {
  switch (dt) {
    case ORC_E4M3: return encode_fp8_satfinite(x, 4, 3);
    case ORC_E5M2: return encode_fp8_satfinite(x, 5, 2);
    case ORC_F16: return encode_binary16like(x, 5, 10);
    case ORC_BF16: return encode_binary16like(x, 8, 7);
    case ORC_F32: {
      float f = (float)x; /* C conversion: round to nearest even */
      uint32_t u;
      memcpy(&u, &f, 4);
      return u;
    }
    default: return 0;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Activations, in fp64.                                                                */
/* ------------------------------------------------------------------------------------ */

double orc_act(int act, double x) {
  switch (act) {
    case ORC_ACT_NONE: return x;
    case ORC_ACT_RELU: return x > 0.0 ? x : 0.0;
    case ORC_ACT_RELU_SQ: { double r = x > 0.0 ? x : 0.0; return r * r; }
    case ORC_ACT_GELU_TANH: {
      /* tanh approximation of GELU: x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))) */
      double c = sqrt(2.0 / M_PI);
      return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
    }
    case ORC_ACT_SILU: return x / (1.0 + exp(-x));
    default: return NAN;
  }
}

/* Derivative act'(x) of each activation above, in fp64, for the activation-backward
 * epilogue (page 6, quack/gemm_dact_sm90.py: dact_fn_map maps relu, relu_sq and
 * gelu_tanh_approx to functions of (x, dout) returning (dx, act(x)); their bodies are not on
 * the pages). Written from the formulas above by the product and chain rules:
 *   relu:     1 for x > 0, else 0 (the derivative at 0 taken as 0)
 *   relu_sq:  2 max(x, 0)
 *   gelu:     with c = sqrt(2/pi), u = c (x + 0.044715 x^3), t = tanh(u):
 *             (1 + t)/2 + x/2 (1 - t^2) c (1 + 3 * 0.044715 x^2)
 *   silu:     with s = 1/(1 + e^-x): s + x s (1 - s)        (an addition: not on the pages)
 *   none:     1 */
double orc_dact(int act, double x) {
  switch (act) {
    case ORC_ACT_NONE: return 1.0;
    case ORC_ACT_RELU: return x > 0.0 ? 1.0 : 0.0;
    case ORC_ACT_RELU_SQ: return x > 0.0 ? 2.0 * x : 0.0;
    case ORC_ACT_GELU_TANH: {
      double c = sqrt(2.0 / M_PI);
      double t = tanh(c * (x + 0.044715 * x * x * x));
      return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x);
    }
    case ORC_ACT_SILU: {
      double sg = 1.0 / (1.0 + exp(-x));
      return sg + x * sg * (1.0 - sg);
    }
    default: return NAN;
  }
}

/* ------------------------------------------------------------------------------------ */
/* The GEMM problem.                                                                    */
/* ------------------------------------------------------------------------------------ */

/* Logical operands (page 5, quack/dense_gemm_sm90.py, gemm_sm90 wrapper): A is (l, m, k),
 * B is (l, n, k), C / D / PostAct are (l, m, n). Each has one contiguous dimension:
 *   a_kmajor = 1: A[l*sa + m*lda + k]          a_kmajor = 0: A[l*sa + k*lda + m]
 *   b_kmajor = 1: B[l*sb + n*ldb + k]          b_kmajor = 0: B[l*sb + k*ldb + n]
 *   x_nmajor = 1: X[l*sx + m*ldx + n]          x_nmajor = 0: X[l*sx + n*ldx + m]
 * Variable-length M (grouped): cu_seqlens has L+1 entries, group g owns global rows
 * [cu[g], cu[g+1]); A, C, D, PostAct are indexed by the global row with batch 0, and
 * B by the group g (page 5, the varlen-M offsets of A, B and D in GemmSm90.kernel).
 * Variable-length K (grouped, page 5 GemmSm90.kernel and the torch-vendored gemm_sm90.py
 * page: cu_seqlens_k offsets the K coordinate of A and B by cu_seqlens_k[l] and the group's
 * K extent is cu_seqlens_k[l+1] - cu_seqlens_k[l]): cu_seqlens_k has L+1 entries, A is
 * (m, total_k) and B is (n, total_k) with no batch index, C / D / PostAct are (l, m, n);
 * group l sums k over [cu_k[l], cu_k[l+1]), an empty range giving acc = 0.
 * Gathered A (mAIdx on the same pages; the gather copies of load_AB_gather_A and
 * _make_gather_A_copy): with varlen-M, the A row read for global output row m is
 * a_idx[m]; with varlen-K, the A column read for global k is a_idx[k]. The pages load only
 * rows that exist and leave the rest of the tile empty; the reading taken here is that an
 * index outside [0, a_rows) (a_rows = the rows, or columns, of A an index may name) reads
 * a zero row (column), i.e. contributes nothing to the sum.
 * Preconditions, checked by every entry point below (they return ORC_ERR_* instead of
 * reading out of bounds): cu_seqlens starts at 0, never decreases and ends at M (every
 * global row belongs to exactly one group); cu_seqlens_k starts at 0, never decreases and
 * ends at most at K; requested (l, m, n) lie inside the output. */
typedef struct {
  int64_t M, N, K, L;
  int32_t a_dt, b_dt, c_dt;
  int32_t a_kmajor, b_kmajor, c_nmajor;
  int64_t lda, ldb, ldc;
  int64_t sa, sb, sc;
  double alpha, beta;
  int32_t has_c;
  int32_t act;
  int32_t varlen;
  const int32_t* cu_seqlens; /* host array, L+1 entries, when varlen */
  int32_t dact;              /* 1: activation-backward epilogue, C holds the pre-activation */
  int32_t varlen_k;          /* 1: grouped K, cu_seqlens_k given */
  const int32_t* cu_seqlens_k; /* host array, L+1 entries, when varlen_k */
  const int32_t* a_idx;      /* host array or NULL: gathered A rows (varlen-M) / columns (varlen-K) */
  int64_t a_rows;            /* with a_idx: the rows (varlen-M) / columns (varlen-K) of A it may name */
} orc_problem;

enum { ORC_OK = 0, ORC_ERR_CU_SEQLENS = -1, ORC_ERR_CU_SEQLENS_K = -2, ORC_ERR_INDEX = -3 };

/* The preconditions above; ORC_OK or the first one violated. */
static int validate(const orc_problem* p) {
  if (p->varlen) {
    if (p->cu_seqlens[0] != 0 || p->cu_seqlens[p->L] != p->M) return ORC_ERR_CU_SEQLENS;
    for (int64_t g = 0; g < p->L; ++g)
      if (p->cu_seqlens[g + 1] < p->cu_seqlens[g]) return ORC_ERR_CU_SEQLENS;
  }
  if (p->varlen_k) {
    if (p->cu_seqlens_k[0] != 0 || p->cu_seqlens_k[p->L] > p->K) return ORC_ERR_CU_SEQLENS_K;
    for (int64_t g = 0; g < p->L; ++g)
      if (p->cu_seqlens_k[g + 1] < p->cu_seqlens_k[g]) return ORC_ERR_CU_SEQLENS_K;
  }
  return ORC_OK;
}

static int point_ok(const orc_problem* p, int64_t l, int64_t m, int64_t n) {
  const int64_t nb = p->varlen ? 1 : p->L;
  return l >= 0 && l < nb && m >= 0 && m < p->M && n >= 0 && n < p->N;
}

static double load_elem(const void* base, int dt, int64_t idx) {
  switch (dt) {
    case ORC_F16:
    case ORC_BF16: return orc_decode(dt, ((const uint16_t*)base)[idx]);
    case ORC_E4M3:
    case ORC_E5M2: return orc_decode(dt, ((const uint8_t*)base)[idx]);
    case ORC_F32: return orc_decode(dt, ((const uint32_t*)base)[idx]);
    default: return NAN;
  }
}

/* Group owning global row r (plain linear search). validate() guarantees one exists for
 * every r in [0, M). */
static int64_t group_of_row(const orc_problem* p, int64_t r) {
  for (int64_t g = 0; g < p->L; ++g)
    if (r >= p->cu_seqlens[g] && r < p->cu_seqlens[g + 1]) return g;
  return -1;
}

/* One output element: pre = alpha * sum_k A*B + beta * C, post = act(pre).
 * Activation-backward (dact, page 6 GemmDActSm90.epi_visit_acc_subtile): the GEMM gives the
 * incoming gradient dout = alpha * sum_k A*B (alpha = 1 on the page, which has none), C is
 * the saved pre-activation x; then pre (the D output) = dout * act'(x) and post (PostAct) =
 * act(x); with no activation D = dout and PostAct = x. beta is not used. */
static void elem(const orc_problem* p, const void* A, const void* B, const void* C, int64_t l,
                 int64_t m, int64_t n, double* pre, double* post) {
  int64_t lb = l;   /* batch index used for B */
  int64_t la = l;   /* batch index used for A */
  int64_t lx = l;   /* batch index used for C */
  int64_t k_lo = 0, k_hi = p->K;
  if (p->varlen) {
    lb = group_of_row(p, m);
    la = lx = 0;
  }
  if (p->varlen_k) {
    k_lo = p->cu_seqlens_k[l];
    k_hi = p->cu_seqlens_k[l + 1];
    la = lb = 0;
  }
  int64_t ma = (p->a_idx && p->varlen) ? (int64_t)p->a_idx[m] : m; /* the A row read */
  const int row_zero = p->a_idx && p->varlen && (ma < 0 || ma >= p->a_rows);
  double acc = 0.0;
  for (int64_t k = k_lo; k < k_hi && !row_zero; ++k) {
    int64_t ka = (p->a_idx && p->varlen_k) ? (int64_t)p->a_idx[k] : k; /* the A column read */
    if (p->a_idx && p->varlen_k && (ka < 0 || ka >= p->a_rows)) continue; /* a zero column */
    int64_t ia = la * p->sa + (p->a_kmajor ? ma * p->lda + ka : ka * p->lda + ma);
    int64_t ib = lb * p->sb + (p->b_kmajor ? n * p->ldb + k : k * p->ldb + n);
    acc += load_elem(A, p->a_dt, ia) * load_elem(B, p->b_dt, ib);
  }
  double v = p->alpha * acc;
  if (p->dact) {
    int64_t ic = lx * p->sc + (p->c_nmajor ? m * p->ldc + n : n * p->ldc + m);
    double x = load_elem(C, p->c_dt, ic);
    *pre = v * orc_dact(p->act, x);
    *post = orc_act(p->act, x);
    return;
  }
  if (p->has_c) {
    int64_t ic = lx * p->sc + (p->c_nmajor ? m * p->ldc + n : n * p->ldc + m);
    v += p->beta * load_elem(C, p->c_dt, ic);
  }
  *pre = v;
  *post = orc_act(p->act, v);
}

/* ---- threading over a list of work items ---- */
typedef struct {
  const orc_problem* p;
  const void *A, *B, *C;
  int64_t npts;
  const int64_t* pts; /* (l, m, n) triples */
  int64_t nrows;
  const int64_t* rows; /* (l, m) pairs: whole rows */
  double *pre, *post;
  int64_t begin, end;
} job_t;

static void* run_points(void* arg) {
  job_t* j = (job_t*)arg;
  for (int64_t i = j->begin; i < j->end; ++i)
    elem(j->p, j->A, j->B, j->C, j->pts[3 * i], j->pts[3 * i + 1], j->pts[3 * i + 2], &j->pre[i],
         &j->post[i]);
  return NULL;
}

static void* run_rows(void* arg) {
  job_t* j = (job_t*)arg;
  int64_t N = j->p->N;
  for (int64_t i = j->begin; i < j->end; ++i)
    for (int64_t n = 0; n < N; ++n)
      elem(j->p, j->A, j->B, j->C, j->rows[2 * i], j->rows[2 * i + 1], n, &j->pre[i * N + n],
           &j->post[i * N + n]);
  return NULL;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long c = sysconf(_SC_NPROCESSORS_ONLN);
  return c > 0 ? (int)c : 1;
}

static void parallel(job_t base, int64_t count, int nthreads, void* (*fn)(void*)) {
  nthreads = resolve_threads(nthreads);
  if (nthreads > count) nthreads = count > 0 ? (int)count : 1;
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = base;
    jobs[t].begin = count * t / nthreads;
    jobs[t].end = count * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, fn, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
}

/* Output elements at the given (l, m, n) triples (varlen: l ignored, m = global row). */
int orc_gemm_points(const orc_problem* p, const void* A, const void* B, const void* C,
                    int64_t npts, const int64_t* pts, double* pre, double* post, int nthreads) {
  int rc = validate(p);
  if (rc != ORC_OK) return rc;
  for (int64_t i = 0; i < npts; ++i)
    if (!point_ok(p, pts[3 * i], pts[3 * i + 1], pts[3 * i + 2])) return ORC_ERR_INDEX;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.p = p; j.A = A; j.B = B; j.C = C; j.npts = npts; j.pts = pts; j.pre = pre; j.post = post;
  parallel(j, npts, nthreads, run_points);
  return 0;
}

/* Whole output rows (l, m): pre/post are [nrows][N]. */
int orc_gemm_rows(const orc_problem* p, const void* A, const void* B, const void* C,
                  int64_t nrows, const int64_t* rows, double* pre, double* post, int nthreads) {
  int rc = validate(p);
  if (rc != ORC_OK) return rc;
  for (int64_t i = 0; i < nrows; ++i)
    if (p->N > 0 && !point_ok(p, rows[2 * i], rows[2 * i + 1], 0)) return ORC_ERR_INDEX;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.p = p; j.A = A; j.B = B; j.C = C; j.nrows = nrows; j.rows = rows; j.pre = pre; j.post = post;
  parallel(j, nrows, nthreads, run_rows);
  return 0;
}

/* Every output: pre/post are logical [L][M][N] (varlen: [M][N] over global rows). */
int orc_gemm_all(const orc_problem* p, const void* A, const void* B, const void* C, double* pre,
                 double* post, int nthreads) {
  int64_t nb = p->varlen ? 1 : p->L;
  int64_t nrows = nb * p->M;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * 2 * (size_t)(nrows > 0 ? nrows : 1));
  for (int64_t l = 0; l < nb; ++l)
    for (int64_t m = 0; m < p->M; ++m) {
      rows[2 * (l * p->M + m)] = l;
      rows[2 * (l * p->M + m) + 1] = m;
    }
  int rc = orc_gemm_rows(p, A, B, C, nrows, rows, pre, post, nthreads);
  free(rows);
  return rc;
}

/* Encode an array of doubles to codes of type dt (16-bit types -> uint16, f32 -> uint32). */
void orc_encode_array(int dt, int64_t n, const double* x, void* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t c = orc_encode(dt, x[i]);
    if (dt == ORC_F32) ((uint32_t*)out)[i] = c;
    else if (dt == ORC_E4M3 || dt == ORC_E5M2) ((uint8_t*)out)[i] = (uint8_t)c;
    else ((uint16_t*)out)[i] = (uint16_t)c;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Persistent tile map, with plain division.                                            */
/* ------------------------------------------------------------------------------------ */

/* Grouped raster inside one batch (page 5, the removed 0.1.10 "CTA Swizzle to promote L2
 * data reuse" in GemmSm90.kernel): with tm M-blocks and tn N-blocks, whole groups of G
 * M-blocks come first, M fastest inside a group, then N, then the next group; the
 * leftover tm % G M-blocks form a tail group with the same order. */
void orc_raster(int64_t r, int64_t tm, int64_t tn, int64_t G, int64_t* m, int64_t* n) {
  int64_t full = (tm / G) * G;
  if (r < full * tn) {
    int64_t grp = r / (G * tn);
    int64_t w = r % (G * tn);
    *m = grp * G + w % G;
    *n = w / G;
  } else {
    int64_t tail = tm - full;
    int64_t w = r - full * tn;
    *m = full + w % tail;
    *n = w / tail;
  }
}

/* Dense batched: linear tile t -> (m_blk, n_blk, l); batches are outermost. */
void orc_tile_dense(int64_t t, int64_t tm, int64_t tn, int64_t G, int64_t* m, int64_t* n,
                    int64_t* l) {
  *l = t / (tm * tn);
  orc_raster(t % (tm * tn), tm, tn, G, m, n);
}

/* Dense batched, raster along N: the same grouped raster with the roles of M and N
 * exchanged (groups of G N-blocks, N fastest inside a group; the order option that page 6's
 * quack/gemm_config.py keeps in its tuning space next to the swizzle size). */
void orc_tile_dense_n(int64_t t, int64_t tm, int64_t tn, int64_t G, int64_t* m, int64_t* n,
                      int64_t* l) {
  *l = t / (tm * tn);
  orc_raster(t % (tm * tn), tn, tm, G, n, m);
}

/* Varlen-M: groups in order, group g owning ceil(M_g/TM) * tn consecutive tile ids; empty
 * groups own none. Returns the group in *l and the block inside the group in *m. */
void orc_tile_varlen(int64_t t, const int32_t* cu, int64_t ngroups, int64_t TM, int64_t tn,
                     int64_t G, int64_t* m, int64_t* n, int64_t* l) {
  int64_t start = 0;
  for (int64_t g = 0; g < ngroups; ++g) {
    int64_t rows = (int64_t)cu[g + 1] - (int64_t)cu[g];
    int64_t tmg = (rows + TM - 1) / TM;
    if (t < start + tmg * tn) {
      *l = g;
      orc_raster(t - start, tmg, tn, G, m, n);
      return;
    }
    start += tmg * tn;
  }
  *m = *n = *l = -1;
}

/* Workgroup b of P takes tiles t = b' + i*P. With the XCD remap on and P % 8 == 0,
 * b' = (b % 8) * (P / 8) + b / 8, so that workgroups dispatched to the same one of the
 * 8 XCDs (round-robin by b) work on consecutive tile ids. */
int64_t orc_wg_tile(int64_t b, int64_t i, int64_t P, int32_t xcd_remap) {
  int64_t bb = b;
  if (xcd_remap && P % 8 == 0) bb = (b % 8) * (P / 8) + b / 8;
  return bb + i * P;
}

/* ------------------------------------------------------------------------------------ */
/* FastDivmod as on the pages (page 6, quack/fast_math.py), in 64-bit arithmetic.       */
/* ------------------------------------------------------------------------------------ */

/* ceil(log2(d)) for d >= 1: 31 - clz(d), plus one when d is not a power of two. */
static uint32_t ceil_log2_u32(uint32_t d) {
  int clz = 32;
  for (int i = 0; i < 32; ++i)
    if (d & (1u << (31 - i))) { clz = i; break; }
  return (uint32_t)(31 - clz) + ((d & (d - 1)) != 0);
}

void orc_fdm_create(uint32_t d, uint32_t* multiplier, uint32_t* shift_right) {
  uint32_t p = 31 + ceil_log2_u32(d);
  *multiplier = (uint32_t)((((uint64_t)1 << p) + d - 1) / d);
  *shift_right = p - 32; /* unused when d == 1 */
}

void orc_fdm_divmod(uint32_t n, uint32_t d, uint32_t mult, uint32_t shift, uint32_t* q,
                    uint32_t* r) {
  uint32_t qq = (d == 1) ? n : (uint32_t)((((uint64_t)n * mult) >> 32) >> shift);
  *q = qq;
  *r = n - qq * d;
}

/* Exhaustive check over d in [d_lo, d_hi], n in [0, n_count): the true quotient and
 * remainder are tracked by counting (no division), so the comparison does not reuse the
 * arithmetic under test. Returns the number of mismatching pairs. */
typedef struct { uint32_t d_lo, d_hi, n_count; uint64_t bad; } fdm_job_t;
static void* fdm_run(void* arg) {
  fdm_job_t* j = (fdm_job_t*)arg;
  uint64_t bad = 0;
  for (uint32_t d = j->d_lo; d <= j->d_hi && d >= j->d_lo; ++d) {
    uint32_t mult, shift;
    orc_fdm_create(d, &mult, &shift);
    uint32_t tq = 0, tr = 0;
    for (uint32_t n = 0; n < j->n_count; ++n) {
      uint32_t q = (d == 1) ? n : (uint32_t)((((uint64_t)n * mult) >> 32) >> shift);
      uint32_t r = n - q * d;
      bad += (q != tq) | (r != tr);
      if (++tr == d) { tr = 0; ++tq; }
    }
    if (d == 0xFFFFFFFFu) break;
  }
  j->bad = bad;
  return NULL;
}

uint64_t orc_fdm_exhaustive(uint32_t d_lo, uint32_t d_hi, uint32_t n_count, int nthreads) {
  nthreads = resolve_threads(nthreads);
  uint64_t span = (uint64_t)d_hi - d_lo + 1;
  if ((uint64_t)nthreads > span) nthreads = (int)span;
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  fdm_job_t* jobs = (fdm_job_t*)calloc((size_t)nthreads, sizeof(fdm_job_t));
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].d_lo = (uint32_t)(d_lo + span * t / nthreads);
    jobs[t].d_hi = (uint32_t)(d_lo + span * (t + 1) / nthreads - 1);
    jobs[t].n_count = n_count;
    pthread_create(&th[t], NULL, fdm_run, &jobs[t]);
  }
  uint64_t bad = 0;
  for (int t = 0; t < nthreads; ++t) {
    pthread_join(th[t], NULL);
    bad += jobs[t].bad;
  }
  free(th);
  free(jobs);
  return bad;
}

/* Edge sweep: every d in [d_lo, d_hi] at n in {0, 1, d-1, d, d+1, 2d-1, 2d, the multiples
 * of d just below 2^31 and their neighbours, 2^31-1}, against C's '/' and '%'. */
uint64_t orc_fdm_edges(uint32_t d_lo, uint32_t d_hi) {
  uint64_t bad = 0;
  for (uint64_t d = d_lo; d <= d_hi; ++d) {
    uint32_t mult, shift;
    orc_fdm_create((uint32_t)d, &mult, &shift);
    uint64_t top = (0x7FFFFFFFull / d) * d;
    uint64_t ns[12] = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, top - 1, top,
                       top + 1 <= 0x7FFFFFFFull ? top + 1 : top, top >= d ? top - d : 0,
                       0x7FFFFFFFull};
    for (int i = 0; i < 12; ++i) {
      uint64_t n = ns[i];
      if (n > 0x7FFFFFFFull) continue;
      uint32_t q, r;
      orc_fdm_divmod((uint32_t)n, (uint32_t)d, mult, shift, &q, &r);
      bad += (q != n / d) | (r != n % d);
    }
  }
  return bad;
}

/* Random pairs over the full domain 0 <= n < 2^31, 1 <= d < 2^31 (splitmix64 stream from
 * `seed`), against C's '/' and '%'. */
uint64_t orc_fdm_random(uint64_t count, uint64_t seed) {
  uint64_t s = seed, bad = 0;
  for (uint64_t i = 0; i < count; ++i) {
    uint64_t z;
    s += 0x9E3779B97F4A7C15ull; z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull; z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    uint32_t n = (uint32_t)(z & 0x7FFFFFFFu);
    /* log-uniform divisor (so that small and large ones are both frequent), even or odd:
     * a second draw gives d in [2^(bits-1), 2^bits) for bits in 1..31 */
    uint32_t bits = (uint32_t)((z >> 32) % 31) + 1;
    uint64_t z2;
    s += 0x9E3779B97F4A7C15ull; z2 = s;
    z2 = (z2 ^ (z2 >> 30)) * 0xBF58476D1CE4E5B9ull; z2 = (z2 ^ (z2 >> 27)) * 0x94D049BB133111EBull;
    z2 ^= z2 >> 31;
    uint32_t top = 1u << (bits - 1);
    uint32_t d = top | ((uint32_t)z2 & (top - 1u));
    uint32_t mult, shift, q, r;
    orc_fdm_create(d, &mult, &shift);
    orc_fdm_divmod(n, d, mult, shift, &q, &r);
    bad += (q != n / d) | (r != n % d);
  }
  return bad;
}
