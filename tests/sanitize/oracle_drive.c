/* Drive every oracle entry point on small problems in every mode, for a sanitizer build:
 * dense (all major modes, batches, C, activations, dact), varlen-M with empty groups and
 * gathered rows (indices in and out of range), varlen-K with gathered columns, malformed
 * cu_seqlens (which must be rejected, not read past), every code of every type, the tile maps
 * and FastDivmod. Exit status 0 when every call returns what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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
  const int32_t* cu_seqlens;
  int32_t dact;
  int32_t varlen_k;
  const int32_t* cu_seqlens_k;
  const int32_t* a_idx;
  int64_t a_rows;
} orc_problem;

double orc_decode(int dt, uint32_t code);
uint32_t orc_encode(int dt, double x);
double orc_act(int act, double x);
double orc_dact(int act, double x);
int orc_gemm_points(const orc_problem* p, const void* A, const void* B, const void* C, int64_t npts,
                    const int64_t* pts, double* pre, double* post, int nthreads);
int orc_gemm_rows(const orc_problem* p, const void* A, const void* B, const void* C, int64_t nrows,
                  const int64_t* rows, double* pre, double* post, int nthreads);
int orc_gemm_all(const orc_problem* p, const void* A, const void* B, const void* C, double* pre, double* post,
                 int nthreads);
void orc_encode_array(int dt, int64_t n, const double* x, void* out);
void orc_tile_dense(int64_t t, int64_t tm, int64_t tn, int64_t G, int64_t* m, int64_t* n, int64_t* l);
void orc_tile_dense_n(int64_t t, int64_t tm, int64_t tn, int64_t G, int64_t* m, int64_t* n, int64_t* l);
void orc_tile_varlen(int64_t t, const int32_t* cu, int64_t ngroups, int64_t TM, int64_t tn, int64_t G, int64_t* m,
                     int64_t* n, int64_t* l);
int64_t orc_wg_tile(int64_t b, int64_t i, int64_t P, int32_t xcd_remap);
void orc_fdm_create(uint32_t d, uint32_t* multiplier, uint32_t* shift_right);
uint64_t orc_fdm_exhaustive(uint32_t d_lo, uint32_t d_hi, uint32_t n_count, int nthreads);
uint64_t orc_fdm_edges(uint32_t d_lo, uint32_t d_hi);
uint64_t orc_fdm_random(uint64_t count, uint64_t seed);

static uint16_t* codes16(int64_t n, uint32_t seed) {
  uint16_t* v = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) v[i] = (uint16_t)(0x3C00u | ((seed + (uint32_t)i * 2654435761u) >> 22));  /* f16/bf16 in [1,2) or so */
  return v;
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d\n", __LINE__); return 1; } } while (0)

int main(void) {
  for (int dt = 1; dt <= 5; ++dt) {
    uint32_t n = dt == 3 ? 0 : (dt <= 2 ? 65536u : 256u);
    for (uint32_t c = 0; c < n; ++c) (void)orc_encode(dt, orc_decode(dt, c));
  }
  for (int a = 0; a <= 4; ++a) { (void)orc_act(a, 0.5); (void)orc_dact(a, -0.5); }
  double xs[5] = {1.0, -1e30, NAN, INFINITY, 3.5};
  uint16_t o16[5]; uint8_t o8[5]; uint32_t o32[5];
  orc_encode_array(1, 5, xs, o16); orc_encode_array(4, 5, xs, o8); orc_encode_array(3, 5, xs, o32);

  /* dense: every major combination, 3 batches, C, GELU; then dact */
  const int64_t M = 9, N = 7, K = 13, L = 3;
  uint16_t* A = codes16(L * M * K, 1);
  uint16_t* B = codes16(L * N * K, 2);
  uint16_t* C = codes16(L * M * N, 3);
  double* pre = (double*)malloc(sizeof(double) * L * M * N * 4);
  double* post = (double*)malloc(sizeof(double) * L * M * N * 4);
  for (int am = 0; am < 2; ++am)
    for (int bm = 0; bm < 2; ++bm)
      for (int cm = 0; cm < 2; ++cm) {
        orc_problem p;
        memset(&p, 0, sizeof(p));
        p.M = M; p.N = N; p.K = K; p.L = L;
        p.a_dt = p.b_dt = 2; p.c_dt = 1;
        p.a_kmajor = am; p.b_kmajor = bm; p.c_nmajor = cm;
        p.lda = am ? K : M; p.ldb = bm ? K : N; p.ldc = cm ? N : M;
        p.sa = M * K; p.sb = N * K; p.sc = M * N;
        p.alpha = 0.5; p.beta = 2.0; p.has_c = 1; p.act = 3;
        CHECK(orc_gemm_all(&p, A, B, C, pre, post, 2) == 0);
        p.dact = 1;
        CHECK(orc_gemm_all(&p, A, B, C, pre, post, 3) == 0);
        int64_t pts[6] = {0, 0, 0, 2, M - 1, N - 1};
        CHECK(orc_gemm_points(&p, A, B, C, 2, pts, pre, post, 1) == 0);
        int64_t bad[3] = {3, 0, 0};
        CHECK(orc_gemm_points(&p, A, B, C, 1, bad, pre, post, 1) != 0);
        int64_t rows[4] = {0, 0, 2, M - 1};
        CHECK(orc_gemm_rows(&p, A, B, C, 2, rows, pre, post, 2) == 0);
      }
  /* varlen-M with empty groups, gathered rows in and out of range, malformed arrays */
  {
    int32_t cu[5] = {0, 4, 4, 9, 9};
    int32_t idx[9] = {0, 8, -1, 3, 1 << 30, 5, 2, 7, 9};
    orc_problem p;
    memset(&p, 0, sizeof(p));
    p.M = 9; p.N = N; p.K = K; p.L = 4;
    p.a_dt = p.b_dt = 1; p.a_kmajor = p.b_kmajor = 1; p.lda = K; p.ldb = K; p.sb = N * K;
    p.alpha = 1.0; p.act = 4; p.varlen = 1; p.cu_seqlens = cu;
    uint16_t* Bv = codes16(4 * N * K, 4);
    CHECK(orc_gemm_all(&p, A, Bv, NULL, pre, post, 2) == 0);
    p.a_idx = idx; p.a_rows = 9;
    CHECK(orc_gemm_all(&p, A, Bv, NULL, pre, post, 2) == 0);
    int32_t bad1[5] = {0, 4, 3, 9, 9}, bad2[5] = {1, 4, 4, 9, 9}, bad3[5] = {0, 4, 4, 9, 12};
    p.cu_seqlens = bad1; CHECK(orc_gemm_all(&p, A, Bv, NULL, pre, post, 1) != 0);
    p.cu_seqlens = bad2; CHECK(orc_gemm_all(&p, A, Bv, NULL, pre, post, 1) != 0);
    p.cu_seqlens = bad3; CHECK(orc_gemm_all(&p, A, Bv, NULL, pre, post, 1) != 0);
    for (int64_t t = 0; t < 6; ++t) { int64_t m, n, l; orc_tile_varlen(t, cu, 4, 2, 2, 2, &m, &n, &l); }
    free(Bv);
  }
  /* varlen-K with gathered columns (in and out of range) and malformed arrays */
  {
    int32_t cuk[4] = {0, 5, 5, 13};
    int32_t kidx[13] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, -3, 99};
    orc_problem p;
    memset(&p, 0, sizeof(p));
    p.M = M; p.N = N; p.K = K; p.L = 3;
    p.a_dt = p.b_dt = 2; p.a_kmajor = 0; p.b_kmajor = 1; p.lda = M; p.ldb = K;
    p.alpha = 1.0; p.varlen_k = 1; p.cu_seqlens_k = cuk;
    CHECK(orc_gemm_all(&p, A, B, NULL, pre, post, 2) == 0);
    p.a_idx = kidx; p.a_rows = 11;
    CHECK(orc_gemm_all(&p, A, B, NULL, pre, post, 2) == 0);
    int32_t badk[4] = {0, 5, 4, 13}, badk2[4] = {0, 5, 5, 14};
    p.cu_seqlens_k = badk; CHECK(orc_gemm_all(&p, A, B, NULL, pre, post, 1) != 0);
    p.cu_seqlens_k = badk2; CHECK(orc_gemm_all(&p, A, B, NULL, pre, post, 1) != 0);
  }
  for (int64_t t = 0; t < 40; ++t) {
    int64_t m, n, l;
    orc_tile_dense(t, 5, 3, 4, &m, &n, &l);
    orc_tile_dense_n(t, 5, 3, 2, &m, &n, &l);
    (void)orc_wg_tile(t % 16, t / 16, 16, (int32_t)(t & 1));
  }
  uint32_t mu, sh;
  orc_fdm_create(1, &mu, &sh);
  orc_fdm_create(0x7FFFFFFFu, &mu, &sh);
  CHECK(orc_fdm_exhaustive(1, 300, 4096, 2) == 0);
  CHECK(orc_fdm_edges(1, 5000) == 0);
  CHECK(orc_fdm_random(100000, 7) == 0);
  free(A); free(B); free(C); free(pre); free(post);
  printf("oracle drive ok\n");
  return 0;
}
