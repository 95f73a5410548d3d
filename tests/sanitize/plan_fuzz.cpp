// Host-only fuzz of the plan builder (gemm_create and the plan queries) for a sanitizer
// build: seeded random descriptors, most near the validation boundaries, some with extreme
// values. Every call must return a status without undefined behaviour or invalid memory use;
// valid plans must report a consistent schedule. Exit status 0 on success.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gemm_mi355x.h"

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint64_t next() {  // splitmix64
  uint64_t z = (rs += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int64_t pick(const int64_t* v, int n) { return v[next() % n]; }

int main() {
  const int64_t sizes[] = {0, 1, 7, 8, 16, 100, 128, 255, 256, 257, 260, 4096, 8192, 65535, 1 << 20, 0x7FFFFFFF, -1};
  const int64_t lds[] = {0, 8, 16, 64, 260, 264, 4096, 8200, 1 << 24, (int64_t)1 << 31, (int64_t)1 << 40, -8};
  int ok = 0, rejected = 0;
  for (int it = 0; it < 200000; ++it) {
    // a valid descriptor of a random kind, then (most of the time) one field perturbed
    gemm_desc d;
    memset(&d, 0, sizeof(d));
    const int kind = (int)(next() % 4);  // dense, varlen-M, varlen-K, fp8 dense
    d.M = (int32_t)(8 * (1 + next() % 1024));
    d.N = (int32_t)(8 * (1 + next() % 1024));
    d.K = (int32_t)(16 * (next() % 512));
    d.L = (int32_t)(1 + next() % 6);
    d.a = d.b = next() % 2 ? GEMM_DT_BF16 : GEMM_DT_F16;
    if (kind == 3) { d.a = GEMM_DT_E4M3; d.b = next() % 2 ? GEMM_DT_E5M2 : GEMM_DT_E4M3; }
    d.a_major = kind == 3 ? GEMM_ROW : (int32_t)(next() % 2);
    d.b_major = kind == 3 ? GEMM_ROW : (int32_t)(next() % 2);
    d.d = (int32_t)(1 + next() % 5);
    if (d.d == GEMM_DT_E4M3 || d.d == GEMM_DT_E5M2) d.N = (d.N + 15) / 16 * 16, d.M = (d.M + 15) / 16 * 16;
    d.c = next() % 2 ? GEMM_DT_NONE : GEMM_DT_F32;
    d.post = next() % 3 ? GEMM_DT_NONE : GEMM_DT_F32;
    d.act = d.post ? (int32_t)(next() % 5) : 0;
    d.c_major = d.d_major = d.post_major = kind == 1 ? GEMM_ROW : (int32_t)(next() % 2);
    const int64_t contig_o = d.d_major == GEMM_ROW ? d.N : d.M, other_o = d.d_major == GEMM_ROW ? d.M : d.N;
    d.lda = d.a_major == GEMM_ROW ? d.K : d.M;
    d.ldb = d.b_major == GEMM_ROW ? d.K : d.N;
    d.ldc = d.ldd = d.ldp = contig_o + 8 * (int64_t)(next() % 3);
    d.sa = (int64_t)d.M * d.K;
    d.sb = (int64_t)d.N * d.K;
    d.sc = d.sd = d.sp = other_o * d.ldd;
    if (kind == 1) { d.varlen_m = 1; d.gather_a = next() % 4 == 0 && d.a_major == GEMM_ROW && kind != 3; d.gather_rows = d.M; }
    if (kind == 2) { d.varlen_k = 1; }
    d.alpha = 1.0f;
    d.beta = 1.0f;
    d.dact = kind == 0 && d.c != GEMM_DT_NONE && next() % 4 == 0;
    d.tile_m = d.tile_n = (int32_t)pick((const int64_t[]){0, 0, 128, 256}, 4);
    d.group_m = (int32_t)pick((const int64_t[]){0, 1, 2, 4, 8, 16}, 6);
    d.xcd_remap = (int32_t)(next() % 3) - 1;
    d.tail_split = (int32_t)(next() % 3) - 1;
    d.raster_order = kind == 1 ? (int32_t)(next() % 2) : (int32_t)(next() % 3);
    if (next() % 4) {  // perturb one field
      switch (next() % 12) {
        case 0: d.M = (int32_t)pick(sizes, 17); break;
        case 1: d.N = (int32_t)pick(sizes, 17); break;
        case 2: d.K = (int32_t)pick(sizes, 17); break;
        case 3: d.L = (int32_t)pick(sizes, 17); break;
        case 4: d.lda = pick(lds, 12); break;
        case 5: d.ldb = pick(lds, 12); break;
        case 6: d.ldd = pick(lds, 12); break;
        case 7: d.sd = pick(lds, 12); d.sa = pick(lds, 12); break;
        case 8: d.a = (int32_t)(next() % 8) - 1; break;
        case 9: d.act = (int32_t)(next() % 7) - 1; break;
        case 10: d.gather_a = 1; d.gather_rows = pick(sizes, 17); break;
        default: d.max_ctas = (int32_t)pick((const int64_t[]){1, 100, -1}, 3); break;
      }
    }
    gemm_plan* p = nullptr;
    gemm_status st = gemm_create(&d, &p);
    if (st == GEMM_OK) {
      ++ok;
      int32_t tm, tn, g, x, P, along;
      int64_t T;
      if (gemm_plan_grid(p, 256, &tm, &tn, &g, &x, &T, &P) != GEMM_OK) return 2;
      if (gemm_plan_raster(p, &along) != GEMM_OK) return 3;
      // the grid holds 1..T workgroups (none for an empty problem; the cap for varlen, T = -1)
      if (T > 0 ? (P < 1 || (int64_t)P > T) : (T == 0 ? P != 0 : P < 1)) {
        fprintf(stderr, "grid %d for %lld tiles (M=%d N=%d K=%d L=%d)\n", P, (long long)T, d.M, d.N, d.K, d.L);
        gemm_destroy(p);
        return 4;
      }
      if (gemm_destroy(p) != GEMM_OK) return 5;
    } else {
      ++rejected;
      if (p != nullptr) return 6;
      if (gemm_last_error()[0] == 0) return 7;
    }
    (void)gemm_status_string(st);
  }
  uint32_t m, s;
  for (uint32_t dv = 1; dv < 70000; dv += 7) gemm_fastdivmod_params(dv, &m, &s);
  gemm_fastdivmod_params(0x7FFFFFFFu, &m, &s);
  if (gemm_fastdivmod_params(0, &m, &s) == GEMM_OK) return 8;
  if (gemm_create(nullptr, nullptr) == GEMM_OK) return 9;
  printf("plans accepted %d, rejected %d\n", ok, rejected);
  return ok > 0 && rejected > 0 ? 0 : 10;
}
