// Host side of the C ABI: validation of a gemm_desc, choice of the kernel and tile, the
// persistent schedule constants (FastDivmod, quack-kernels 0.1.10 -> 0.2.0 diff, page 6,
// quack/fast_math.py) and status/error reporting. No HIP call is made here.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>

#include "../../include/gemm_mi355x.h"
#include "params.hpp"

namespace gep {

static thread_local std::string g_last_error;

gemm_status fail(gemm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }
const char* last_error() { return g_last_error.c_str(); }

static int elem_bytes(int32_t dt) {
  switch (dt) {
    case DT_F16:
    case DT_BF16: return 2;
    case DT_F32: return 4;
    case DT_E4M3:
    case DT_E5M2: return 1;
    default: return 0;
  }
}

static bool is_input_type(int32_t dt) {
  return dt == DT_F16 || dt == DT_BF16 || dt == DT_E4M3 || dt == DT_E5M2;
}
// C: 16-bit or f32; D and PostAct also OCP fp8 (page 5 is_valid_dtypes), saturating
static bool is_output_type(int32_t dt, bool c) {
  return dt == DT_NONE || dt == DT_F16 || dt == DT_BF16 || dt == DT_F32 || (!c && (dt == DT_E4M3 || dt == DT_E5M2));
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest stride (elements) and operand span (bytes) accepted: products of a stride with any
// index stay far inside int64 on the host and in the kernels.
constexpr int64_t kMaxStride = (int64_t)1 << 48;
constexpr int64_t kMaxSpan = (int64_t)1 << 62;

// Check one operand: contiguous extent and strides in whole 16-byte chunks, leading
// dimension covering the contiguous extent, the whole addressed span (nb batches) bounded.
static gemm_status check_operand(const char* name, int es, int64_t contig, int64_t ld,
                                 int64_t other_extent, int64_t batch_stride, int64_t nb) {
  if (ld < 0 || batch_stride < 0) return fail(GEMM_ERR_INVALID_ARG, "%s: negative stride", name);
  if (ld > kMaxStride || batch_stride > kMaxStride)
    return fail(GEMM_ERR_UNSUPPORTED, "%s: stride beyond 2^48 elements", name);
  if (contig > 0 && other_extent > 0 && nb > 0) {
    const __int128 span = ((__int128)(nb - 1) * batch_stride + (__int128)(other_extent - 1) * ld + contig) * es;
    if (span > kMaxSpan) return fail(GEMM_ERR_UNSUPPORTED, "%s: addresses more than 2^62 bytes", name);
  }
  if (other_extent > 1 && ld < contig)
    return fail(GEMM_ERR_INVALID_ARG, "%s: leading dimension %lld smaller than the contiguous extent %lld",
                name, (long long)ld, (long long)contig);
  if ((contig * es) % 16 != 0)
    return fail(GEMM_ERR_ALIGNMENT, "%s: contiguous extent %lld x %d bytes is not a multiple of 16 bytes",
                name, (long long)contig, es);
  if ((ld * es) % 16 != 0)
    return fail(GEMM_ERR_ALIGNMENT, "%s: leading dimension %lld x %d bytes is not a multiple of 16 bytes",
                name, (long long)ld, es);
  if ((batch_stride * es) % 16 != 0)
    return fail(GEMM_ERR_ALIGNMENT, "%s: batch stride is not a multiple of 16 bytes", name);
  return GEMM_OK;
}

gemm_status create_plan(const gemm_desc* d_in, gemm_plan** out) {
  if (out) *out = nullptr;
  if (!d_in || !out) return fail(GEMM_ERR_INVALID_ARG, "gemm_create: NULL argument");
  gemm_desc d = *d_in;

  if (d.M < 0 || d.N < 0 || d.K < 0 || d.L < 0)
    return fail(GEMM_ERR_INVALID_ARG, "negative size (M=%d N=%d K=%d L=%d)", d.M, d.N, d.K, d.L);
  if (d.varlen_m != 0 && d.varlen_m != 1) return fail(GEMM_ERR_INVALID_ARG, "varlen_m must be 0 or 1");
  if (d.varlen_k != 0 && d.varlen_k != 1) return fail(GEMM_ERR_INVALID_ARG, "varlen_k must be 0 or 1");
  if (d.gather_a != 0 && d.gather_a != 1) return fail(GEMM_ERR_INVALID_ARG, "gather_a must be 0 or 1");
  if (d.varlen_m && d.varlen_k) return fail(GEMM_ERR_INVALID_ARG, "varlen_m and varlen_k are exclusive");
  if (d.gather_a && !d.varlen_m && !d.varlen_k)
    return fail(GEMM_ERR_INVALID_ARG, "gathered A needs varlen-M or varlen-K");
  if (d.gather_a && d.gather_rows < 0) return fail(GEMM_ERR_INVALID_ARG, "gather_rows < 0");
  const int32_t majors[5] = {d.a_major, d.b_major, d.c_major, d.d_major, d.post_major};
  for (int i = 0; i < 5; ++i)
    if (majors[i] != GEMM_ROW && majors[i] != GEMM_COL)
      return fail(GEMM_ERR_INVALID_ARG, "unknown major mode %d", majors[i]);
  if (d.act < GEMM_ACT_NONE || d.act > GEMM_ACT_SILU) return fail(GEMM_ERR_INVALID_ARG, "unknown activation %d", d.act);

  // ---- types (page 5, GemmSm90.is_valid_dtypes and the __call__ type checks)
  if (!is_input_type(d.a) || !is_input_type(d.b))
    return fail(d.a < 0 || d.a > 5 || d.b < 0 || d.b > 5 ? GEMM_ERR_INVALID_ARG : GEMM_ERR_UNSUPPORTED,
                "A/B type must be f16, bf16, e4m3 or e5m2 (got %d, %d)", d.a, d.b);
  const int es_a = elem_bytes(d.a), es_b = elem_bytes(d.b);
  if (es_a != es_b) return fail(GEMM_ERR_UNSUPPORTED, "A and B must have the same width");
  if (es_a == 2 && d.a != d.b) return fail(GEMM_ERR_UNSUPPORTED, "16-bit A and B must have the same type");
  if (es_a == 1 && (d.a_major != GEMM_ROW || d.b_major != GEMM_ROW))
    return fail(GEMM_ERR_UNSUPPORTED, "fp8 A and B must be K-major");
  const int32_t outs[3] = {d.c, d.d, d.post};
  for (int i = 0; i < 3; ++i) {
    if (outs[i] < 0 || outs[i] > 5) return fail(GEMM_ERR_INVALID_ARG, "unknown dtype %d", outs[i]);
    if (!is_output_type(outs[i], i == 0))
      return fail(GEMM_ERR_UNSUPPORTED, "C must be f16, bf16 or f32; D and PostAct f16, bf16, f32, e4m3 or e5m2");
  }
  if (d.d == DT_NONE && d.post == DT_NONE) return fail(GEMM_ERR_INVALID_ARG, "neither D nor PostAct requested");
  if (d.dact != 0 && d.dact != 1) return fail(GEMM_ERR_INVALID_ARG, "dact must be 0 or 1");
  if (d.dact) {
    // activation backward (page 6, gemm_dact_sm90): C is the saved pre-activation, D the
    // gradient dout * act'(C); beta has no role there
    if (d.c == DT_NONE) return fail(GEMM_ERR_INVALID_ARG, "dact: C (the pre-activation) is required");
    if (d.d == DT_NONE) return fail(GEMM_ERR_INVALID_ARG, "dact: D (the gradient) is required");
    if (d.beta != 1.0f) return fail(GEMM_ERR_INVALID_ARG, "dact: beta is not used and must be 1");
    if (d.varlen_k || d.gather_a)
      return fail(GEMM_ERR_UNSUPPORTED, "dact: not offered with varlen-K or gathered A");
  } else if (d.act != GEMM_ACT_NONE && d.post == DT_NONE) {
    return fail(GEMM_ERR_INVALID_ARG, "an activation needs a PostAct output");
  }

  // ---- output majors: D and PostAct share one; C may have either (page 5, gemm_sm90 reads
  // each operand's major mode from its own strides)
  int32_t out_major = -1;
  const int32_t omaj[3] = {d.c_major, d.d_major, d.post_major};
  for (int i = 1; i < 3; ++i) {
    if (outs[i] == DT_NONE) continue;
    if (out_major == -1) out_major = omaj[i];
    else if (out_major != omaj[i]) return fail(GEMM_ERR_UNSUPPORTED, "D and PostAct must share one major mode");
  }
  const bool c_trans = d.c != DT_NONE && d.c_major != out_major;
  if (d.varlen_m && (out_major == GEMM_COL || c_trans))
    return fail(GEMM_ERR_UNSUPPORTED, "varlen-M needs N-major C/D/PostAct");
  if (d.gather_a && d.varlen_m && (es_a != 2 || d.a_major != GEMM_ROW))
    return fail(GEMM_ERR_UNSUPPORTED, "gathered A rows (varlen-M): A must be a 16-bit K-major operand");
  if (d.gather_a && d.varlen_k && (es_a != 2 || d.a_major != GEMM_COL || out_major == GEMM_COL))
    return fail(GEMM_ERR_UNSUPPORTED,
                "gathered A columns (varlen-K): A must be a 16-bit M-major operand and the outputs N-major");

  // ---- tuning fields
  int32_t G = d.group_m == 0 ? 8 : d.group_m;
  if (G < 1 || G > (1 << kMaxGroupLog2) || (G & (G - 1)) != 0)
    return fail(GEMM_ERR_INVALID_ARG, "group_m must be a power of two in [1, 16]");
  if (d.max_ctas < 0) return fail(GEMM_ERR_INVALID_ARG, "max_ctas < 0");
  if (d.xcd_remap < -1 || d.xcd_remap > 1) return fail(GEMM_ERR_INVALID_ARG, "xcd_remap must be -1, 0 or 1");
  if (d.tail_split < -1 || d.tail_split > 1) return fail(GEMM_ERR_INVALID_ARG, "tail_split must be -1, 0 or 1");
  if (d.raster_order < 0 || d.raster_order > 2) return fail(GEMM_ERR_INVALID_ARG, "raster_order must be 0, 1 or 2");
  if (d.raster_order == 2 && d.varlen_m)
    return fail(GEMM_ERR_UNSUPPORTED, "raster along N is not offered for varlen-M (its M-blocks vary per group)");
  if (d.varlen_m && d.L > kMaxVarlenGroups)
    return fail(GEMM_ERR_UNSUPPORTED, "varlen-M supports at most %d groups", kMaxVarlenGroups);

  // ---- strides and alignment, in the caller's (unswapped) terms
  const int64_t M = d.M, N = d.N, K = d.K;
  const bool batched = !d.varlen_m && d.L > 1;  // batched outputs (dense and varlen-K)
  const bool a_batched = batched && !d.varlen_k;
  const int64_t rows_a = (d.gather_a && d.varlen_m) ? d.gather_rows : M;  // rows A's pointer addresses
  const int64_t cols_a = (d.gather_a && d.varlen_k) ? d.gather_rows : K;  // its K extent
  gemm_status st;
  const int64_t nb_a = a_batched ? d.L : 1;
  if (d.a_major == GEMM_ROW) st = check_operand("A", es_a, K, d.lda, rows_a, a_batched ? d.sa : 0, nb_a);
  else st = check_operand("A", es_a, M, d.lda, cols_a, a_batched ? d.sa : 0, nb_a);
  if (st != GEMM_OK) return st;
  const bool b_batched = d.varlen_m ? d.L > 1 : (batched && !d.varlen_k);
  const int64_t nb_b = b_batched ? d.L : 1;
  if (d.b_major == GEMM_ROW) st = check_operand("B", es_b, K, d.ldb, N, b_batched ? d.sb : 0, nb_b);
  else st = check_operand("B", es_b, N, d.ldb, K, b_batched ? d.sb : 0, nb_b);
  if (st != GEMM_OK) return st;
  struct { const char* n; int32_t dt; int64_t ld, s; } xo[3] = {
      {"C", d.c, d.ldc, d.sc}, {"D", d.d, d.ldd, d.sd}, {"PostAct", d.post, d.ldp, d.sp}};
  for (int i = 0; i < 3; ++i) {
    if (xo[i].dt == DT_NONE) continue;
    int es = elem_bytes(xo[i].dt);
    const int32_t maj = i == 0 ? d.c_major : out_major;
    int64_t contig = maj == GEMM_ROW ? N : M, other = maj == GEMM_ROW ? M : N;
    st = check_operand(xo[i].n, es, contig, xo[i].ld, other, batched ? xo[i].s : 0, batched ? d.L : 1);
    if (st != GEMM_OK) return st;
    // written outputs of different batches must not overlap
    if (i > 0 && batched && other > 0 && (__int128)xo[i].s < (__int128)other * xo[i].ld)
      return fail(GEMM_ERR_INVALID_ARG, "%s: batch stride overlaps the previous batch", xo[i].n);
  }

  // ---- the kernel's view: M-major outputs are computed as the transposed problem
  gemm_plan* p = new (std::nothrow) gemm_plan;
  if (!p) return fail(GEMM_ERR_NO_MEMORY, "plan allocation failed");
  memset(p, 0, sizeof(*p));
  const bool swap = out_major == GEMM_COL;
  p->swapped = swap ? 1 : 0;
  KParams& k = p->base;
  int32_t ta = d.a, tb = d.b;
  int32_t amaj = d.a_major, bmaj = d.b_major;
  int64_t lda = d.lda, ldb = d.ldb, sa = d.sa, sb = d.sb;
  k.M = d.M;
  k.N = d.N;
  if (swap) {
    int32_t t = ta; ta = tb; tb = t;
    t = amaj; amaj = bmaj; bmaj = t;
    int64_t x = lda; lda = ldb; ldb = x;
    x = sa; sa = sb; sb = x;
    k.M = d.N;
    k.N = d.M;
  }
  k.K = d.K;
  k.L = d.L;
  k.lda = lda; k.ldb = ldb; k.ldc = d.ldc; k.ldd = d.ldd; k.ldp = d.ldp;
  k.sa = a_batched ? sa : 0;
  k.sb = b_batched ? sb : 0;
  k.sc = batched ? d.sc : 0;
  k.sd = batched ? d.sd : 0;
  k.sp = batched ? d.sp : 0;
  {
    // addressable extents (bytes) of A and B in the kernel's terms; 0 when empty
    const int64_t ra = swap ? k.M : rows_a, rb = swap ? rows_a : k.N;  // (no swap with gather)
    const int64_t la = a_batched ? d.L : 1, lb = b_batched ? d.L : 1;
    auto extent = [&](bool kmaj, int64_t rows, int64_t ld, int64_t s, int64_t nb, int es, int64_t kx) -> int64_t {
      if (rows == 0 || kx == 0 || nb == 0) return 0;
      const int64_t last = kmaj ? (rows - 1) * ld + kx : (kx - 1) * ld + rows;
      return ((nb - 1) * s + last) * es;
    };
    k.a_bytes = extent(amaj == GEMM_ROW, ra, lda, k.sa, la, es_a, cols_a);
    k.b_bytes = extent(bmaj == GEMM_ROW, rb, ldb, k.sb, lb, es_b, K);
  }
  if (d.gather_a) {
    // gathered rows are addressed from A's base with 32-bit offsets
    if (k.a_bytes >= ((int64_t)1 << 31) || d.gather_rows >= ((int64_t)1 << 31)) {
      delete p;
      return fail(GEMM_ERR_UNSUPPORTED, "gathered A must span less than 2^31 bytes");
    }
    k.a_rows = (int32_t)d.gather_rows;
  }
  k.alpha = d.alpha;
  k.beta = d.beta;
  k.c_dt = d.c;
  k.c_trans = c_trans ? 1 : 0;
  k.d_dt = d.d;
  k.p_dt = d.post;
  k.act = d.act;

  KernelKey& key = p->key;
  key.op = es_a == 1 ? OP_FP8 : (ta == DT_F16 ? OP_F16 : OP_BF16);
  key.fmt_a = ta == DT_E5M2 ? 1 : 0;
  key.fmt_b = tb == DT_E5M2 ? 1 : 0;
  key.a_kmajor = amaj == GEMM_ROW ? 1 : 0;
  key.b_kmajor = bmaj == GEMM_ROW ? 1 : 0;
  key.varlen = d.varlen_m ? 1 : (d.varlen_k ? 2 : 0);
  key.dact = d.dact;
  key.gather = d.gather_a;

  // ---- tile choice
  int32_t tmn = 0;
  if (d.tile_m == 0 && d.tile_n == 0) {
    int64_t rows = k.M;
    int64_t t256 = cdiv(rows, 256) * cdiv(k.N, 256) * (d.varlen_m ? 1 : d.L);
    tmn = t256 >= 128 ? 256 : 128;
  } else if (d.tile_m == d.tile_n && (d.tile_m == 256 || d.tile_m == 128)) {
    tmn = d.tile_m;
  } else {
    delete p;
    return fail(GEMM_ERR_UNSUPPORTED, "tile %dx%d not offered (256x256 or 128x128)", d.tile_m, d.tile_n);
  }
  key.tile = tmn == 256 ? 0 : 1;
  p->tile_m = p->tile_n = tmn;
  p->wg_per_cu = tmn == 256 ? 1 : 2;

  // ---- byte offsets inside one tile must stay below 2^31 (32-bit buffer offsets)
  const int64_t lim = (int64_t)1 << 31;
  if ((key.a_kmajor ? (int64_t)tmn * lda : 64 * lda) * es_a >= lim ||
      (key.b_kmajor ? (int64_t)tmn * ldb : 64 * ldb) * es_b >= lim) {
    delete p;
    return fail(GEMM_ERR_UNSUPPORTED, "leading dimension too large for 32-bit tile offsets");
  }

  // ---- schedule constants
  const int64_t tm = cdiv(k.M, tmn), tn = cdiv(k.N, tmn);
  int log2G = 0;
  while ((1 << log2G) < G) ++log2G;
  k.log2G = log2G;
  k.tn = (int32_t)tn;
  k.fd_Gtn = make_fastdiv((uint32_t)std::max<int64_t>(1, G * tn));
  k.fd_Gtm = make_fastdiv((uint32_t)std::max<int64_t>(1, G * tm));
  // default: along N for a single dense GEMM that reads C (measured, same box: 4096^3 with C,
  // D and GELU PostAct +5%, its activation backward +2.4%), else along M, the page's order
  // (8192^3 bf16 and f16 without C +4%, fp8 neutral; batches +0.9%)
  k.raster_n = (d.raster_order == 2 ||
                (d.raster_order == 0 && !d.varlen_m && d.L == 1 && d.c != DT_NONE)) ? 1 : 0;
  for (int w = 1; w < (1 << kMaxGroupLog2); ++w) k.fd_tail[w] = make_fastdiv((uint32_t)w);
  k.fd_tail[0] = make_fastdiv(1);
  if (d.varlen_m) {
    // worst case over any split of M rows into L groups
    int64_t tmax = (cdiv(k.M, tmn) + d.L) * tn;
    if (tmax >= lim) { delete p; return fail(GEMM_ERR_UNSUPPORTED, "too many tiles"); }
    k.tm = 0;
    k.T = 0;
    p->T = -1;
    k.fd_mn = make_fastdiv(1);
  } else {
    int64_t T = tm * tn * d.L;
    if (T >= lim) { delete p; return fail(GEMM_ERR_UNSUPPORTED, "too many tiles (%lld)", (long long)T); }
    k.tm = (int32_t)tm;
    k.T = (int32_t)T;
    p->T = T;
    k.fd_mn = make_fastdiv((uint32_t)std::max<int64_t>(1, tm * tn));
  }
  k.xcd_remap = d.xcd_remap == -1 ? 0 : 1;
  k.tail = 0;
  k.P_big = 0;
  p->tail_split = (d.tail_split != -1 && key.tile == 0) ? 1 : 0;
  p->max_ctas = d.max_ctas;
  p->varlen = d.varlen_m;
  p->varlen_k = d.varlen_k;
  p->gather = d.gather_a;
  p->L = d.L;
  p->has_c = d.c != DT_NONE;
  p->has_d = d.d != DT_NONE;
  p->has_p = d.post != DT_NONE;
  *out = p;
  clear_error();
  return GEMM_OK;
}

int32_t grid_size(const gemm_plan* p, int32_t num_cus) {
  int64_t cap = (int64_t)num_cus * p->wg_per_cu;
  if (p->max_ctas > 0 && p->max_ctas < cap) cap = p->max_ctas;
  if (cap < 1) cap = 1;
  if (p->varlen) return (int32_t)cap;
  return (int32_t)(p->T < cap ? p->T : cap);
}

}  // namespace gep

extern "C" {

gemm_status gemm_create(const gemm_desc* desc, gemm_plan** out) { return gep::create_plan(desc, out); }

gemm_status gemm_destroy(gemm_plan* plan) {
  delete plan;
  return GEMM_OK;
}

gemm_status gemm_plan_grid(const gemm_plan* p, int32_t num_cus, int32_t* tile_m, int32_t* tile_n,
                           int32_t* group_m, int32_t* xcd_remap, int64_t* tiles, int32_t* grid) {
  if (!p) return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_plan_grid: NULL plan");
  if (num_cus <= 0) return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_plan_grid: num_cus <= 0");
  if (tile_m) *tile_m = p->tile_m;
  if (tile_n) *tile_n = p->tile_n;
  if (group_m) *group_m = 1 << p->base.log2G;
  if (xcd_remap) *xcd_remap = p->base.xcd_remap;
  if (tiles) *tiles = p->T;
  if (grid) *grid = gep::grid_size(p, num_cus);
  return GEMM_OK;
}

gemm_status gemm_plan_raster(const gemm_plan* p, int32_t* along_n) {
  if (!p || !along_n) return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_plan_raster: NULL argument");
  *along_n = p->base.raster_n;
  return GEMM_OK;
}

gemm_status gemm_fastdivmod_params(uint32_t d, uint32_t* multiplier, uint32_t* shift) {
  if (d < 1 || d > 0x7FFFFFFFu) return gep::fail(GEMM_ERR_INVALID_ARG, "divisor out of [1, 2^31)");
  FastDiv f = make_fastdiv(d);
  if (multiplier) *multiplier = f.multiplier;
  if (shift) *shift = f.shift;
  return GEMM_OK;
}

const char* gemm_status_string(gemm_status s) {
  switch (s) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_ERR_UNSUPPORTED: return "unsupported";
    case GEMM_ERR_ALIGNMENT: return "misaligned";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_NO_MEMORY: return "out of host memory";
    default: return "unknown status";
  }
}

const char* gemm_last_error(void) { return gep::last_error(); }

}  // extern "C"
