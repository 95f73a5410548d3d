/*
 * gemm_mi355x.h - C ABI of the MI355X (gfx950) batched GEMM with fused epilogue.
 *
 *   D       = alpha * A x B + beta * C          (the pre-activation output)
 *   PostAct = act(alpha * A x B + beta * C)
 *
 * The operation is the one defined by the quack-kernels pages (0.1.10 -> 0.2.0 diff):
 *   - page 5, quack/dense_gemm_sm90.py: the gemm_sm90 wrapper takes A (l, m, k), B (l, n, k),
 *     D and C (l, m, n); GemmSm90.epi_visit_acc_subtile scales the fp32 accumulator by alpha
 *     and adds beta * C (beta absent means +C);
 *   - page 6, quack/gemm_act_sm90.py: GemmActSm90.epi_visit_acc_subtile applies the
 *     activation to that same fp32 value and writes it as PostAct next to D; act_fn_map lists
 *     relu, relu_sq and gelu_tanh_approx;
 *   - page 5, GemmSm90.__call__ and kernel: the varlen-M (grouped) mode, where cu_seqlens_m
 *     splits the rows of A / C / D into groups and group g multiplies by its own B[g];
 *   - page 5, GemmSm90.is_valid_dtypes: fp16 / bf16 / e4m3 / e5m2 inputs, fp32 accumulation,
 *     fp8 operands K-major only;
 *   - page 5, GemmSm90.kernel, and the torch-vendored quack/gemm_sm90.py page: the varlen-K
 *     (grouped K) mode, where cu_seqlens_k splits the K range of A and B into groups that
 *     each produce one output batch, and gathered A (mAIdx: A rows read through an index
 *     array).
 * SiLU is an addition of this library (x * sigmoid(x)).
 *
 * Conventions used by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or retains them. gemm_run writes only D, PostAct and (debug) the
 *     tile log; it reads A, B, C, alpha/beta pointers and cu_seqlens_m.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Launches are
 *     asynchronous; no entry point synchronises a stream or the device.
 *   - Errors are returned as gemm_status, never thrown; gemm_last_error() gives a
 *     thread-local message describing the last failure on the calling thread.
 *   - A gemm_plan holds host memory only. gemm_create makes no HIP call. A plan may be used
 *     from several threads and streams at once (gemm_run does not modify it).
 */
#ifndef GEMM_MI355X_H
#define GEMM_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, inconsistent strides  */
  GEMM_ERR_UNSUPPORTED = 2, /* valid request this library does not implement          */
  GEMM_ERR_ALIGNMENT = 3,   /* contiguous dimension / pointer not 16-byte aligned     */
  GEMM_ERR_HIP = 4,         /* a HIP runtime call failed (message in gemm_last_error) */
  GEMM_ERR_NO_MEMORY = 5    /* host allocation of the plan failed                    */
} gemm_status;

typedef enum {
  GEMM_DT_NONE = 0, /* operand absent (C, D or PostAct only)          */
  GEMM_DT_F16 = 1,  /* IEEE binary16                                  */
  GEMM_DT_BF16 = 2, /* bfloat16                                       */
  GEMM_DT_F32 = 3,  /* IEEE binary32 (C, D, PostAct only)             */
  GEMM_DT_E4M3 = 4, /* OCP fp8 E4M3 ("fn": no inf, max 448)           */
  GEMM_DT_E5M2 = 5  /* OCP fp8 E5M2 (IEEE-like inf/NaN, max 57344)    */
} gemm_dtype;

/* Which logical dimension is contiguous in memory (page 5, gemm_sm90: majors from strides).
 *   A (l, m, k):  GEMM_ROW = K contiguous ("K-major"):  A[l*sa + m*lda + k]
 *                 GEMM_COL = M contiguous ("M-major"):  A[l*sa + k*lda + m]
 *   B (l, n, k):  GEMM_ROW = K contiguous:              B[l*sb + n*ldb + k]
 *                 GEMM_COL = N contiguous:              B[l*sb + k*ldb + n]
 *   C, D, PostAct (l, m, n):
 *                 GEMM_ROW = N contiguous:              X[l*sx + m*ldx + n]
 *                 GEMM_COL = M contiguous:              X[l*sx + n*ldx + m]            */
typedef enum { GEMM_ROW = 0, GEMM_COL = 1 } gemm_major;

/* Activation applied to the fp32 pre-activation value to form PostAct
 * (page 6, gemm_act_sm90.py, act_fn_map; SiLU added by this library). */
typedef enum {
  GEMM_ACT_NONE = 0,      /* PostAct = pre                                            */
  GEMM_ACT_RELU = 1,      /* max(pre, 0)                                              */
  GEMM_ACT_RELU_SQ = 2,   /* max(pre, 0)^2                                            */
  GEMM_ACT_GELU_TANH = 3, /* pre/2 * (1 + tanh(sqrt(2/pi) * (pre + 0.044715 pre^3)))  */
  GEMM_ACT_SILU = 4       /* pre / (1 + exp(-pre))                                    */
} gemm_act;

/* Problem description. Sizes and strides are in ELEMENTS.
 *
 * Dense batched mode (varlen_m == 0): A is (L, M, K), B is (L, N, K), C/D/PostAct are
 * (L, M, N); sa/sb/sc/sd/sp are the batch strides (ignored when L == 1).
 *
 * Varlen-M mode (varlen_m == 1, page 5, GemmSm90 with VarlenMTileScheduler): L is the
 * number of groups G and M the total number of rows. A is (M, K), C/D/PostAct are (M, N),
 * B is (G, N, K) with batch stride sb; cu_seqlens_m (passed to gemm_run, device int32[G+1])
 * gives the row range [cu[g], cu[g+1]) of group g. sa/sc/sd/sp are ignored.
 *
 * Types: a, b in {F16, BF16, E4M3, E5M2}. 16-bit inputs need a == b; 8-bit inputs may mix
 * E4M3 and E5M2 and must both be GEMM_ROW (K-major) (page 5, is_valid_dtypes).
 * c in {NONE, F16, BF16, F32}; d, post in {NONE, F16, BF16, F32, E4M3, E5M2} (page 5
 * is_valid_dtypes admits fp8 D); at least one of d, post is not NONE. fp8 outputs round
 * to nearest even and saturate: magnitudes past the largest finite value (448 for E4M3,
 * 57344 for E5M2), infinities included, become it; NaN stays NaN.
 * The C term is present iff c != NONE; beta multiplies it (beta = 1 gives +C; beta = 0
 * still reads C, so NaN/inf in C propagate).
 * C, D and PostAct that are present must share one major mode.
 * Varlen mode supports only GEMM_ROW outputs.
 *
 * Varlen-K mode (varlen_k == 1; page 5, GemmSm90.kernel offsets A and B along K by
 * cu_seqlens_k[l] and ends the group's K range at cu_seqlens_k[l+1]): L is the number of
 * groups and K the total K extent of A and B. A is (M, K) and B is (N, K) with no batch
 * index (sa, sb ignored); C/D/PostAct are (L, M, N) with batch strides sc/sd/sp, batch l
 * holding group l: D[l] = alpha * A[:, k in group l] x B[:, k in group l]^T (+ beta C[l]),
 * an empty group giving alpha * 0. cu_seqlens_k (device int32[L+1], in gemm_args) gives
 * the ranges; precondition (not checked): cu[0] == 0, non-decreasing, cu[L] <= K, and when
 * A or B is K-major, every cu[g] times the element size a multiple of 16 bytes (the group
 * starts on a 16-byte chunk). Any major modes and output majors; no activation backward.
 * varlen_m and varlen_k are exclusive.
 *
 * Gathered A (gather_a == 1; the pages' mAIdx, load_AB_gather_A and the torch-vendored
 * page's gather copies), 16-bit A at most 2^31 bytes from its pointer, no activation backward:
 *   - varlen-M: output row r (global, in [0, M)) reads A row a_idx[r] instead of row r. A is
 *     (gather_rows, K), K-major; a_idx is device int32[M].
 *   - varlen-K: global k (in [0, K)) reads A column a_idx[k] instead of column k. A is
 *     (M, gather_rows), M-major (each column one contiguous row of storage); a_idx is device
 *     int32[K]; C/D/PostAct N-major. B is not gathered.
 * a_idx (in gemm_args) may repeat indices; an index outside [0, gather_rows) reads zeros.
 *
 * Activation backward (dact = 1; page 6, quack/gemm_dact_sm90.py, GemmDActSm90): the product
 * is the incoming gradient dout = alpha * A x B, C holds the saved pre-activation x (its
 * own type), and the outputs are D = dout * act'(x) (required) and PostAct = act(x)
 * (optional); with act NONE, D = dout and PostAct = x. act'(x): relu [x > 0], relu_sq
 * 2 max(x, 0), gelu_tanh the derivative of the tanh form above, silu s (1 + x (1 - s)) with
 * s = 1 / (1 + exp(-x)) (silu is an addition: the page maps relu, relu_sq and gelu only).
 * beta has no role: it must be 1 and gemm_run takes no beta_dev. C is required.
 *
 * Alignment (page 5, constraints of the dense GEMM docstring): the contiguous dimension
 * of every operand must hold a whole number of 16-byte chunks (a multiple of 8 elements
 * for 16-bit types, 16 for fp8, 4 for f32), and every leading-dimension and batch stride
 * must be a multiple of 16 bytes. Pointers must be 16-byte aligned (checked by gemm_run).
 *
 * Tuning fields (0 = library default):
 *   tile_m, tile_n  output tile per workgroup; supported pairs: 256x256, 128x128.
 *   group_m         raster group size G of the tile map, power of two in [1, 16], default 8.
 *   max_ctas        cap on the persistent grid size.
 *   xcd_remap       -1: off, 0: default (on), 1: on. See gemm_plan_grid.
 *   tail_split      -1: off, 0: default (on), 1: on. With 256x256 tiles, when the last
 *                   round of the persistent schedule is partial and at most half full
 *                   (T > P, 0 < T mod P <= P/2), gemm_run stops the persistent launch before
 *                   those T mod P tiles and enqueues a second launch that computes each of
 *                   them as four 128x128 quarters (quarters wholly outside the output are
 *                   skipped). Varlen plans decide on the device, where T is known; their
 *                   second launch exits at once when there is no such tail. Same results.
 *                   gemm_run_logged never splits.
 *   raster_order    0: default (along N for dense L == 1 with C, else along M), 1: along M,
 *                   2: along N (dense only). The grouped
 *                   raster takes groups of group_m blocks along M, M fastest inside a group
 *                   (page 5's swizzle); along N the roles of M and N are exchanged (page 6,
 *                   quack/gemm_config.py, keeps the raster order and the swizzle size in
 *                   its tuning space).                                                   */
typedef struct {
  int32_t M, N, K, L;
  int32_t a, b, c, d, post;                              /* gemm_dtype */
  int32_t a_major, b_major, c_major, d_major, post_major; /* gemm_major */
  int64_t lda, ldb, ldc, ldd, ldp;
  int64_t sa, sb, sc, sd, sp;
  float alpha, beta;
  int32_t act;      /* gemm_act */
  int32_t varlen_m; /* 0 or 1 */
  int32_t tile_m, tile_n;
  int32_t group_m;
  int32_t max_ctas;
  int32_t xcd_remap;
  int32_t tail_split;
  int32_t raster_order;
  int32_t dact;     /* 1: activation-backward epilogue (see above) */
  int32_t varlen_k; /* 0 or 1: grouped K (see above) */
  int32_t gather_a; /* 0 or 1: A rows gathered through a_idx (varlen-M) */
  int64_t gather_rows; /* gather_a: rows (varlen-M) or columns (varlen-K) of A that a_idx may name */
} gemm_desc;

/* Run-time arguments of gemm_run_ex (all device pointers, owned by the caller; NULL where
 * the plan does not use them). */
typedef struct {
  const void* A;
  const void* B;
  const void* C;
  void* D;
  void* PostAct;
  const float* alpha_dev;        /* optional device fp32, replaces desc.alpha            */
  const float* beta_dev;         /* optional device fp32, replaces desc.beta             */
  const int32_t* cu_seqlens_m;   /* varlen-M plans: int32[L+1]                           */
  const int32_t* cu_seqlens_k;   /* varlen-K plans: int32[L+1]                           */
  const int32_t* a_idx;          /* gather_a plans: int32[M] (varlen-M) or int32[K] (varlen-K) */
  int32_t* tile_counters;        /* NULL: static schedule; else as in gemm_run_dynamic  */
} gemm_args;

typedef struct gemm_plan gemm_plan;

/* Validate `desc` and build a plan (host memory only, no HIP call). On success *out owns a
 * new plan to release with gemm_destroy; on failure *out is set to NULL and the status
 * says why: INVALID_ARG (NULL desc/out, a negative size, strides smaller than the
 * extents they skip, unknown enum value), UNSUPPORTED (dtype or major combination the
 * pages exclude or this library does not build, tile pair not offered, tile count >= 2^31,
 * a tile's operand byte offsets >= 2^31, a stride beyond 2^48 elements, an operand whose
 * addressed span exceeds 2^62 bytes), ALIGNMENT (contiguous extent or stride not a
 * multiple of 16 bytes), NO_MEMORY. Zero sizes are valid: M, N or L == 0 is an empty
 * problem, and K == 0 makes the product zero (page 5, GemmSm90.mma sets the accumulator
 * to zero when there is no k-tile). */
gemm_status gemm_create(const gemm_desc* desc, gemm_plan** out);

/* Enqueue the GEMM on `stream`. A, B, D / PostAct (those the plan declares present) must
 * be non-NULL device pointers (A and B may be NULL when K == 0: they are not read);
 * C must be non-NULL iff the plan has a C type. A plan with no output element (M, N or L
 * zero) returns GEMM_OK without launching anything.
 * alpha_dev / beta_dev: optional device pointers to one fp32 each; when non-NULL they
 * replace desc.alpha / desc.beta and are read by the kernel at run time (page 5,
 * gemm_sm90 passes a tensor alpha/beta to the kernel as a pointer).
 * cu_seqlens_m: device int32[L+1], required iff varlen_m; precondition: cu[0] == 0,
 * non-decreasing, cu[L] == M (checked by the kernel: an array that breaks it runs no tile and
 * writes nothing; gemm_check_cu_seqlens reports it). Returns INVALID_ARG for a missing pointer,
 * ALIGNMENT for a pointer that is not 16-byte aligned, HIP if the launch fails. */
gemm_status gemm_run(const gemm_plan* plan, const void* A, const void* B, const void* C, void* D,
                     void* PostAct, const float* alpha_dev, const float* beta_dev,
                     const int32_t* cu_seqlens_m, void* stream);

/* As gemm_run, and additionally record the persistent schedule: for workgroup b and its
 * i-th tile (i < max_iters) the kernel writes int32 {m_blk, n_blk, l, t} at
 * tile_log[(b * max_iters + i) * 4]; entries it does not reach are left untouched
 * (callers pre-fill them). For varlen plans l is the group and m_blk the block inside it.
 * tile_log is a device buffer of at least P * max_iters * 4 int32 (P from gemm_plan_grid
 * with the device's CU count). Used to check the tile map bit for bit. */
gemm_status gemm_run_logged(const gemm_plan* plan, const void* A, const void* B, const void* C,
                            void* D, void* PostAct, const float* alpha_dev, const float* beta_dev,
                            const int32_t* cu_seqlens_m, int32_t* tile_log, int32_t max_iters,
                            void* stream);

/* The general entry point: every plan, including varlen-K and gathered-A plans, which
 * gemm_run, gemm_run_logged and gemm_run_dynamic reject with INVALID_ARG. The fields of
 * `args` mean what the same-named arguments of gemm_run mean; cu_seqlens_k and a_idx are
 * required iff the plan has varlen_k / gather_a, and a device array the plan does not use
 * must be NULL (INVALID_ARG otherwise). tile_counters non-NULL selects the dynamic schedule
 * exactly as gemm_run_dynamic (its counters must be zero before the first call and are left
 * zero). Asynchronous on `stream`; ALIGNMENT for operand pointers not 16-byte aligned or
 * index arrays not 4-byte aligned, HIP if a launch fails. */
gemm_status gemm_run_ex(const gemm_plan* plan, const gemm_args* args, void* stream);

/* As gemm_run (or, with tile_log non-NULL, gemm_run_logged), with the dynamic persistent
 * schedule: the page 5 GEMM's optional tile_count_semaphore, a device counter from which
 * persistent workgroups claim their next tile. Here the grid keeps the static schedule's
 * queues (eight, one per group of P/8 workgroups that the XCD remap keeps on one XCD, or
 * one queue when the remap is off or P is not a multiple of 8): each workgroup starts on
 * its static first tile and then claims the next unclaimed tile of its own queue, so a
 * slow or late compute unit takes fewer tiles while each queue keeps the tiles (and L2
 * reuse) of the static schedule. Results equal gemm_run's bit for bit; only the tile ->
 * workgroup assignment changes.
 * tile_counters: device int32[8], all zero before the first call. Every call returns them
 * to zero before it completes, so calls in sequence on a stream need no reset; calls that
 * may run at the same time need separate counters. A call that does not complete (a
 * faulted context) leaves them undefined. The split tail (tail_split) still applies and
 * its quarter tiles run statically. Returns INVALID_ARG for NULL tile_counters, ALIGNMENT
 * if they are not 4-byte aligned, otherwise as gemm_run / gemm_run_logged. */
gemm_status gemm_run_dynamic(const gemm_plan* plan, const void* A, const void* B, const void* C,
                             void* D, void* PostAct, const float* alpha_dev, const float* beta_dev,
                             const int32_t* cu_seqlens_m, int32_t* tile_counters, int32_t* tile_log,
                             int32_t max_iters, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): gemm_run_dynamic without the
 * tile_counters argument (and without a tile log). The queue counters live in a 256-byte
 * array of the library's own device memory, one per GPU, held until the process ends; the
 * dynamic schedule uses 8 int32 of it at any problem size, so no size is rejected for
 * scratch. Each call first zeroes those counters with a one-workgroup fill kernel on
 * `stream`, then launches exactly as gemm_run_dynamic; results equal gemm_run's bit for bit.
 * No hipMalloc, hipFree or other allocating call is made. Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (other streams, other threads) race on it
 * and must be serialised by the caller. The first call on a device looks the array's
 * address up (hipGetSymbolAddress) with that device current. Returns as gemm_run_dynamic
 * (INVALID_ARG for varlen-K and gathered-A plans), UNSUPPORTED on a device index >= 64. */
gemm_status gemm_run_dynamic_noalloc(const gemm_plan* plan, const void* A, const void* B, const void* C,
                                     void* D, void* PostAct, const float* alpha_dev,
                                     const float* beta_dev, const int32_t* cu_seqlens_m, void* stream);

/* Debug check of a cu_seqlens array (page 5: cu_seqlens_m / cu_seqlens_k delimit the groups
 * of the varlen modes; their well-formedness is the caller's precondition there). Enqueues one
 * small kernel that writes int32 *status_dev = 0 when cu[0] == 0, cu never decreases and
 * cu[L] == total (exact_end = 1, varlen-M: total = M) or cu[L] <= total (exact_end = 0,
 * varlen-K: total = K); otherwise 1 + the index of the first entry that breaks a rule.
 * cu_seqlens: device int32[L+1]; status_dev: device int32, caller-owned. Asynchronous on
 * `stream`: read the status after synchronising. The varlen-M kernels make the same check on
 * every launch and, for an array that fails it, run no tile and write nothing. INVALID_ARG for
 * a NULL pointer, L < 0, total < 0 or exact_end not 0/1; ALIGNMENT for pointers not 4-byte
 * aligned; HIP if the launch fails. */
gemm_status gemm_check_cu_seqlens(const int32_t* cu_seqlens, int32_t L, int32_t total, int32_t exact_end,
                                  int32_t* status_dev, void* stream);

/* Release a plan (NULL is accepted). */
gemm_status gemm_destroy(gemm_plan* plan);

/* The schedule a plan uses on a device with `num_cus` compute units:
 *   tile_m, tile_n: the output tile; group_m: raster group G; xcd_remap: 0/1;
 *   tiles: T = ceil(M/tile_m) * ceil(N/tile_n) * L for dense plans, -1 for varlen plans
 *          (their T depends on cu_seqlens_m, known only on the device);
 *   grid:  P = min(T, num_cus * workgroups_per_cu) (varlen: num_cus * workgroups_per_cu).
 * Workgroup b handles linear tiles t = b' + i * P while t < T, where b' = b, or with the
 * XCD remap and P % 8 == 0, b' = (b % 8) * (P / 8) + b / 8. Tile t maps to (m_blk, n_blk,
 * l) by the grouped raster of page 5 (the removed 0.1.10 "CTA swizzle" in GemmSm90.kernel):
 * l = t / (tm * tn); inside a batch, groups of G M-blocks with M fastest, then N, then the
 * next group; the tm % G leftover M-blocks form a last group of that width (raster along
 * M; along N, see raster_order and gemm_plan_raster, M and N swap roles). Varlen plans
 * concatenate the groups' tiles in group order (ceil(M_g / tile_m) * tn tiles each) and use
 * the same raster inside a group. All device divisions use FastDivmod (page 6,
 * quack/fast_math.py). Any output pointer may be NULL. */
gemm_status gemm_plan_grid(const gemm_plan* plan, int32_t num_cus, int32_t* tile_m,
                           int32_t* tile_n, int32_t* group_m, int32_t* xcd_remap,
                           int64_t* tiles, int32_t* grid);

/* The raster order the plan's tile map uses: *along_n = 1 along N, 0 along M (see
 * raster_order in gemm_desc). INVALID_ARG for a NULL argument. */
gemm_status gemm_plan_raster(const gemm_plan* plan, int32_t* along_n);

/* FastDivmod constants the library computes for divisor d (1 <= d < 2^31), as page 6,
 * quack/fast_math.py, FastDivmod.create: p = 31 + ceil(log2 d),
 * multiplier = ceil(2^p / d) (as uint32), shift = p - 32. */
gemm_status gemm_fastdivmod_params(uint32_t d, uint32_t* multiplier, uint32_t* shift);

/* Device self-check of the library's FastDivmod: for every d in [d_lo, d_hi] and
 * n in [0, n_count) the kernel compares the library's quotient/remainder with the device's
 * integer '/' and '%', and atomically adds the number of mismatching pairs to *bad_dev
 * (device uint64, not cleared by the call). Requires 1 <= d_lo <= d_hi < 2^31 and
 * n_count <= 2^31. */
gemm_status gemm_fastdivmod_check(uint32_t d_lo, uint32_t d_hi, uint32_t n_count,
                                  unsigned long long* bad_dev, void* stream);

/* Static description of a status code (never NULL). */
const char* gemm_status_string(gemm_status status);

/* Message about the last failure on the calling thread ("" if none). */
const char* gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_MI355X_H */
