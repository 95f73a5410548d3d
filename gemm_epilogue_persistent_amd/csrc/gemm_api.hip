// gemm_run / gemm_run_ex / gemm_run_logged / gemm_run_dynamic and the device FastDivmod self-check (C ABI).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/gemm_mi355x.h"
#include "launch.hpp"

namespace gep {
gemm_status fail(gemm_status st, const char* fmt, ...);
void clear_error();
int32_t grid_size(const gemm_plan* p, int32_t num_cus);

// Compute units of the current device, cached per device id.
static gemm_status current_cus(int32_t* cus) {
  static std::atomic<int32_t> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) {
    int32_t v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) { *cus = v; return GEMM_OK; }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || n <= 0) return fail(GEMM_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return GEMM_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int OP>
static hipError_t launch_op(const KernelKey& key, const KParams& k, hipStream_t s) {
  if (key.dact) {
    if (key.varlen == 0) return launch_family<OP, true, 0>(key, k, s);
    if (key.varlen == 1) return launch_family<OP, true, 1>(key, k, s);
    return hipErrorInvalidValue;
  }
  if (key.varlen == 0) return launch_family<OP, false, 0>(key, k, s);
  if (key.varlen == 1) return launch_family<OP, false, 1>(key, k, s);
  return launch_family<OP, false, 2>(key, k, s);
}

static hipError_t launch_key(const KernelKey& key, const KParams& k, hipStream_t s) {
  switch (key.op) {
    case OP_F16: return launch_op<OP_F16>(key, k, s);
    case OP_BF16: return launch_op<OP_BF16>(key, k, s);
    default: return launch_op<OP_FP8>(key, k, s);
  }
}

// cu: cu_seqlens_m (varlen-M plans) or cu_seqlens_k (varlen-K plans); a_idx: gathered A rows.
static gemm_status run_impl(const gemm_plan* plan, const void* A, const void* B, const void* C, void* D,
                            void* Post, const float* alpha_dev, const float* beta_dev, const int32_t* cu,
                            const int32_t* a_idx, int32_t* counters, int32_t* tile_log, int32_t max_iters,
                            void* stream) {
  if (!plan) return fail(GEMM_ERR_INVALID_ARG, "gemm_run: NULL plan");
  // nothing to compute: no tiles (dense) or no rows / columns / groups (varlen)
  const bool empty = plan->varlen ? (plan->base.M == 0 || plan->base.N == 0 || plan->L == 0) : plan->T == 0;
  if (empty) { clear_error(); return GEMM_OK; }
  if (plan->base.K > 0 && (!A || !B)) return fail(GEMM_ERR_INVALID_ARG, "gemm_run: A and B are required");
  if (plan->has_c != (C != nullptr)) return fail(GEMM_ERR_INVALID_ARG, "gemm_run: C must be given iff the plan has a C type");
  if (plan->has_d != (D != nullptr)) return fail(GEMM_ERR_INVALID_ARG, "gemm_run: D must be given iff the plan has a D type");
  if (plan->has_p != (Post != nullptr)) return fail(GEMM_ERR_INVALID_ARG, "gemm_run: PostAct must be given iff the plan has a PostAct type");
  if (plan->varlen && !cu) return fail(GEMM_ERR_INVALID_ARG, "gemm_run: cu_seqlens_m is required for a varlen plan");
  if (plan->varlen_k && !cu) return fail(GEMM_ERR_INVALID_ARG, "gemm_run_ex: cu_seqlens_k is required for a varlen-K plan");
  if (plan->gather && !a_idx) return fail(GEMM_ERR_INVALID_ARG, "gemm_run_ex: a_idx is required for a gathered-A plan");
  if (((uintptr_t)cu & 3u) != 0 || ((uintptr_t)a_idx & 3u) != 0)
    return fail(GEMM_ERR_ALIGNMENT, "gemm_run: cu_seqlens / a_idx not 4-byte aligned");
  if (plan->key.dact && beta_dev) return fail(GEMM_ERR_INVALID_ARG, "gemm_run: a dact plan takes no beta");
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(D) || !aligned16(Post))
    return fail(GEMM_ERR_ALIGNMENT, "gemm_run: operand pointers must be 16-byte aligned");
  if (tile_log && max_iters <= 0) return fail(GEMM_ERR_INVALID_ARG, "gemm_run_logged: max_iters <= 0");
  if (((uintptr_t)counters & 3u) != 0) return fail(GEMM_ERR_ALIGNMENT, "gemm_run_dynamic: tile_counters not 4-byte aligned");

  KParams k = plan->base;
  k.A = plan->swapped ? B : A;
  k.B = plan->swapped ? A : B;
  k.C = C;
  k.D = D;
  k.Post = Post;
  k.alpha_ptr = alpha_dev;
  k.beta_ptr = beta_dev;
  k.cu_seqlens = cu;
  k.a_idx = a_idx;
  k.tile_counters = counters;
  k.tile_log = tile_log;
  k.tile_log_iters = tile_log ? max_iters : 0;
  int32_t cus = 0;
  gemm_status st = current_cus(&cus);
  if (st != GEMM_OK) return st;
  k.P = grid_size(plan, cus);

  // Split tail (see tail_split in the header): grid of the quarter-tile launch, 0 for none.
  int32_t p_tail = 0;
  if (plan->tail_split && !tile_log) {
    int64_t cap = 2 * (int64_t)cus;  // 128x128 kernels run two workgroups per CU
    if (plan->max_ctas > 0 && plan->max_ctas < cap) cap = plan->max_ctas;
    if (plan->varlen) {
      // the device knows T; launch only if T can exceed one round at all
      const int64_t t_max = ((int64_t)plan->base.M / plan->tile_m + 1 + plan->L) * plan->base.tn;
      if (t_max > k.P) p_tail = (int32_t)cap;
    } else {
      const int64_t rem = plan->T % k.P;
      if (plan->T > k.P && rem > 0 && 2 * rem <= k.P) p_tail = (int32_t)(4 * rem < cap ? 4 * rem : cap);
    }
  }
  if (p_tail > 0) {
    k.tail = 1;
    k.P_big = k.P;
  }

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_key(plan->key, k, s);
  if (e == hipSuccess && p_tail > 0) {
    KParams kt = k;
    kt.tail = 2;
    kt.tile_counters = nullptr;  // the quarter tiles run the static schedule
    kt.P = p_tail;
    KernelKey key = plan->key;
    key.tile = 1;
    e = launch_key(key, kt, s);
  }
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  clear_error();
  return GEMM_OK;
}

// For every divisor d in [d_lo, d_hi] (blocks, grid-stride) and dividend n < n_count
// (threads), compare FastDivmod with the device's integer '/' and '%'.
__global__ __launch_bounds__(256) void fastdivmod_check_kernel(uint32_t d_lo, uint32_t d_hi, uint32_t n_count,
                                                               unsigned long long* bad) {
  unsigned long long local = 0;
  for (uint64_t d = (uint64_t)d_lo + blockIdx.x; d <= d_hi; d += gridDim.x) {
    const FastDiv f = make_fastdiv((uint32_t)d);
    for (uint64_t n = threadIdx.x; n < n_count; n += blockDim.x) {
      uint32_t q, r;
      fd_divmod(f, (uint32_t)n, q, r);
      local += (q != (uint32_t)n / (uint32_t)d) | (r != (uint32_t)n % (uint32_t)d);
    }
  }
  if (local) atomicAdd(bad, local);
}

// ---- the dynamic schedule's queue counters for callers that cannot allocate
// (gemm_run_dynamic_noalloc): one array per device, held for the life of the process. Only
// its first kQueueCounters entries are used (one counter per XCD queue); the rest is slack.
constexpr int kQueueCounters = 8;
constexpr int kScratchInts = 64;  // 256 bytes
static_assert(kQueueCounters <= kScratchInts, "the queue counters must fit the scratch array");
static __device__ __align__(256) int32_t scratch[kScratchInts];

// Device address of `scratch` on each device, looked up once with that device current.
// (In host code the array's name is only a host-side stand-in, never a device address.)
constexpr int kMaxDevices = 64;
static std::atomic<int32_t*> g_scratch_ptr[kMaxDevices];

static gemm_status scratch_of_current_device(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GEMM_ERR_UNSUPPORTED, "gemm_run_dynamic_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !addr)
      return fail(GEMM_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    p = (int32_t*)addr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // (a racing lookup stores the same value)
  }
  *out = p;
  return GEMM_OK;
}

// Zero the counters with a vector store (a fill kernel rather than hipMemsetAsync, so that
// the call can sit in a captured graph).
__global__ __launch_bounds__(64) void zero_counters_kernel(int32_t* c, int n) {
  if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}

// cu_seqlens check: one workgroup; *status = 0 when cu[0] == 0, cu never decreases and cu[L]
// is total (exact_end) or at most total; else 1 + the index of the first offending entry.
__global__ __launch_bounds__(256) void check_cu_seqlens_kernel(const int32_t* cu, int32_t L, int32_t total,
                                                               int32_t exact_end, int32_t* status) {
  __shared__ int32_t first;
  if (threadIdx.x == 0) first = 0x7FFFFFFF;
  __syncthreads();
  for (int32_t i = threadIdx.x; i <= L; i += blockDim.x) {
    const int32_t v = cu[i];
    const bool ok = (i == 0 ? v == 0 : v >= cu[i - 1]) && (i < L || (exact_end ? v == total : v <= total));
    if (!ok) atomicMin(&first, i);
  }
  __syncthreads();
  if (threadIdx.x == 0) *status = first == 0x7FFFFFFF ? 0 : first + 1;
}

// The entry points of the C ABI that predate varlen-K and gathered A take no place for their
// device arrays: such plans must go through gemm_run_ex.
static gemm_status legacy_ok(const gemm_plan* plan, const char* fn) {
  if (plan && (plan->varlen_k || plan->gather))
    return fail(GEMM_ERR_INVALID_ARG, "%s: varlen-K and gathered-A plans run through gemm_run_ex", fn);
  return GEMM_OK;
}

}  // namespace gep

extern "C" {

gemm_status gemm_run(const gemm_plan* plan, const void* A, const void* B, const void* C, void* D, void* PostAct,
                     const float* alpha_dev, const float* beta_dev, const int32_t* cu_seqlens_m, void* stream) {
  if (gep::legacy_ok(plan, "gemm_run") != GEMM_OK) return GEMM_ERR_INVALID_ARG;
  return gep::run_impl(plan, A, B, C, D, PostAct, alpha_dev, beta_dev, cu_seqlens_m, nullptr, nullptr, nullptr, 0,
                       stream);
}

gemm_status gemm_run_ex(const gemm_plan* plan, const gemm_args* a, void* stream) {
  if (!a) return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_run_ex: NULL args");
  if (plan && !plan->varlen_k && a->cu_seqlens_k)
    return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_run_ex: cu_seqlens_k given to a plan without varlen_k");
  if (plan && !plan->varlen && a->cu_seqlens_m)
    return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_run_ex: cu_seqlens_m given to a plan without varlen_m");
  if (plan && !plan->gather && a->a_idx)
    return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_run_ex: a_idx given to a plan without gather_a");
  const int32_t* cu = (plan && plan->varlen_k) ? a->cu_seqlens_k : a->cu_seqlens_m;
  return gep::run_impl(plan, a->A, a->B, a->C, a->D, a->PostAct, a->alpha_dev, a->beta_dev, cu, a->a_idx,
                       a->tile_counters, nullptr, 0, stream);
}

gemm_status gemm_run_dynamic(const gemm_plan* plan, const void* A, const void* B, const void* C, void* D,
                             void* PostAct, const float* alpha_dev, const float* beta_dev,
                             const int32_t* cu_seqlens_m, int32_t* tile_counters, int32_t* tile_log,
                             int32_t max_iters, void* stream) {
  if (!tile_counters) return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_run_dynamic: NULL tile_counters");
  if (gep::legacy_ok(plan, "gemm_run_dynamic") != GEMM_OK) return GEMM_ERR_INVALID_ARG;
  return gep::run_impl(plan, A, B, C, D, PostAct, alpha_dev, beta_dev, cu_seqlens_m, nullptr, tile_counters,
                       tile_log, max_iters, stream);
}

gemm_status gemm_run_dynamic_noalloc(const gemm_plan* plan, const void* A, const void* B, const void* C, void* D,
                                     void* PostAct, const float* alpha_dev, const float* beta_dev,
                                     const int32_t* cu_seqlens_m, void* stream) {
  if (gep::legacy_ok(plan, "gemm_run_dynamic_noalloc") != GEMM_OK) return GEMM_ERR_INVALID_ARG;
  if (!plan) return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_run_dynamic_noalloc: NULL plan");
  int32_t* ctr = nullptr;
  gemm_status st = gep::scratch_of_current_device(&ctr);
  if (st != GEMM_OK) return st;
  // the counters start every call at zero (each call also leaves them at zero)
  hipLaunchKernelGGL(gep::zero_counters_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ctr,
                     gep::kQueueCounters);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return gep::fail(GEMM_ERR_HIP, "counter reset launch: %s", hipGetErrorString(e));
  return gep::run_impl(plan, A, B, C, D, PostAct, alpha_dev, beta_dev, cu_seqlens_m, nullptr, ctr, nullptr, 0,
                       stream);
}

gemm_status gemm_check_cu_seqlens(const int32_t* cu_seqlens, int32_t L, int32_t total, int32_t exact_end,
                                  int32_t* status_dev, void* stream) {
  if (!cu_seqlens || !status_dev || L < 0 || total < 0 || (exact_end != 0 && exact_end != 1))
    return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_check_cu_seqlens: NULL array or status, L < 0, total < 0 or bad mode");
  if (((uintptr_t)cu_seqlens & 3u) != 0 || ((uintptr_t)status_dev & 3u) != 0)
    return gep::fail(GEMM_ERR_ALIGNMENT, "gemm_check_cu_seqlens: arrays must be 4-byte aligned");
  hipLaunchKernelGGL(gep::check_cu_seqlens_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, cu_seqlens, L, total,
                     exact_end, status_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return gep::fail(GEMM_ERR_HIP, "cu_seqlens check launch: %s", hipGetErrorString(e));
  gep::clear_error();
  return GEMM_OK;
}

gemm_status gemm_run_logged(const gemm_plan* plan, const void* A, const void* B, const void* C, void* D,
                            void* PostAct, const float* alpha_dev, const float* beta_dev,
                            const int32_t* cu_seqlens_m, int32_t* tile_log, int32_t max_iters, void* stream) {
  if (!tile_log) return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_run_logged: NULL tile_log");
  if (gep::legacy_ok(plan, "gemm_run_logged") != GEMM_OK) return GEMM_ERR_INVALID_ARG;
  return gep::run_impl(plan, A, B, C, D, PostAct, alpha_dev, beta_dev, cu_seqlens_m, nullptr, nullptr, tile_log,
                       max_iters, stream);
}

gemm_status gemm_fastdivmod_check(uint32_t d_lo, uint32_t d_hi, uint32_t n_count, unsigned long long* bad_dev,
                                  void* stream) {
  if (!bad_dev || d_lo < 1 || d_lo > d_hi || d_hi > 0x7FFFFFFFu || n_count > 0x80000000u)
    return gep::fail(GEMM_ERR_INVALID_ARG, "gemm_fastdivmod_check: bad range or NULL counter");
  uint64_t span = (uint64_t)d_hi - d_lo + 1;
  unsigned blocks = (unsigned)(span < 65536 ? span : 65536);
  hipLaunchKernelGGL(gep::fastdivmod_check_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, d_lo, d_hi,
                     n_count, bad_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return gep::fail(GEMM_ERR_HIP, "fastdivmod check launch: %s", hipGetErrorString(e));
  gep::clear_error();
  return GEMM_OK;
}

}  // extern "C"
