// Kernel arguments and the host-side plan, shared by plan.cpp and the HIP kernels.
#pragma once
#include <stdint.h>

#include "fastdivmod.hpp"

namespace gep {

// Element types, numbered as gemm_dtype in the public header.
enum : int32_t { DT_NONE = 0, DT_F16 = 1, DT_BF16 = 2, DT_F32 = 3, DT_E4M3 = 4, DT_E5M2 = 5 };
enum : int32_t { ACT_NONE = 0, ACT_RELU = 1, ACT_RELU_SQ = 2, ACT_GELU_TANH = 3, ACT_SILU = 4 };

constexpr int kMaxGroupLog2 = 4;           // raster group G <= 16
constexpr int kMaxVarlenGroups = 1024;     // groups held in LDS by the varlen kernels
constexpr uint32_t kOOB = 0x80000000u;     // buffer offset that reads as zero

// Everything a kernel launch needs; passed by value as the kernel argument.
struct KParams {
  const void* A;
  const void* B;
  const void* C;
  void* D;
  void* Post;  // PostAct
  int64_t lda, ldb, ldc, ldd, ldp;  // elements
  int64_t sa, sb, sc, sd, sp;       // elements
  int64_t a_bytes, b_bytes;         // addressable extent of A and B from their base pointers
  int32_t M, N, K, L;
  float alpha, beta;
  const float* alpha_ptr;
  const float* beta_ptr;
  const int32_t* cu_seqlens;  // cu_seqlens_m (varlen-M) or cu_seqlens_k (varlen-K)
  const int32_t* a_idx;       // gathered A rows (varlen-M), or NULL
  int32_t a_rows;             // rows of A that a_idx may name
  int32_t c_dt, d_dt, p_dt;
  int32_t c_trans;  // C's contiguous dimension is the kernel's M (the outputs' is N)
  int32_t act;
  // persistent schedule
  int32_t tm, tn;   // M- and N-blocks (tm unused for varlen)
  int32_t T;        // tiles (dense); varlen computes it on the device
  int32_t P;        // workgroups in the grid
  int32_t log2G;    // raster group size G = 1 << log2G
  int32_t xcd_remap;
  int32_t tail;     // 0: the whole map; 1: all but a split tail; 2: the split tail's quarter tiles
  int32_t P_big;    // tail != 0: grid of the first launch (the map's round size)
  FastDiv fd_mn;    // tm * tn
  FastDiv fd_Gtn;   // G * tn
  FastDiv fd_Gtm;   // G * tm (raster along N)
  int32_t raster_n; // 1: grouped raster along N (dense only)
  FastDiv fd_tail[1 << kMaxGroupLog2];  // index w: divisor w (1 <= w < G); [0] unused
  int32_t* tile_counters;  // dynamic schedule: 8 queue counters (zero at launch), or NULL
  int32_t* tile_log;
  int32_t tile_log_iters;
};

// Kernel families the plan can pick.
enum KernelOp : int32_t { OP_F16 = 0, OP_BF16 = 1, OP_FP8 = 2 };

struct KernelKey {
  int32_t op;        // KernelOp
  int32_t fmt_a;     // fp8 only: 0 = e4m3, 1 = e5m2
  int32_t fmt_b;
  int32_t a_kmajor;  // 1: K contiguous
  int32_t b_kmajor;
  int32_t tile;      // 0: 256x256, 1: 128x128
  int32_t varlen;    // 0 dense, 1 varlen-M, 2 varlen-K
  int32_t dact;      // activation-backward epilogue
  int32_t gather;    // A rows gathered through a_idx (varlen-M)
};

}  // namespace gep

struct gemm_plan {
  // problem as the kernel sees it (after an optional A<->B swap for M-major outputs)
  gep::KParams base;  // pointers left NULL; filled per run
  gep::KernelKey key;
  int32_t tile_m, tile_n;
  int32_t wg_per_cu;
  int32_t swapped;    // 1: the kernel computes the transposed problem
  int32_t has_c, has_d, has_p;
  int64_t T;          // -1 for varlen
  int32_t max_ctas;
  int32_t varlen;     // varlen-M: T known only on the device
  int32_t varlen_k;
  int32_t gather;
  int32_t L;          // groups (varlen) or batches
  int32_t tail_split; // 1: gemm_run may split the last partial round into quarter tiles
};
