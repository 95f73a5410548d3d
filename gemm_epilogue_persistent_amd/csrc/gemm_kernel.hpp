// Persistent batched GEMM with fused epilogue for gfx950 (CDNA4):
//   D = alpha * A x B + beta * C,  PostAct = act(D before rounding).
//
// Operation: quack-kernels 0.1.10 -> 0.2.0 diff, page 5, quack/dense_gemm_sm90.py (GemmSm90:
// persistent tile loop, k-tile mainloop, epi_visit_acc_subtile) and page 6,
// quack/gemm_act_sm90.py (GemmActSm90: PostAct = act(fp32 pre-activation) next to D).
// The design is this file's own:
//   * 256 threads = 4 wave64s in a 2x2 grid; each wave owns a (BM/2) x (BN/2) block of the
//     output tile, computed with v_mfma_f32_32x32x16_{f16,bf16} or, for fp8,
//     v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales; per-operand e4m3/e5m2 format fields).
//   * A and B k-tiles of 128 bytes per row travel global -> LDS with buffer_load ... lds
//     (no VGPR staging), STAGES deep. Out-of-range rows / k-chunks use an offset past the
//     buffer's num_records, which the hardware reads as zero (tails in M, N and K).
//   * K-major tiles are stored [row][8 x 16-byte chunks] with the chunk index XOR-swizzled
//     by the row, so the 32-row MFMA fragment reads (ds_read_b128) hit distinct banks.
//     M/N-major (16-bit) tiles are stored [k][row] and read with ds_read_b64_tr_b16, which
//     transposes 16x4 blocks across each 16-lane group into K-contiguous fragments.
//   * Persistent grid: workgroup b takes tiles t = b' + i*P; t -> (m_blk, n_blk, l) by the
//     grouped raster with FastDivmod (page 6, quack/fast_math.py); b' optionally remaps b so
//     that the workgroups of one XCD (dispatched round-robin) take consecutive tile ids.
//   * Epilogue straight from the accumulators: the MFMA is issued as (B fragment,
//     A fragment) so each lane holds 4 consecutive N values of one row, which it scales,
//     adds beta*C to, activates and stores as 8- or 16-byte vectors.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.hpp"

namespace gep {

#define GEP_LDS __attribute__((address_space(3)))

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------
// MFMA flavours. Frag = the per-lane operand registers of one 32-row fragment.
// Lane l holds row (l % 32) and, inside the MFMA's K slice, elements [8*(l/32), +8) for
// 16-bit types or bytes [32*(l/32), +32) for fp8; A and B use the same K assignment.
// ------------------------------------------------------------------------------------
template <int OP, int FA, int FB>
struct Mfma;

template <int FA, int FB>
struct Mfma<OP_F16, FA, FB> {
  static constexpr int kES = 2;       // bytes per element
  static constexpr int kKStep = 16;   // K per instruction
  using Frag = i32x4;
  static __device__ __forceinline__ f32x16 mma(Frag b, Frag a, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a),
                                                  c, 0, 0, 0);
  }
};

template <int FA, int FB>
struct Mfma<OP_BF16, FA, FB> {
  static constexpr int kES = 2;
  static constexpr int kKStep = 16;
  using Frag = i32x4;
  static __device__ __forceinline__ f32x16 mma(Frag b, Frag a, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                   c, 0, 0, 0);
  }
};

template <int FA, int FB>
struct Mfma<OP_FP8, FA, FB> {
  static constexpr int kES = 1;
  static constexpr int kKStep = 64;
  using Frag = i32x8;
  // cbsz / blgp select the format of the instruction's first / second source
  // (0 = e4m3, 1 = e5m2). The kernel passes the B fragment first (see the epilogue
  // layout note), so B's format goes in cbsz and A's in blgp.
  // Scales of 127 are 2^0 in the E8M0 scale encoding (no scaling).
  static __device__ __forceinline__ f32x16 mma(Frag b, Frag a, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, 0, 127, 0, 127);
  }
};

// ------------------------------------------------------------------------------------
// LDS tile layouts
// ------------------------------------------------------------------------------------
constexpr int kRowBytes = 128;  // one k-tile row of a K-major tile

// K-major: chunk (16 bytes) c of row r lives at chunk c ^ swz(r). Rows r..r+15 of one
// fragment read then cover all banks for both 8-lane (128 B) and 16-lane (256 B) phases.
__device__ __forceinline__ int kswz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }
// M/N-major: chunk c of k-row k lives at chunk c ^ mswz(k); the 4 k-rows that one 16-lane
// transpose group reads land in 4 disjoint 64-byte bank ranges.
__device__ __forceinline__ int mswz(int k) { return (k & 3) << 2; }

// Buffer resource over [base, base + bytes); reads at offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Loader of one operand's k-tile: ROWS rows (M or N) by 128 bytes of K.
// Each wave issues kInstr instructions of 64 lanes x 16 bytes (1 KB of LDS each).
template <int ROWS, bool KMAJ, int ES>
struct TileLoader {
  static constexpr int kTileBytes = ROWS * kRowBytes;
  static constexpr int kInstr = kTileBytes / 1024 / 4;
  static constexpr int kCPR = ROWS * ES / 16;          // MN-major: chunks per k-row
  static constexpr int kKPI = KMAJ ? 1 : 1024 / (ROWS * ES);  // MN-major: k-rows per instruction
  uint32_t off[kInstr];
  int32_t kidx[kInstr];   // K-major: element k of the chunk; MN-major: the k-row
  bool ok[kInstr];        // row (K-major) / column chunk (MN-major) inside the operand

  // rows_valid: rows of this tile that exist (K-major) or MN elements that exist (MN-major).
  __device__ __forceinline__ void init(int wave, int lane, int rows_valid, int64_t ld_bytes) {
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int blk = q * 4 + wave;
      if constexpr (KMAJ) {
        const int row = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ kswz(row);
        off[q] = (uint32_t)(row * ld_bytes + c * 16);
        kidx[q] = c * (16 / ES);
        ok[q] = row < rows_valid;
      } else {
        const int krow = blk * kKPI + lane / kCPR;
        const int c = (lane % kCPR) ^ mswz(krow);
        off[q] = (uint32_t)(krow * ld_bytes + c * 16);
        kidx[q] = krow;
        ok[q] = c * (16 / ES) < rows_valid;
      }
    }
  }

  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, GEP_LDS char* lds, int wave, int k0,
                                        int K) const {
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const uint32_t o = (ok[q] && k0 + kidx[q] < K) ? off[q] : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GEP_LDS void*)(lds + (q * 4 + wave) * 1024), 16, o, 0, 0,
                                               0);
    }
  }
};

// Fragment reader: rows [r0, r0+32) of a tile, MFMA k-step s (16-bit: 32 bytes; fp8: 64).
template <bool KMAJ, int ROWS, class Op>
__device__ __forceinline__ typename Op::Frag read_frag(const GEP_LDS char* tile, int r0, int s, int lane) {
  using Frag = typename Op::Frag;
  if constexpr (KMAJ) {
    const int row = r0 + (lane & 31);
    const int sw = kswz(row);
    const GEP_LDS char* rp = tile + row * kRowBytes;
    if constexpr (Op::kES == 2) {
      const int c = s * 2 + (lane >> 5);
      return *(const GEP_LDS i32x4*)(rp + ((c ^ sw) << 4));
    } else {
      const int c = s * 4 + (lane >> 5) * 2;
      i32x4 lo = *(const GEP_LDS i32x4*)(rp + ((c ^ sw) << 4));
      i32x4 hi = *(const GEP_LDS i32x4*)(rp + (((c + 1) ^ sw) << 4));
      return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  } else {
    static_assert(Op::kES == 2, "M/N-major operands are 16-bit only");
    // Source lane (in its 16-lane group) 4j + a reads the 4 row-contiguous elements at
    // k-row kb + j, rows r0 + 16*(group & 1) + 4a; after the transpose lane 4a + e holds
    // row 4a + e, k-rows kb + 0..3.
    const int g = lane >> 4, sl = lane & 15;
    const int row = r0 + 16 * (g & 1) + 4 * (sl & 3);
    const int c = row >> 3, within = (row & 7) * 2;
    s16x4 v[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int krow = s * 16 + 8 * (g >> 1) + 4 * rd + (sl >> 2);
      const GEP_LDS char* p = tile + krow * (ROWS * 2) + ((c ^ mswz(krow)) << 4) + within;
      v[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GEP_LDS s16x4*)p);
    }
    i32x4 out;
    out[0] = (int)((uint16_t)v[0][0] | ((uint32_t)(uint16_t)v[0][1] << 16));
    out[1] = (int)((uint16_t)v[0][2] | ((uint32_t)(uint16_t)v[0][3] << 16));
    out[2] = (int)((uint16_t)v[1][0] | ((uint32_t)(uint16_t)v[1][1] << 16));
    out[3] = (int)((uint16_t)v[1][2] | ((uint32_t)(uint16_t)v[1][3] << 16));
    return out;
  }
}

// ------------------------------------------------------------------------------------
// Epilogue helpers
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Activation of the fp32 pre-activation value (page 6, gemm_act_sm90.py, act_fn_map; SiLU
// added here). Both smooth activations are x * sigmoid(z): GELU-tanh uses
// 0.5 * (1 + tanh(u)) = sigmoid(2u) with u = sqrt(2/pi) * (x + 0.044715 x^3).
__device__ __forceinline__ float apply_act(int act, float x) {
  switch (act) {
    case ACT_RELU: return x > 0.f ? x : 0.f;
    case ACT_RELU_SQ: { float r = x > 0.f ? x : 0.f; return r * r; }
    case ACT_GELU_TANH: {
      const float u2 = 1.5957691216057308f * (x + 0.044715f * x * x * x);  // 2u
      return x / (1.f + fast_exp(-u2));
    }
    case ACT_SILU: return x / (1.f + fast_exp(-x));
    default: return x;
  }
}

__device__ __forceinline__ void load4(const void* p, int dt, float v[4]) {
  if (dt == DT_F32) {
    float4 x = *(const float4*)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else if (dt == DT_BF16) {
    uint2 x = *(const uint2*)p;
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
  } else {
    uint2 x = *(const uint2*)p;
    _Float16 h[4];
    __builtin_memcpy(h, &x, 8);
    v[0] = (float)h[0]; v[1] = (float)h[1]; v[2] = (float)h[2]; v[3] = (float)h[3];
  }
}

__device__ __forceinline__ void store4(void* p, int dt, const float v[4]) {
  if (dt == DT_F32) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  } else if (dt == DT_BF16) {
    __bf16 h[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    uint2 x;
    __builtin_memcpy(&x, h, 8);
    *(uint2*)p = x;
  } else {
    _Float16 h[4] = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    uint2 x;
    __builtin_memcpy(&x, h, 8);
    *(uint2*)p = x;
  }
}

__device__ __forceinline__ int dt_bytes(int dt) { return dt == DT_F32 ? 4 : 2; }

// Wait until at most N vector-memory operations of this wave are outstanding, then
// synchronise the workgroup. The "memory" clobber keeps LDS accesses on their side.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// ------------------------------------------------------------------------------------
// Tile scheduler: linear tile id -> (m_blk, n_blk) inside one batch / group
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void raster(const KParams& p, uint32_t r, uint32_t tm, uint32_t& m, uint32_t& n) {
  const uint32_t G = 1u << p.log2G;
  const uint32_t full = (tm >> p.log2G) << p.log2G;
  const uint32_t tn = (uint32_t)p.tn;
  if (r < full * tn) {
    uint32_t grp, w;
    fd_divmod(p.fd_Gtn, r, grp, w);
    m = (grp << p.log2G) + (w & (G - 1));
    n = w >> p.log2G;
  } else {
    const uint32_t tail = tm - full;  // 1 <= tail < G
    // select the constants with static indices (a dynamic index would spill the kernel
    // argument block to scratch)
    FastDiv f = p.fd_tail[1];
#pragma unroll
    for (int w = 2; w < (1 << kMaxGroupLog2); ++w)
      if (tail == (uint32_t)w) f = p.fd_tail[w];
    uint32_t nn, mm;
    fd_divmod(f, r - full * tn, nn, mm);
    m = full + mm;
    n = nn;
  }
}

template <int BM, int BN, int OP, int FA, int FB, bool A_K, bool B_K, bool VARLEN, int STAGES>
struct GemmKernel {
  using Op = Mfma<OP, FA, FB>;
  using Frag = typename Op::Frag;
  static constexpr int kES = Op::kES;
  static constexpr int kBK = kRowBytes / kES;             // K elements per k-tile
  static constexpr int kSteps = kBK / Op::kKStep;          // MFMA k-steps per k-tile
  static constexpr int kWM = BM / 2, kWN = BN / 2;         // per-wave output block
  static constexpr int kMI = kWM / 32, kNI = kWN / 32;     // 32x32 MFMA blocks per wave
  using LA = TileLoader<BM, A_K, kES>;
  using LB = TileLoader<BN, B_K, kES>;
  static constexpr int kABytes = LA::kTileBytes, kBBytes = LB::kTileBytes;
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kLdsBytes = kStageBytes * STAGES;
  static constexpr int kLoadsPerKTile = LA::kInstr + LB::kInstr;
  static constexpr int kStripPitch = kWN + 4;  // floats per staged row (pad: no bank conflicts)
  static_assert(4 * 32 * kStripPitch * 4 <= kLdsBytes, "epilogue strips must fit in the ring");

  // Scale, add beta*C, activate, convert and store one 32 x kWN strip staged in LDS.
  static __device__ __forceinline__ void epilogue_strip(const KParams& p, const float GEP_LDS* strip, int lane,
                                                        int mrow0, int ncol0, int row_end, int l, float alpha,
                                                        float beta) {
    constexpr int kLanesPerRow = kWN / 4;
    constexpr int kRowsPerIt = 64 / kLanesPerRow;
    const int rr = lane / kLanesPerRow, cc = (lane % kLanesPerRow) * 4;
    const int n = ncol0 + cc;
    if (n >= p.N) return;
    const int64_t c_lb = VARLEN ? 0 : (int64_t)l * p.sc;
    const int64_t d_lb = VARLEN ? 0 : (int64_t)l * p.sd;
    const int64_t p_lb = VARLEN ? 0 : (int64_t)l * p.sp;
    const int cb = dt_bytes(p.c_dt), db = dt_bytes(p.d_dt), pb = dt_bytes(p.p_dt);
#pragma unroll 1
    for (int it = 0; it < 32 / kRowsPerIt; ++it) {
      const int row = it * kRowsPerIt + rr;
      const int m = mrow0 + row;
      if (m >= row_end) break;
      const f32x4 x = *(const f32x4 GEP_LDS*)(strip + row * kStripPitch + cc);
      float v[4] = {x[0] * alpha, x[1] * alpha, x[2] * alpha, x[3] * alpha};
      if (p.c_dt != DT_NONE) {
        float c[4];
        load4((const char*)p.C + (c_lb + (int64_t)m * p.ldc + n) * cb, p.c_dt, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(beta, c[e], v[e]);
      }
      if (p.d_dt != DT_NONE) store4((char*)p.D + (d_lb + (int64_t)m * p.ldd + n) * db, p.d_dt, v);
      if (p.p_dt != DT_NONE) {
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = apply_act(p.act, v[e]);
        store4((char*)p.Post + (p_lb + (int64_t)m * p.ldp + n) * pb, p.p_dt, w);
      }
    }
  }

  static __device__ __forceinline__ void run(const KParams& p) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes];
    GEP_LDS char* smem = (GEP_LDS char*)smem_raw;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave >> 1) * kWM, wn0 = (wave & 1) * kWN;

    const int P = p.P;
    const int bid = blockIdx.x;
    const int bb = (p.xcd_remap && (P & 7) == 0) ? (bid & 7) * (P >> 3) + (bid >> 3) : bid;

    // ---- varlen: tile offsets of the groups, in LDS
    [[maybe_unused]] int32_t* gstart = nullptr;
    int T = p.T;
    if constexpr (VARLEN) {
      __shared__ int32_t s_start[kMaxVarlenGroups + 1];
      __shared__ int32_t s_part[256];
      const int G = p.L;
      constexpr int kPer = (kMaxVarlenGroups + 255) / 256;
      int32_t local[kPer];
      int32_t sum = 0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int g = tid * kPer + q;
        int32_t tiles = 0;
        if (g < G) {
          const int rows = p.cu_seqlens[g + 1] - p.cu_seqlens[g];
          tiles = ((rows + BM - 1) / BM) * p.tn;
        }
        local[q] = sum;
        sum += tiles;
      }
      s_part[tid] = sum;
      __syncthreads();
      // inclusive scan of the 256 partial sums (Hillis-Steele)
      for (int off = 1; off < 256; off <<= 1) {
        const int32_t add = tid >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += add;
        __syncthreads();
      }
      const int32_t excl = s_part[tid] - sum;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int g = tid * kPer + q;
        if (g < G) s_start[g] = excl + local[q];
      }
      if (tid == 255) s_start[G] = s_part[255];
      __syncthreads();
      gstart = s_start;
      T = s_start[G];
    }

    float alpha = p.alpha_ptr ? *p.alpha_ptr : p.alpha;
    float beta = p.beta_ptr ? *p.beta_ptr : p.beta;

    LA la;
    LB lb;
    int iter = 0;
    for (int t = bb; t < T; t += P, ++iter) {
      // ---- decode the tile
      uint32_t mb, nb;
      int l, row_base, row_end;
      if constexpr (VARLEN) {
        int lo = 0, hi = p.L - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (gstart[mid] <= t) lo = mid; else hi = mid - 1;
        }
        l = lo;
        row_base = p.cu_seqlens[l];
        row_end = p.cu_seqlens[l + 1];
        const uint32_t tmg = (uint32_t)((row_end - row_base + BM - 1) / BM);
        raster(p, (uint32_t)(t - gstart[l]), tmg, mb, nb);
      } else {
        uint32_t ll, r;
        fd_divmod(p.fd_mn, (uint32_t)t, ll, r);
        raster(p, r, (uint32_t)p.tm, mb, nb);
        l = (int)ll;
        row_base = 0;
        row_end = p.M;
      }
      if (p.tile_log && iter < p.tile_log_iters && tid == 0) {
        int32_t* e = p.tile_log + ((int64_t)bid * p.tile_log_iters + iter) * 4;
        e[0] = (int32_t)mb; e[1] = (int32_t)nb; e[2] = l; e[3] = t;
      }
      const int m0 = row_base + (int)mb * BM;  // first row of the tile
      const int n0 = (int)nb * BN;

      // ---- operand tile bases (bytes) and loaders
      const int64_t a_lb = VARLEN ? 0 : (int64_t)l * p.sa;
      const int64_t b_lb = (int64_t)l * p.sb;
      const char* a_tile;
      const char* b_tile;
      int64_t a_room, b_room;  // bytes from the tile base to the operand's end
      {
        const int64_t a_off = (a_lb + (A_K ? (int64_t)m0 * p.lda : (int64_t)m0)) * kES;
        const int64_t b_off = (b_lb + (B_K ? (int64_t)n0 * p.ldb : (int64_t)n0)) * kES;
        a_tile = (const char*)p.A + a_off;
        b_tile = (const char*)p.B + b_off;
        a_room = p.a_bytes - a_off;
        b_room = p.b_bytes - b_off;
      }
      const int64_t lda_b = p.lda * kES, ldb_b = p.ldb * kES;
      la.init(wave, lane, row_end - m0, lda_b);
      lb.init(wave, lane, p.N - n0, ldb_b);
      const int64_t a_kstep = A_K ? (int64_t)kRowBytes : (int64_t)kBK * lda_b;
      const int64_t b_kstep = B_K ? (int64_t)kRowBytes : (int64_t)kBK * ldb_b;

      const int nk = (p.K + kBK - 1) / kBK;
      auto issue = [&](int kt) {
        GEP_LDS char* st = smem + (kt % STAGES) * kStageBytes;
        const int64_t ao = (int64_t)kt * a_kstep, bo = (int64_t)kt * b_kstep;
        la.issue(make_rsrc(a_tile + ao, a_room - ao), st, wave, kt * kBK, p.K);
        lb.issue(make_rsrc(b_tile + bo, b_room - bo), st + kABytes, wave, kt * kBK, p.K);
      };

      f32x16 acc[kMI][kNI];
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNI; ++j) acc[i][j] = f32x16{};

      // every wave is done with the previous tile's LDS before it is overwritten
      barrier_only();
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue(s);

      for (int kt = 0; kt < nk; ++kt) {
        if (kt + STAGES - 2 < nk) wait_vm_barrier<(STAGES - 2) * kLoadsPerKTile>();
        else wait_vm_barrier<0>();
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
        const GEP_LDS char* sa = smem + (kt % STAGES) * kStageBytes;
        const GEP_LDS char* sb = sa + kABytes;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          Frag af[kMI], bf[kNI];
#pragma unroll
          for (int i = 0; i < kMI; ++i) af[i] = read_frag<A_K, BM, Op>(sa, wm0 + i * 32, s, lane);
#pragma unroll
          for (int j = 0; j < kNI; ++j) bf[j] = read_frag<B_K, BN, Op>(sb, wn0 + j * 32, s, lane);
#pragma unroll
          for (int i = 0; i < kMI; ++i)
#pragma unroll
            for (int j = 0; j < kNI; ++j) acc[i][j] = Op::mma(bf[j], af[i], acc[i][j]);
        }
      }

      // ---- epilogue. Lane l holds, for block (i, j) and register group g, the values at
      // row wm0 + 32i + (l % 32), columns wn0 + 32j + 8g + 4(l / 32) + [0, 4). Each
      // 32-row strip goes through this wave's part of the (now idle) LDS ring as fp32 and
      // comes back row-contiguous: 4 consecutive columns per lane, so C loads and D /
      // PostAct stores are coalesced.
      barrier_only();  // every wave is done reading the ring
      float GEP_LDS* strip = (float GEP_LDS*)smem + wave * 32 * kStripPitch;
#pragma unroll
      for (int i = 0; i < kMI; ++i) {
#pragma unroll
        for (int j = 0; j < kNI; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                             acc[i][j][4 * g + 3]};
            *(f32x4 GEP_LDS*)(strip + (lane & 31) * kStripPitch + j * 32 + 8 * g + 4 * (lane >> 5)) = v;
          }
        // LDS operations of one wave complete in order; keep the compiler from reordering
        asm volatile("" ::: "memory");
        epilogue_strip(p, strip, lane, m0 + wm0 + i * 32, n0 + wn0, row_end, l, alpha, beta);
        asm volatile("" ::: "memory");
      }
    }
  }
};

}  // namespace gep
