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
//   * A and B k-tiles of 64 bytes per row travel global -> LDS with buffer_load ... lds
//     (no VGPR staging) into a STAGES-deep ring, issued STAGES-1 k-tiles ahead.
//     Out-of-range rows / k-chunks use an offset past the buffer's num_records, which the
//     hardware reads as zero (tails in M, N and K).
//   * K-major tiles are stored [row][4 x 16-byte chunks] with the chunk index XOR-swizzled
//     by the row, so the 32-row MFMA fragment reads (ds_read_b128) hit distinct banks.
//     M/N-major (16-bit) tiles are stored [k][row] and read with ds_read_b64_tr_b16, which
//     transposes 16x4 blocks across each 16-lane group into K-contiguous fragments.
//   * Fragments are double-buffered in registers: the LDS reads of the next k-step are
//     interleaved with the MFMAs of the current one. The once-per-k-tile barrier sits before
//     the last k-step's MFMAs, so the next k-tile's first fragments load under them.
//   * Persistent grid: workgroup b takes tiles t = b' + i*P; t -> (m_blk, n_blk, l) by the
//     grouped raster with FastDivmod (page 6, quack/fast_math.py); b' optionally remaps b so
//     that the workgroups of one XCD (dispatched round-robin) take consecutive tile ids.
//   * Epilogue: the accumulators go, 16 rows at a time, through one stage-sized region of
//     the ring as fp32 and come back row-contiguous (4 columns per lane) for scaling,
//     beta*C, the activation, conversion and coalesced stores. The next tile's first k-tile
//     loads are already in flight in the other stages meanwhile.
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
// Lane l holds row (l % 32) and, inside the instruction's K slice, elements [8*(l/32), +8)
// for 16-bit types or bytes [32*(l/32), +32) for fp8; A and B use the same K assignment.
// The kernel passes the B fragment as the instruction's first source and the A fragment as
// its second, so that each output lane holds 4 consecutive N values (see the epilogue).
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
  // cbsz / blgp select the format of the first / second source (0 = e4m3, 1 = e5m2):
  // B's format goes in cbsz and A's in blgp. Scales of 127 are 2^0 in E8M0 (no scaling).
  static __device__ __forceinline__ f32x16 mma(Frag b, Frag a, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, 0, 127, 0, 127);
  }
};

// ------------------------------------------------------------------------------------
// LDS tile layouts
// ------------------------------------------------------------------------------------
constexpr int kRowBytes = 64;  // bytes of K per row of a K-major k-tile
constexpr int kChunks = kRowBytes / 16;

// K-major: 16-byte chunk c of row r lives at chunk c ^ kswz(r). Measured on gfx950, a
// ds_read_b128 is served in 4 phases of 16 lanes (the lanes sharing lane bit 5 and
// bit 2 ^ bit 4) over 64 four-byte banks, i.e. one 256-byte window per phase. A fragment
// read puts rows r0 + (l % 32) of one logical chunk in a phase; 64-byte rows sharing r & 3
// land in the same 64-byte quarter of the window, so the key must differ between them:
// (r >> 2) & 3 does, for both phase parities.
__device__ __forceinline__ int kswz(int row) { return (row >> 2) & 3; }
// M/N-major: chunk c of k-row k lives at chunk c ^ mswz(k); the 4 k-rows that one 16-lane
// transpose group reads land in 4 disjoint 64-byte bank ranges.
__device__ __forceinline__ int mswz(int k) { return (k & 3) << 2; }

// Buffer resource over [base, base + bytes); reads at offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Loader of one operand's k-tile: ROWS rows (M or N) by kRowBytes of K, staged through
// VGPRs: each lane loads kInstr 16-byte chunks (buffer_load_dwordx4) and later writes them
// with ds_write_b128 to fixed LDS positions (block q*4+wave of 1 KB, lane*16 inside it).
// The global address of a lane is the inverse of the LDS swizzle, so LDS writes are
// contiguous and conflict-free. Measured on gfx950, this path keeps the MFMA pipe full at
// twice the bandwidth the mainloop needs, where LDS-DMA loads (buffer_load ... lds) slow it.
template <int ROWS, bool KMAJ, int ES>
struct TileLoader {
  static constexpr int kTileBytes = ROWS * kRowBytes;
  static constexpr int kInstr = kTileBytes / 1024 / 4;
  static constexpr int kCPR = ROWS * ES / 16;                  // MN-major: chunks per k-row
  static constexpr int kKPI = KMAJ ? 1 : 1024 / (ROWS * ES);   // MN-major: k-rows per instruction
  static_assert(kInstr >= 1, "tile too small for 4 waves");
  uint32_t offv[kInstr];   // byte offset of this lane's chunk in the k-tile, or kOOB when the
                           // row / column chunk lies outside the operand
  int32_t klim[kInstr];    // the chunk exists while k0 < klim (K minus its k offset in the k-tile)
  i32x4 reg[2][kInstr];    // two staging sets (k-tile parity)

  // rows_valid: rows of this tile that exist (K-major) or MN elements that exist (MN-major).
  __device__ __forceinline__ void init(int wave, int lane, int rows_valid, int64_t ld_bytes, int K) {
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int blk = q * 4 + wave;
      if constexpr (KMAJ) {
        const int row = blk * (1024 / kRowBytes) + lane / kChunks;
        const int c = (lane % kChunks) ^ kswz(row);
        offv[q] = row < rows_valid ? (uint32_t)(row * ld_bytes + c * 16) : kOOB;
        klim[q] = K - c * (16 / ES);
      } else {
        const int krow = blk * kKPI + lane / kCPR;
        const int c = (lane % kCPR) ^ mswz(krow);
        offv[q] = c * (16 / ES) < rows_valid ? (uint32_t)(krow * ld_bytes + c * 16) : kOOB;
        klim[q] = K - krow;
      }
    }
  }

  // Global -> registers. Chunks at k >= K (the K tail, and whole k-tiles past the end) read
  // as zero through the buffer range check.
  template <int SET>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int k0) {
#pragma unroll
    for (int q = 0; q < kInstr; ++q)
      reg[SET][q] = __builtin_amdgcn_raw_buffer_load_b128(rs, k0 < klim[q] ? offv[q] : kOOB, 0, 0);
  }

  // Registers -> LDS (tile base `lds`).
  template <int SET>
  __device__ __forceinline__ void store(GEP_LDS char* lds, int wave, int lane) const {
#pragma unroll
    for (int q = 0; q < kInstr; ++q) *(GEP_LDS i32x4*)(lds + (q * 4 + wave) * 1024 + lane * 16) = reg[SET][q];
  }
};

// LDS reads per fragment (for the scheduling pattern).
template <bool KMAJ, int ES>
constexpr int reads_per_frag() { return KMAJ ? (ES == 2 ? 1 : 2) : 2; }

// Fragment reader: rows [r0, r0+32) of a tile, MFMA k-step s of the k-tile.
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
      const int c = (lane >> 5) * 2;  // one fp8 k-step spans the whole 64-byte row
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

// Complete this wave's LDS operations, then synchronise the workgroup. The "memory"
// clobber keeps LDS accesses on their side of it.
// sched_barrier(0) on both sides also keeps register-only instructions (MFMAs) from
// drifting across, so each MFMA step stays one scheduling region.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

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

// Everything the loop needs about one output tile.
struct TileInfo {
  int l, m0, n0, row_end;
  int mb, nb;          // block coordinates inside the batch / group
  const char* a_tile;  // first byte of the tile's A rows (K-major) / columns (M-major)
  const char* b_tile;
  int64_t a_room, b_room;  // bytes from the tile base to the end of the operand
};

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
  static constexpr int kEpiBytes = 4 * 16 * (BN / 2) * 4;      // 16-row fp32 strip per wave
  static constexpr int kLdsBytes = kStageBytes * STAGES + kEpiBytes;
  static constexpr int kLoadsPerKTile = LA::kInstr + LB::kInstr;
  static constexpr int kMfmaPerStep = kMI * kNI;
  static constexpr int kDsPerStep = kMI * reads_per_frag<A_K, kES>() + kNI * reads_per_frag<B_K, kES>();
  // Epilogue: 16-row fp32 strips, one per wave, XOR-swizzled by row in 16-byte chunks.
  static constexpr int kStripRows = 16;
  static constexpr int kStripChunks = kWN / 4;
  static_assert(STAGES == 2, "the mainloop alternates two LDS stages");
  // k-tile kt+kW is written to LDS in k-tile kt, and loaded into registers kLead k-tiles
  // before that (two register sets)
  static constexpr int kW = kSteps == 2 ? 1 : 2;

  // ---- scheduling hints: interleave LDS reads (and VMEM loads) with the MFMAs ----
  // Scheduling pattern of one MFMA step, in groups that each start with one MFMA. Without
  // staging (NST == 0) the step's LDS reads are spread over all its MFMAs. With staging the
  // first half of the MFMAs carries the LDS reads and the second half the LDS writes and
  // the VMEM loads: the reads must stay ahead of the writes (the compiler cannot prove
  // them disjoint), and they are what the next step waits for. The builtin needs literal
  // arguments, hence the compile-time recursion.
  template <int NST, int I = 0>
  static __device__ __forceinline__ void sched_step() {
    constexpr int M = kMfmaPerStep, D = kDsPerStep;
    constexpr int H = NST ? (M / 2 > 0 ? M / 2 : 1) : M;   // MFMAs that carry the reads
    constexpr int rper = (D + H - 1) / H;
    constexpr int wper = NST ? (NST + (M - H) - 1) / (M - H > 0 ? M - H : 1) : 0;
    if constexpr (I < M) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if constexpr (I < H && I * rper < D) {
        constexpr int n = (D - I * rper) < rper ? (D - I * rper) : rper;
        __builtin_amdgcn_sched_group_barrier(0x100, n, 0);  // LDS reads
      }
      if constexpr (I >= H && (I - H) * wper < NST) {
        constexpr int n = (NST - (I - H) * wper) < wper ? (NST - (I - H) * wper) : wper;
        __builtin_amdgcn_sched_group_barrier(0x200, n, 0);  // LDS writes
        __builtin_amdgcn_sched_group_barrier(0x020, n, 0);  // VMEM loads
      }
      sched_step<NST, I + 1>();
    }
  }

  static __device__ __forceinline__ void read_step(Frag (&fa)[kMI], Frag (&fb)[kNI], const GEP_LDS char* st,
                                                   int s, int wm0, int wn0, int lane) {
#pragma unroll
    for (int i = 0; i < kMI; ++i) fa[i] = read_frag<A_K, BM, Op>(st, wm0 + i * 32, s, lane);
#pragma unroll
    for (int j = 0; j < kNI; ++j) fb[j] = read_frag<B_K, BN, Op>(st + kABytes, wn0 + j * 32, s, lane);
  }

  static __device__ __forceinline__ void mma_step(f32x16 (&acc)[kMI][kNI], const Frag (&fa)[kMI],
                                                  const Frag (&fb)[kNI]) {
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < kNI; ++j) acc[i][j] = Op::mma(fb[j], fa[i], acc[i][j]);
  }

  static __device__ __forceinline__ TileInfo decode(const KParams& p, int t, const int32_t* gstart) {
    TileInfo ti;
    uint32_t mb, nb;
    int row_base;
    if constexpr (VARLEN) {
      int lo = 0, hi = p.L - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (gstart[mid] <= t) lo = mid; else hi = mid - 1;
      }
      ti.l = lo;
      row_base = p.cu_seqlens[lo];
      ti.row_end = p.cu_seqlens[lo + 1];
      const uint32_t tmg = (uint32_t)((ti.row_end - row_base + BM - 1) / BM);
      raster(p, (uint32_t)(t - gstart[lo]), tmg, mb, nb);
    } else {
      uint32_t ll, r;
      fd_divmod(p.fd_mn, (uint32_t)t, ll, r);
      raster(p, r, (uint32_t)p.tm, mb, nb);
      ti.l = (int)ll;
      row_base = 0;
      ti.row_end = p.M;
    }
    ti.mb = (int)mb;
    ti.nb = (int)nb;
    ti.m0 = row_base + (int)mb * BM;
    ti.n0 = (int)nb * BN;
    const int64_t a_lb = VARLEN ? 0 : (int64_t)ti.l * p.sa;
    const int64_t b_lb = (int64_t)ti.l * p.sb;
    const int64_t a_off = (a_lb + (A_K ? (int64_t)ti.m0 * p.lda : (int64_t)ti.m0)) * kES;
    const int64_t b_off = (b_lb + (B_K ? (int64_t)ti.n0 * p.ldb : (int64_t)ti.n0)) * kES;
    ti.a_tile = (const char*)p.A + a_off;
    ti.b_tile = (const char*)p.B + b_off;
    ti.a_room = p.a_bytes - a_off;
    ti.b_room = p.b_bytes - b_off;
    return ti;
  }

  // Global loads of k-tile j into register set SET (k-tiles past the end read as zero).
  template <int SET>
  static __device__ __forceinline__ void load_kt(const KParams& p, const TileInfo& ti, LA& la, LB& lb, int j) {
    const int64_t a_step = A_K ? (int64_t)kRowBytes : (int64_t)kBK * p.lda * kES;
    const int64_t b_step = B_K ? (int64_t)kRowBytes : (int64_t)kBK * p.ldb * kES;
    const int64_t ao = (int64_t)j * a_step, bo = (int64_t)j * b_step;
    la.template load<SET>(make_rsrc(ti.a_tile + ao, ti.a_room - ao), j * kBK);
    lb.template load<SET>(make_rsrc(ti.b_tile + bo, ti.b_room - bo), j * kBK);
  }
  // Register set SET -> LDS stage of k-tile j.
  template <int SET>
  static __device__ __forceinline__ void store_kt(const LA& la, const LB& lb, GEP_LDS char* smem, int j, int wave,
                                                  int lane) {
    GEP_LDS char* st = smem + (j % STAGES) * kStageBytes;
    la.template store<SET>(st, wave, lane);
    lb.template store<SET>(st + kABytes, wave, lane);
  }

  // First loads of a tile into registers: k-tile 0 (set 0) and 1 (set 1).
  static __device__ __forceinline__ void prologue_loads(const KParams& p, const TileInfo& ti, LA& la, LB& lb,
                                                        int wave, int lane) {
    la.init(wave, lane, ti.row_end - ti.m0, p.lda * kES, p.K);
    lb.init(wave, lane, p.N - ti.n0, p.ldb * kES, p.K);
    load_kt<0>(p, ti, la, lb, 0);
    load_kt<1>(p, ti, la, lb, 1);
  }
  // Rest of a tile's start (every wave is done reading the ring): k-tiles 0 .. kW-1 to LDS,
  // their register sets reloaded with k-tiles 2 .. kW+1.
  static __device__ __forceinline__ void prologue_stores(const KParams& p, const TileInfo& ti, LA& la, LB& lb,
                                                         GEP_LDS char* smem, int wave, int lane) {
    store_kt<0>(la, lb, smem, 0, wave, lane);
    load_kt<0>(p, ti, la, lb, 2);
    if constexpr (kW == 2) {
      store_kt<1>(la, lb, smem, 1, wave, lane);
      load_kt<1>(p, ti, la, lb, 3);
    }
  }

  // MFMAs on fragment buffer CUR while the next fragments are read into the other buffer,
  // and (STAGE) the register set of k-tile js is written to LDS and reloaded with k-tile jl.
  // Program order puts the reads first: the compiler keeps LDS reads behind LDS writes it
  // cannot prove disjoint, and the reads are the ones the next step waits for.
  template <int CUR, bool STAGE, int SET>
  static __device__ __forceinline__ void step(const KParams& p, const TileInfo& ti, LA& la, LB& lb,
                                              GEP_LDS char* smem, f32x16 (&acc)[kMI][kNI], Frag (&fa)[2][kMI],
                                              Frag (&fb)[2][kNI], const GEP_LDS char* st, int s, int js, int jl,
                                              int wave, int lane, int wm0, int wn0) {
    read_step(fa[CUR ^ 1], fb[CUR ^ 1], st, s, wm0, wn0, lane);
    if constexpr (STAGE) {
      store_kt<SET>(la, lb, smem, js, wave, lane);
      load_kt<SET>(p, ti, la, lb, jl);
    }
    mma_step(acc, fa[CUR], fb[CUR]);
    sched_step<STAGE ? LA::kInstr + LB::kInstr : 0>();
  }

  // One k-tile kt (PAR = kt & 1), the same code for every kt. k-tiles past the end are
  // zero-filled and never used, so there is no branch and the LDS writes, loads and reads
  // interleave with the MFMAs.
  //   two MFMA steps (16-bit): step 0 writes k-tile kt+1 to LDS from its register set and
  //     reloads that set with kt+3, while its MFMAs run on fragments of (kt, 0) and it reads
  //     (kt, 1); barrier; step 1 runs (kt, 1) and reads (kt+1, 0).
  //   one MFMA step (fp8): barrier; write kt+2, reload its set with kt+4, MFMAs on kt, read
  //     kt+1.
  // The barrier is preceded by lgkmcnt(0): this wave's LDS writes are complete and its
  // reads of the stage about to be overwritten have returned.
  template <int PAR>
  static __device__ __forceinline__ void ktile(const KParams& p, const TileInfo& ti, LA& la, LB& lb,
                                               GEP_LDS char* smem, f32x16 (&acc)[kMI][kNI], Frag (&fa)[2][kMI],
                                               Frag (&fb)[2][kNI], int kt, int wave, int lane, int wm0, int wn0) {
    const GEP_LDS char* st = smem + (kt % STAGES) * kStageBytes;
    const GEP_LDS char* st1 = smem + ((kt + 1) % STAGES) * kStageBytes;
    if constexpr (kSteps == 2) {
      constexpr int SET = (PAR + 1) & 1;  // register set of k-tile kt+1 (and kt+3)
      step<0, true, SET>(p, ti, la, lb, smem, acc, fa, fb, st, 1, kt + 1, kt + 3, wave, lane, wm0, wn0);
      lds_barrier();
      step<1, false, 0>(p, ti, la, lb, smem, acc, fa, fb, st1, 0, 0, 0, wave, lane, wm0, wn0);
    } else {
      constexpr int SET = PAR;  // register set of k-tile kt+2 (and kt+4)
      lds_barrier();
      step<PAR, true, SET>(p, ti, la, lb, smem, acc, fa, fb, st1, 0, kt + 2, kt + 4, wave, lane, wm0, wn0);
    }
  }

  // Scale, add beta*C, activate, convert and store one kStripRows x kWN strip staged in LDS.
  static __device__ __forceinline__ void epilogue_strip(const KParams& p, const float GEP_LDS* strip, int lane,
                                                        int mrow0, int ncol0, int row_end, int l, float alpha,
                                                        float beta) {
    constexpr int kRowsPerIt = 64 / kStripChunks;
    const int rr = lane / kStripChunks, q = lane % kStripChunks;
    const int n = ncol0 + q * 4;
    if (n >= p.N) return;
    const int64_t c_lb = VARLEN ? 0 : (int64_t)l * p.sc;
    const int64_t d_lb = VARLEN ? 0 : (int64_t)l * p.sd;
    const int64_t p_lb = VARLEN ? 0 : (int64_t)l * p.sp;
    const int cb = dt_bytes(p.c_dt), db = dt_bytes(p.d_dt), pb = dt_bytes(p.p_dt);
#pragma unroll 1
    for (int it = 0; it < kStripRows / kRowsPerIt; ++it) {
      const int row = it * kRowsPerIt + rr;
      const int m = mrow0 + row;
      if (m >= row_end) break;
      const f32x4 x = *(const f32x4 GEP_LDS*)(strip + row * kWN + ((q ^ (row & 7)) << 2));
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

  // Accumulator lane layout: for block (i, j) and register group g, lane l holds row
  // wm0 + 32i + (l % 32) and columns wn0 + 32j + 8g + 4(l / 32) + [0, 4).
  static __device__ __forceinline__ void epilogue(const KParams& p, const TileInfo& ti,
                                                  const f32x16 (&acc)[kMI][kNI], float GEP_LDS* region, int wave,
                                                  int lane, int wm0, int wn0, float alpha, float beta) {
    float GEP_LDS* strip = region + wave * kStripRows * kWN;
    const int r16 = lane & 15;
    const bool mine_lo = ((lane >> 4) & 1) == 0;  // lane holds rows 0..15 of its 32-row block
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (mine_lo == (h == 0)) {
#pragma unroll
          for (int j = 0; j < kNI; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                               acc[i][j][4 * g + 3]};
              const int q = j * 8 + 2 * g + (lane >> 5);
              *(f32x4 GEP_LDS*)(strip + r16 * kWN + ((q ^ (r16 & 7)) << 2)) = v;
            }
        }
        // LDS operations of one wave complete in order; keep the compiler from reordering
        asm volatile("" ::: "memory");
        epilogue_strip(p, strip, lane, ti.m0 + wm0 + i * 32 + h * 16, ti.n0 + wn0, ti.row_end, ti.l, alpha, beta);
        asm volatile("" ::: "memory");
      }
    }
  }

  static __device__ __forceinline__ void run(const KParams& p) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes];
    GEP_LDS char* smem = (GEP_LDS char*)smem_raw;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
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

    const float alpha = p.alpha_ptr ? *p.alpha_ptr : p.alpha;
    const float beta = p.beta_ptr ? *p.beta_ptr : p.beta;
    // k-tiles, run in pairs (the register sets alternate): an odd count gets one padding
    // k-tile past K, whose loads read zeros and which adds nothing.
    int nk = (p.K + kBK - 1) / kBK;
    nk = (nk + 1) & ~1;
    float GEP_LDS* epi_region = (float GEP_LDS*)(smem + STAGES * kStageBytes);

    LA la;
    LB lb;
    Frag fa[2][kMI], fb[2][kNI];
    TileInfo ti;
    if (bb < T) {
      ti = decode(p, bb, gstart);
      prologue_loads(p, ti, la, lb, wave, lane);
    }
    int iter = 0;
    for (int t = bb; t < T; t += P, ++iter) {
      if (p.tile_log && iter < p.tile_log_iters && tid == 0) {
        int32_t* e = p.tile_log + ((int64_t)bid * p.tile_log_iters + iter) * 4;
        e[0] = ti.mb; e[1] = ti.nb; e[2] = ti.l; e[3] = t;
      }
      f32x16 acc[kMI][kNI];
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNI; ++j) acc[i][j] = f32x16{};

      if (nk > 0) {
        prologue_stores(p, ti, la, lb, smem, wave, lane);
        lds_barrier();
        read_step(fa[0], fb[0], smem, 0, wm0, wn0, lane);
        for (int kt = 0; kt < nk; kt += 2) {
          ktile<0>(p, ti, la, lb, smem, acc, fa, fb, kt, wave, lane, wm0, wn0);
          ktile<1>(p, ti, la, lb, smem, acc, fa, fb, kt + 1, wave, lane, wm0, wn0);
        }
      }

      // ---- the next tile's first loads go in flight (into registers), then this tile's
      // epilogue, in its own LDS region. The barrier ends every wave's reads of the ring,
      // which the next tile's first LDS writes overwrite.
      lds_barrier();
      const TileInfo cur = ti;
      const int tnext = t + P;
      if (tnext < T) {
        ti = decode(p, tnext, gstart);
        prologue_loads(p, ti, la, lb, wave, lane);
      }
      epilogue(p, cur, acc, epi_region, wave, lane, wm0, wn0, alpha, beta);
    }
  }
};

}  // namespace gep
