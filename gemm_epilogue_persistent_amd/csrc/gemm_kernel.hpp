// Persistent batched GEMM with fused epilogue for gfx950 (CDNA4):
//   D = alpha * A x B + beta * C,  PostAct = act(D before rounding).
//
// Operation: quack-kernels 0.1.10 -> 0.2.0 diff, page 5, quack/dense_gemm_sm90.py (GemmSm90:
// persistent tile loop, k-tile mainloop, epi_visit_acc_subtile) and page 6,
// quack/gemm_act_sm90.py (GemmActSm90: PostAct = act(fp32 pre-activation) next to D).
// The design is this file's own:
//   * 512 threads = 8 wave64s in a 2x4 grid for operands that are both K-major with 256x256
//     tiles: two waves per SIMD, each owning a 128x64 block of the output tile, computed with
//     v_mfma_f32_16x16x32_{f16,bf16} or v_mfma_f32_16x16x128_f8f6f4. Otherwise 256 threads =
//     4 wave64s in a 2x2 grid, each owning a (BM/2) x (BN/2) block computed with
//     v_mfma_f32_32x32x16_{f16,bf16} or v_mfma_f32_32x32x64_f8f6f4 (fp8: per-operand
//     e4m3/e5m2 format fields, no scaling).
//   * A k-tile is 128 bytes of K per row (64 16-bit or 128 fp8 elements): every global load
//     instruction reads whole 128-byte lines. A and B k-tiles go into a two-stage LDS ring,
//     global -> LDS directly (buffer_load_dwordx4 ... lds; the 8-wave and fp8 kernels) or
//     through a staging register set (buffer_load_dwordx4 -> ds_write_b128). Out-of-range
//     rows / k-chunks use an offset past the buffer's num_records, which the hardware reads
//     as zero (tails in M, N and K).
//   * One barrier per k-tile, placed before the first fragment read from the next stage
//     (before the last MFMA step, or inside it with 8 waves); the transfers (or staging
//     writes) into the stage that barrier frees follow it.
//   * K-major tiles are stored [row][8 x 16-byte chunks] with the chunk index XOR-swizzled
//     by the row, so the fragment reads (ds_read_b128) hit distinct banks. M/N-major (16-bit)
//     tiles are stored [k][row] and read with ds_read_b64_tr_b16, which transposes 16x4
//     blocks across each 16-lane group into K-contiguous fragments.
//   * The LDS reads of the next k-step are interleaved with the MFMAs of the current one
//     (double-buffered fragments; with 8 waves a rolling set of 12, or for fp8 the 4 B
//     fragments and a ring of 2 A fragments).
//   * Persistent grid: workgroup b takes tiles t = b' + i*P; t -> (m_blk, n_blk, l) by the
//     grouped raster with FastDivmod (page 6, quack/fast_math.py); b' optionally remaps b so
//     that the workgroups of one XCD (dispatched round-robin) take consecutive tile ids.
//   * Epilogue: the accumulators go through per-wave buffers in the (then idle) ring and come
//     back row-contiguous (8 columns per lane) for scaling, beta*C, the activation,
//     conversion and 16-byte stores.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "params.hpp"

namespace gep {

#define GEP_LDS __attribute__((address_space(3)))

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------------------------
// MFMA flavours, in blocks of kBlk x kBlk outputs. Frag = the per-lane operand registers of
// one kBlk-row fragment: lane l holds row (l % kBlk) and, inside the instruction's K slice,
// the (l / kBlk)-th run of 8 16-bit elements or 32 fp8 bytes; A and B use the same K
// assignment. The kernel passes the B fragment as the instruction's first source and the A
// fragment as its second, so that each output lane holds 4 consecutive N values (see the
// epilogue).
// Measured on gfx950 with full-entropy operands and no memory traffic, the chip sustains the
// 16x16 forms at a higher clock than the 32x32 ones (the same FLOPs take less energy):
// bf16 16x16x32 2.06 against 32x32x16 1.84 PFLOP/s with two waves per SIMD; fp8 16x16x128
// 4.41 against 32x32x64 4.07 PFLOP/s with one.
// ------------------------------------------------------------------------------------
template <int OP, int FA, int FB, int BLK = 32>
struct Mfma;

template <int FA, int FB>
struct Mfma<OP_F16, FA, FB, 32> {
  static constexpr int kES = 2;       // bytes per element
  static constexpr int kKStep = 16;   // K per instruction
  static constexpr int kBlk = 32;
  using Frag = i32x4;
  using Acc = f32x16;
  static __device__ __forceinline__ Acc mma(Frag b, Frag a, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a),
                                                  c, 0, 0, 0);
  }
};

template <int FA, int FB>
struct Mfma<OP_BF16, FA, FB, 32> {
  static constexpr int kES = 2;
  static constexpr int kKStep = 16;
  static constexpr int kBlk = 32;
  using Frag = i32x4;
  using Acc = f32x16;
  static __device__ __forceinline__ Acc mma(Frag b, Frag a, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                   c, 0, 0, 0);
  }
};

template <int FA, int FB>
struct Mfma<OP_F16, FA, FB, 16> {
  static constexpr int kES = 2;
  static constexpr int kKStep = 32;
  static constexpr int kBlk = 16;
  using Frag = i32x4;
  using Acc = f32x4;
  static __device__ __forceinline__ Acc mma(Frag b, Frag a, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a),
                                                  c, 0, 0, 0);
  }
};

template <int FA, int FB>
struct Mfma<OP_BF16, FA, FB, 16> {
  static constexpr int kES = 2;
  static constexpr int kKStep = 32;
  static constexpr int kBlk = 16;
  using Frag = i32x4;
  using Acc = f32x4;
  static __device__ __forceinline__ Acc mma(Frag b, Frag a, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                   c, 0, 0, 0);
  }
};

template <int FA, int FB>
struct Mfma<OP_FP8, FA, FB, 32> {
  static constexpr int kES = 1;
  static constexpr int kKStep = 64;
  static constexpr int kBlk = 32;
  using Frag = i32x8;
  using Acc = f32x16;
  // cbsz / blgp select the format of the first / second source (0 = e4m3, 1 = e5m2):
  // B's format goes in cbsz and A's in blgp. Zero scale operands make the compiler emit the
  // unscaled instruction, which needs no register for them.
  static __device__ __forceinline__ Acc mma(Frag b, Frag a, Acc c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, 0, 0, 0, 0);
  }
};

// 16x16x128 (the 8-wave fp8 kernels), the same way
template <int FA, int FB>
struct Mfma<OP_FP8, FA, FB, 16> {
  static constexpr int kES = 1;
  static constexpr int kKStep = 128;
  static constexpr int kBlk = 16;
  using Frag = i32x8;
  using Acc = f32x4;
  static __device__ __forceinline__ Acc mma(Frag b, Frag a, Acc c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, FB, FA, 0, 0, 0, 0);
  }
};

// ------------------------------------------------------------------------------------
// LDS tile layouts
// ------------------------------------------------------------------------------------
constexpr int kRowBytes = 128;  // bytes of K per row of a K-major k-tile
constexpr int kChunks = kRowBytes / 16;

// K-major: 16-byte chunk c of row r lives at chunk c ^ kswz(r). Measured on gfx950, a
// ds_read_b128 is served in 4 phases of 16 lanes (the lanes sharing lane bit 5 and
// bit 2 ^ bit 4) over 64 four-byte banks, i.e. one 256-byte window per phase. A fragment
// read puts rows r0 + (l % 32) of one logical chunk in a phase: per value of row bit 0
// (which 128-byte half of the window a row falls in), eight rows that differ in bits 1..3.
// Keyed by those bits, the chunk lands in eight distinct 16-byte slots of its half.
__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 7; }
// M/N-major: chunk c of k-row k lives at chunk c ^ mswz(k); the 4 k-rows that one 16-lane
// transpose group reads land in 4 disjoint 64-byte bank ranges.
__device__ __forceinline__ int mswz(int k) { return (k & 3) << 2; }

// Buffer resource over [base, base + bytes); reads at offsets >= bytes return zero.
// The base and extent are the same in every lane (they depend on the tile only); reading
// them through readfirstlane states that, so the descriptor stays in SGPRs. (Where the
// compiler cannot tell and has moved them to VGPRs, it otherwise wraps every buffer
// instruction in a loop over the distinct descriptor values.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// Loader of one operand's k-tile: ROWS rows (M or N) by kRowBytes of K, staged through
// VGPRs: each lane loads kInstr 16-byte chunks (buffer_load_dwordx4) and later writes them
// with ds_write_b128 to fixed LDS positions (block q*NW+wave of 1 KB, lane*16 inside it).
// The global address of a lane is the inverse of the LDS swizzle, so LDS writes are
// contiguous and conflict-free, and the 8 (K-major) or 32/16 (M/N-major) lanes that fill
// one LDS row read one contiguous 128/512/256-byte run of global memory.
template <int ROWS, bool KMAJ, int ES, int NW, bool PAD>
struct TileLoader {
  // K-major rows in LDS: kRowBytes of K, either padded to kPitch (PAD; 9 16-byte slots
  // per row, an odd count, so the 16 rows of a fragment read phase hit 16 distinct slots)
  // or XOR-swizzled (kswz; the layout global -> LDS transfers can produce).
  static constexpr int kPitch = (KMAJ && PAD) ? kRowBytes + 16 : kRowBytes;
  static constexpr int kTileBytes = ROWS * kPitch;  // LDS bytes of one k-tile
  static constexpr int kInstr = ROWS * kRowBytes / 1024 / NW;
  static constexpr int kCPR = ROWS * ES / 16;                  // MN-major: chunks per k-row
  static constexpr int kKPI = KMAJ ? 1 : 1024 / (ROWS * ES);   // MN-major: k-rows per instruction
  static_assert(kInstr >= 1, "tile too small for the waves");
  uint32_t offv[kInstr];   // byte offset of this lane's chunk in the k-tile, or kOOB when the
                           // row / column chunk lies outside the operand
  int32_t klim;            // chunk q exists while k0 + q * kDK < klim (K minus the chunk's
                           // k offset in the k-tile)
  i32x4 reg[kInstr];       // staging registers
  // k offset between consecutive chunks of a lane: K-major chunks of one lane share their
  // k offset (the swizzle key repeats every 16 rows); M/N-major ones step NW*kKPI k-rows
  static constexpr int kDK = KMAJ ? 0 : NW * kKPI;

  // rows_valid: rows of this tile that exist (K-major) or MN elements that exist (MN-major).
  __device__ __forceinline__ void init(int wave, int lane, int rows_valid, int64_t ld_bytes, int K) {
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int blk = q * NW + wave;
      if constexpr (KMAJ) {
        const int row = blk * (1024 / kRowBytes) + lane / kChunks;
        const int c = PAD ? lane % kChunks : (lane % kChunks) ^ kswz(row);
        offv[q] = row < rows_valid ? (uint32_t)(row * ld_bytes + c * 16) : kOOB;
      } else {
        const int krow = blk * kKPI + lane / kCPR;
        const int c = (lane % kCPR) ^ mswz(krow);
        offv[q] = c * (16 / ES) < rows_valid ? (uint32_t)(krow * ld_bytes + c * 16) : kOOB;
      }
    }
    if constexpr (KMAJ && PAD) {
      klim = K - (lane % kChunks) * (16 / ES);
    } else if constexpr (KMAJ) {
      klim = K - (((lane % kChunks) ^ kswz(wave * (1024 / kRowBytes) + lane / kChunks)) * (16 / ES));
    } else {
      klim = K - (wave * kKPI + lane / kCPR);
    }
  }

  // K-major operand with gathered rows: tile row r reads operand row ridx[r] (a row index
  // in [0, nrows); others read as zero), so offsets count from the operand's base, not the
  // tile's (the plan keeps the operand below 2^31 bytes).
  __device__ __forceinline__ void init_gather(int wave, int lane, int rows_valid, int64_t ld_bytes, int K,
                                              const int32_t* ridx, int32_t nrows) {
    static_assert(KMAJ, "gathered rows need a K-major operand");
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int blk = q * NW + wave;
      const int row = blk * (1024 / kRowBytes) + lane / kChunks;
      const int c = PAD ? lane % kChunks : (lane % kChunks) ^ kswz(row);
      const int32_t src = row < rows_valid ? ridx[row] : -1;
      offv[q] = (uint32_t)src < (uint32_t)nrows ? (uint32_t)(src * ld_bytes + c * 16) : kOOB;
    }
    if constexpr (PAD) klim = K - (lane % kChunks) * (16 / ES);
    else klim = K - (((lane % kChunks) ^ kswz(wave * (1024 / kRowBytes) + lane / kChunks)) * (16 / ES));
  }

  // M/N-major operand with gathered k-rows: k-row k of the group reads operand row
  // kidx[k]. The row of each chunk changes with the k-tile, so the loader keeps the index of
  // its chunks' rows for the k-tile it loads next (gidx, fetched one k-tile ahead) and
  // only the column offset (coff) of each chunk.
  int32_t gidx[kInstr];
  uint32_t coff[kInstr];
  int32_t krow0;  // k-row of chunk 0 inside a k-tile; chunk q is krow0 + q * kDK
  __device__ __forceinline__ void init_gather_k(int wave, int lane, int rows_valid, int K) {
    static_assert(!KMAJ, "gathered k-rows need an M/N-major operand");
    krow0 = wave * kKPI + lane / kCPR;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int krow = q * kDK + krow0;
      const int c = (lane % kCPR) ^ mswz(krow);
      coff[q] = c * (16 / ES) < rows_valid ? (uint32_t)(c * 16) : kOOB;
    }
    klim = K - krow0;
  }
  // Operand row indices of chunk Q's k-row in the k-tile at k0 (reads past the group's
  // index range return 0; those chunks are not loaded).
  template <int Q>
  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t irs, int k0) {
    gidx[Q] = __builtin_amdgcn_raw_buffer_load_b32(irs, (k0 + krow0 + Q * kDK) * 4, 0, 0);
  }
  // Global -> registers, chunk Q of the k-tile at k0 whose rows gidx holds; `rows` bounds
  // the operand rows an index may name (others read as zero).
  template <int Q>
  __device__ __forceinline__ void load_gather(__amdgpu_buffer_rsrc_t rs, int k0, uint32_t ld_bytes, uint32_t rows) {
    const bool ok = k0 + Q * kDK < klim && coff[Q] != kOOB && (uint32_t)gidx[Q] < rows;
    reg[Q] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? (uint32_t)gidx[Q] * ld_bytes + coff[Q] : kOOB, 0, 0);
  }

  // Global -> registers, chunk Q of the k-tile starting at element k0 of K. Chunks at
  // k >= K (the K tail, and whole k-tiles past the end) read as zero.
  template <int Q>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int k0) {
    reg[Q] = __builtin_amdgcn_raw_buffer_load_b128(rs, k0 + Q * kDK < klim ? offv[Q] : kOOB, 0, 0);
  }

  // Global -> LDS directly (buffer_load_dwordx4 ... lds), chunk Q: the wave's 64 lanes
  // fill the 1 KB block Q*NW+wave of the tile at `lds` in lane order, the layout the
  // register path writes.
  template <int Q>
  __device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, int k0, GEP_LDS char* lds, int wave) const {
    static_assert(!(KMAJ && PAD), "transfers fill whole 1 KB blocks: no row padding");
#if defined(__HIP_DEVICE_COMPILE__)  // the builtin exists for the gfx950 pass only
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GEP_LDS void*)(lds + (Q * NW + wave) * 1024), 16,
                                             k0 + Q * kDK < klim ? offv[Q] : kOOB, 0, 0, 0);
#else
    (void)rs, (void)k0, (void)lds, (void)wave;
#endif
  }

  // Registers -> LDS (tile base `lds`), chunk Q.
  template <int Q>
  __device__ __forceinline__ void store(GEP_LDS char* lds, int wave, int lane) const {
    if constexpr (KMAJ && PAD)
      *(GEP_LDS i32x4*)(lds + ((Q * NW + wave) * (1024 / kRowBytes) + lane / kChunks) * kPitch +
                        (lane % kChunks) * 16) = reg[Q];
    else
      *(GEP_LDS i32x4*)(lds + (Q * NW + wave) * 1024 + lane * 16) = reg[Q];
  }
};

// LDS reads per fragment (for the scheduling pattern).
template <bool KMAJ, int ES>
constexpr int reads_per_frag() { return KMAJ ? (ES == 2 ? 1 : 2) : 2; }

// Fragment reader: rows [r0, r0 + kBlk) of a tile, MFMA k-step s of the k-tile.
// (16x16 reads: the 16 lanes of a ds_read_b128 phase hold rows {0-3, 8-11} of one chunk and
// rows {4-7, 12-15} of the next, which the K-major key also spreads over 16 distinct slots.)
template <bool KMAJ, int ROWS, class Op, bool PAD>
__device__ __forceinline__ typename Op::Frag read_frag(const GEP_LDS char* tile, int r0, int s, int lane) {
  using Frag = typename Op::Frag;
  constexpr int kB = Op::kBlk;
  if constexpr (KMAJ) {
    const int row = r0 + (lane & (kB - 1));
    const int kg = lane / kB;  // the lane's run of K inside the instruction's K slice
    const int sw = PAD ? 0 : kswz(row);
    const GEP_LDS char* rp = tile + row * (PAD ? kRowBytes + 16 : kRowBytes);
    if constexpr (Op::kES == 2) {
      const int c = s * (64 / kB) + kg;
      return *(const GEP_LDS i32x4*)(rp + ((c ^ sw) << 4));
    } else {
      static_assert(kB == 32, "fp8 fragments are read for the 32x32 form");
      const int c = s * 4 + kg * 2;  // 32 bytes per lane: two chunks
      i32x4 lo = *(const GEP_LDS i32x4*)(rp + ((c ^ sw) << 4));
      i32x4 hi = *(const GEP_LDS i32x4*)(rp + (((c + 1) ^ sw) << 4));
      return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  } else {
    static_assert(Op::kES == 2, "M/N-major operands are 16-bit only");
    static_assert(kB == 32, "M/N-major fragments are read for the 32x32 form");
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
// 0.5 * (1 + tanh(u)) = sigmoid(2u) with u = sqrt(2/pi) * (x + 0.044715 x^3). The
// reciprocal is v_rcp_f32 (1 ulp), far below the bf16/f16 rounding of the result.
template <int ACT>
__device__ __forceinline__ float act_fn(float x) {
  if constexpr (ACT == ACT_RELU) {
    return x > 0.f ? x : 0.f;
  } else if constexpr (ACT == ACT_RELU_SQ) {
    const float r = x > 0.f ? x : 0.f;
    return r * r;
  } else if constexpr (ACT == ACT_GELU_TANH) {
    const float u2 = 1.5957691216057308f * (x + 0.044715f * x * x * x);  // 2u
    return x * __builtin_amdgcn_rcpf(1.f + fast_exp(-u2));
  } else if constexpr (ACT == ACT_SILU) {
    return x * __builtin_amdgcn_rcpf(1.f + fast_exp(-x));
  } else {
    return x;
  }
}

// act'(x) for the activation-backward epilogue (page 6, quack/gemm_dact_sm90.py: dact_fn_map
// pairs each activation with a function of (x, dout) returning (dout * act'(x), act(x)); the
// derivative bodies are not on the pages and follow from the forms above): relu: [x > 0];
// relu_sq: 2 max(x, 0); GELU-tanh x * s with s = sigmoid(2u): s + x s (1 - s) * 2u', where
// 2u' = 2 sqrt(2/pi) (1 + 3 * 0.044715 x^2); SiLU (added here): s + x s (1 - s), s = sigmoid(x).
template <int ACT>
__device__ __forceinline__ float dact_fn(float x) {
  if constexpr (ACT == ACT_RELU) {
    return x > 0.f ? 1.f : 0.f;
  } else if constexpr (ACT == ACT_RELU_SQ) {
    return x > 0.f ? 2.f * x : 0.f;
  } else if constexpr (ACT == ACT_GELU_TANH) {
    const float x2 = x * x;
    const float sg = __builtin_amdgcn_rcpf(1.f + fast_exp(-1.5957691216057308f * (x + 0.044715f * x2 * x)));
    return sg + x * sg * (1.f - sg) * (1.5957691216057308f * (1.f + 0.134145f * x2));
  } else if constexpr (ACT == ACT_SILU) {
    const float sg = __builtin_amdgcn_rcpf(1.f + fast_exp(-x));
    return sg + x * sg * (1.f - sg);
  } else {
    return 1.f;
  }
}

// Four fp32 values as the 8 bytes of 4 bf16 / f16 (round to nearest even).
__device__ __forceinline__ uint2 pack4_16(int dt, const float v[4]) {
  uint2 x;
  if (dt == DT_BF16) {
    __bf16 h[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    __builtin_memcpy(&x, h, 8);
  } else {
    _Float16 h[4] = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    __builtin_memcpy(&x, h, 8);
  }
  return x;
}

// Four fp32 values as the 4 bytes of 4 OCP fp8 codes (e4m3fn or e5m2), round to nearest even,
// saturating: magnitudes past the largest finite value (448 / 57344), infinities included,
// become it; NaN passes the clamp (comparisons with NaN are false) and converts to NaN.
__device__ __forceinline__ uint32_t pack4_8(int dt, const float v[4]) {
  const float mx = dt == DT_E4M3 ? 448.f : 57344.f;
  float c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = v[e] > mx ? mx : (v[e] < -mx ? -mx : v[e]);
  int w;
  if (dt == DT_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], w, true);
  }
  return (uint32_t)w;
}

// Four fp32 values to an output element type (not fp32) at p.
__device__ __forceinline__ void store4(int dt, char* ptr, const float v[4]) {
  if (dt == DT_E4M3 || dt == DT_E5M2) *(uint32_t*)ptr = pack4_8(dt, v);
  else *(uint2*)ptr = pack4_16(dt, v);
}

// Four consecutive 16-bit values (bf16 or f16) to fp32.
__device__ __forceinline__ void unpack4_16(int dt, uint2 x, float v[4]) {
  if (dt == DT_BF16) {
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
  } else {
    _Float16 h[4];
    __builtin_memcpy(h, &x, 8);
    v[0] = (float)h[0]; v[1] = (float)h[1]; v[2] = (float)h[2]; v[3] = (float)h[3];
  }
}

__device__ __forceinline__ int dt_bytes(int dt) {
  return dt == DT_F32 ? 4 : (dt == DT_NONE ? 0 : ((dt == DT_E4M3 || dt == DT_E5M2) ? 1 : 2));
}

// Complete this wave's LDS operations, then synchronise the workgroup. The "memory"
// clobber keeps LDS accesses on their side of it.
// sched_barrier(0) on both sides also keeps register-only instructions (MFMAs) from
// drifting across, so each MFMA step stays one scheduling region.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// As lds_barrier, after this wave's global -> LDS transfers (buffer_load ... lds) have
// landed too: after it, every wave's transfers issued before it are visible.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------------------------
// Tile scheduler: linear tile id -> (m_blk, n_blk) inside one batch / group
// ------------------------------------------------------------------------------------
// Grouped raster over a grid of ta x tb blocks: groups of G blocks along a (the last group
// holds the ta % G left over), a fastest inside a group, then b. Raster along M: a = m;
// along N the roles of M and N are exchanged. fd_Gtb divides by G * tb.
__device__ __forceinline__ void raster(const KParams& p, uint32_t r, uint32_t ta, uint32_t tb, const FastDiv& fd_Gtb,
                                       uint32_t& a, uint32_t& b) {
  const uint32_t G = 1u << p.log2G;
  const uint32_t full = (ta >> p.log2G) << p.log2G;
  if (r < full * tb) {
    uint32_t grp, w;
    fd_divmod(fd_Gtb, r, grp, w);
    a = (grp << p.log2G) + (w & (G - 1));
    b = w >> p.log2G;
  } else {
    const uint32_t tail = ta - full;  // 1 <= tail < G
    // select the constants with static indices (a dynamic index would spill the kernel
    // argument block to scratch)
    FastDiv f = p.fd_tail[1];
#pragma unroll
    for (int w = 2; w < (1 << kMaxGroupLog2); ++w)
      if (tail == (uint32_t)w) f = p.fd_tail[w];
    uint32_t bb, aa;
    fd_divmod(f, r - full * tb, bb, aa);
    a = full + aa;
    b = bb;
  }
}

// Everything the loop needs about one output tile.
struct TileInfo {
  int l, m0, n0, row_end;
  int klen;            // K extent of the tile's problem (varlen-K: of its group)
  int kb;              // varlen-K: the group's first k
  int mb, nb;          // block coordinates inside the batch / group
  const char* a_tile;  // first byte of the tile's A rows (K-major) / columns (M-major)
  const char* b_tile;
  int64_t a_room, b_room;  // bytes from the tile base to the end of the operand
};


// VM: 0 dense batched, 1 varlen-M (cu_seqlens splits the rows), 2 varlen-K (cu_seqlens
// splits K; one output batch per group). GA: A rows gathered through a_idx (varlen-M).
template <int BM, int BN, int OP, int FA, int FB, bool A_K, bool B_K, int VM, int NW, bool DACT = false,
          bool GA = false>
struct GemmKernel {
  static constexpr bool VARLEN = VM == 1;
  static constexpr bool VARK = VM == 2;
  static_assert(!GA || (VARLEN && A_K) || (VARK && !A_K), "gathered A: rows of a K-major A (varlen-M) or k-rows of an M-major A (varlen-K)");
  static constexpr bool GAK = GA && VARK;  // gathered k-rows of A
  // NW wave64s in a 2 x (NW/2) grid over the output tile
  static constexpr int kThreads = NW * 64;
  // MFMA block: 16x16 for the 8-wave kernels (two waves per SIMD, K-major operands), 32x32
  // for the 4-wave ones (whose 256 accumulators must live in AGPRs, where the compiler
  // keeps 32x32 blocks but not 16x16 ones)
  static constexpr int kBlk = NW == 8 ? 16 : 32;
  using Op = Mfma<OP, FA, FB, kBlk>;
  using Frag = typename Op::Frag;
  using Acc = typename Op::Acc;
  static constexpr int kES = Op::kES;
  static constexpr int kBK = kRowBytes / kES;             // K elements per k-tile
  static constexpr int kSteps = kBK / Op::kKStep;          // MFMA k-steps per k-tile (4, 2 or 1)
  static constexpr int kWM = BM / 2, kWN = BN / (NW / 2);  // per-wave output block
  static constexpr int kMI = kWM / kBlk, kNI = kWN / kBlk;  // MFMA blocks per wave
  // kDMA: k-tiles go global -> LDS directly (buffer_load ... lds; with 4 waves all chunks of
  // k-tile kt+2 issued in the last MFMA step of k-tile kt); else through the staging registers
  // over the first kWriteSteps steps. Measured: direct transfers win for fp8 (they free the
  // staging registers, which fp8's 32-byte fragments need) and for 16-bit operands with
  // 8 waves (the staging registers do not fit next to two waves' accumulators); with 4
  // waves they lose for 16-bit operands (batched M/N-major -30%).
  static constexpr bool kDMA = kES == 1 || NW == 8;
  // Padded K-major rows (PAD) cost the register path two-way bank conflicts on its LDS
  // writes: measured 3% slower than the XOR swizzle with 4 waves. They only pay where
  // the per-step address registers of the swizzle do not fit (8 waves).
  static constexpr bool kPadRows = !kDMA && NW == 8;
  using LA = TileLoader<BM, A_K, kES, NW, kPadRows>;
  using LB = TileLoader<BN, B_K, kES, NW, kPadRows>;
  static constexpr int kABytes = LA::kTileBytes, kBBytes = LB::kTileBytes;
  // Ring layout [A stage 0 | A stage 1 | B stage 0 | B stage 1]: a stage is named by its A
  // tile (at s * kABytes) and its B tile sits kBOff further. The offsets between stages and
  // fragments then fit the 16-bit immediate of the LDS instructions, so one address
  // register per (k-step, operand) serves both stages and every fragment.
  static constexpr int kStageBytes = kABytes > kBBytes ? kABytes : kBBytes;  // stage s at s * kStageBytes
  static constexpr int kBOff = 2 * kStageBytes;
  static constexpr int kLdsBytes = 4 * kStageBytes;
  // varlen group table (tile offsets of the groups, scan partials) past the ring
  static constexpr int kVarlenLds = (kMaxVarlenGroups + 1 + kThreads + 1) * 4;  // (+1: the validity flag)
  static constexpr int kSlotBytes = 16;  // dynamic schedule: next queue position
  static constexpr int kFrags = kMI + kNI;
  static constexpr int kMfmaPerStep = kMI * kNI;
  static constexpr int kRA = reads_per_frag<A_K, kES>(), kRB = reads_per_frag<B_K, kES>();
  // register chunks of one k-tile, written to LDS (and reloaded) over the first kWriteSteps
  // MFMA steps, kCPF chunks next to each fragment read
  static constexpr int kChunksPerKt = LA::kInstr + LB::kInstr;
  static constexpr int kWriteSteps = kDMA ? 1 : (kSteps >= 4 ? 2 : 1);
  static constexpr int kChunksPerStep = kChunksPerKt / kWriteSteps;
  // fragment slot f carries MFMAs [mlo(f), mlo(f+1)) and register chunks [clo(f), clo(f+1))
  static constexpr int mlo(int f) { return f * kMfmaPerStep / kFrags; }
  static constexpr int clo(int f) { return f * kChunksPerStep / kFrags; }
  static_assert(kSteps % 2 == 0 || (NW == 8 && kSteps == 1), "a k-tile ends on fragment buffer 0");
  static_assert(kChunksPerKt % kWriteSteps == 0, "register chunks must spread evenly over the write steps");
  static_assert(kMfmaPerStep >= kFrags, "every fragment slot needs an MFMA");

  // ---- scheduling hints: one slot per fragment, each carrying its MFMAs, the fragment's
  // LDS reads and (WR) its register chunks' LDS writes and global loads, in that order. Program order
  // already interleaves the memory operations the same way (the compiler keeps LDS reads
  // and writes it cannot prove disjoint in program order). The builtin needs literal
  // arguments, hence the compile-time recursion.
  template <bool WR, int F = 0>
  static __device__ __forceinline__ void sched_step() {
    if constexpr (F < kFrags) {
      constexpr int nm = mlo(F + 1) - mlo(F), nc = clo(F + 1) - clo(F);
      __builtin_amdgcn_sched_group_barrier(0x008, nm, 0);                       // MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, F < kMI ? kRA : kRB, 0);      // LDS reads
      if constexpr (WR && nc > 0) {
        if constexpr (!kDMA) __builtin_amdgcn_sched_group_barrier(0x200, nc, 0);  // LDS writes
        __builtin_amdgcn_sched_group_barrier(0x020, nc, 0);                       // VMEM loads
      }
      sched_step<WR, F + 1>();
    }
  }

  static __device__ __forceinline__ void mma_step(Acc (&acc)[kMI][kNI], const Frag (&fa)[kMI],
                                                  const Frag (&fb)[kNI]) {
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < kNI; ++j) acc[i][j] = Op::mma(fb[j], fa[i], acc[i][j]);
  }

  static __device__ __forceinline__ void read_all(Frag (&fa)[kMI], Frag (&fb)[kNI], const GEP_LDS char* st, int s,
                                                  int wm0, int wn0, int lane) {
#pragma unroll
    for (int i = 0; i < kMI; ++i) fa[i] = read_frag<A_K, BM, Op, kPadRows>(st, wm0 + i * kBlk, s, lane);
#pragma unroll
    for (int j = 0; j < kNI; ++j) fb[j] = read_frag<B_K, BN, Op, kPadRows>(st + kBOff, wn0 + j * kBlk, s, lane);
  }

  // Work item u of this launch -> output tile. Tiles are numbered in the map's tiling (MT x
  // (BN * MT / BM)): BM itself, or twice BM for the quarter tiles of a split tail (p.tail == 2,
  // item u = quarter (u & 3) of map tile t_lo + (u >> 2); quarter q covers rows
  // (q & 1) * BM and columns (q >> 1) * BN of it, and may lie wholly outside the output).
  static __device__ __forceinline__ TileInfo decode(const KParams& p, int u, const int32_t* gstart, int t_lo) {
    const bool quarter = BM == 128 && p.tail == 2;  // (split tails run 128x128 kernels)
    const int MT = quarter ? 2 * BM : BM, NT = quarter ? 2 * BN : BN;
    const int t = quarter ? t_lo + (u >> 2) : u;
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
      const uint32_t tmg = (uint32_t)((ti.row_end - row_base + MT - 1) / MT);
      raster(p, (uint32_t)(t - gstart[lo]), tmg, (uint32_t)p.tn, p.fd_Gtn, mb, nb);
    } else {
      uint32_t ll, r;
      fd_divmod(p.fd_mn, (uint32_t)t, ll, r);
      if (p.raster_n) raster(p, r, (uint32_t)p.tn, (uint32_t)p.tm, p.fd_Gtm, nb, mb);
      else raster(p, r, (uint32_t)p.tm, (uint32_t)p.tn, p.fd_Gtn, mb, nb);
      ti.l = (int)ll;
      row_base = 0;
      ti.row_end = p.M;
    }
    ti.mb = (int)mb;
    ti.nb = (int)nb;
    ti.m0 = row_base + (int)mb * MT;
    ti.n0 = (int)nb * NT;
    if (quarter) {
      ti.m0 += (u & 1) * BM;
      ti.n0 += ((u >> 1) & 1) * BN;
    }
    // varlen-K: the group's K range [cu[l], cu[l+1]) offsets A and B along K
    int64_t kb = 0;
    ti.klen = p.K;
    if constexpr (VARK) {
      kb = p.cu_seqlens[ti.l];
      ti.klen = p.cu_seqlens[ti.l + 1] - (int)kb;
    }
    const int64_t a_lb = (VARLEN || VARK) ? 0 : (int64_t)ti.l * p.sa;
    const int64_t b_lb = VARK ? 0 : (int64_t)ti.l * p.sb;
    // gathered A: the loader's offsets count from A's base (rows come from a_idx), or for
    // gathered k-rows from the tile's first column
    ti.kb = (int)kb;
    const int64_t a_off =
        (GA && VARLEN) ? 0
                       : (GAK ? (int64_t)ti.m0 * kES
                              : (a_lb + (A_K ? (int64_t)ti.m0 * p.lda + kb : kb * p.lda + (int64_t)ti.m0)) * kES);
    const int64_t b_off = (b_lb + (B_K ? (int64_t)ti.n0 * p.ldb + kb : kb * p.ldb + (int64_t)ti.n0)) * kES;
    ti.a_tile = (const char*)p.A + a_off;
    ti.b_tile = (const char*)p.B + b_off;
    ti.a_room = p.a_bytes - a_off;
    ti.b_room = p.b_bytes - b_off;
    // Everything above is the same in every lane, but grouped tiles derive it from LDS and
    // global loads (the group table, cu_seqlens), whose results the compiler keeps per lane:
    // the buffer descriptors of every k-tile were then rebuilt with 64-bit vector adds and
    // readfirstlane in the main loop. Stating uniformity here keeps the tile in SGPRs.
    if constexpr (VARLEN || VARK) {
      ti.l = uni(ti.l);
      ti.m0 = uni(ti.m0);
      ti.n0 = uni(ti.n0);
      ti.row_end = uni(ti.row_end);
      ti.klen = uni(ti.klen);
      ti.kb = uni(ti.kb);
      ti.mb = uni(ti.mb);
      ti.nb = uni(ti.nb);
      ti.a_tile = (const char*)uni64((int64_t)ti.a_tile);
      ti.b_tile = (const char*)uni64((int64_t)ti.b_tile);
      ti.a_room = uni64(ti.a_room);
      ti.b_room = uni64(ti.b_room);
    }
    return ti;
  }
  static __device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
  static __device__ __forceinline__ int64_t uni64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  }

  // Buffer resources of k-tile j of the current tile (k-tiles past the end read as zero).
  struct KtSrc {
    __amdgpu_buffer_rsrc_t a, b;
    int k0;
    // gathered k-rows only: the group's index range, A's leading dimension in bytes and the
    // number of rows of A an index may name
    __amdgpu_buffer_rsrc_t ia;
    uint32_t ld, rows;
  };
  static __device__ __forceinline__ KtSrc kt_src(const KParams& p, const TileInfo& ti, int j) {
    // (gathered k-rows: one resource for all k-tiles, the rows come from the index)
    const int64_t a_step = GAK ? 0 : (A_K ? (int64_t)kRowBytes : (int64_t)kBK * p.lda * kES);
    const int64_t b_step = B_K ? (int64_t)kRowBytes : (int64_t)kBK * p.ldb * kES;
    const int64_t ao = (int64_t)j * a_step, bo = (int64_t)j * b_step;
    KtSrc r;
    r.a = make_rsrc(ti.a_tile + ao, ti.a_room - ao);
    r.b = make_rsrc(ti.b_tile + bo, ti.b_room - bo);
    r.k0 = j * kBK;
    if constexpr (GAK) {
      r.ia = make_rsrc(p.a_idx + ti.kb, (int64_t)ti.klen * 4);
      r.ld = (uint32_t)(p.lda * kES);
      r.rows = (uint32_t)p.a_rows;
    }
    return r;
  }

  // Register chunk C (A chunks first, then B): write it to the LDS stage `wr`, then reload it
  // from the k-tile described by `src`.
  template <int C>
  static __device__ __forceinline__ void cycle_chunk(LA& la, LB& lb, GEP_LDS char* wr, const KtSrc& src, int wave,
                                                     int lane) {
    if constexpr (C < LA::kInstr) {
      la.template store<C>(wr, wave, lane);
      if constexpr (GAK) {
        la.template load_gather<C>(src.a, src.k0, src.ld, src.rows);
        la.template fetch<C>(src.ia, src.k0 + kBK);
      } else {
        la.template load<C>(src.a, src.k0);
      }
    } else {
      lb.template store<C - LA::kInstr>(wr + kBOff, wave, lane);
      lb.template load<C - LA::kInstr>(src.b, src.k0);
    }
  }
  template <int C0, int N>
  static __device__ __forceinline__ void cycle_chunks(LA& la, LB& lb, GEP_LDS char* wr, const KtSrc& src, int wave,
                                                      int lane) {
    if constexpr (N > 0) {
      cycle_chunk<C0>(la, lb, wr, src, wave, lane);
      cycle_chunks<C0 + 1, N - 1>(la, lb, wr, src, wave, lane);
    }
  }
  // Gathered k-rows: the row indices of a tile's k-tile 0.
  template <int C = 0>
  static __device__ __forceinline__ void fetch_all(LA& la, __amdgpu_buffer_rsrc_t irs) {
    if constexpr (C < LA::kInstr) {
      la.template fetch<C>(irs, 0);
      fetch_all<C + 1>(la, irs);
    }
  }

  // Only the loads (the tile's first k-tile).
  template <int C = 0>
  static __device__ __forceinline__ void load_all(LA& la, LB& lb, const KtSrc& src) {
    if constexpr (C < kChunksPerKt) {
      if constexpr (C < LA::kInstr) {
        if constexpr (GAK) {
          la.template load_gather<C>(src.a, src.k0, src.ld, src.rows);
          la.template fetch<C>(src.ia, src.k0 + kBK);
        } else {
          la.template load<C>(src.a, src.k0);
        }
      } else {
        lb.template load<C - LA::kInstr>(src.b, src.k0);
      }
      load_all<C + 1>(la, lb, src);
    }
  }

  // Global -> LDS transfers of register-chunk positions [C0, C0 + N) of the k-tile `src`
  // into the stage at `st`.
  template <int C0, int N>
  static __device__ __forceinline__ void dma_chunks(const LA& la, const LB& lb, GEP_LDS char* st, const KtSrc& src,
                                                    int wave) {
    if constexpr (N > 0) {
      if constexpr (C0 < LA::kInstr) la.template dma<C0>(src.a, src.k0, st, wave);
      else lb.template dma<C0 - LA::kInstr>(src.b, src.k0, st + kBOff, wave);
      dma_chunks<C0 + 1, N - 1>(la, lb, st, src, wave);
    }
  }

  // Fragment slot F of a step: read fragment F (A fragments first) of k-step s into `fa`/
  // `fb`, then (WR) cycle register chunks C0 + [clo(F), clo(F+1)).
  template <bool WR, int C0, int F = 0>
  static __device__ __forceinline__ void slots(Frag (&fa)[kMI], Frag (&fb)[kNI], const GEP_LDS char* rd, int s,
                                               int wm0, int wn0, LA& la, LB& lb, GEP_LDS char* wr,
                                               const KtSrc& src, int wave, int lane) {
    if constexpr (F < kFrags) {
      if constexpr (F < kMI) fa[F] = read_frag<A_K, BM, Op, kPadRows>(rd, wm0 + F * kBlk, s, lane);
      else fb[F - kMI] = read_frag<B_K, BN, Op, kPadRows>(rd + kBOff, wn0 + (F - kMI) * kBlk, s, lane);
      if constexpr (WR) {
        if constexpr (kDMA) dma_chunks<C0 + clo(F), clo(F + 1) - clo(F)>(la, lb, wr, src, wave);
        else cycle_chunks<C0 + clo(F), clo(F + 1) - clo(F)>(la, lb, wr, src, wave, lane);
      }
      slots<WR, C0, F + 1>(fa, fb, rd, s, wm0, wn0, la, lb, wr, src, wave, lane);
    }
  }

  // register chunk / transfer range of slot i of an 8-wave step
  static constexpr int rlo(int i) { return i * kChunksPerStep / kMI; }

  // ---- column halves (kRoll3; 16x16 blocks, kMI = 2 kNI): one A and one B buffer, 12
  // fragments live (double-buffered B with rolling A, the 32x32 scheme, needs 16 and spills
  // next to two waves' accumulators). Slots 0 .. kNI-1 run column I over the first kH block
  // rows, and after the last of them the A fragments of those rows are re-read; slots kNI + J
  // run column J over the other kH rows and re-read B fragment J; the A fragments of those
  // rows are re-read at the end. Every fragment of the next k-step is read at least kNI * kH
  // MFMAs before its first use. (Rows first, then columns, left the last B fragment read
  // three MFMAs before its use.)
  static constexpr bool kRoll3 = NW == 8 && kBlk == 16 && kSteps >= 2;
  // transfer placement over the slots of a step, DM 0: spread (rlo); 1: the second half of a
  // k-tile's chunks, one per slot in slots 0 .. kNI-1; 2: the first half, one per slot in
  // slots kNI .. kMI-1
  static constexpr int dlo(int dm, int i) {
    return dm == 0 ? rlo(i) : (dm == 1 ? kChunksPerKt / 2 + (i < kNI ? i : kNI) : (i < kNI ? 0 : i - kNI));
  }
  static constexpr int dn(int dm, int i) { return dlo(dm, i + 1) - dlo(dm, i); }
  static_assert(!kRoll3 || kChunksPerKt == 2 * kNI, "8 waves: a k-tile's transfers fill two half steps, one per slot");
  static constexpr int kH = kMI / 2;
  template <bool WR, int I, int E, int DM = 0, bool SKIPA = false>
  static __device__ __forceinline__ void sched_roll3() {
    if constexpr (I < E) {
      constexpr int nc = dn(DM, I);
      constexpr int nr = I < kNI ? ((I == kNI - 1 && !SKIPA) ? kH * kRA : 0) : (kRB + (I == kMI - 1 ? kH * kRA : 0));
      __builtin_amdgcn_sched_group_barrier(0x008, kH, 0);                         // MFMAs
      if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);  // LDS reads
      if constexpr (WR && nc > 0) __builtin_amdgcn_sched_group_barrier(0x020, nc, 0);  // transfers
      sched_roll3<WR, I + 1, E, DM, SKIPA>();
    }
  }
  // slots [I, E) of a step; oa / ob: this lane's fragment offsets of the k-step read, A and B;
  // MM = false: only the slots' transfers (a wave whose rows all lie past the output); DM: the
  // transfer placement (dlo); SKIPA: slot kNI-1 leaves the re-read of its A fragments to the
  // caller
  template <bool WR, int C0, int I, int E, bool MM = true, int DM = 0, bool SKIPA = false>
  static __device__ __forceinline__ void roll3_slots(Acc (&acc)[kMI][kNI], Frag (&fa)[kMI], Frag (&fb)[kNI],
                                                     const GEP_LDS char* rd, int oa, int ob, LA& la, LB& lb,
                                                     GEP_LDS char* wr, const KtSrc& src, int wave) {
    static_assert(kMI == 2 * kNI && kDMA, "two halves of kNI block rows, global -> LDS transfers");
    if constexpr (I < E) {
      if constexpr (!MM) {
      } else if constexpr (I < kNI) {
#pragma unroll
        for (int i = 0; i < kH; ++i) acc[i][I] = Op::mma(fb[I], fa[i], acc[i][I]);
        if constexpr (I == kNI - 1 && !SKIPA) {
#pragma unroll
          for (int i = 0; i < kH; ++i) fa[i] = *(const GEP_LDS Frag*)(rd + oa + i * kBlk * kRowBytes);
        }
      } else {
        constexpr int J = I - kNI;
#pragma unroll
        for (int i = kH; i < kMI; ++i) acc[i][J] = Op::mma(fb[J], fa[i], acc[i][J]);
        fb[J] = *(const GEP_LDS Frag*)(rd + ob + J * kBlk * kRowBytes);
        if constexpr (I == kMI - 1) {
#pragma unroll
          for (int i = kH; i < kMI; ++i) fa[i] = *(const GEP_LDS Frag*)(rd + oa + i * kBlk * kRowBytes);
        }
      }
      if constexpr (WR) dma_chunks<C0 + dlo(DM, I), dn(DM, I)>(la, lb, wr, src, wave);
      roll3_slots<WR, C0, I + 1, E, MM, DM, SKIPA>(acc, fa, fb, rd, oa, ob, la, lb, wr, src, wave);
    }
  }
  // Byte offset in a stage of this lane's chunk of the 16x16 fragment of rows r0 + [0, 16),
  // k-step s (K-major, XOR-swizzled rows).
  static __device__ __forceinline__ int frag_off16(int r0, int s, int lane) {
    const int row = r0 + (lane & 15);
    return row * kRowBytes + (((s * (64 / kBlk) + (lane >> 4)) ^ kswz(row)) << 4);
  }

  // One MFMA step: MFMAs on fragment buffer CUR while the fragments of k-step s of the stage
  // at `rd` are read into the other buffer; WR: register chunks [C0, C0 + kChunksPerStep)
  // are written to the stage at `wr` and reloaded from `src` (global -> LDS: issued to `wr`).
  // (kRoll3: one fragment buffer, the 0 of each pair.)
  template <int CUR, bool WR, int C0, bool MM = true, int DM = 0>
  static __device__ __forceinline__ void step(Acc (&acc)[kMI][kNI], Frag (&fa)[2][kMI], Frag (&fb)[2][kNI],
                                              const GEP_LDS char* rd, int s, LA& la, LB& lb, GEP_LDS char* wr,
                                              const KtSrc& src, int wave, int lane, int wm0, int wn0) {
    if constexpr (!MM) {
      static_assert(kRoll3, "only the 8-wave steps skip their MFMAs");
      roll3_slots<WR, C0, 0, kMI, false, DM>(acc, fa[0], fb[0], rd, 0, 0, la, lb, wr, src, wave);
    } else if constexpr (kRoll3) {
      // The fragment offsets of k-step s are made opaque: the stage, fragment and (for B)
      // operand offsets then fold into the 16-bit immediates of the reads, one address
      // register per operand and k-step. (Folded by the compiler, B's offsets past 64 KB took
      // a register per fragment and stage.)
      int oa = frag_off16(wm0, s, lane), ob = kBOff + frag_off16(wn0, s, lane);
      asm volatile("" : "+v"(oa), "+v"(ob));
      // Wave priority 1 for the first half of the step, 0 for the second: of the two waves
      // sharing a SIMD, the one ahead yields to the one behind, which otherwise (the issue
      // arbiter favours the older wave) finishes each k-tile alone while its partner waits at
      // the barrier (8192^3 bf16: the older waves' barrier time per tile 152 K -> 99 K cycles,
      // +2.5% throughput).
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      roll3_slots<WR, C0, 0, kNI, true, DM>(acc, fa[0], fb[0], rd, oa, ob, la, lb, wr, src, wave);
      sched_roll3<WR, 0, kNI, DM>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      roll3_slots<WR, C0, kNI, kMI, true, DM>(acc, fa[0], fb[0], rd, oa, ob, la, lb, wr, src, wave);
      sched_roll3<WR, kNI, kMI, DM>();
    } else {
      slots<WR, C0>(fa[CUR ^ 1], fb[CUR ^ 1], rd, s, wm0, wn0, la, lb, wr, src, wave, lane);
      mma_step(acc, fa[CUR], fb[CUR]);
      sched_step<WR>();
    }
  }

  // The last step of an 8-wave k-tile with the k-tile barrier after its first half: that half
  // runs on fragments read before, the barrier comes before the first read of stage `rd` (the
  // next k-tile: the A fragments of the first block rows, taken out of slot kNI-1), and the
  // second half issues the first half of k-tile kt+2's transfers into `wr`, whose last reads
  // the barrier ended. MM = false: the barrier and the transfers only.
  template <bool MM>
  static __device__ __forceinline__ void last_step_midbar(Acc (&acc)[kMI][kNI], Frag (&fa)[2][kMI],
                                                          Frag (&fb)[2][kNI], const GEP_LDS char* rd, LA& la, LB& lb,
                                                          GEP_LDS char* wr, const KtSrc& src, int wave, int lane,
                                                          int wm0, int wn0) {
    int oa = frag_off16(wm0, 0, lane), ob = kBOff + frag_off16(wn0, 0, lane);
    asm volatile("" : "+v"(oa), "+v"(ob));
    if constexpr (MM) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      roll3_slots<false, 0, 0, kNI, true, 0, true>(acc, fa[0], fb[0], rd, oa, ob, la, lb, wr, src, wave);
      sched_roll3<false, 0, kNI, 0, true>();
    }
    dma_barrier();
    if constexpr (MM) {
#pragma unroll
      for (int i = 0; i < kH; ++i) fa[0][i] = *(const GEP_LDS Frag*)(rd + oa + i * kBlk * kRowBytes);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    roll3_slots<true, 0, kNI, kMI, MM, 2>(acc, fa[0], fb[0], rd, oa, ob, la, lb, wr, src, wave);
    if constexpr (MM) sched_roll3<true, kNI, kMI, 2>();
  }

  // ---- 8 waves, one k-step per k-tile (fp8: a 16x16x128 instruction takes all 128 bytes of
  // K of a k-tile). A fragment is 8 registers, too many for the 12 fragments of the column
  // halves next to the 128 accumulators; this loop keeps 6: the 4 B fragments and a ring of 2
  // A fragments (block row r in register r & 1). The 32 MFMAs run row by row, position p
  // being block row p / kNI, column p % kNI. The A fragment of row r >= 2 is read right after
  // the last MFMA of row r-2 (row 1 after the first MFMA), 5 MFMAs before its first use. The
  // k-tile barrier precedes the last row: by then every wave has read its last fragment of
  // this k-tile's stage. After it, the first MFMA of the last row is followed by the read of
  // the next k-tile's row-0 A fragment, and each MFMA by that k-tile's B fragment of its
  // column: 4 MFMAs before their first use. A k-tile's 8 transfers go out in two halves: one
  // per MFMA of the last row of the k-tile two before it (into the stage its barrier freed),
  // and one per two MFMAs over the first two rows of the k-tile before it, landing before that
  // k-tile's barrier. Positions [0, kPrioP) run at wave priority 1.
  static constexpr bool kStream = NW == 8 && kSteps == 1;
  static constexpr int kLastP = kMfmaPerStep - kNI;  // first position of the last block row
  static constexpr int kHalfKt = kChunksPerKt / 2;
  static constexpr int kPrioP = kLastP / 2;
  static_assert(!kStream || (kMI >= 4 && kHalfKt == kNI && 2 * kHalfKt <= kLastP),
                "one transfer per MFMA of the last row, one per two over the first rows");
  // rows of this k-tile whose A fragments are read after position p (bit r)
  static constexpr int s_rd_cur(int p) {
    int m = 0;
    for (int r = 1; r < kMI; ++r) m |= ((r == 1 ? 0 : (r - 1) * kNI - 1) == p) << r;
    return m;
  }
  static constexpr int s_nreads(int p) { return 2 * (popc(s_rd_cur(p)) + (p == kLastP) + (p >= kLastP)); }
  static constexpr int popc(int m) { return m ? (m & 1) + popc(m >> 1) : 0; }
  static constexpr bool s_head_dma(int p) { return p % 2 == 0 && p < 2 * kHalfKt; }

  // a fragment from its two 16-byte halves (lane offsets o0, o1 from the block-row base)
  static __device__ __forceinline__ Frag s_frag(const GEP_LDS char* base, int o0, int o1) {
    const i32x4 lo = *(const GEP_LDS i32x4*)(base + o0);
    const i32x4 hi = *(const GEP_LDS i32x4*)(base + o1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  template <int M, int R = 0>
  static __device__ __forceinline__ void s_read_rows(Frag (&fa)[kMI], const GEP_LDS char* st, int o0, int o1) {
    if constexpr (R < kMI) {
      if constexpr ((M >> R) & 1) fa[R & 1] = s_frag(st + R * kBlk * kRowBytes, o0, o1);
      s_read_rows<M, R + 1>(fa, st, o0, o1);
    }
  }
  // Positions [P, E) of k-tile kt: stage `cur` holds kt and receives the last row's transfers
  // of kt+2 (from s2); stage `nxt` holds kt+1, whose second half the first rows issue (from
  // s1). MM = false: the transfers only.
  template <bool MM, int P, int E>
  static __device__ __forceinline__ void s_run(Acc (&acc)[kMI][kNI], Frag (&fa)[kMI], Frag (&fb)[kNI],
                                               GEP_LDS char* cur, GEP_LDS char* nxt, int oa0, int oa1, int ob0,
                                               int ob1, LA& la, LB& lb, const KtSrc& s1, const KtSrc& s2, int wave) {
    if constexpr (P < E) {
      if constexpr (MM) {
        constexpr int r = P / kNI, c = P % kNI;
        acc[r][c] = Op::mma(fb[c], fa[r & 1], acc[r][c]);
        s_read_rows<s_rd_cur(P)>(fa, cur, oa0, oa1);
        if constexpr (P == kLastP) fa[0] = s_frag(nxt, oa0, oa1);
        if constexpr (P >= kLastP) fb[P - kLastP] = s_frag(nxt + (P - kLastP) * kBlk * kRowBytes, ob0, ob1);
      }
      if constexpr (s_head_dma(P)) dma_chunks<kHalfKt + P / 2, 1>(la, lb, nxt, s1, wave);
      if constexpr (P >= kLastP) dma_chunks<P - kLastP, 1>(la, lb, cur, s2, wave);
      s_run<MM, P + 1, E>(acc, fa, fb, cur, nxt, oa0, oa1, ob0, ob1, la, lb, s1, s2, wave);
    }
  }
  template <int P, int E>
  static __device__ __forceinline__ void s_sched() {
    if constexpr (P < E) {
      constexpr int nt = s_head_dma(P) + (P >= kLastP);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                // MFMA
      if constexpr (s_nreads(P) > 0) __builtin_amdgcn_sched_group_barrier(0x100, s_nreads(P), 0);  // LDS reads
      if constexpr (nt > 0) __builtin_amdgcn_sched_group_barrier(0x020, nt, 0);                  // transfers
      s_sched<P + 1, E>();
    }
  }
  // Lane offsets of the two 16-byte halves of a lane's fragment in block row r0: row
  // r0 + (l % 16), K chunks l / 16 and l / 16 + 4. A and B take the same K assignment, so the
  // MFMA sums the same products; chunks l / 16 + {0, 4} (rather than 2 (l / 16) + {0, 1})
  // keep the 16 rows of a read phase on distinct banks.
  static __device__ __forceinline__ void s_offs(int r0, int lane, int& o0, int& o1) {
    const int row = r0 + (lane & 15);
    o0 = row * kRowBytes + (((lane >> 4) ^ kswz(row)) << 4);
    o1 = o0 ^ 64;
  }
  // the fragments a tile's first k-tile starts with: all of B, and A's block row 0
  static __device__ __forceinline__ void s_first(Frag (&fa)[kMI], Frag (&fb)[kNI], const GEP_LDS char* st, int lane,
                                                 int wm0, int wn0) {
    int oa0, oa1, ob0, ob1;
    s_offs(wm0, lane, oa0, oa1);
    s_offs(wn0, lane, ob0, ob1);
    fa[0] = s_frag(st, oa0, oa1);
#pragma unroll
    for (int c = 0; c < kNI; ++c) fb[c] = s_frag(st + kBOff + c * kBlk * kRowBytes, ob0, ob1);
  }
  template <bool MM>
  static __device__ __forceinline__ void s_ktile(Acc (&acc)[kMI][kNI], Frag (&fa)[kMI], Frag (&fb)[kNI],
                                                 GEP_LDS char* cur, GEP_LDS char* nxt, LA& la, LB& lb, const KtSrc& s1,
                                                 const KtSrc& s2, int wave, int lane, int wm0, int wn0) {
    // opaque offsets: stage, block-row and (B) operand offsets fold into the reads' immediates
    int oa0, oa1, ob0, ob1;
    s_offs(wm0, lane, oa0, oa1);
    s_offs(wn0, lane, ob0, ob1);
    ob0 += kBOff;
    ob1 += kBOff;
    asm volatile("" : "+v"(oa0), "+v"(oa1), "+v"(ob0), "+v"(ob1));
    if constexpr (MM) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      s_run<true, 0, kPrioP>(acc, fa, fb, cur, nxt, oa0, oa1, ob0, ob1, la, lb, s1, s2, wave);
      s_sched<0, kPrioP>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      s_run<true, kPrioP, kLastP>(acc, fa, fb, cur, nxt, oa0, oa1, ob0, ob1, la, lb, s1, s2, wave);
      s_sched<kPrioP, kLastP>();
      dma_barrier();
      s_run<true, kLastP, kMfmaPerStep>(acc, fa, fb, cur, nxt, oa0, oa1, ob0, ob1, la, lb, s1, s2, wave);
      s_sched<kLastP, kMfmaPerStep>();
      __builtin_amdgcn_sched_barrier(0);
    } else {
      s_run<false, 0, kLastP>(acc, fa, fb, cur, nxt, oa0, oa1, ob0, ob1, la, lb, s1, s2, wave);
      dma_barrier();
      s_run<false, kLastP, kMfmaPerStep>(acc, fa, fb, cur, nxt, oa0, oa1, ob0, ob1, la, lb, s1, s2, wave);
    }
  }

  // Steps S .. kSteps-2 of a k-tile (stage `cur`): step S runs the MFMAs of k-step S on
  // buffer S & 1 and reads k-step S+1; the first kWriteSteps steps also cycle their share of
  // the register chunks through the stage `nxt`.
  template <int S = 0, bool WRITES = true>
  static __device__ __forceinline__ void first_steps(Acc (&acc)[kMI][kNI], Frag (&fa)[2][kMI],
                                                     Frag (&fb)[2][kNI], const GEP_LDS char* cur, LA& la, LB& lb,
                                                     GEP_LDS char* nxt, const KtSrc& src, int wave, int lane,
                                                     int wm0, int wn0) {
    if constexpr (S + 1 < kSteps) {
      step<S & 1, (WRITES && S < kWriteSteps), S * kChunksPerStep>(acc, fa, fb, cur, S + 1, la, lb, nxt, src,
                                                                   wave, lane, wm0, wn0);
      first_steps<S + 1, WRITES>(acc, fa, fb, cur, la, lb, nxt, src, wave, lane, wm0, wn0);
    }
  }

  // Steps S .. E-1 of a k-tile without register chunk writes (the global -> LDS path).
  template <int S, int E, bool MM = true>
  static __device__ __forceinline__ void first_steps_range(Acc (&acc)[kMI][kNI], Frag (&fa)[2][kMI],
                                                           Frag (&fb)[2][kNI], const GEP_LDS char* cur, LA& la, LB& lb,
                                                           GEP_LDS char* nxt, const KtSrc& src, int wave, int lane,
                                                           int wm0, int wn0) {
    if constexpr (S < E) {
      step<S & 1, false, S * kChunksPerStep, MM>(acc, fa, fb, cur, S + 1, la, lb, nxt, src, wave, lane, wm0, wn0);
      first_steps_range<S + 1, E, MM>(acc, fa, fb, cur, la, lb, nxt, src, wave, lane, wm0, wn0);
    }
  }

  // k-tile kt, held in stage PAR (= kt & 1); fragments (kt, 0) are in buffer 0 and the
  // staging registers hold k-tile kt+1. The first kWriteSteps steps write kt+1 into the
  // other stage (free: its last reads were issued before the previous barrier) and reload
  // the registers with kt+2. The barrier (after lgkmcnt(0): this wave's writes landed and
  // its reads of stage PAR returned) comes before the last step, which reads (kt+1, 0).
  // MM = false: the k-tile's transfers and barrier only (the 8-wave kernels' waves whose rows all
  // lie past the output: they keep the workgroup's transfers and barriers, and leave their SIMD's
  // MFMA pipe to their partner wave)
  template <int PAR, bool MM = true>
  static __device__ __forceinline__ void ktile(const KParams& p, const TileInfo& ti, LA& la, LB& lb,
                                               GEP_LDS char* smem, Acc (&acc)[kMI][kNI], Frag (&fa)[2][kMI],
                                               Frag (&fb)[2][kNI], int kt, int wave, int lane, int wm0, int wn0) {
    GEP_LDS char* cur = smem + PAR * kStageBytes;
    GEP_LDS char* nxt = smem + (PAR ^ 1) * kStageBytes;
    const KtSrc src = kt_src(p, ti, kt + 2);
    if constexpr (kStream) {
      s_ktile<MM>(acc, fa[0], fb[0], cur, nxt, la, lb, kt_src(p, ti, kt + 1), src, wave, lane, wm0, wn0);
    } else if constexpr (kRoll3) {
      // 8 waves, two steps per k-tile. Step 0 reads the fragments of step 1 from stage PAR and
      // issues the second half of k-tile kt+1's transfers into stage PAR^1, which received the
      // first half in the second half of k-tile kt-1's last step. The barrier sits in the middle
      // of the last step, before its first read of stage PAR^1; the step's second half then
      // issues the first half of k-tile kt+2's transfers into stage PAR. Each half has at least
      // one step to land, the address path carries transfers in both steps, and the waves of
      // a SIMD meet at the barrier half a step later than with the barrier before the last
      // step (8192^3 bf16 +2.5-3%, same binary, bit-identical results).
      step<0, true, 0, MM, 1>(acc, fa, fb, cur, 1, la, lb, nxt, kt_src(p, ti, kt + 1), wave, lane, wm0, wn0);
      last_step_midbar<MM>(acc, fa, fb, nxt, la, lb, cur, src, wave, lane, wm0, wn0);
    } else if constexpr (kDMA) {
      // fp8: stage PAR^1 (k-tile kt+1) received its transfers in the last step of k-tile kt-1
      // and nobody reads it before this k-tile's barrier, which waits for them; k-tile kt+2
      // goes into stage PAR once its last fragments have been read, in the last step (split
      // with the first step of the next k-tile, fp8 8192^3 ran 8% slower).
      first_steps_range<0, kSteps - 1, MM>(acc, fa, fb, cur, la, lb, nxt, src, wave, lane, wm0, wn0);
      dma_barrier();
      step<1, true, 0, MM>(acc, fa, fb, nxt, 0, la, lb, cur, src, wave, lane, wm0, wn0);
    } else {
      first_steps(acc, fa, fb, cur, la, lb, nxt, src, wave, lane, wm0, wn0);
      lds_barrier();
      step<1, false, 0>(acc, fa, fb, nxt, 0, la, lb, nxt, src, wave, lane, wm0, wn0);
    }
  }

  // ---- epilogue -----------------------------------------------------------------------
  // Accumulator lane layout: 32x32 blocks: for block (i, j) and register group g, lane l
  // holds row wm0 + 32i + (l % 32) and columns wn0 + 32j + 8g + 4(l / 32) + [0, 4). 16x16
  // blocks: lane l holds row wm0 + 16i + (l % 16) and columns wn0 + 16j + 4(l / 16) + [0, 4).
  // Per pass of kBPP block rows, the wave writes its raw fp32 accumulators (straight from
  // the accumulator registers) to a row-major buffer in its share of the idle ring, then
  // reads them back 8 consecutive columns per lane, so that C loads and D / PostAct stores
  // are 16-byte, row-contiguous accesses: alpha, beta * C, the activation and the
  // conversion run there. Common type combinations (C / D / PostAct all bf16 or all f16)
  // take a branch-free path with the C loads of a pass issued together; the others a
  // generic one.
  static constexpr int kEpiRegion = kLdsBytes / NW;
  static constexpr int kNC8 = kWN / 8;                             // 8-column groups per row
  static constexpr int kBPP = (kEpiRegion / (kBlk * kWN * 4)) < kMI ? (kEpiRegion / (kBlk * kWN * 4)) : kMI;
  static_assert(kBPP >= 1 && kMI % kBPP == 0, "epilogue passes must cover the wave tile");
  static constexpr int kRPI = 64 / kNC8;                           // rows per read instruction
  static constexpr int kIt = kBPP * kBlk / kRPI;                   // read instructions per pass

  // Byte offset of half `hf` (columns 8*c8 + 4*hf + [0, 4)) of row r in the wave's fp32
  // buffer: the first halves of all groups fill the first half of the row, the second
  // halves the second, each chunk index XOR-swizzled by the row. Acc-layout writes (32 rows,
  // one group) and row reads (one or two rows, all groups) then fall in distinct banks.
  // (16x16 blocks with 8 groups per row: a write phase holds rows {0-3, 8-11} of one half,
  // which the key maps to 8 distinct chunks.)
  static __device__ __forceinline__ int ekey(int r) {
    if constexpr (kBlk == 16 && kNC8 == 8) return (r & 3) | ((r >> 1) & 4);
    else return r & (kNC8 - 1);
  }
  static __device__ __forceinline__ int ebuf(int r, int c8, int hf) {
    return r * (kWN * 4) + hf * (kWN * 2) + ((c8 ^ ekey(r)) << 4);
  }

  template <int DT>
  static __device__ __forceinline__ i32x4 pack8(const f32x8& v) {
    if constexpr (DT == DT_BF16) return __builtin_bit_cast(i32x4, __builtin_convertvector(v, bf16x8));
    else return __builtin_bit_cast(i32x4, __builtin_convertvector(v, f16x8));
  }
  template <int DT>
  static __device__ __forceinline__ f32x8 unpack8(const i32x4& x) {
    if constexpr (DT == DT_BF16) return __builtin_convertvector(__builtin_bit_cast(bf16x8, x), f32x8);
    else return __builtin_convertvector(__builtin_bit_cast(f16x8, x), f32x8);
  }
  static __device__ __forceinline__ f32x8 act8(int act, const f32x8& v) {
    f32x8 w;
    switch (act) {
      case ACT_RELU:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = act_fn<ACT_RELU>(v[e]);
        break;
      case ACT_RELU_SQ:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = act_fn<ACT_RELU_SQ>(v[e]);
        break;
      case ACT_GELU_TANH:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = act_fn<ACT_GELU_TANH>(v[e]);
        break;
      case ACT_SILU:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = act_fn<ACT_SILU>(v[e]);
        break;
      default:
        w = v;
    }
    return w;
  }

  static __device__ __forceinline__ f32x8 dact8(int act, const f32x8& v) {
    f32x8 w;
    switch (act) {
      case ACT_RELU:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = dact_fn<ACT_RELU>(v[e]);
        break;
      case ACT_RELU_SQ:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = dact_fn<ACT_RELU_SQ>(v[e]);
        break;
      case ACT_GELU_TANH:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = dact_fn<ACT_GELU_TANH>(v[e]);
        break;
      case ACT_SILU:
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = dact_fn<ACT_SILU>(v[e]);
        break;
      default:
        w = f32x8{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    }
    return w;
  }

  // Everything a pass needs about the wave's part of the output tile.
  struct EpiArgs {
    const char* cb;  // C, D, PostAct at the wave tile's first row and column
    char* db;
    char* pb;
    int rows_valid, cols_valid;
    float alpha, beta;
  };

  // Branch-free pass: C (HC), D and PostAct (those present) all of type DT (bf16 or f16).
  // Without C the pass issues no global load, so no wait in it covers its own stores (a
  // wait on a load after a store is a vmcnt(0): loads and stores share the counter); with
  // C the loads of a batch of kCB row groups are issued together, one wait per batch.
  // BWD (activation backward; C present): D = (alpha * acc) * act'(C), PostAct = act(C).
  template <int DT, bool HC, bool BWD = false>
  static __device__ __forceinline__ void pass_fast(const KParams& p, const EpiArgs& ea, const GEP_LDS char* buf,
                                                   int m0, int lane) {
    constexpr int kCB = kIt < 4 ? kIt : 4;  // row groups per batch
    const int rl = lane / kNC8, c8 = lane % kNC8;
    const bool col_ok = 8 * c8 < ea.cols_valid;
    const bool hd = p.d_dt != DT_NONE, hp = p.p_dt != DT_NONE;
#pragma unroll 1
    for (int it0 = 0; it0 < kIt; it0 += kCB) {
      [[maybe_unused]] i32x4 cv[kCB];
      if constexpr (HC) {
#pragma unroll
        for (int u = 0; u < kCB; ++u) {
          const int m = m0 + (it0 + u) * kRPI + rl;
          cv[u] = i32x4{0, 0, 0, 0};
          if (col_ok && m < ea.rows_valid) cv[u] = *(const i32x4*)(ea.cb + ((int64_t)m * p.ldc + 8 * c8) * 2);
        }
      }
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        const int r = (it0 + u) * kRPI + rl, m = m0 + r;
        const f32x4 x0 = *(const f32x4 GEP_LDS*)(buf + ebuf(r, c8, 0));
        const f32x4 x1 = *(const f32x4 GEP_LDS*)(buf + ebuf(r, c8, 1));
        f32x8 v = f32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]} * ea.alpha;
        if constexpr (BWD) {
          const f32x8 pre = unpack8<DT>(cv[u]);
          if (col_ok && m < ea.rows_valid) {
            if (hd) *(i32x4*)(ea.db + ((int64_t)m * p.ldd + 8 * c8) * 2) = pack8<DT>(v * dact8(p.act, pre));
            if (hp) *(i32x4*)(ea.pb + ((int64_t)m * p.ldp + 8 * c8) * 2) = pack8<DT>(act8(p.act, pre));
          }
          // one row group at a time: interleaved, their temporaries would crowd out the
          // registers the main loop keeps
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        if constexpr (HC) v += ea.beta * unpack8<DT>(cv[u]);
        if (col_ok && m < ea.rows_valid) {
          if (hd) *(i32x4*)(ea.db + ((int64_t)m * p.ldd + 8 * c8) * 2) = pack8<DT>(v);
          if (hp) *(i32x4*)(ea.pb + ((int64_t)m * p.ldp + 8 * c8) * 2) = pack8<DT>(act8(p.act, v));
        }
      }
    }
  }

  // Four outputs of the generic pass (any C / D / PostAct types), at 4-element pointers. With
  // a transposed C (c_trans) its four values lie cstride bytes apart.
  static __device__ __forceinline__ void finish4(const KParams& p, const char* cp, char* dp, char* pp,
                                                 const f32x4& x, float alpha, float beta, int64_t cstride) {
    float v[4] = {x[0] * alpha, x[1] * alpha, x[2] * alpha, x[3] * alpha};
    float c[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.c_dt != DT_NONE && p.c_trans) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const char* q = cp + e * cstride;
        if (p.c_dt == DT_F32) c[e] = *(const float*)q;
        else if (p.c_dt == DT_BF16) c[e] = __uint_as_float((uint32_t)*(const uint16_t*)q << 16);
        else c[e] = (float)*(const _Float16*)q;
      }
      if constexpr (!DACT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(beta, c[e], v[e]);
      }
    } else if (p.c_dt != DT_NONE) {
      if (p.c_dt == DT_F32) {
        const f32x4 y = *(const f32x4*)cp;
        c[0] = y[0]; c[1] = y[1]; c[2] = y[2]; c[3] = y[3];
      } else {
        unpack4_16(p.c_dt, *(const uint2*)cp, c);
      }
      if constexpr (!DACT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(beta, c[e], v[e]);
      }
    }
    if constexpr (DACT) {
      // activation backward: D = dout * act'(C), PostAct = act(C)
      const f32x8 c8 = f32x8{c[0], c[1], c[2], c[3], 0.f, 0.f, 0.f, 0.f};
      const f32x8 g = dact8(p.act, c8), w8 = act8(p.act, c8);
      float d[4] = {v[0] * g[0], v[1] * g[1], v[2] * g[2], v[3] * g[3]};
      float w[4] = {w8[0], w8[1], w8[2], w8[3]};
      if (p.d_dt == DT_F32) *(f32x4*)dp = f32x4{d[0], d[1], d[2], d[3]};
      else if (p.d_dt != DT_NONE) store4(p.d_dt, dp, d);
      if (p.p_dt == DT_F32) *(f32x4*)pp = f32x4{w[0], w[1], w[2], w[3]};
      else if (p.p_dt != DT_NONE) store4(p.p_dt, pp, w);
      return;
    }
    if (p.d_dt == DT_F32) *(f32x4*)dp = f32x4{v[0], v[1], v[2], v[3]};
    else if (p.d_dt != DT_NONE) store4(p.d_dt, dp, v);
    if (p.p_dt != DT_NONE) {
      const f32x8 w8 = act8(p.act, f32x8{v[0], v[1], v[2], v[3], 0.f, 0.f, 0.f, 0.f});
      float w[4] = {w8[0], w8[1], w8[2], w8[3]};
      if (p.p_dt == DT_F32) *(f32x4*)pp = f32x4{w[0], w[1], w[2], w[3]};
      else store4(p.p_dt, pp, w);
    }
  }

  // Each lane covers 8 columns as two 4-column halves, each checked on its own: with only
  // f32 outputs the contiguous extent is a multiple of 4 elements, so the right edge may
  // end after the first half.
  static __device__ __forceinline__ void pass_generic(const KParams& p, const EpiArgs& ea, const GEP_LDS char* buf,
                                                      int m0, int lane) {
    const int rl = lane / kNC8, c8 = lane % kNC8;
    const int esc = dt_bytes(p.c_dt), esd = dt_bytes(p.d_dt), esp = dt_bytes(p.p_dt);
#pragma unroll 1
    for (int it = 0; it < kIt; ++it) {
      const int r = it * kRPI + rl, m = m0 + r;
      if (m >= ea.rows_valid) continue;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int n = 8 * c8 + 4 * hf;
        if (n + 4 > ea.cols_valid) continue;
        const f32x4 x = *(const f32x4 GEP_LDS*)(buf + ebuf(r, c8, hf));
        const int64_t coff = p.c_trans ? (int64_t)n * p.ldc + m : (int64_t)m * p.ldc + n;
        finish4(p, ea.cb + coff * esc, ea.db + ((int64_t)m * p.ldd + n) * esd,
                ea.pb + ((int64_t)m * p.ldp + n) * esp, x, ea.alpha, ea.beta, p.ldc * esc);
      }
    }
  }

  // ---- single 16-bit output without C: the values are final in the accumulator layout
  // (alpha, then the activation for a PostAct output), so they are converted there and only
  // the 16-bit results go through LDS: half the bytes of the fp32 path and the whole wave tile
  // in one pass. Buffer: kWM rows of kWN 16-bit values, 16-byte chunk c of row r at c ^ swz(r),
  // so that the 32 rows one accumulator write covers and the rows one read covers fall in
  // distinct 16-byte slots of the 256-byte bank window.
  static constexpr int kNC16 = kWN / 8;          // 16-byte chunks per row (8 or 16)
  // (the swizzle key below spans 8 or 16 chunks: a narrower row would need it masked)
  static_assert(kNC16 == 8 || kNC16 == 16, "single-output epilogue rows hold 8 or 16 chunks");
  static constexpr int kRPI16 = 64 / kNC16;      // rows per read instruction
  static constexpr bool kOnePass16 = kWM * kWN * 2 <= kEpiRegion;
  static __device__ __forceinline__ int ebuf16(int r, int c) {
    const int sw = kNC16 == 16 ? (r & 15) : ((r >> 1) & 7);
    return r * (kWN * 2) + ((c ^ sw) << 4);
  }

  template <int DT, bool ACT>
  static __device__ __forceinline__ void epilogue16(const KParams& p, const Acc (&acc)[kMI][kNI],
                                                    GEP_LDS char* region, int lane, char* ob, int64_t ld,
                                                    int rows_valid, int cols_valid, float alpha) {
    // the LDS addresses below depend on the lane only; computed here (an opaque copy of the
    // lane id), not hoisted to the kernel's start where they would stay live, and spill,
    // across the main loop
    asm volatile("" : "+v"(lane));
    if constexpr (kBlk == 16) {
      // blocks j and j + 1: columns 16j + 4q + [0, 4) and the same 16 further
      const int q = lane >> 4;
#pragma unroll
      for (int i = 0; i < kMI; ++i) {
        const int lr = i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < kNI; j += 2) {
          const Acc& a = acc[i][j];
          const Acc& b = acc[i][j + 1];
          f32x8 v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]} * alpha;
          if constexpr (ACT) v = act8(p.act, v);
          const i32x4 w = pack8<DT>(v);
          *(GEP_LDS i32x2*)(region + ebuf16(lr, 2 * j + (q >> 1)) + 8 * (q & 1)) = i32x2{w[0], w[1]};
          *(GEP_LDS i32x2*)(region + ebuf16(lr, 2 * j + 2 + (q >> 1)) + 8 * (q & 1)) = i32x2{w[2], w[3]};
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
    const int h = lane >> 5;
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const int lr = i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < kNI; ++j)
#pragma unroll
        for (int g = 0; g < 4; g += 2) {
          // groups g, g + 1: columns 32j + 8g + 4h + [0, 4) and the same 8 further
          const Acc& a = acc[i][j];
          f32x8 v = f32x8{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3],
                          a[4 * g + 4], a[4 * g + 5], a[4 * g + 6], a[4 * g + 7]} * alpha;
          if constexpr (ACT) v = act8(p.act, v);
          const i32x4 w = pack8<DT>(v);
          *(GEP_LDS i32x2*)(region + ebuf16(lr, 4 * j + g) + 8 * h) = i32x2{w[0], w[1]};
          *(GEP_LDS i32x2*)(region + ebuf16(lr, 4 * j + g + 1) + 8 * h) = i32x2{w[2], w[3]};
          // one group pair at a time: keeps the converted values from crowding the registers
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    }
    asm volatile("" ::: "memory");
    const int rl = lane / kNC16, c = lane % kNC16;
    const bool col_ok = 8 * c < cols_valid;
#pragma unroll 4
    for (int it = 0; it < kWM / kRPI16; ++it) {
      const int r = it * kRPI16 + rl;
      const i32x4 x = *(const GEP_LDS i32x4*)(region + ebuf16(r, c));
      if (col_ok && r < rows_valid) *(i32x4*)(ob + ((int64_t)r * ld + 8 * c) * 2) = x;
    }
    asm volatile("" ::: "memory");
  }

  static __device__ __forceinline__ void epilogue(const KParams& p, const TileInfo& ti,
                                                  const Acc (&acc)[kMI][kNI], GEP_LDS char* region, int lane,
                                                  int wm0, int wn0, float alpha, float beta) {
    const int h = lane >> 5;
    const int row0 = ti.m0 + wm0, col0 = ti.n0 + wn0;
    const int esc = dt_bytes(p.c_dt), esd = dt_bytes(p.d_dt), esp = dt_bytes(p.p_dt);
    EpiArgs ea;
    ea.cb = (const char*)p.C + ((VARLEN ? 0 : (int64_t)ti.l * p.sc) +
                                (p.c_trans ? (int64_t)col0 * p.ldc + row0 : (int64_t)row0 * p.ldc + col0)) * esc;
    ea.db = (char*)p.D + ((VARLEN ? 0 : (int64_t)ti.l * p.sd) + (int64_t)row0 * p.ldd + col0) * esd;
    ea.pb = (char*)p.Post + ((VARLEN ? 0 : (int64_t)ti.l * p.sp) + (int64_t)row0 * p.ldp + col0) * esp;
    ea.rows_valid = ti.row_end - row0;
    ea.cols_valid = p.N - col0;
    ea.alpha = alpha;
    ea.beta = beta;
    if constexpr (!DACT && kOnePass16) {
      // no C and one 16-bit output: D = alpha acc, or PostAct = act(alpha acc)
      if (p.c_dt == DT_NONE && (p.d_dt == DT_NONE) != (p.p_dt == DT_NONE)) {
        const bool post = p.p_dt != DT_NONE;
        const int ot = post ? p.p_dt : p.d_dt;
        char* ob = post ? ea.pb : ea.db;
        const int64_t ld = post ? p.ldp : p.ldd;
        if (ot == DT_BF16) {
          if (post && p.act != ACT_NONE) epilogue16<DT_BF16, true>(p, acc, region, lane, ob, ld, ea.rows_valid, ea.cols_valid, alpha);
          else epilogue16<DT_BF16, false>(p, acc, region, lane, ob, ld, ea.rows_valid, ea.cols_valid, alpha);
          return;
        }
        if (ot == DT_F16) {
          if (post && p.act != ACT_NONE) epilogue16<DT_F16, true>(p, acc, region, lane, ob, ld, ea.rows_valid, ea.cols_valid, alpha);
          else epilogue16<DT_F16, false>(p, acc, region, lane, ob, ld, ea.rows_valid, ea.cols_valid, alpha);
          return;
        }
      }
    }
    // one output type for C, D and PostAct (those present), 16-bit: the branch-free path
    const int ot = p.d_dt != DT_NONE ? p.d_dt : p.p_dt;
    const bool same = (p.c_dt == DT_NONE || (p.c_dt == ot && !p.c_trans)) && (p.p_dt == DT_NONE || p.p_dt == ot);
    const int path = !same ? 0 : (ot == DT_BF16 ? 1 : (ot == DT_F16 ? 2 : 0));
#pragma unroll 1
    for (int pass = 0; pass < kMI / kBPP; ++pass) {
      // raw accumulators of kBPP block rows -> LDS (the accumulator index must be literal)
#pragma unroll
      for (int pc = 0; pc < kMI / kBPP; ++pc) {
        if (pc != pass) continue;
#pragma unroll
        for (int ii = 0; ii < kBPP; ++ii) {
          if constexpr (kBlk == 16) {
            const int lr = ii * 16 + (lane & 15), q = lane >> 4;
#pragma unroll
            for (int j = 0; j < kNI; ++j)
              *(f32x4 GEP_LDS*)(region + ebuf(lr, 2 * j + (q >> 1), q & 1)) = acc[pc * kBPP + ii][j];
          } else {
            const int lr = ii * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < kNI; ++j)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const Acc& a = acc[pc * kBPP + ii][j];
                const f32x4 v = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
                *(f32x4 GEP_LDS*)(region + ebuf(lr, 4 * j + g, h)) = v;
              }
          }
        }
      }
      // LDS operations of one wave complete in order; keep the compiler from reordering
      asm volatile("" ::: "memory");
      const int m0 = pass * kBPP * kBlk;
      if constexpr (DACT) {
        // (C is always present)
        if (path == 1) pass_fast<DT_BF16, true, true>(p, ea, region, m0, lane);
        else if (path == 2) pass_fast<DT_F16, true, true>(p, ea, region, m0, lane);
        else pass_generic(p, ea, region, m0, lane);
      } else if (path == 1) {
        if (p.c_dt != DT_NONE) pass_fast<DT_BF16, true>(p, ea, region, m0, lane);
        else pass_fast<DT_BF16, false>(p, ea, region, m0, lane);
      } else if (path == 2) {
        if (p.c_dt != DT_NONE) pass_fast<DT_F16, true>(p, ea, region, m0, lane);
        else pass_fast<DT_F16, false>(p, ea, region, m0, lane);
      }
      else pass_generic(p, ea, region, m0, lane);
      asm volatile("" ::: "memory");
    }
  }

  static __device__ __forceinline__ void run(const KParams& p) {
    // One LDS object: the varlen group table sits past the ring. (With a second LDS array in
    // the kernel the compiler no longer separates fragment reads from pending global -> LDS
    // transfers and waits for all of them before every read.)
    __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes + kSlotBytes + (VARLEN ? kVarlenLds : 0)];
    GEP_LDS char* smem = (GEP_LDS char*)smem_raw;
    // the dynamic schedule's next queue position, published by thread 0
    volatile int32_t* next_slot = (volatile int32_t*)(smem_raw + kLdsBytes);
    const int tid = threadIdx.x, lane = tid & 63, lane_id = lane;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
    // 8 waves: waves w and w + 4, which share a SIMD, take the two row halves of one column
    // block, so that a tile whose second row half lies past the output leaves one active wave
    // per SIMD; 4 waves: a 2 x 2 grid
    const int wm0 = (NW == 8 ? ((wave >> 2) & 1) : (wave & 1)) * kWM;
    const int wn0 = (NW == 8 ? (wave & 3) : (wave >> 1)) * kWN;

    const int P = p.P;
    const int bid = blockIdx.x;
    // With the XCD remap, the P workgroups form 8 queues of Q = P/8 (workgroup b in queue
    // b % 8 at position b / 8), else one queue of P. Position k of queue x is tile
    // (k / Q) * P + x * Q + k % Q: the static schedule walks k = j, j + Q, j + 2Q, ...; the
    // dynamic one (tile_counters given) starts at k = j and then takes k = Q + the value of
    // an atomic counter per queue, so each queue still holds the same tiles (and L2 reuse)
    // while its workgroups balance among themselves.
    const bool xq = p.xcd_remap && (P & 7) == 0;
    const int Q = xq ? (P >> 3) : P;
    const int qx = xq ? (bid & 7) : 0;
    const int qj = xq ? (bid >> 3) : bid;
    const int bb = qx * Q + qj;
    auto qtile = [&](int k) { return (k / Q) * P + qx * Q + k % Q; };

    // ---- varlen: tile offsets of the groups (in map tiles), in LDS
    [[maybe_unused]] int32_t* gstart = nullptr;
    [[maybe_unused]] const int MT = (BM == 128 && p.tail == 2) ? 2 * BM : BM;
    int T = p.T;
    if constexpr (VARLEN) {
      int32_t* s_start = (int32_t*)(smem_raw + kLdsBytes + kSlotBytes);
      int32_t* s_part = s_start + kMaxVarlenGroups + 1;
      // the validity flag lives in the same LDS array (__syncthreads_or would add an LDS object
      // of its own, and with two the compiler waits for every pending global -> LDS transfer
      // before each fragment read)
      volatile int32_t* s_bad = s_part + kThreads;
      if (tid == 0) *s_bad = 0;
      __syncthreads();
      const int G = p.L;
      constexpr int kPer = (kMaxVarlenGroups + kThreads - 1) / kThreads;
      int32_t local[kPer];
      int32_t sum = 0;
      // cu_seqlens must start at 0, never decrease and end at M; otherwise no tile is run and
      // nothing is written (a decreasing or overlong array would address rows outside D)
      int bad = 0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int g = tid * kPer + q;
        int32_t tiles = 0;
        if (g < G) {
          const int c0 = p.cu_seqlens[g], c1 = p.cu_seqlens[g + 1];
          const int rows = c1 - c0;
          bad |= rows < 0 || (g == 0 && c0 != 0) || (g == G - 1 && c1 != p.M);
          tiles = rows > 0 ? ((rows + MT - 1) / MT) * p.tn : 0;
        }
        local[q] = sum;
        sum += tiles;
      }
      if (bad) *s_bad = 1;
      s_part[tid] = sum;
      __syncthreads();
      bad = __builtin_amdgcn_readfirstlane(*s_bad);
      // inclusive scan of the partial sums (Hillis-Steele)
      for (int off = 1; off < kThreads; off <<= 1) {
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
      if (tid == kThreads - 1) s_start[G] = s_part[kThreads - 1];
      __syncthreads();
      gstart = s_start;
      T = __builtin_amdgcn_readfirstlane(bad ? 0 : s_start[G]);
    }
    // Split tail: when the last round of map tiles is partial and at most half full, a second
    // launch (tail == 2, BM x BN kernel over the map of 2BM x 2BN tiles) takes it as quarter
    // tiles, and the first launch (tail == 1) stops before it. Both decide from T alone.
    int t_lo = 0, U = T;
    if (p.tail != 0) {
      const int rem = T % p.P_big;
      const bool split = T > p.P_big && rem > 0 && 2 * rem <= p.P_big;
      if (p.tail == 1) {
        U = split ? T - rem : T;
      } else {
        t_lo = T - rem;
        U = split ? 4 * rem : 0;
      }
    }
    // The quarter-tile launch can hold more workgroups than items (a varlen grid is sized
    // before T is known): its XCD queues then take ceil(U / 8) consecutive items each, so the
    // items spread over all eight XCDs rather than filling the first queues (the workgroups
    // past them take none).
    int b0 = bb;
    if (p.tail == 2 && xq && U <= P) {
      const int Qu = (U + 7) >> 3;
      b0 = qj < Qu ? qx * Qu + qj : U;
    }

    const float alpha = p.alpha_ptr ? *p.alpha_ptr : p.alpha;
    const float beta = p.beta_ptr ? *p.beta_ptr : p.beta;
    LA la;
    LB lb;
    Frag fa[2][kMI], fb[2][kNI];
    TileInfo ti;
    // a tile's first k-tile goes into the staging registers as early as possible
    auto begin_tile = [&](int t) {
      ti = decode(p, t, gstart, t_lo);
      // the loaders' lane offsets are recomputed here from an opaque copy of the lane id: hoisted
      // out of the tile loop they stay live across the main loop and spill
      int lane = lane_id;
      asm volatile("" : "+v"(lane));
      if constexpr (GAK) la.init_gather_k(wave, lane, ti.row_end - ti.m0, ti.klen);
      else if constexpr (GA) la.init_gather(wave, lane, ti.row_end - ti.m0, p.lda * kES, ti.klen, p.a_idx + ti.m0, p.a_rows);
      else la.init(wave, lane, ti.row_end - ti.m0, p.lda * kES, ti.klen);
      lb.init(wave, lane, p.N - ti.n0, p.ldb * kES, ti.klen);
      if constexpr (GAK) {
        static_assert(!kDMA, "gathered k-rows go through the staging registers");
        const KtSrc s0 = kt_src(p, ti, 0);
        fetch_all(la, s0.ia);
        load_all(la, lb, s0);
      } else if constexpr (!kDMA) {
        load_all(la, lb, kt_src(p, ti, 0));
      }
    };
    // dynamic schedule: this queue's counter, and the number of tiles it holds (the fetch
    // that returns the last value returns the counter to zero for the next launch)
    int32_t* const ctr = p.tile_counters ? p.tile_counters + qx : nullptr;
    const int q_tiles = (U / P) * Q + min(max(U % P - qx * Q, 0), Q);
    int32_t fetched = 0;

    if (b0 < U) begin_tile(b0);
    int iter = 0;
    for (int t = b0; t < U; ++iter) {
      // claim the tile after this one (its result is first waited for where it is published)
      if (ctr && tid == 0) fetched = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ti.m0 >= ti.row_end || ti.n0 >= p.N) {  // a quarter tile wholly outside the output
        // (split-tail launches only, which are static)
        t += P;
        if (t < U) begin_tile(t);
        continue;
      }
      if (p.tile_log && iter < p.tile_log_iters && tid == 0) {
        int32_t* e = p.tile_log + ((int64_t)bid * p.tile_log_iters + iter) * 4;
        e[0] = ti.mb; e[1] = ti.nb; e[2] = ti.l; e[3] = t;
      }
      Acc acc[kMI][kNI];
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNI; ++j) acc[i][j] = Acc{};

      // An 8-wave wave whose rows all lie past the output (the last M-block of a varlen group,
      // or of M) runs only the k-tiles' transfers and barriers: its SIMD partner, on the other
      // half of the rows, then has the MFMA pipe to itself (uniform per wave).
      const bool idle = (kRoll3 || kStream) && ti.m0 + wm0 >= ti.row_end;
      // the previous tile's epilogue buffers (and the published queue position) are free
      lds_barrier();
      // k-tiles, run in pairs (the stages alternate): an odd count gets one more k-tile past
      // K, whose loads read zeros and which adds nothing
      const int nk = (((ti.klen + kBK - 1) / kBK) + 1) & ~1;
      if (nk > 0) {
        if constexpr (kDMA) {
          // k-tiles 0 and 1 -> stages 0 and 1 (8 waves: the first half of k-tile 1; the first
          // k-tile's step 0 issues the rest)
          dma_chunks<0, kChunksPerKt>(la, lb, smem, kt_src(p, ti, 0), wave);
          dma_chunks<0, (kRoll3 || kStream) ? kChunksPerKt / 2 : kChunksPerKt>(la, lb, smem + kStageBytes, kt_src(p, ti, 1), wave);
          dma_barrier();
        } else {
          // k-tile 0 -> stage 0, registers <- k-tile 1
          cycle_chunks<0, kChunksPerKt>(la, lb, smem, kt_src(p, ti, 1), wave, lane);
          lds_barrier();
        }
        if constexpr (kRoll3 || kStream) {
          if (idle) {
            __builtin_amdgcn_s_setprio(0);
            for (int kt = 0; kt < nk; kt += 2) {
              ktile<0, false>(p, ti, la, lb, smem, acc, fa, fb, kt, wave, lane, wm0, wn0);
              ktile<1, false>(p, ti, la, lb, smem, acc, fa, fb, kt + 1, wave, lane, wm0, wn0);
            }
          }
        }
        if (!idle) {
          if constexpr (kStream) s_first(fa[0], fb[0], smem, lane, wm0, wn0);
          else read_all(fa[0], fb[0], smem, 0, wm0, wn0, lane);
          for (int kt = 0; kt < nk; kt += 2) {
            ktile<0>(p, ti, la, lb, smem, acc, fa, fb, kt, wave, lane, wm0, wn0);
            ktile<1>(p, ti, la, lb, smem, acc, fa, fb, kt + 1, wave, lane, wm0, wn0);
          }
        }
      }

      // ---- this tile's epilogue, through per-wave buffers in the ring (the barrier ends every
      // wave's reads of it), then the next tile's first loads. (Issued before the epilogue,
      // those loads would gain nothing: a wait on them after the epilogue's stores also
      // waits for the stores, and their registers would crowd the epilogue.)
      // (global -> LDS transfers of the padding k-tiles past K must land before the ring is
      // reused)
      if (ctr && tid == 0) {
        *next_slot = fetched;
        if (fetched == q_tiles - 1) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if constexpr (kDMA) dma_barrier();
      else lds_barrier();
      // (uniform: keeps the tile loop's state in scalar registers)
      const int tnext = ctr ? qtile(Q + __builtin_amdgcn_readfirstlane(*next_slot)) : t + P;
      if (!idle) epilogue(p, ti, acc, smem + wave * kEpiRegion, lane, wm0, wn0, alpha, beta);
      t = tnext;
      if (t < U) begin_tile(t);
    }
  }
};

}  // namespace gep
