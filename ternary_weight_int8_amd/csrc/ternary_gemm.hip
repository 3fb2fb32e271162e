// ternary_gemm.hip -- gfx950 (CDNA4) kernels and C ABI of the ternary x int8
// GEMM library.  The ABI and the stored-weight format are documented in
// include/ternary_gemm.h.
//
// Sources (cited by page title and section):
//   [P10425] t27 pull request #10425, "t27c PTX backend: ternary x int8 GEMM
//            kernel emitted by a .t27 spec (int8 mma.sync), ptx-run glue".
//   [P10855] t27 pull request #10855, "spec(igla): hslm_bwd_ptx -- HSLM
//            backward dX and dW as int8 tensor-core PTX written by t27".
//
// One kernel template computes all three products.  Every product writes a
// row-major int32 output O[R][Cc] = sum over a contraction of length L:
//
//   product   O      R   Cc  L   Q operand (rows of O)      P operand (cols of O)
//   forward   C      M   N   K   A[m][.]   contraction-     W(., n) decoded, contraction-
//                                          contiguous rows  contiguous rows
//   dX        dX     M   K   N   dC[m][.]  same             Wpacked rows n decoded as they
//                                                           lie (rows = contraction)
//   dW        dW     K   N   M   A[.][k]   rows as they     dC[.][n] rows as they lie
//                                          lie (contraction)
//
// A workgroup of 4 waves owns a BM x BN tile of O.  Per step of 64 along the
// contraction it stages the step's Q and P data into LDS (decoding the 2-bit
// codes once per global->LDS tile load [P10425 "What this adds"]), then each
// wave runs v_mfma_i32_16x16x64_i8 over its sub-tile with int32 accumulators
// held in registers for the whole contraction.  Contraction-contiguous rows
// are read as fragments with 16-byte LDS reads; rows indexed by the
// contraction are read with the transposing LDS read (TrRead), which yields
// the same byte order, so any pairing of the two kinds is valid.
//
// Pipeline: global loads run PF steps ahead of the MFMAs through a ring of PF
// register slots; the step after the current one is written from its slot
// into the other of two LDS buffers once the current step's MFMAs are issued,
// with one barrier per step.  (The pages' kernel loads synchronously with one
// stage and names asynchronous double buffering with a 64-wide step as its
// next lever [P10425 "What this says"].)
//
// MFMA operand roles: the P fragment is the instruction's A operand and the Q
// fragment its B operand, so lane l of a 16x16 result holds O[row l%16][cols
// 4*(l/16) .. +3]: four consecutive int32 of one output row, stored with one
// 16-byte store.  Both fragments take the same 16 contraction bytes per lane
// (chunk l/16 of the 64), so whatever order the instruction assigns to those
// bytes is shared by both operands and the dot products are unchanged.
//
// Exactness: every partial sum is bounded by the final bound the host checks
// (L * 128 for ternary, L * 128^2 for int8 x int8), so int32 accumulation in
// any order is exact [P10425 "What this adds", "i32 overflow bound"; P10855
// PR body, "k <= 131071"], and every reduction order below gives the same
// bits on every call, with no atomics.  Most kernels reduce each output
// serially in one wave's registers.  Three split the contraction, each into
// a fixed number of parts added in a fixed order:
//   - tgemm_split (dW at long contractions, dX with few tiles): two halves of
//     one workgroup take alternate steps; half 1 hands its sums to half 0
//     through LDS;
//   - the skinny kernels (M <= 32): the eight waves of a workgroup take
//     interleaved steps and add their sums through LDS in wave order;
//   - the workspace dX calls (ternary_gemm_s8_dx_ws, _scaled_ws, _noalloc):
//     S workgroups take contiguous runs of the contraction and write int32
//     partial sums; a second kernel adds them in split order.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "ternary_gemm.h"

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int BK = 64;         // contraction per step (one 16x16x64 MFMA)
constexpr int LP = BK;         // LDS row pitch (bytes): rows are not padded

// LDS layout of a staged tile: row r holds its four 16-byte contraction
// chunks in the order chunk c at slot c ^ ((r >> 1) & 3).  Measured on gfx950:
// with this swizzle both the MFMA fragment reads (16 rows x 4 chunks per
// wave) and the 4-threads-per-row tile copies run at the full ~220 B/clk/CU
// ds_read_b128 rate, while an unswizzled or padded (80-byte) pitch halves it.
__host__ __device__ constexpr int swz(int r, int c) { return r * LP + 16 * (c ^ ((r >> 1) & 3)); }

// Workgroup barrier for LDS only: waits for this wave's LDS operations, not
// for its outstanding global loads (which __syncthreads() would also drain,
// defeating the prefetch).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Byte c of this word is the int8 weight of code c: 00, 01, FF, 00, i.e.
// (c & 1) - ((c >> 1) & 1) [P10425 "What this adds"; P10855 PR body].
constexpr uint32_t kCodeTable = 0x00FF0100u;

enum Op { FWD = 0, DX = 1, DW = 2 };

template <bool B>
struct Flag {
  static constexpr bool value = B;
};


// ---------------------------------------------------------------------------
// The output of a call: the int32 sums as computed, or the sums scaled into
// f32 or bf16 (the dequantization step that follows the integer product:
// activations quantized per row for the forward and dX, X and dY per column
// for dW [P10855 PR body]).  A scaled element is
//     y = (float(acc) * rs[row]) * cs[col]          (cs null: cscal)
// with the int32 -> float conversion and each product rounded to nearest-even
// in IEEE single precision, in that order; bf16 output then rounds y to the
// nearest bf16, ties to even (v_cvt_pk_bf16_f32; a NaN stays a NaN).
// ---------------------------------------------------------------------------
enum OutKind { OUT_I32 = 0, OUT_F32 = TGEMM_OUT_F32, OUT_BF16 = TGEMM_OUT_BF16 };
static_assert(OUT_F32 != OUT_I32 && OUT_BF16 != OUT_I32 && OUT_F32 != OUT_BF16, "output kinds");

struct Out {
  void *ptr;          // [R][Cc] elements of the kind
  const float *rs;    // per output row (scaled kinds)
  const float *cs;    // per output column, or null: cscal for every column
  float cscal;
  int32_t kind;       // OutKind
  int32_t vec;        // Cc % 4 == 0 and ptr aligned to 4 elements: 4-element stores
  int32_t vec8;       // bf16, Cc % 8 == 0 and ptr 16-byte aligned: 8-element stores
};

__device__ __forceinline__ float scaled(int32_t x, float r, float c) {
  return __fmul_rn(__fmul_rn((float)x, r), c);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even) packed low, high
__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// columns col .. col + 3 of row `row`, all inside the output (o.vec); r is
// the row's scale (read by the caller; unused for int32)
__device__ __forceinline__ void put4(const Out &o, int64_t Cc, int64_t row, int64_t col, const v4i &v, float r) {
  const int64_t e = row * Cc + col;
  if (o.kind == OUT_I32) {
    *reinterpret_cast<v4i *>(static_cast<int32_t *>(o.ptr) + e) = v;
    return;
  }
  float y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) y[k] = scaled(v[k], r, o.cs ? o.cs[col + k] : o.cscal);
  if (o.kind == OUT_F32) {
    *reinterpret_cast<float4 *>(static_cast<float *>(o.ptr) + e) = make_float4(y[0], y[1], y[2], y[3]);
  } else {
    uint2 b;
    b.x = bf16_pack(y[0], y[1]);
    b.y = bf16_pack(y[2], y[3]);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o.ptr) + e) = b;
  }
}
__device__ __forceinline__ void put1(const Out &o, int64_t Cc, int64_t row, int64_t col, int32_t x, float r) {
  const int64_t e = row * Cc + col;
  if (o.kind == OUT_I32) {
    static_cast<int32_t *>(o.ptr)[e] = x;
    return;
  }
  const float y = scaled(x, r, o.cs ? o.cs[col] : o.cscal);
  if (o.kind == OUT_F32)
    static_cast<float *>(o.ptr)[e] = y;
  else
    static_cast<uint16_t *>(o.ptr)[e] = __builtin_bit_cast(uint16_t, (__bf16)y);
}
__device__ __forceinline__ float row_scale(const Out &o, int64_t row) {
  return o.kind == OUT_I32 ? 0.f : o.rs[row];
}

struct Args {
  const int8_t *q;    // Q source
  const void *p;      // P source (Wpacked for FWD/DX, dC for DW)
  Out o;
  int64_t R, Cc, L;   // output rows, output cols, contraction length
  int64_t ldq, ldp;   // row strides (bytes) of the Q and P sources
  int32_t tiles_c;    // column tiles
  int32_t band_cols;  // tile columns per band of the workgroup -> tile order
  int32_t tiles;      // total tiles (= workgroups)
  int32_t xcds;       // workgroup b runs on XCD b % xcds
};

// ---------------------------------------------------------------------------
// Workgroup -> tile order.  The hardware hands workgroup ids to the XCDs
// round-robin (id % xcds; MI355X has eight), and each XCD has its own L2.
// xcd_tile gives each
// XCD a contiguous range of positions in a linear tile order (a bijection on
// [0, tiles)).  That order runs row by row inside bands of band_cols tile
// columns, band after band, so the tiles an XCD runs together share input
// rows, and with several bands an XCD also touches only its band's columns.
// The host picks the band count that minimises the operand bytes the eight
// XCDs fetch between them.
// ---------------------------------------------------------------------------
__host__ __device__ inline int32_t xcd_tile(int32_t wg, int32_t tiles, int32_t xcds) {
  const int32_t q = tiles / xcds, r = tiles % xcds;
  const int32_t x = wg % xcds, j = wg / xcds;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

__host__ __device__ inline void tile_rc(int32_t pos, int32_t tiles_r, int32_t tiles_c,
                                        int32_t band_cols, int32_t *tr, int32_t *tc) {
  const int32_t per_band = tiles_r * band_cols;
  const int32_t band = pos / per_band, rem = pos % per_band;
  const int32_t c0 = band * band_cols;
  const int32_t w = tiles_c - c0 < band_cols ? tiles_c - c0 : band_cols;
  *tr = rem / w;
  *tc = c0 + rem % w;
}

// ---------------------------------------------------------------------------
// Code decode: one packed dword x (code i at bits 2i) -> 16 int8 weights.
// For output dword j (codes 4j .. 4j + 3, byte j of x), one v_perm_b32
// gathers byte j of x and byte j of y = x >> 2 as [x_j, y_j, x_j, y_j]; a
// packed 16-bit right shift by (0, 4) leaves code 4j + k in the low two bits
// of byte k (byte 1: bits 2-3 of x_j, byte 2: bits 4-5, byte 3: bits 6-7);
// masked to those bits, each byte selects its weight from kCodeTable with a
// second v_perm_b32.  Four codes -> four weights in four instructions.
// ---------------------------------------------------------------------------
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4i decode16(uint32_t x) {
  const uint32_t y = x >> 2;
  v4i w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // selector bytes [j, 4 + j, j, 4 + j]: bytes 0-3 of the pool are x, 4-7 are y
    const uint32_t sel = (uint32_t)j * 0x00010001u + (uint32_t)(4 + j) * 0x01000100u;
    const u16x2 h = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(y, x, sel)) >> (u16x2){0, 4};
    w[j] = (int32_t)__builtin_amdgcn_perm(0u, kCodeTable, __builtin_bit_cast(uint32_t, h) & 0x03030303u);
  }
  return w;
}

// ---------------------------------------------------------------------------
// Stagers.  init() fixes a thread's source addresses for the workgroup's
// tile; load() issues the global reads of the step starting at contraction
// index c0 into a register slot; store() writes a slot (decoded / transposed)
// into an LDS tile of BT rows of LP bytes.  `full` is true when the whole step
// lies inside the contraction; otherwise positions >= L are loaded as 0, so a
// ragged last step contributes nothing.  Rows beyond the output are clamped to
// the last valid row (in bounds, computed, never stored).
// ---------------------------------------------------------------------------

// Rows of an int8 matrix that run along the contraction (A or dC as the Q
// operand): 16-byte chunks, 4 per row per step, 4 threads per row; a thread's
// i-th chunk is in tile row i*64 + tid/4 (the last pass may cover fewer rows).
template <int BT, bool FAST>
struct CopyOp {
  static constexpr int kPer = (BT + kThreads / 4 - 1) / (kThreads / 4);
  static_assert(BT % 16 == 0, "tile shape");
  struct Slot { v4i r[kPer]; };
  const int8_t *ptr[kPer];
  int64_t L;
  int cc, row0;

  // pass i of this thread covers a tile row; `wave` is wave-uniform (rows of
  // a wave are 16 consecutive ones and BT % 16 == 0), so this is a scalar test
  __device__ __forceinline__ static bool has(int i, int wave) {
    return BT % (kThreads / 4) == 0 || i * (kThreads / 4) + 16 * wave < BT;
  }

  __device__ __forceinline__ void init(const int8_t *src, int64_t ld, int64_t nrows, int64_t L_,
                                       int64_t t0, int tid) {
    L = L_;
    cc = tid & 3;
    row0 = tid >> 2;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t row = t0 + i * (kThreads / 4) + row0;
      ptr[i] = src + (row < nrows ? row : nrows - 1) * ld + cc * 16;
    }
  }

  __device__ __forceinline__ void load(Slot &s, int64_t c0, bool full) const {
    const int64_t gc = c0 + cc * 16;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      // every thread loads every pass (rows past the tile are clamped to valid
      // rows, never stored), so the number of loads in flight is the same on
      // every path and the compiler can wait for exactly the ones it needs
      const int8_t *p = ptr[i] + c0;
      if (FAST && full) {
        s.r[i] = *reinterpret_cast<const v4i *>(p);
      } else if (FAST) {  // L % 16 == 0: a chunk is all in or all out
        // branch-free: read an in-bounds chunk (the row start), keep it only if in
        const v4i v = *reinterpret_cast<const v4i *>(gc < L ? p : ptr[i]);
        s.r[i] = gc < L ? v : v4i{0, 0, 0, 0};
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < 16; ++b)
          if (full || gc + b < L) w[b >> 2] |= (uint32_t)(uint8_t)p[b] << (8 * (b & 3));
        s.r[i] = v4i{(int32_t)w[0], (int32_t)w[1], (int32_t)w[2], (int32_t)w[3]};
      }
    }
  }

  __device__ __forceinline__ static void store(const Slot &s, int8_t *lds, int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!has(i, wave)) break;
      *reinterpret_cast<v4i *>(lds + swz(i * (kThreads / 4) + (tid >> 2), tid & 3)) = s.r[i];
    }
  }
};

// Stored ternary weights as the P operand of the forward product: row n of
// Wpacked holds the codes of column n along K, so a step's 64 codes of a row
// are 16 contiguous bytes = 4 dwords, one per thread (4 threads per row, same
// row assignment as CopyOp).  Decoded once here, one 16-B LDS store per dword.
template <int BT, bool FAST>
struct DecodeOp {
  static constexpr int kPer = (BT + kThreads / 4 - 1) / (kThreads / 4);
  static_assert(BT % 16 == 0, "tile shape");
  struct Slot { uint32_t r[kPer]; };
  const uint8_t *ptr[kPer];
  int64_t L;
  int uc, row0;

  __device__ __forceinline__ static bool has(int i, int wave) {
    return BT % (kThreads / 4) == 0 || i * (kThreads / 4) + 16 * wave < BT;
  }

  __device__ __forceinline__ void init(const uint8_t *wp, int64_t ld, int64_t nrows, int64_t L_,
                                       int64_t t0, int tid) {
    L = L_;
    uc = tid & 3;
    row0 = tid >> 2;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t row = t0 + i * (kThreads / 4) + row0;
      ptr[i] = wp + (row < nrows ? row : nrows - 1) * ld + uc * 4;
    }
  }

  __device__ __forceinline__ void load(Slot &s, int64_t c0, bool full) const {
    const int64_t gk = c0 + uc * 16;  // first code of this thread's dword
#pragma unroll
    for (int i = 0; i < kPer; ++i) {  // every pass, as in CopyOp
      const uint8_t *p = ptr[i] + (c0 >> 2);
      if (FAST && full) {
        s.r[i] = *reinterpret_cast<const uint32_t *>(p);
      } else if (FAST) {  // L % 16 == 0, 4-B aligned rows; branch-free as above
        const uint32_t v = *reinterpret_cast<const uint32_t *>(gk < L ? p : ptr[i]);
        s.r[i] = gk < L ? v : 0u;
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (full || gk + 4 * b < L) w |= (uint32_t)p[b] << (8 * b);
        s.r[i] = w;
      }
    }
  }

  __device__ __forceinline__ static void store(const Slot &s, int8_t *lds, int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!has(i, wave)) break;
      *reinterpret_cast<v4i *>(lds + swz(i * (kThreads / 4) + (tid >> 2), tid & 3)) =
          decode16(s.r[i]);
    }
  }
};

// An int8 matrix whose rows are indexed by the contraction (A[m][k] and
// dC[m][n] for dW), staged as it lies in memory: LDS row = contraction index m
// (BK rows per step), BT bytes of output index o per row in 16-byte chunks.
// The MFMA fragments, which need 16 contraction bytes per output index, are
// read from it with the transposing LDS read (see Frags<DW>).  A unit is one
// 16-byte chunk; thread tid takes units tid, tid + 256, ...
//
// Placement of chunk c of row m (RowLayout).  The fragment reads (Frags)
// take 16 rows per half-wave, rows {16g + 8h + b} for g in a pair of lane
// groups and b < 8, all at one chunk c; the unit stores write 16 consecutive
// units.  With a power-of-two number of chunks per row, chunk c goes to slot
// c ^ sw(m), sw mapping each such row set onto distinct 16-byte bank groups.
// With an odd number (144-byte rows: 9), rows are packed and every second
// block of 16 rows is shifted by a further 128 bytes, which does the same;
// with twice an odd number (160-byte rows: 10) the shift is 16 bytes.  A model of the 64 banks (checked for all five row
// lengths) and the counters on MI355X both show no conflicts.
template <int BT>
struct RowLayout {
  static constexpr int kChunks = BT / 16;
  static_assert(BT % 16 == 0 && (BK * kChunks) % 64 == 0, "row length");
  static_assert(kChunks == 4 || kChunks == 8 || kChunks == 16 || kChunks % 2 == 1 || kChunks == 10,
                "row length");
  static constexpr bool kOdd = kChunks % 2 == 1;
  static constexpr bool kTwiceOdd = kChunks == 10;
  __host__ __device__ static constexpr int sw(int m) {
    return kChunks == 16  ? (m & 7) | (((m >> 4) & 1) << 3)
           : kChunks == 8 ? ((m >> 1) & 3) | (((m >> 4) & 1) << 2)
           : kChunks == 4 ? ((m >> 2) & 1) | (((m >> 4) & 1) << 1)
                          : 0;
  }
  __host__ __device__ static constexpr int base(int m) {
    return m * BT + (kOdd ? 128 : kTwiceOdd ? 16 : 0) * (((m >> 4) + 1) >> 1);
  }
  __host__ __device__ static constexpr int at(int m, int c) { return base(m) + 16 * (c ^ sw(m)); }
  static constexpr int kBytes = BK * BT + (kOdd ? 256 : kTwiceOdd ? 32 : 0);  // one stage
};

template <int BT, bool FAST>
struct RowCopyOp {
  typedef RowLayout<BT> Lay;
  static constexpr int kUnits = BK * Lay::kChunks;  // a multiple of 64: whole waves
  static constexpr int kPer = (kUnits + kThreads - 1) / kThreads;
  struct Slot { v4i r[kPer]; };
  const int8_t *base;          // the matrix, row 0 (an always-valid address)
  const int8_t *ptr[kPer];     // chunk of unit i in contraction row 0
  int64_t ld, L, nout;
  int64_t o[kPer];             // first output index of unit i's chunk
  int m[kPer];                 // contraction row of unit i within a step

  // unit i of a thread exists for whole waves; `wave` is wave-uniform, so the
  // store test is a scalar branch
  __device__ __forceinline__ static bool has(int i, int wave) {
    return kUnits % kThreads == 0 || i * kThreads + wave * 64 < kUnits;
  }

  __device__ __forceinline__ void init(const int8_t *src, int64_t ld_, int64_t nout_, int64_t L_,
                                       int64_t t0, int tid) {
    base = src;
    ld = ld_;
    L = L_;
    nout = nout_;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      // a thread without a unit in pass i repeats its pass i - 1 unit (loaded,
      // never stored): every path then has the same loads in flight
      const int u = i * kThreads + tid < kUnits ? i * kThreads + tid : (i - 1) * kThreads + tid;
      const int c = u % Lay::kChunks;
      m[i] = u / Lay::kChunks;
      o[i] = t0 + 16 * c;
      // FAST: nout % 16 == 0, so a chunk is all inside the output range or all
      // outside; outside ones read the last valid chunk (computed, never stored)
      const int64_t oc = (FAST && o[i] >= nout) ? nout - 16 : o[i];
      ptr[i] = src + m[i] * ld + oc;
    }
  }

  __device__ __forceinline__ void load(Slot &s, int64_t c0, bool full) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int8_t *p = ptr[i] + c0 * ld;
      if (FAST && full) {
        s.r[i] = *reinterpret_cast<const v4i *>(p);
      } else if (FAST) {
        // branch-free: rows past the contraction read row 0 and are zeroed
        const bool in = c0 + m[i] < L;
        const v4i v = *reinterpret_cast<const v4i *>(in ? p : base);
        s.r[i] = in ? v : v4i{0, 0, 0, 0};
      } else {
        const bool in = full || c0 + m[i] < L;
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < 16; ++b)
          if (in && o[i] + b < nout) w[b >> 2] |= (uint32_t)(uint8_t)p[b] << (8 * (b & 3));
        s.r[i] = v4i{(int32_t)w[0], (int32_t)w[1], (int32_t)w[2], (int32_t)w[3]};
      }
    }
  }

  __device__ __forceinline__ static void store(const Slot &s, int8_t *lds, int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!has(i, wave)) break;
      const int u = i * kThreads + tid;
      *reinterpret_cast<v4i *>(lds + Lay::at(u / Lay::kChunks, u % Lay::kChunks)) = s.r[i];
    }
  }
};

// Stored ternary weights as the P operand of dX, staged as they lie: Wpacked
// row n holds the codes of contraction index n along the output index k, so
// LDS row = n and one packed dword (16 codes, k .. k + 15) decodes into one
// 16-byte chunk of that row.  Layout, units and clamping as RowCopyOp; the
// fragments are read transposed (Frags<DX>).
template <int BT, bool FAST>
struct DecodeRowOp {
  typedef RowLayout<BT> Lay;
  static constexpr int kUnits = BK * Lay::kChunks;
  static constexpr int kPer = (kUnits + kThreads - 1) / kThreads;
  struct Slot { uint32_t r[kPer]; };
  const uint8_t *base;         // Wpacked, row 0 (an always-valid address)
  const uint8_t *ptr[kPer];    // unit i's dword in contraction row 0
  int64_t ld, L, kbytes;       // row stride, contraction length, packed bytes per row
  int64_t gb[kPer];            // first packed byte of unit i's dword
  int m[kPer];                 // contraction row of unit i within a step

  __device__ __forceinline__ static bool has(int i, int wave) {
    return kUnits % kThreads == 0 || i * kThreads + wave * 64 < kUnits;
  }

  __device__ __forceinline__ void init(const uint8_t *wp, int64_t ld_, int64_t kbytes_, int64_t L_,
                                       int64_t t0, int tid) {
    base = wp;
    ld = ld_;
    L = L_;
    kbytes = kbytes_;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = i * kThreads + tid < kUnits ? i * kThreads + tid : (i - 1) * kThreads + tid;
      const int c = u % Lay::kChunks;
      m[i] = u / Lay::kChunks;
      gb[i] = (t0 >> 2) + 4 * c;
      // FAST: kbytes % 4 == 0, so a dword is all inside the row or all outside;
      // outside ones read the last valid dword (computed, never stored)
      const int64_t gbc = (FAST && gb[i] >= kbytes) ? kbytes - 4 : gb[i];
      ptr[i] = wp + m[i] * ld + gbc;
    }
  }

  __device__ __forceinline__ void load(Slot &s, int64_t c0, bool full) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint8_t *p = ptr[i] + c0 * ld;
      if (FAST && full) {
        s.r[i] = *reinterpret_cast<const uint32_t *>(p);
      } else if (FAST) {
        const bool in = c0 + m[i] < L;
        const uint32_t v = *reinterpret_cast<const uint32_t *>(in ? p : base);
        s.r[i] = in ? v : 0u;
      } else {
        const bool in = full || c0 + m[i] < L;
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (in && gb[i] + b < kbytes) w |= (uint32_t)p[b] << (8 * b);
        s.r[i] = w;
      }
    }
  }

  __device__ __forceinline__ static void store(const Slot &s, int8_t *lds, int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!has(i, wave)) break;
      const int u = i * kThreads + tid;
      *reinterpret_cast<v4i *>(lds + Lay::at(u / Lay::kChunks, u % Lay::kChunks)) = decode16(s.r[i]);
    }
  }
};

// ---------------------------------------------------------------------------
// Tile shapes: BM x BN outputs per workgroup, WM x WN waves, each wave a
// (BM/WM) x (BN/WN) block of 16x16 MFMA results; PF = steps of global-load
// prefetch (register slots); OCC = waves per SIMD the registers are sized for;
// PIN = keep each step's global loads ahead of its MFMAs (without it the
// compiler may sink them below, shortening the prefetch distance).
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_, int PF_, int OCC_, bool PIN_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, PF = PF_, OCC = OCC_;
  static constexpr bool PIN = PIN_;
  static_assert(WM * WN * 64 == kThreads, "4 waves");
  static constexpr int TM = BM / WM, TN = BN / WN;  // per wave
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 blocks per wave
  static_assert(FM * 16 == TM && FN * 16 == TN, "wave tile must be a multiple of 16");
};

template <int OP, class T, bool FAST>
struct Stages;

template <class T, bool FAST>
struct Stages<FWD, T, FAST> {
  CopyOp<T::BM, FAST> q;
  DecodeOp<T::BN, FAST> p;
  struct Slot {
    typename CopyOp<T::BM, FAST>::Slot q;
    typename DecodeOp<T::BN, FAST>::Slot p;
  };
  __device__ __forceinline__ void init(const Args &a, int64_t q0, int64_t p0, int tid) {
    q.init(a.q, a.ldq, a.R, a.L, q0, tid);
    p.init(static_cast<const uint8_t *>(a.p), a.ldp, a.Cc, a.L, p0, tid);
  }
  __device__ __forceinline__ void load(Slot &s, int64_t c0, bool full) const {
    q.load(s.q, c0, full);
    p.load(s.p, c0, full);
  }
  __device__ __forceinline__ static void store(const Slot &s, int8_t *lq, int8_t *lp, int tid) {
    CopyOp<T::BM, FAST>::store(s.q, lq, tid);
    DecodeOp<T::BN, FAST>::store(s.p, lp, tid);
  }
};

template <class T, bool FAST>
struct Stages<DX, T, FAST> {
  CopyOp<T::BM, FAST> q;
  DecodeRowOp<T::BN, FAST> p;
  struct Slot {
    typename CopyOp<T::BM, FAST>::Slot q;
    typename DecodeRowOp<T::BN, FAST>::Slot p;
  };
  __device__ __forceinline__ void init(const Args &a, int64_t q0, int64_t p0, int tid) {
    q.init(a.q, a.ldq, a.R, a.L, q0, tid);
    p.init(static_cast<const uint8_t *>(a.p), a.ldp, a.Cc >> 2, a.L, p0, tid);
  }
  __device__ __forceinline__ void load(Slot &s, int64_t c0, bool full) const {
    q.load(s.q, c0, full);
    p.load(s.p, c0, full);
  }
  __device__ __forceinline__ static void store(const Slot &s, int8_t *lq, int8_t *lp, int tid) {
    CopyOp<T::BM, FAST>::store(s.q, lq, tid);
    DecodeRowOp<T::BN, FAST>::store(s.p, lp, tid);
  }
};

template <class T, bool FAST>
struct Stages<DW, T, FAST> {
  RowCopyOp<T::BM, FAST> q;
  RowCopyOp<T::BN, FAST> p;
  struct Slot {
    typename RowCopyOp<T::BM, FAST>::Slot q;
    typename RowCopyOp<T::BN, FAST>::Slot p;
  };
  __device__ __forceinline__ void init(const Args &a, int64_t q0, int64_t p0, int tid) {
    q.init(a.q, a.ldq, a.R, a.L, q0, tid);
    p.init(static_cast<const int8_t *>(a.p), a.ldp, a.Cc, a.L, p0, tid);
  }
  __device__ __forceinline__ void load(Slot &s, int64_t c0, bool full) const {
    q.load(s.q, c0, full);
    p.load(s.p, c0, full);
  }
  __device__ __forceinline__ static void store(const Slot &s, int8_t *lq, int8_t *lp, int tid) {
    RowCopyOp<T::BM, FAST>::store(s.q, lq, tid);
    RowCopyOp<T::BN, FAST>::store(s.p, lp, tid);
  }
};

// One contraction step of a wave's sub-tile: fragments from LDS, FM x FN
// MFMAs.  Frags<OP, T> holds the lane's fragment addresses inside one LDS
// stage; step() reads the fragments of the stage at (qb, pb) and accumulates.
template <class T>
__device__ __forceinline__ void mfma_block(v4i (&acc)[T::FM][T::FN], const v4i (&fp)[T::FN],
                                           const v4i &fq, int i) {
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fp[j], fq, acc[i][j], 0, 0, 0);
}

// Forward and dX: contraction-contiguous LDS rows (swz layout), one 16-byte
// read per fragment: row lane % 16 of the 16-row block, chunk lane / 16.
template <int OP, class T>
struct Frags {
  int qoff, poff;
  __device__ __forceinline__ void init(int lane, int wm, int wn) {
    // block bases are multiples of 16 rows, so the swizzle depends on the lane only
    const int frag = swz(lane & 15, lane >> 4);
    qoff = wm * T::TM * LP + frag;
    poff = wn * T::TN * LP + frag;
  }
  __device__ __forceinline__ void step(v4i (&acc)[T::FM][T::FN], const int8_t *qb,
                                       const int8_t *pb) const {
    v4i fp[T::FN];
#pragma unroll
    for (int j = 0; j < T::FN; ++j) fp[j] = *reinterpret_cast<const v4i *>(pb + poff + j * 16 * LP);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
      mfma_block<T>(acc, fp, *reinterpret_cast<const v4i *>(qb + qoff + i * 16 * LP), i);
  }
};

// Transposing fragment reads from a RowLayout tile (rows = contraction).
// ds_read_b64_tr_b8 transposes 8x8 bytes inside each 16-lane group: result
// byte b of lane i is byte i % 8 of the 8 bytes that lane 2b + i / 8 of the
// group addressed.  So if lanes 2r and 2r + 1 address the two halves of a
// 16-byte chunk (16 output indices) in contraction row m_r, lane i receives
// output index i at the 8 rows m_0 .. m_7.  Lane group g takes rows
// 16g .. 16g + 7 in the first read and 16g + 8 .. 16g + 15 in the second, so
// byte p of lane group g holds contraction index 16g + p: the same order as a
// 16-byte read of chunk g of a contraction-contiguous row (swz layout), and
// the two kinds of fragment can be paired in one MFMA.
struct TrRead {
  template <class Lay>
  __device__ __forceinline__ static int off(int c, int lane) {
    const int g = lane >> 4, i = lane & 15;
    return Lay::at(16 * g + (i >> 1), c) + 8 * (i & 1);
  }
  // second: byte distance of 8 rows (8 * BT: sw and the block shift repeat)
  __device__ __forceinline__ static v4i frag(const int8_t *p, int second) {
    typedef int32_t v2i __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i lds_v2i;
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(p));
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(p + second));
    return v4i{lo.x, lo.y, hi.x, hi.y};
  }
};

// dX: Q (dC rows) contraction-contiguous in the swz layout, P (decoded W,
// rows = contraction n) in a RowLayout, read transposed.
template <class T>
struct Frags<DX, T> {
  typedef RowLayout<T::BN> PL;
  int qoff, poff[T::FN];
  __device__ __forceinline__ void init(int lane, int wm, int wn) {
    qoff = wm * T::TM * LP + swz(lane & 15, lane >> 4);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) poff[j] = TrRead::off<PL>(wn * T::FN + j, lane);
  }
  __device__ __forceinline__ void step(v4i (&acc)[T::FM][T::FN], const int8_t *qb,
                                       const int8_t *pb) const {
    v4i fp[T::FN];
#pragma unroll
    for (int j = 0; j < T::FN; ++j) fp[j] = TrRead::frag(pb + poff[j], 8 * T::BN);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
      mfma_block<T>(acc, fp, *reinterpret_cast<const v4i *>(qb + qoff + i * 16 * LP), i);
  }
};

// dW: both operands in RowLayouts (rows = contraction m), both read transposed.
template <class T>
struct Frags<DW, T> {
  typedef RowLayout<T::BM> QL;
  typedef RowLayout<T::BN> PL;
  int qoff[T::FM], poff[T::FN];
  __device__ __forceinline__ void init(int lane, int wm, int wn) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) qoff[i] = TrRead::off<QL>(wm * T::FM + i, lane);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) poff[j] = TrRead::off<PL>(wn * T::FN + j, lane);
  }
  __device__ __forceinline__ void step(v4i (&acc)[T::FM][T::FN], const int8_t *qb,
                                       const int8_t *pb) const {
    v4i fp[T::FN];
#pragma unroll
    for (int j = 0; j < T::FN; ++j) fp[j] = TrRead::frag(pb + poff[j], 8 * T::BN);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) mfma_block<T>(acc, fp, TrRead::frag(qb + qoff[i], 8 * T::BM), i);
  }
};

// LDS bytes of one pipeline stage of each operand, and of the kernel's two stages.
template <int OP, class T>
struct StageBytes {
  static constexpr int Q = OP == DW ? RowLayout<T::BM>::kBytes : T::BM * LP;
  static constexpr int P = OP == FWD ? T::BN * LP : RowLayout<T::BN>::kBytes;
  static constexpr int kLds = 2 * (Q + P);
};

// Epilogue: lane holds O[row][col .. col+3] of each 16x16 block of a wave's
// sub-tile starting at (r0, c0); `inside` says the workgroup's whole tile is
// inside the output.
template <class T>
__device__ __forceinline__ void store_tile(const Args &a, const v4i (&acc)[T::FM][T::FN], int64_t r0,
                                           int64_t c0, bool inside, int lane) {
  const int64_t rbase = r0 + (lane & 15);
  const int64_t cbase = c0 + (lane >> 4) * 4;
  if (a.o.vec && inside) {
    // Lane l of a fragment holds row l % 16, so neighbouring lanes would hit
    // different rows, which a CU drains at a third of the rate of
    // row-contiguous stores.  A lane permutation (ds_bpermute, no LDS memory;
    // every lane is active here) moves row L / 4, columns 4 (L % 4) .. + 3 to
    // lane L, so four neighbouring lanes write one 16-column run of a row.
    const int src = 4 * ((lane >> 2) + 16 * (lane & 3));
    const int64_t rp = r0 + (lane >> 2), cp = c0 + 4 * (lane & 3);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int64_t row = rp + i * 16;
      const float r = row_scale(a.o, row);
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        v4i v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_ds_bpermute(src, acc[i][j][e]);
        put4(a.o, a.Cc, row, cp + j * 16, v, r);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int64_t row = rbase + i * 16;
    if (row >= a.R) continue;
    const float r = row_scale(a.o, row);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int64_t col = cbase + j * 16;
      if (a.o.vec && col + 3 < a.Cc) {
        put4(a.o, a.Cc, row, col, acc[i][j], r);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < a.Cc) put1(a.o, a.Cc, row, col + e, acc[i][j][e], r);
      }
    }
  }
}

template <int OP, class T, bool FAST>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(T::OCC)))
void tgemm_kernel(Args a) {
  typedef StageBytes<OP, T> SB;
  __shared__ __attribute__((aligned(16))) int8_t smem[SB::kLds];
  int8_t *const sq = smem;               // two Q stages
  int8_t *const sp = smem + 2 * SB::Q;   // two P stages

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;

  int32_t tr, tc;
  tile_rc(xcd_tile((int32_t)blockIdx.x, a.tiles, a.xcds), a.tiles / a.tiles_c, a.tiles_c, a.band_cols,
          &tr, &tc);
  const int64_t q0 = (int64_t)tr * T::BM;
  const int64_t p0 = (int64_t)tc * T::BN;

  v4i acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  typedef Stages<OP, T, FAST> S;
  S st;
  st.init(a, q0, p0, tid);
  typename S::Slot slot[T::PF];

  const int32_t nk = (int32_t)((a.L + BK - 1) / BK);  // steps
  const int32_t nfull = (int32_t)(a.L / BK);          // steps entirely inside L
  // The loop runs whole groups of PF steps.  Steps past the contraction load
  // zeros (their loads are guarded off), so padding the last group adds
  // nothing to the sums and the loop has no early exit.
  const int32_t ngroups = (nk + T::PF - 1) / T::PF;

#pragma unroll
  for (int s = 0; s < T::PF; ++s) st.load(slot[s], (int64_t)s * BK, s < nfull);
  S::store(slot[0], sq, sp, tid);
  lds_barrier();

  Frags<OP, T> fr;
  fr.init(lane, wm, wn);

  // one group of PF steps; `full` says that every step it loads lies inside
  // the contraction (then the loads carry no guard at all)
  auto group = [&](int32_t g, auto full) {
#pragma unroll
    for (int u = 0; u < T::PF; ++u) {
      const int32_t j = g * T::PF + u;
      // refill the slot this step's data came from with step j + PF
      st.load(slot[u], (int64_t)(j + T::PF) * BK, decltype(full)::value || j + T::PF < nfull);
      if constexpr (T::PIN) __builtin_amdgcn_sched_barrier(0);
      const int cur = j & 1;
      fr.step(acc, sq + cur * SB::Q, sp + cur * SB::P);
      S::store(slot[(u + 1) % T::PF], sq + (cur ^ 1) * SB::Q, sp + (cur ^ 1) * SB::P, tid);
      lds_barrier();
    }
  };
  // groups g whose loads (steps up to (g + 2) * PF - 1) are all full
  const int32_t gfull = nfull / T::PF - 1 > 0 ? nfull / T::PF - 1 : 0;
  int32_t g = 0;
  for (; g < gfull; ++g) group(g, Flag<true>());
  for (; g < ngroups; ++g) group(g, Flag<false>());

  store_tile<T>(a, acc, q0 + wm * T::TM, p0 + wn * T::TN, q0 + T::BM <= a.R && p0 + T::BN <= a.Cc,
                lane);
}

// ---------------------------------------------------------------------------
// Host side: validation, planning, launch.
// ---------------------------------------------------------------------------

// Tile shapes per product.  Prefetch depth, occupancy and load pinning are
// chosen per product from measured MI355X runs, such that no instantiation
// spills registers.  At occupancy
// 2 the dW accumulators stay in VGPRs; at 1 the compiler moves them to AGPRs
// and copies them between sets every step.
template <int OP>
struct Tiles;
template <>
struct Tiles<FWD> {
  typedef Tile<256, 128, 2, 2, 2, 2> L;  // large outputs
  typedef Tile<128, 144, 4, 1, 2, 2> W;  // outputs of ~240 tiles of this size
  typedef Tile<64, 64, 2, 2, 2, 4> S;    // small / ragged
};
template <>
struct Tiles<DX> {
  typedef Tile<256, 128, 2, 2, 2, 2, true> L;
  typedef Tile<128, 144, 4, 1, 1, 2, true> W;
  typedef Tile<64, 64, 2, 2, 2, 2, true> S;
};
template <>
struct Tiles<DW> {
  typedef Tile<256, 128, 2, 2, 4, 1> L;
  typedef Tile<128, 144, 4, 1, 2, 2> W;
  typedef Tile<64, 64, 2, 2, 2, 2> S;
};
typedef Tiles<FWD> TileShapes;  // the shapes (not the tuning) are common

enum TileId { TL = 0, TW = 1, TS = 2, kTiles = 3 };

struct TileInfo {
  int bm, bn;
  double eff;  // relative MFMA efficiency (operand bytes per MAC read from LDS)
};

const TileInfo kTileInfo[kTiles] = {
    // efficiencies relative to the large tile, from measured MI355X runs
    // (operand bytes staged per MAC grow as the tile shrinks)
    {TileShapes::L::BM, TileShapes::L::BN, 1.0},
    {TileShapes::W::BM, TileShapes::W::BN, 0.8},
    {TileShapes::S::BM, TileShapes::S::BN, 0.3},
};

template <int OP>
int lds_of_tile(int tile) {
  return tile == TL   ? StageBytes<OP, typename Tiles<OP>::L>::kLds
         : tile == TW ? StageBytes<OP, typename Tiles<OP>::W>::kLds
                      : StageBytes<OP, typename Tiles<OP>::S>::kLds;
}


struct Shape {
  int64_t R, Cc, L;
};

Shape shape_of(int op, int64_t M, int64_t N, int64_t K) {
  if (op == FWD) return {M, N, K};
  if (op == DX) return {M, K, N};
  return {K, N, M};
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Pick the tile with the least estimated time: rounds of one workgroup per
// CU times the MACs of one tile at that tile's efficiency.  dX of at least
// 512 rows is the exception: when its 128 x 144 tiles would leave more than
// half the CUs idle even with the contraction split inside each workgroup,
// and its 64 x 64 tiles fill every CU, the small tiles win (several small
// workgroups share a CU).  Measured on MI355X, dX at 1782 x 3456 x 1280 takes 24 against
// 27.5 us, at 640 x 8192 x 2048 36 against 66 us; at 3000 x 3456 x 1280 (216
// tiles of 128 x 144) the split tile stays faster, 30 against 34 us.
int pick_tile(const Shape &s, int64_t cus);
int pick_tile_for(int op, const Shape &s, int64_t cus) {
  const int t = pick_tile(s, cus);
  if (op != DX || t != TW) return t;
  const TileInfo &w = kTileInfo[TW], &sm = kTileInfo[TS];
  const int64_t tw = ceil_div(s.R, w.bm) * ceil_div(s.Cc, w.bn);
  const int64_t ts = ceil_div(s.R, sm.bm) * ceil_div(s.Cc, sm.bn);
  return s.R >= 4 * w.bm && 2 * tw <= cus && ts >= cus ? TS : t;
}

int pick_tile(const Shape &s, int64_t cus) {
  int best = TS;
  double best_cost = 0;
  for (int t = 0; t < kTiles; ++t) {
    const TileInfo &ti = kTileInfo[t];
    const int64_t tiles = ceil_div(s.R, ti.bm) * ceil_div(s.Cc, ti.bn);
    const double cost = (double)ceil_div(tiles, cus) * ti.bm * ti.bn / ti.eff;
    if (t == 0 || cost < best_cost) {
      best = t;
      best_cost = cost;
    }
  }
  return best;
}

// Bands of tile columns for the workgroup order: with nb bands, each of the
// x XCDs reads about nb/x of the Q operand (rows) and 1/nb of the P operand
// (columns); the XCDs fetch about nb*Q + x*P/nb bytes between them.
int32_t pick_band_cols(int op, int64_t M, int64_t N, int64_t K, int32_t tiles_c, int32_t xcds) {
  const double q = op == DX ? (double)M * N : (double)M * K;          // Q operand bytes
  const double p = op == DW ? (double)M * N : (double)N * (K / 4);    // P operand bytes
  int best_nb = 1;
  double best = 0;
  for (int nb = 1; nb <= xcds; nb *= 2) {
    if (nb > tiles_c) break;
    const double bytes = nb * q + (double)xcds * p / nb;
    if (nb == 1 || bytes < best) {
      best = bytes;
      best_nb = nb;
    }
  }
  return (int32_t)ceil_div(tiles_c, best_nb);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  if (a > 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// dimension, packing and bound checks shared by the calls and the plan query
int check_dims(int op, int64_t M, int64_t N, int64_t K) {
  if (op < FWD || op > DW) return TGEMM_ERR_DIM;
  if (M < 1 || N < 1 || K < 1) return TGEMM_ERR_DIM;
  int64_t t;
  // every operand and output byte count (int32 outputs: 4 bytes) fits int64
  if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &t) || !mul_ok(M, N, &t) || !mul_ok(t, 4, &t) ||
      !mul_ok(K, N, &t) || !mul_ok(t, 4, &t))
    return TGEMM_ERR_DIM;
  if (op != DW && K % 4 != 0) return TGEMM_ERR_PACK;
  const Shape s = shape_of(op, M, N, K);
  const int64_t bound = op == DW ? TGEMM_INT8_MAX_CONTRACTION : TGEMM_TERNARY_MAX_CONTRACTION;
  if (s.L > bound) return TGEMM_ERR_BOUND;
  // smallest tile must keep the workgroup count within a 1-D grid
  if (ceil_div(s.R, TileShapes::S::BM) * ceil_div(s.Cc, TileShapes::S::BN) > INT32_MAX)
    return TGEMM_ERR_DIM;
  return TGEMM_OK;
}

bool fast_ok(int op, int64_t M, int64_t N, int64_t K, uintptr_t qalign, uintptr_t palign) {
  (void)M;
  if (op == FWD) return K % 16 == 0 && qalign % 16 == 0 && palign % 4 == 0;
  if (op == DX) return N % 16 == 0 && K % 16 == 0 && qalign % 16 == 0 && palign % 4 == 0;
  return K % 16 == 0 && N % 16 == 0 && qalign % 16 == 0 && palign % 16 == 0;
}

uintptr_t align_of(const void *p) {
  const uintptr_t v = (uintptr_t)p;
  return v ? (v & (~v + 1)) : ((uintptr_t)1 << 20);
}

// ---------------------------------------------------------------------------
// The contraction split inside the workgroup (dW, and dX with few tiles).
// dW's output is small (K x N) and its contraction long (M), so at the large
// shapes there are only about as many tiles as CUs; dX of a few thousand rows
// (the pages' backward batch of 1782) has fewer.  One 4-wave workgroup per CU
// then leaves each SIMD a single wave, whose MFMAs stop at every barrier and
// LDS wait.  Here a workgroup has two 4-wave halves on the same tile: half h
// takes the contraction steps j = 2t + h, each half with its own LDS stages,
// so every SIMD runs two waves.  At the end half 1 hands its int32 sums to
// half 0 through LDS and half 0 adds and stores them: a fixed order, so the
// result is exact and identical on every call, with no atomics and no
// scratch memory.
// ---------------------------------------------------------------------------
template <int OP, class T, bool FAST>
__global__ __attribute__((amdgpu_flat_work_group_size(2 * kThreads, 2 * kThreads), amdgpu_waves_per_eu(2)))
void tgemm_split(Args a) {
  typedef StageBytes<OP, T> SB;
  constexpr int kHalf = 2 * (SB::Q + SB::P);                      // a half's two stages
  constexpr int kRed = T::FM * T::FN * kThreads * 16;             // half 1's sums
  constexpr int kBytes = 2 * kHalf > kRed ? 2 * kHalf : kRed;
  __shared__ __attribute__((aligned(16))) int8_t smem[kBytes];

  const int h = (int)(threadIdx.x >> 8);         // half (wave-uniform)
  const int tid = (int)(threadIdx.x & (kThreads - 1));
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
  int8_t *const sq = smem + h * kHalf;
  int8_t *const sp = sq + 2 * SB::Q;

  int32_t tr, tc;
  tile_rc(xcd_tile((int32_t)blockIdx.x, a.tiles, a.xcds), a.tiles / a.tiles_c, a.tiles_c, a.band_cols,
          &tr, &tc);
  const int64_t q0 = (int64_t)tr * T::BM;
  const int64_t p0 = (int64_t)tc * T::BN;

  v4i acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  typedef Stages<OP, T, FAST> S;
  S st;
  st.init(a, q0, p0, tid);
  typename S::Slot slot[T::PF];
  Frags<OP, T> fr;
  fr.init(lane, wm, wn);

  const int32_t nk = (int32_t)((a.L + BK - 1) / BK);
  const int32_t nfull = (int32_t)(a.L / BK);
  const int32_t nt = (nk + 1) / 2;                        // steps per half (same for both)
  const int32_t ngroups = (nt + T::PF - 1) / T::PF;
  auto c0_of = [&](int32_t t) { return (int64_t)(2 * t + h) * BK; };
  auto full_of = [&](int32_t t) { return 2 * t + h < nfull; };

#pragma unroll
  for (int s = 0; s < T::PF; ++s) st.load(slot[s], c0_of(s), full_of(s));
  S::store(slot[0], sq, sp, tid);
  lds_barrier();

  auto group = [&](int32_t g, auto full) {
#pragma unroll
    for (int u = 0; u < T::PF; ++u) {
      const int32_t t = g * T::PF + u;
      st.load(slot[u], c0_of(t + T::PF), decltype(full)::value || full_of(t + T::PF));
      if constexpr (T::PIN) __builtin_amdgcn_sched_barrier(0);
      const int cur = t & 1;
      fr.step(acc, sq + cur * SB::Q, sp + cur * SB::P);
      S::store(slot[(u + 1) % T::PF], sq + (cur ^ 1) * SB::Q, sp + (cur ^ 1) * SB::P, tid);
      lds_barrier();
    }
  };
  // groups whose loads (half steps up to (g + 2) * PF - 1, i.e. steps up to
  // 2 ((g + 2) PF - 1) + 1) are all full, for both halves
  const int32_t gfull = nfull / (2 * T::PF) - 1 > 0 ? nfull / (2 * T::PF) - 1 : 0;
  int32_t g = 0;
  for (; g < gfull; ++g) group(g, Flag<true>());
  for (; g < ngroups; ++g) group(g, Flag<false>());

  // half 1 -> LDS -> half 0 (the last barrier above ends every read of the stages)
  v4i *red = reinterpret_cast<v4i *>(smem);
  if (h == 1) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) red[(i * T::FN + j) * kThreads + tid] = acc[i][j];
  }
  lds_barrier();
  if (h == 1) return;
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] += red[(i * T::FN + j) * kThreads + tid];
  store_tile<T>(a, acc, q0 + wm * T::TM, p0 + wn * T::TN, q0 + T::BM <= a.R && p0 + T::BN <= a.Cc,
                lane);
}

// ---------------------------------------------------------------------------
// Streaming kernels: forward and dX on large outputs.
//
// One workgroup of 8 waves per CU, persistent over its tiles of 512 output
// rows x BN output columns (forward 16384 x 3456: 768 tiles of 512 x 144,
// three per CU; dX 16384 x 1280: 256 tiles of 512 x 160, one per CU).  The
// waves are stacked 8 x 1, each a 64 x BN sub-tile, two waves per SIMD; the
// tall tile spreads each decoded weight over 512 rows, which halves the
// decode work per MAC of a 256-row tile.
//
// The row operand Q (A for the forward, dC for dX: rows of the output, along
// the contraction) and the packed weight rows go straight from global memory
// into LDS (never through VGPRs): Q with 16-byte loads into a ring of three
// stages, packed codes with 4-byte loads into a ring of two.  Each wave
// decodes the packed dwords it loaded itself (16 codes -> a 16-byte chunk,
// decode16) into a ring of three decoded stages, two steps ahead, so the
// codes are decoded once per tile load [P10425 "What this adds"] and the
// decode needs only the wave's own load count, no extra barrier.
//   forward: decoded stage = rows n of the tile, 64 codes of k each (swz
//            layout), read as fragments with 16-byte LDS reads;
//   dX:      decoded stage = rows n of the contraction, BN codes of k each
//            (RowLayout), read as fragments with the transposing LDS read
//            (TrRead), as the packed rows of W lie along k [P10855 PR body].
//
// Register pipeline: during the MFMAs of step g a wave reads the Q fragments
// and the first weight fragments of step g + 1 (Q fragments stay in
// registers for the whole step; weight fragments stream through, kPD ahead),
// so the MFMA issue does not wait for LDS at a step boundary.  The barrier
// that starts step g therefore publishes Q(g + 1) and decoded W(g + 1), and a
// Q stage is free once the step before its own has read it: three stages
// keep the loads two steps ahead.
//
// The loads come from inline assembly, so the compiler does not drain them
// at every LDS read; each wave waits for its own loads with explicit vmcnt
// counts (memory operations of a wave complete in issue order, so vmcnt(N),
// N = the operations issued after the awaited one, is exactly that wait):
//
//   step g  cols 0 .. 4: issue batch B(g + 3) = packed W, then Q, of step g + 3
//           col 5:  wait for the packed W of step g + 2, fetch it for decoding
//           end:    decode it; wait for Q(g + 2); barrier
//
// The loads of a step are spread over the MFMA columns so that the eight
// waves do not queue them all at once behind the barrier.  A tile's output is
// stored right after its last step, while loads of the next tile are in
// flight; its kStores stores are younger than what the next two waits await,
// and those waits count them.  The last steps re-load the final step (valid
// addresses, never used), which keeps the counts uniform; the kernel waits
// for every load before it ends, so no transfer into LDS outlives it.
// ---------------------------------------------------------------------------
namespace fs {

constexpr int S = 3;                              // Q stages
constexpr int DS = 3;                             // decoded weight stages
constexpr int PS = 2;                             // packed weight stages
constexpr int kWaves = 8, kNT = 64 * kWaves;
constexpr int BM = 512, TM = 64, FM = TM / 16;    // 8 x 1 waves of 64 rows
constexpr int kAStage = BM * LP;                  // Q rows of one step
constexpr int kALoads = kAStage / 1024 / kWaves;  // 16-byte loads per wave per step
constexpr int kPD = 3;                            // weight fragments read ahead

template <int OP>
struct Geo;

template <int OP>
struct GeoBase {
  static constexpr int BN = OP == FWD ? 144 : 160;
  static constexpr int FN = BN / 16;
  // forward: decoded rows n of the tile (swz layout); dX: decoded rows = the
  // step's 64 contraction indices n, BN bytes each (RowLayout)
  static constexpr int kWdStage = OP == FWD ? BN * LP : RowLayout<BN>::kBytes;
  // packed dwords of one step: forward BN rows x 4 (64 codes of k); dX 64
  // rows x BN / 16 (BN codes of k); in units of one 64-lane load
  static constexpr int kDwPerRow = OP == FWD ? BK / 16 : BN / 16;
  static constexpr int kUnits = (OP == FWD ? BN * BK / 16 : BK * BN / 16) / 64;
  // Units (loads and their decode) per wave: q or q + 1, the extra ones on
  // the last waves; waves w and w + 4 share a SIMD, so per-SIMD decode work
  // differs by at most one unit.
  static constexpr int kUnitQ = kUnits / kWaves, kUnitR = kUnits % kWaves;
  static constexpr int kWpLoads = kUnitQ + (kUnitR ? 1 : 0);
  __host__ __device__ static constexpr int units_of(int w) {
    return kUnitQ + (w >= kWaves - kUnitR ? 1 : 0);
  }
  __host__ __device__ static constexpr int first_unit(int w) {
    return kUnitQ * w + (w > kWaves - kUnitR ? w - (kWaves - kUnitR) : 0);
  }
  static constexpr int kWpStage = kUnits * 256;   // unit u at byte 256 u
  static constexpr int kOffWd = S * kAStage;
  static constexpr int kOffWp = kOffWd + DS * kWdStage;
  static constexpr int kLds = kOffWp + PS * kWpStage;
  static constexpr int kBatch = kALoads + kUnitQ; // loads of a step, fewest over the waves
  static constexpr int kStores = FM * FN;
  static constexpr int kStoresPair = FM * (FN / 2 + FN % 2);   // bf16 stores of fragment pairs
  // Waits count the operations issued after the awaited one; a wave with an
  // extra unit has one more, and counting fewer than there are is safe.
  static constexpr int kWaitMid = kALoads + kBatch;  // own packed W(g + 2): Q(g + 2), B(g + 3) after it
  static constexpr int kWaitEnd = kBatch;            // own Q(g + 2): B(g + 3) after it
  static_assert(kALoads * kWaves * 1024 == kAStage, "Q stage = whole 1 KB wave loads");
  static_assert(kUnits * 64 * 4 == (OP == FWD ? BN * 16 : BK * BN / 4) && kUnitQ >= 1, "packed stage");
  static_assert(first_unit(kWaves - 1) + units_of(kWaves - 1) == kUnits, "units");
  static_assert(kLds <= 160 * 1024, "LDS");
  static_assert(kWaitMid + kStores <= 63, "vmcnt field");
  static_assert(kPD < FN - FM && kALoads + 1 < FN, "prefetch distance, load columns");
};
template <>
struct Geo<FWD> : GeoBase<FWD> {};
template <>
struct Geo<DX> : GeoBase<DX> {};

// 16 bytes per lane from sbase + voff into LDS at lds + 16 * lane
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const void *sbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
// 4 bytes per lane from sbase + voff into LDS at lds + 4 * lane
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, const void *sbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
// wait until at most N of this wave's memory operations are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// the same, then this wave's LDS operations, then meet the other waves
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace fs

struct SArgs {
  const int8_t *Q;    // A (forward) or dC (dX): rows of the output along the contraction
  const uint8_t *Wp;  // packed weights
  Out o;              // column scale, when scaled: o.cscal (o.cs is null)
  int32_t R, Cc, L;   // output rows, output columns, contraction
  int32_t ldq;        // Q row stride (= L)
  int32_t kb;         // packed row stride (K / 4)
  int32_t tiles_c, tiles;
  int32_t nk;         // L / 64
  int32_t xcds;       // workgroup b runs on XCD b % xcds
};

// The decode of a wave's own packed dwords, in two halves so that the reads
// can go out well before their results are used: fs_decode_read fetches the
// dwords (16 codes each), fs_decode_write turns each into a 16-byte chunk of
// int8 weights (decode16) and stores it in the decoded stage.
template <int OP>
__device__ __forceinline__ void fs_decode_read(uint32_t (&x)[fs::Geo<OP>::kWpLoads], const int8_t *src,
                                               int wave, int lane) {
  typedef fs::Geo<OP> G;
#pragma unroll
  for (int i = 0; i < G::kWpLoads; ++i)
    if (i < G::units_of(wave))
      x[i] = *reinterpret_cast<const uint32_t *>(src + 256 * (G::first_unit(wave) + i) + 4 * lane);
}
template <int OP>
__device__ __forceinline__ void fs_decode_write(const uint32_t (&x)[fs::Geo<OP>::kWpLoads], int8_t *dst,
                                                int wave, int lane) {
  typedef fs::Geo<OP> G;
#pragma unroll
  for (int i = 0; i < G::kWpLoads; ++i)
    if (i < G::units_of(wave)) {
      const int d = 64 * (G::first_unit(wave) + i) + lane;  // packed dword of the step
      const int off = OP == FWD ? swz(d >> 2, d & 3)        // row n = d / 4, 16 codes of k
                                : RowLayout<G::BN>::at(d / G::kDwPerRow, d % G::kDwPerRow);
      *reinterpret_cast<v4i *>(dst + off) = decode16(x[i]);
    }
}

template <int OP>
__global__ __attribute__((amdgpu_flat_work_group_size(fs::kNT, fs::kNT), amdgpu_waves_per_eu(2)))
void tgemm_stream(SArgs a) {
  using namespace fs;
  typedef Geo<OP> G;
  constexpr int BN = G::BN, FN = G::FN;
  __shared__ __attribute__((aligned(1024))) int8_t smem[G::kLds];
  // row scales of the tile (scaled output): each wave loads those of its own
  // 64 rows straight into LDS at the tile's first step, and reads them back
  // when it stores the tile
  __shared__ __attribute__((aligned(256))) float rs_s[BM];
  const bool scaled_out = a.o.kind != OUT_I32;
  const uint32_t lbase = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Tiles of this workgroup: the tile positions (row-major over the tile
  // grid) are split into one contiguous run per XCD (workgroup b runs on XCD
  // b % xcds), and the nx workgroups of an XCD take every nx-th position of
  // its run, so the tiles an XCD works on at one time share Q rows and the
  // weight columns in its L2.
  const int32_t nx = (int32_t)gridDim.x / a.xcds, xcd = (int32_t)blockIdx.x % a.xcds;
  const int32_t j0 = (int32_t)blockIdx.x / a.xcds;
  const int32_t q8 = a.tiles / a.xcds, r8 = a.tiles % a.xcds;
  const int32_t start = xcd * q8 + (xcd < r8 ? xcd : r8) + j0;
  const int32_t cnt = q8 + (xcd < r8 ? 1 : 0);
  const int32_t ntile = cnt > j0 ? (cnt - j0 + nx - 1) / nx : 0;
  if (ntile == 0) return;

  // Load offsets of a tile (recomputed per tile, not kept live across the
  // loop).  Q load i of this wave fills tile rows 16 L .. 16 L + 15 (L =
  // kALoads * wave + i); lane l lands in slot l % 4 of row 16 L + l / 4 and so
  // fetches the chunk the swizzle puts there.  Packed load i (i <
  // units_of(wave)) fills unit u = first_unit(wave) + i of the step, 256
  // bytes at 256 u of the packed stage: dwords d = 64 u + l.  Forward: row
  // d / 4 of the tile's columns, dword d % 4 of the step's 16 bytes.  dX:
  // contraction row d / kDwPerRow of the step, dword d % kDwPerRow of the
  // tile's BN / 4 bytes.  Rows and columns past the output load a valid
  // neighbour (computed, never stored).
  uint32_t offA[kALoads], offW[G::kWpLoads];
  auto set_loads = [&](int32_t it) {
    const int32_t pos = start + it * nx;
    const int32_t m0 = pos / a.tiles_c * BM, n0 = pos % a.tiles_c * BN;
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const int r = 16 * (kALoads * wave + i) + (lane >> 2);
      const int32_t m = m0 + r < a.R ? m0 + r : a.R - 1;
      offA[i] = (uint32_t)(m * a.ldq + 16 * ((lane & 3) ^ ((r >> 1) & 3)));
    }
#pragma unroll
    for (int i = 0; i < G::kWpLoads; ++i) {
      const int d = 64 * (G::first_unit(wave) + (i < G::units_of(wave) ? i : 0)) + lane;
      if constexpr (OP == FWD) {
        const int32_t n = n0 + (d >> 2) < a.Cc ? n0 + (d >> 2) : a.Cc - 1;
        offW[i] = (uint32_t)(n * a.kb + 4 * (d & 3));
      } else {
        const int32_t kw = n0 / 4 + 4 * (d % G::kDwPerRow);
        offW[i] = (uint32_t)((d / G::kDwPerRow) * a.kb + (kw + 4 <= a.kb ? kw : a.kb - 4));
      }
    }
  };
  // packed-code and Q base addresses of step s of the load tile
  auto wbase = [&](int32_t s) {
    return OP == FWD ? a.Wp + 16 * s : a.Wp + (int64_t)BK * s * a.kb;
  };
  auto issue = [&](int32_t st, int32_t ps, int32_t s) {
    const uint32_t lw = lbase + G::kOffWp + ps * G::kWpStage + 256 * G::first_unit(wave);
#pragma unroll
    for (int i = 0; i < G::kWpLoads; ++i)
      if (i < G::units_of(wave)) dma4(lw + 256 * i, offW[i], wbase(s));
    const uint32_t la = lbase + st * kAStage + wave * (kALoads * 1024);
#pragma unroll
    for (int i = 0; i < kALoads; ++i) dma16(la + 1024 * i, offA[i], a.Q + 64 * s);
  };

  v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) acc[i][jj] = v4i{0, 0, 0, 0};

  // load cursor (tile it_ld, step s_ld): the next step whose loads go out;
  // past the end it stays on the last step
  int32_t it_ld = 0, s_ld = 0;
  auto next_load = [&]() {
    if (s_ld + 1 < a.nk) {
      ++s_ld;
    } else if (it_ld + 1 < ntile) {
      ++it_ld;
      s_ld = 0;
      set_loads(it_ld);
    }
  };
  set_loads(0);
  // prologue: steps 0 and 1 land and are decoded (each wave its own units,
  // whose loads it has waited for), then step 2 goes out into packed stage 0
  issue(0, 0, s_ld);
  next_load();
  issue(1, 1, s_ld);
  next_load();
  wait_vm<0>();
  {
    uint32_t x0[G::kWpLoads], x1[G::kWpLoads];
    fs_decode_read<OP>(x0, smem + G::kOffWp, wave, lane);
    fs_decode_read<OP>(x1, smem + G::kOffWp + G::kWpStage, wave, lane);
    fs_decode_write<OP>(x0, smem + G::kOffWd, wave, lane);
    fs_decode_write<OP>(x1, smem + G::kOffWd + G::kWdStage, wave, lane);
  }
  issue(2, 0, s_ld);
  next_load();
  wait_barrier<G::kBatch>();

  // fragment offsets: Q rows of this wave (swz layout); weight fragment jj of
  // a decoded stage at poff + jj * pstep
  const int qoff = wave * TM * LP + swz(lane & 15, lane >> 4);
  const int poff = G::kOffWd + (OP == FWD ? swz(lane & 15, lane >> 4) : TrRead::off<RowLayout<BN>>(0, lane));
  constexpr int pstep = OP == FWD ? 16 * LP : 16;
  auto pfrag = [&](const int8_t *p) -> v4i {
    if constexpr (OP == FWD)
      return *reinterpret_cast<const v4i *>(p);
    else
      return TrRead::frag(p, 8 * BN);
  };

  v4i qc[FM], pf[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) qc[i] = *reinterpret_cast<const v4i *>(smem + qoff + i * 16 * LP);
#pragma unroll
  for (int jj = 0; jj < kPD; ++jj) pf[jj] = pfrag(smem + poff + jj * pstep);
  // every wave's reads of Q stage 0 are done before step 0 loads into it
  wait_barrier<G::kBatch>();

  // Per step g: stage index t = g % 3 of the Q and decoded rings, g % 2 of the
  // packed ring.  Step g loads step g + 3 into Q stage t (read as step g's
  // fragments during step g - 1) and packed stage (g + 1) % 2 (whose codes
  // this wave decoded in step g - 1), computes step g from decoded stage t
  // with Q fragments already in registers, reads step g + 1's fragments from
  // stages t + 1, and decodes step g + 2 from packed stage g % 2 into decoded
  // stage t + 2.
  int32_t gt = 0, gp = 0;
  // stores a tile's vector path issued right before this step: 0, or
  // kStoresPair (bf16 in fragment pairs), or kStores
  int after = 0;
  for (int32_t it = 0; it < ntile; ++it) {
    for (int32_t s = 0; s < a.nk; ++s) {
      const int t1 = gt == 2 ? 0 : gt + 1, t2 = t1 == 2 ? 0 : t1 + 1;
      const uint32_t lw3 = lbase + G::kOffWp + (gp ^ 1) * G::kWpStage + 256 * G::first_unit(wave);
      const uint32_t la3 = lbase + gt * kAStage + wave * (kALoads * 1024);
      const uint8_t *wb3 = wbase(s_ld);
      const int8_t *ab3 = a.Q + 64 * s_ld;
      const int8_t *pc = smem + poff + gt * G::kWdStage;
      const int8_t *pn_ = smem + poff + t1 * G::kWdStage;
      const int8_t *qn_ = smem + qoff + t1 * kAStage;
      if (scaled_out && s == 0) {
        // this wave's row scales of tile it: older than the loads this step
        // issues below, so landed once step 1 has waited for those
        const int32_t m = (start + it * nx) / a.tiles_c * BM + wave * TM + lane;
        dma4((uint32_t)(uintptr_t)rs_s + 4 * TM * wave, 4 * (uint32_t)(m < a.R ? m : a.R - 1), a.o.rs);
      }
      v4i qn[FM], pn[kPD];
#pragma unroll
      for (int i = 0; i < FM; ++i) qn[i] = *reinterpret_cast<const v4i *>(qn_ + i * 16 * LP);
      uint32_t x[G::kWpLoads];
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) {
        // loads of step g + 3, spread over the columns: packed codes at
        // column 0, Q load i at column 1 + i
        if (jj == 0) {
#pragma unroll
          for (int i = 0; i < G::kWpLoads; ++i)
            if (i < G::units_of(wave)) dma4(lw3 + 256 * i, offW[i], wb3);
        }
        if (jj >= 1 && jj <= kALoads) dma16(la3 + 1024 * (jj - 1), offA[jj - 1], ab3);
        if (jj + kPD < FN)
          pf[jj + kPD] = pfrag(pc + (jj + kPD) * pstep);
        else
          pn[jj + kPD - FN] = pfrag(pn_ + (jj + kPD - FN) * pstep);
        if (jj == kALoads + 1) {
          // every load of step g + 3 is out; this wave's packed codes of step
          // g + 2 have landed: fetch them
          if (after == G::kStores)
            wait_vm<G::kWaitMid + G::kStores>();
          else if (after == G::kStoresPair)
            wait_vm<G::kWaitMid + G::kStoresPair>();
          else
            wait_vm<G::kWaitMid>();
          fs_decode_read<OP>(x, smem + G::kOffWp + gp * G::kWpStage, wave, lane);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][jj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pf[jj], qc[i], acc[i][jj], 0, 0, 0);
      }
      fs_decode_write<OP>(x, smem + G::kOffWd + t2 * G::kWdStage, wave, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i) qc[i] = qn[i];
#pragma unroll
      for (int jj = 0; jj < kPD; ++jj) pf[jj] = pn[jj];
      next_load();

      // end of step g: Q(g + 2) has landed and decoded W(g + 2) is written.
      // Stores issued right before this step are younger than Q(g + 2);
      // counting fewer operations than are younger is always safe.
      if (after == G::kStores)
        wait_barrier<G::kWaitEnd + G::kStores>();
      else if (after == G::kStoresPair)
        wait_barrier<G::kWaitEnd + G::kStoresPair>();
      else
        wait_barrier<G::kWaitEnd>();
      after = 0;
      gt = t1;
      gp ^= 1;
    }

    // the tile's output, on its way while the next tile's loads are in flight
    const int32_t pos = start + it * nx;
    const int32_t m0 = pos / a.tiles_c * BM, n0 = pos % a.tiles_c * BN;
    const int32_t rb = m0 + wave * TM + (lane & 15);
    const int32_t cb = n0 + (lane >> 4) * 4;
    // a one-step tile has not waited for anything issued after its row scales
    if (scaled_out && a.nk < 2) wait_vm<0>();
    const float *rsw = rs_s + TM * wave;
    if (a.o.vec8 && m0 + BM <= a.R && n0 + BN <= a.Cc) {
      // bf16: scale and convert in the MFMA layout (lane l: row l % 16, four
      // columns -> two dwords), then give each lane 8 columns of a fragment
      // pair's 32: lane L takes row L / 4, columns 8 (L % 4) .. + 7 (fragment
      // jj for L % 4 < 2, jj + 1 otherwise), so four neighbouring lanes write
      // one 64-byte run with 16-byte stores.  An odd last fragment moves four
      // columns (8 bytes) to each lane, as the int32 path below does.
      const int p4 = lane & 3;
      const int sA = 4 * ((lane >> 2) + 32 * (p4 & 1)), sB = sA + 64;
      const int src = 4 * ((lane >> 2) + 16 * p4);
      const bool hi = p4 >= 2;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const float r = rsw[(lane & 15) + 16 * i];
        uint16_t *orow = static_cast<uint16_t *>(a.o.ptr) +
                         (int64_t)(m0 + wave * TM + (lane >> 2) + 16 * i) * a.Cc + n0;
        uint32_t d[FN][2];
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          d[jj][0] = bf16_pack(scaled(acc[i][jj][0], r, a.o.cscal), scaled(acc[i][jj][1], r, a.o.cscal));
          d[jj][1] = bf16_pack(scaled(acc[i][jj][2], r, a.o.cscal), scaled(acc[i][jj][3], r, a.o.cscal));
        }
#pragma unroll
        for (int jj = 0; jj + 1 < FN; jj += 2) {
          uint4 w;
          const uint32_t a0 = __builtin_amdgcn_ds_bpermute(sA, d[jj][0]), a1 = __builtin_amdgcn_ds_bpermute(sA, d[jj][1]);
          const uint32_t b0 = __builtin_amdgcn_ds_bpermute(sB, d[jj][0]), b1 = __builtin_amdgcn_ds_bpermute(sB, d[jj][1]);
          const uint32_t c0 = __builtin_amdgcn_ds_bpermute(sA, d[jj + 1][0]), c1 = __builtin_amdgcn_ds_bpermute(sA, d[jj + 1][1]);
          const uint32_t e0 = __builtin_amdgcn_ds_bpermute(sB, d[jj + 1][0]), e1 = __builtin_amdgcn_ds_bpermute(sB, d[jj + 1][1]);
          w.x = hi ? c0 : a0;
          w.y = hi ? c1 : a1;
          w.z = hi ? e0 : b0;
          w.w = hi ? e1 : b1;
          *reinterpret_cast<uint4 *>(orow + 16 * jj + 8 * p4) = w;
        }
        if constexpr (FN % 2 == 1) {
          uint2 w;
          w.x = __builtin_amdgcn_ds_bpermute(src, d[FN - 1][0]);
          w.y = __builtin_amdgcn_ds_bpermute(src, d[FN - 1][1]);
          *reinterpret_cast<uint2 *>(orow + 16 * (FN - 1) + 4 * p4) = w;
        }
      }
      after = G::kStoresPair;
    } else if (a.o.vec && m0 + BM <= a.R && n0 + BN <= a.Cc) {
      // Lane l of a fragment holds row l % 16, so neighbouring lanes hit
      // different rows and a CU's stores drain at a third of the rate of
      // row-contiguous ones.  A lane permutation (ds_bpermute, no LDS memory)
      // first moves row L / 4, columns 4 (L % 4) .. + 3 to lane L: four
      // neighbouring lanes then write one 64-byte run.
      const int src = 4 * ((lane >> 2) + 16 * (lane & 3));
      const int32_t rp = m0 + wave * TM + (lane >> 2), cp = n0 + (lane & 3) * 4;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const float r = scaled_out ? rsw[(lane >> 2) + 16 * i] : 0.f;
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          v4i v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_ds_bpermute(src, acc[i][jj][e]);
          put4(a.o, a.Cc, rp + 16 * i, cp + 16 * jj, v, r);
        }
      }
      after = G::kStores;
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int32_t row = rb + 16 * i;
        if (row >= a.R) continue;
        const float r = scaled_out ? rsw[(lane & 15) + 16 * i] : 0.f;
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          const int32_t col = cb + 16 * jj;
          if (a.o.vec && col + 3 < a.Cc) {
            put4(a.o, a.Cc, row, col, acc[i][jj], r);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < a.Cc) put1(a.o, a.Cc, row, col + e, acc[i][jj][e], r);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) acc[i][jj] = v4i{0, 0, 0, 0};
  }
  // no transfer into LDS may outlive the workgroup
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Skinny forward kernel (tgemm_skinny): C[M][N] with at most 32 rows.  Here
// the packed weights are nearly all of the bytes moved, so the product is
// bound by reading them from HBM, and keeping W as 2-bit codes reads a
// quarter of the bytes of int8 weights [P10425 "How each column was
// measured"].
//
// A workgroup of 8 waves owns BN = 16 NB output columns and all the rows.
// Its waves split the contraction into super-steps of 256 (wave w takes
// super-steps w, w + 8, ...); the eight partial sums are added at the end in
// LDS, in wave order.  Per super-step each lane loads, a super-step ahead,
// straight into registers
//   W: 16 bytes (64 codes) of packed row n0 + 16 nb + lane % 16, per block nb,
//      at contraction 256 s + 64 g (g = lane / 16),
//   A: the super-step's 256 bytes of each of the 16 MF rows, either
//      (AL false) as 64 bytes of row 16 mf + lane % 16 at 64 g, or
//      (AL true, more than 8 rows) in whole 128-byte lines, instruction i of
//      block mf taking row 16 mf + 4 i + g, 16-byte chunk lane % 16; the lines
//      go through a wave-private LDS tile into the MFMA layout (partial-line
//      requests, 16 rows x 4 pieces per instruction, held the L1 to a third
//      of its whole-line rate),
// and decodes the weights in registers (decode16).  Sub-step q pairs packed
// dword q with A chunk 4 g + q of the super-step: the same 16 contraction
// indices, so each of the four MFMA sub-steps covers 64 distinct indices and
// together they cover the super-step.  A contraction that ends inside a
// super-step (K % 256 != 0, K % 64 == 0) is finished by one more step whose
// lanes past the end load in-range bytes and zero their codes (code 0 is
// weight 0).  Rows and columns past the output load the last valid row
// (computed, never stored).
// ---------------------------------------------------------------------------
namespace sk {
constexpr int kWaves = 8, kNT = 64 * kWaves;
constexpr int SK = 256;   // contraction per super-step: four MFMA steps of 64
}  // namespace sk

struct KArgs {
  const int8_t *A;
  const uint8_t *Wp;
  Out o;              // column scale, when scaled: o.cscal (o.cs is null)
  int32_t M, N, K;
  int32_t nfull;      // whole super-steps, K / 256
  int32_t vq;         // 64-steps of the last, partial super-step (K % 256 / 64), or 0
  int32_t xcds;       // workgroup b runs on XCD b % xcds
};

// LDS: the reduction buffer (per wave, the tile's 16 MF rows of 4 NB column
// quads, each row padded by one quad so that the MFMA-layout writes, lanes on
// 16 rows, hit 16 distinct bank groups); with AL, first the waves' A tiles
// (16 MF rows of 256 bytes, chunk c of row m at slot c ^ (m & 15), so that
// both the line writes and the fragment reads are conflict-free), in the same
// memory.
template <int MF, int NB, bool AL>
struct SkLds {
  static constexpr int kPitch = 4 * NB + 1;
  static constexpr int kWave = 16 * MF * kPitch;
  static constexpr int kRed = sk::kWaves * kWave * 16;
  static constexpr int kATile = 16 * MF * 256;
  static constexpr int kTiles = AL ? sk::kWaves * kATile : 0;
  static constexpr int kBytes = kRed > kTiles ? kRed : kTiles;
  static_assert(kBytes <= 80 * 1024, "two workgroups per CU");
};

template <int MF, bool AL>
struct SkA {
  typedef const int8_t *Ptr[MF][AL ? 4 : 1];
};

template <int MF, int NB, bool AL>
__device__ __forceinline__ void sk_load(v4i (&w)[NB], v4i (&x)[MF][4], const uint8_t *const (&wr)[NB],
                                        const typename SkA<MF, AL>::Ptr &ar, int64_t wo, int64_t ao) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) w[nb] = *reinterpret_cast<const v4i *>(wr[nb] + wo);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[mf][i] = *reinterpret_cast<const v4i *>(AL ? ar[mf][AL ? i : 0] + ao : ar[mf][0] + ao + 16 * i);
}

template <int MF, int NB, bool AL>
__device__ __forceinline__ void sk_step(v4i (&acc)[MF][NB], const v4i (&w)[NB], const v4i (&x)[MF][4],
                                        int8_t *tile, int lane) {
  const int r = lane & 15, g = lane >> 4;
  if constexpr (AL) {
    // lines -> tile: row 16 mf + 4 i + g, chunk r
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<v4i *>(tile + (16 * mf + 4 * i + g) * 256 + 16 * (r ^ (4 * i + g))) = x[mf][i];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v4i xa[MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
      xa[mf] = AL ? *reinterpret_cast<const v4i *>(tile + (16 * mf + r) * 256 + 16 * ((4 * g + q) ^ r))
                  : x[mf][q];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const v4i d = decode16((uint32_t)w[nb][q]);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
        acc[mf][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(d, xa[mf], acc[mf][nb], 0, 0, 0);
    }
  }
}

// The skinny kernels' end: each wave's partial sums go to LDS (row
// 16 mf + lane % 16, quad 4 nb + lane / 16 of the tile, rows padded by one
// quad); thread t then sums quad t % (4 NB) of tile row t / (4 NB) over the
// eight waves, in wave order, and stores it at output row m, columns
// c0 + 4 (t % (4 NB)) .. + 3 of a row-major output with `width` columns:
// neighbouring threads write neighbouring 16-byte pieces of one output row.
template <int MF, int NB>
__device__ __forceinline__ void sk_epilogue(int8_t *smem, const v4i (&acc)[MF][NB], const Out &o, int wave, int lane,
                                            int tid, int32_t c0, int32_t M, int32_t width) {
  constexpr int kPitch = 4 * NB + 1, kWave = 16 * MF * kPitch;
  const int r = lane & 15, g = lane >> 4;
  v4i *red = reinterpret_cast<v4i *>(smem);
  v4i *mine = red + wave * kWave;
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mine[(16 * mf + r) * kPitch + 4 * nb + g] = acc[mf][nb];
  __syncthreads();
  constexpr int kQuads = 4 * NB, kOut = 16 * MF * kQuads;
  static_assert(kOut <= sk::kNT, "one quad per thread");
  if (tid < kOut) {
    const int m = tid / kQuads, cq = tid % kQuads;
    v4i sum = red[m * kPitch + cq];
#pragma unroll
    for (int w = 1; w < sk::kWaves; ++w) sum += red[w * kWave + m * kPitch + cq];
    const int32_t col = c0 + 4 * cq;
    if (m < M) {
      const float rsc = row_scale(o, m);
      if (o.vec && col + 3 < width) {
        put4(o, width, m, col, sum, rsc);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < width) put1(o, width, m, col + e, sum[e], rsc);
      }
    }
  }
}

template <int MF, int NB, bool AL>
__global__ __attribute__((amdgpu_flat_work_group_size(sk::kNT, sk::kNT), amdgpu_waves_per_eu(2)))
void tgemm_skinny(KArgs a) {
  typedef SkLds<MF, NB, AL> L;
  __shared__ __attribute__((aligned(256))) int8_t smem[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  // column block in the XCD-contiguous order (as the skinny dX kernel)
  const int32_t n0 = xcd_tile((int32_t)blockIdx.x, (int32_t)gridDim.x, a.xcds) * 16 * NB;
  const int64_t kb = a.K / 4;

  const uint8_t *wr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int32_t n = n0 + 16 * nb + r;
    wr[nb] = a.Wp + (int64_t)(n < a.N ? n : a.N - 1) * kb + 16 * g;
  }
  typename SkA<MF, AL>::Ptr ar;
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int i = 0; i < (AL ? 4 : 1); ++i) {
      const int32_t m = AL ? 16 * mf + 4 * i + g : 16 * mf + r;
      ar[mf][i] = a.A + (int64_t)(m < a.M ? m : a.M - 1) * a.K + (AL ? 16 * r : 64 * g);
    }
  int8_t *tile = smem + (AL ? wave * L::kATile : 0);
  v4i acc[MF][NB];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mf][nb] = v4i{0, 0, 0, 0};

  // whole super-steps: the wave's are wave + 8 i, i < cnt.  Two per
  // iteration through two register sets; each load is issued a super-step
  // before its use (past the wave's last super-step the load repeats it: in
  // range, never used).
  const int32_t cnt = a.nfull > wave ? (a.nfull - wave + sk::kWaves - 1) / sk::kWaves : 0;
  if (cnt > 0) {
    v4i w0[NB], x0[MF][4], w1[NB], x1[MF][4];
    const int32_t last = wave + sk::kWaves * (cnt - 1);
    sk_load<MF, NB, AL>(w0, x0, wr, ar, 64 * (int64_t)wave, sk::SK * (int64_t)wave);
    int32_t s = wave;
    for (int32_t i = 0; i + 2 <= cnt; i += 2) {
      const int32_t s1 = s + sk::kWaves;
      const int32_t s2 = s1 + sk::kWaves < last ? s1 + sk::kWaves : last;
      sk_load<MF, NB, AL>(w1, x1, wr, ar, 64 * (int64_t)s1, sk::SK * (int64_t)s1);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
      sk_step<MF, NB, AL>(acc, w0, x0, tile, lane);
      sk_load<MF, NB, AL>(w0, x0, wr, ar, 64 * (int64_t)s2, sk::SK * (int64_t)s2);
      __builtin_amdgcn_sched_barrier(0);
      sk_step<MF, NB, AL>(acc, w1, x1, tile, lane);
      s += 2 * sk::kWaves;
    }
    if (cnt & 1) sk_step<MF, NB, AL>(acc, w0, x0, tile, lane);   // super-step `last`
  }
  // the partial super-step, on the wave whose turn it is: weights of lanes
  // with g >= vq (codes past K) are zeroed, and every lane loads in range:
  // W at the last group in range, A at the last chunk in range
  if (a.vq && wave == a.nfull % sk::kWaves) {
    const int32_t s = a.nfull;
    const int gd = (g < a.vq ? g : a.vq - 1) - g;
    const int ad = AL ? (r < 4 * a.vq ? r : 4 * a.vq - 1) - r : 4 * gd;
    v4i w[NB], x[MF][4];
    sk_load<MF, NB, AL>(w, x, wr, ar, 64 * (int64_t)s + 16 * gd, sk::SK * (int64_t)s + 16 * ad);
    if (g >= a.vq) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) w[nb] = v4i{0, 0, 0, 0};
    }
    sk_step<MF, NB, AL>(acc, w, x, tile, lane);
  }

  // partial sums -> LDS; with AL the buffer reuses the A tiles, once every
  // wave is done with them
  if constexpr (AL) __syncthreads();
  sk_epilogue<MF, NB>(smem, acc, a.o, wave, lane, tid, n0, a.M, a.N);
}

// ---------------------------------------------------------------------------
// Skinny dX kernel (tgemm_skinny_dx): dX[M][K] = dC x W^T with at most 32
// rows [P10855 PR body, kernel 1; the pages run it at 27 rows, "Measured"].
// A workgroup of 8 waves owns BK = 16 NB output columns (contraction index k
// of the forward) and all the rows; its waves split the contraction n into
// steps of 64 (wave w takes steps w, w + 8, ...), and the partial sums are
// added in LDS in wave order (sk_epilogue).  Per step each lane loads, a step
// ahead, the 4 NB packed bytes (16 NB codes) of W row n = 64 s + lane for the
// block's columns, and 16 bytes of dC row 16 mf + lane % 16 at n = 64 s +
// 16 g.  The codes are decoded (decode16) into a wave-private LDS tile with
// one row per contraction index (RowLayout<16 NB>), and the weight fragments
// are read from it with the transposing read (TrRead), which yields the byte
// order of a plain 16-byte dC read, so the two pair in one MFMA.  N % 64 == 0
// (whole steps) and K % (16 NB) == 0 (whole column blocks): nothing is ragged
// but the rows, which past M load the last row (computed, never stored).
// ---------------------------------------------------------------------------
struct XArgs {
  const int8_t *dC;
  const uint8_t *Wp;
  Out o;              // column scale, when scaled: o.cscal (o.cs is null)
  int32_t M, N, K;
  int32_t nsteps;     // N / 64
  int32_t xcds;       // workgroup b runs on XCD b % xcds
};

template <int NB>
struct SkW;   // a lane's packed bytes of one W row: 4 NB bytes
template <>
struct SkW<1> {
  typedef uint32_t T;
  __device__ __forceinline__ static uint32_t dw(const T &v, int) { return v; }
};
template <>
struct SkW<4> {
  typedef v4i T;
  __device__ __forceinline__ static uint32_t dw(const T &v, int c) { return (uint32_t)v[c]; }
};

template <int MF, int NB>
__device__ __forceinline__ void skx_load(typename SkW<NB>::T &w, v4i (&x)[MF], const uint8_t *wl,
                                         const int8_t *const (&cl)[MF], int64_t wo, int64_t co) {
  w = *reinterpret_cast<const typename SkW<NB>::T *>(wl + wo);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) x[mf] = *reinterpret_cast<const v4i *>(cl[mf] + co);
}

template <int MF, int NB>
__device__ __forceinline__ void skx_step(v4i (&acc)[MF][NB], const typename SkW<NB>::T &w, const v4i (&x)[MF],
                                         int8_t *tile, int lane) {
  typedef RowLayout<16 * NB> Lay;
  // row `lane` of the tile: the decoded weights of contraction index 64 s + lane
#pragma unroll
  for (int c = 0; c < NB; ++c) *reinterpret_cast<v4i *>(tile + Lay::at(lane, c)) = decode16(SkW<NB>::dw(w, c));
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const v4i fw = TrRead::frag(tile + TrRead::off<Lay>(c, lane), 8 * 16 * NB);
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
      acc[mf][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw, x[mf], acc[mf][c], 0, 0, 0);
  }
}

template <int MF, int NB>
struct SkxLds {
  static constexpr int kTile = RowLayout<16 * NB>::kBytes;
  static constexpr int kRed = sk::kWaves * 16 * MF * (4 * NB + 1) * 16;
  static constexpr int kTiles = sk::kWaves * kTile;
  static constexpr int kBytes = kRed > kTiles ? kRed : kTiles;
  static_assert(kBytes <= 80 * 1024, "two workgroups per CU");
};

template <int MF, int NB>
__global__ __attribute__((amdgpu_flat_work_group_size(sk::kNT, sk::kNT), amdgpu_waves_per_eu(2)))
void tgemm_skinny_dx(XArgs a) {
  typedef SkxLds<MF, NB> L;
  __shared__ __attribute__((aligned(256))) int8_t smem[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  // column block: each XCD (workgroup b runs on XCD b % 8) takes a
  // contiguous run of blocks, so the blocks that share a 128-byte line of a
  // packed row read it through one L2 (in the plain order, eight XCDs each
  // fetched every line)
  const int32_t k0 = xcd_tile((int32_t)blockIdx.x, (int32_t)gridDim.x, a.xcds) * 16 * NB;
  const int64_t kb = a.K / 4;
  const uint8_t *wl = a.Wp + (int64_t)lane * kb + k0 / 4;       // row 64 s + lane: + 64 s kb
  const int8_t *cl[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int32_t m = 16 * mf + r;
    cl[mf] = a.dC + (int64_t)(m < a.M ? m : a.M - 1) * a.N + 16 * g;
  }
  int8_t *tile = smem + wave * L::kTile;
  v4i acc[MF][NB];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[mf][c] = v4i{0, 0, 0, 0};

  // the wave's steps wave + 8 i, i < cnt, two per iteration through two
  // register sets, each load a step ahead (past the last step the load
  // repeats it: in range, never used)
  const int32_t cnt = a.nsteps > wave ? (a.nsteps - wave + sk::kWaves - 1) / sk::kWaves : 0;
  if (cnt > 0) {
    typename SkW<NB>::T w0, w1;
    v4i x0[MF], x1[MF];
    const int32_t last = wave + sk::kWaves * (cnt - 1);
    const int64_t ws = 64 * kb;                                   // bytes of W per step
    skx_load<MF, NB>(w0, x0, wl, cl, ws * wave, (int64_t)64 * wave);
    int32_t s = wave;
    for (int32_t i = 0; i + 2 <= cnt; i += 2) {
      const int32_t s1 = s + sk::kWaves;
      const int32_t s2 = s1 + sk::kWaves < last ? s1 + sk::kWaves : last;
      skx_load<MF, NB>(w1, x1, wl, cl, ws * s1, (int64_t)64 * s1);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
      skx_step<MF, NB>(acc, w0, x0, tile, lane);
      skx_load<MF, NB>(w0, x0, wl, cl, ws * s2, (int64_t)64 * s2);
      __builtin_amdgcn_sched_barrier(0);
      skx_step<MF, NB>(acc, w1, x1, tile, lane);
      s += 2 * sk::kWaves;
    }
    if (cnt & 1) skx_step<MF, NB>(acc, w0, x0, tile, lane);
  }
  __syncthreads();   // the reduction buffer reuses the tiles
  sk_epilogue<MF, NB>(smem, acc, a.o, wave, lane, tid, k0, a.M, a.K);
}

// ---------------------------------------------------------------------------
// Split skinny dX (tgemm_skinny_dx_split + skinny_dx_sum), the same product
// as tgemm_skinny_dx for the same few rows, when the caller lends a
// workspace.  What bounds tgemm_skinny_dx at long rows is the number of W
// rows one load instruction touches: 64 rows of 16 bytes, each row in its own
// page when K is large.  Here a workgroup owns 256 output columns, so a W row
// contributes 64 contiguous bytes, and four neighbouring lanes load them:
// one instruction covers 16 rows x 64 bytes.  With K / 256 column blocks too
// few to fill the chip, the contraction n is split S ways across workgroups
// (S column-block copies, each over a contiguous range of steps); each writes
// its int32 partial sums to the workspace, and a second kernel adds the S
// partials in split order and applies the output kind.  Integer addition is
// exact, so the bits equal those of the one-pass kernels.
//   Per step (64 contraction indices) a wave loads four 16-row slabs of W
// (lane l: row 16 i + l / 4, bytes 16 (l % 4) .. + 15 of the block) and the
// dC fragments as in tgemm_skinny_dx, decodes its 64 x 256 codes into a
// wave-private LDS tile (RowLayout<256>: chunk 4 (l % 4) + j of row
// 16 i + l / 4; a 16-lane pass then writes 16 distinct chunk slots) and reads
// the 16 weight fragments back transposed.  The waves' partials meet in LDS
// (one 16-row block at a time, 128 KB) and are stored as whole 16-byte
// pieces.  Requirements (checked by the plan): M <= 32, N % 64 == 0,
// K % 256 == 0, 16-byte aligned dC and Wpacked.
// ---------------------------------------------------------------------------
namespace sxs {
constexpr int kBK = 256;                         // output columns per workgroup
constexpr int kTile = RowLayout<kBK>::kBytes;    // 64 x 256 decoded codes
constexpr int kLds = sk::kWaves * kTile;         // 128 KB: tiles, then the reduction
}  // namespace sxs

template <int MF>
__device__ __forceinline__ void sxs_load(v4i (&w)[4], v4i (&x)[MF], const uint8_t *wl, int64_t kb,
                                         const int8_t *const (&cl)[MF], int32_t st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const v4i *>(wl + ((int64_t)64 * st + 16 * i) * kb);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) x[mf] = *reinterpret_cast<const v4i *>(cl[mf] + (int64_t)64 * st);
}

template <int MF>
__device__ __forceinline__ void sxs_step(v4i (&acc)[MF][16], const v4i (&w)[4], const v4i (&x)[MF],
                                         int8_t *tile, int lane) {
  typedef RowLayout<sxs::kBK> Lay;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<v4i *>(tile + Lay::at(16 * i + (lane >> 2), 4 * (lane & 3) + j)) =
          decode16((uint32_t)w[i][j]);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const v4i fw = TrRead::frag(tile + TrRead::off<Lay>(c, lane), 8 * sxs::kBK);
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
      acc[mf][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw, x[mf], acc[mf][c], 0, 0, 0);
  }
}

template <int MF>
__global__ __attribute__((amdgpu_flat_work_group_size(sk::kNT, sk::kNT), amdgpu_waves_per_eu(2)))
void tgemm_skinny_dx_split(XArgs a, int32_t *part, int32_t S) {
  __shared__ __attribute__((aligned(256))) int8_t smem[sxs::kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  // the S splits of a column block are neighbours in the XCD-contiguous
  // order, so they run on one XCD and share its L2 for dC
  const int32_t b = xcd_tile((int32_t)blockIdx.x, (int32_t)gridDim.x, a.xcds);
  const int32_t blk = b / S, sp = b % S;
  const int32_t k0 = blk * sxs::kBK;
  const int64_t kb = a.K / 4;
  const int32_t st0 = (int32_t)((int64_t)sp * a.nsteps / S);
  const int32_t st1 = (int32_t)((int64_t)(sp + 1) * a.nsteps / S);
  const uint8_t *wl = a.Wp + (int64_t)(lane >> 2) * kb + k0 / 4 + 16 * (lane & 3);
  const int8_t *cl[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int32_t m = 16 * mf + r;
    cl[mf] = a.dC + (int64_t)(m < a.M ? m : a.M - 1) * a.N + 16 * g;
  }
  int8_t *tile = smem + wave * sxs::kTile;
  v4i acc[MF][16];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[mf][c] = v4i{0, 0, 0, 0};

  // the wave's steps st0 + wave + 8 i < st1, two per iteration through two
  // register sets, each load a step ahead (past the last step the load
  // repeats it: in range, never used)
  const int32_t first = st0 + wave;
  const int32_t cnt = st1 > first ? (st1 - first + sk::kWaves - 1) / sk::kWaves : 0;
  if (cnt > 0) {
    v4i w0[4], w1[4], x0[MF], x1[MF];
    const int32_t last = first + sk::kWaves * (cnt - 1);
    sxs_load<MF>(w0, x0, wl, kb, cl, first);
    int32_t st = first;
    for (int32_t i = 0; i + 2 <= cnt; i += 2) {
      const int32_t s1 = st + sk::kWaves;
      const int32_t s2 = s1 + sk::kWaves < last ? s1 + sk::kWaves : last;
      sxs_load<MF>(w1, x1, wl, kb, cl, s1);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
      sxs_step<MF>(acc, w0, x0, tile, lane);
      sxs_load<MF>(w0, x0, wl, kb, cl, s2);
      __builtin_amdgcn_sched_barrier(0);
      sxs_step<MF>(acc, w1, x1, tile, lane);
      st += 2 * sk::kWaves;
    }
    if (cnt & 1) sxs_step<MF>(acc, w0, x0, tile, lane);
  }

  // partials: the eight waves' sums of one 16-row block go to LDS as
  // [wave][fragment][lane] (conflict-free 16-byte pieces), then thread t adds
  // the eight copies of two (fragment, lane) pieces in wave order.  Lane l of
  // fragment c holds row l % 16, columns 16 c + 4 (l / 16) .. + 3.
  v4i *red = reinterpret_cast<v4i *>(smem);
  int32_t *out = part + (int64_t)sp * a.M * a.K;
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    __syncthreads();   // the tiles (or the previous block's partials) are free
#pragma unroll
    for (int c = 0; c < 16; ++c) red[(wave * 16 + c) * 64 + lane] = acc[mf][c];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + sk::kNT * u, c = idx >> 6, ln = idx & 63;
      v4i t = red[c * 64 + ln];
#pragma unroll
      for (int w = 1; w < sk::kWaves; ++w) t += red[(w * 16 + c) * 64 + ln];
      const int32_t m = 16 * mf + (ln & 15);
      if (m < a.M) *reinterpret_cast<v4i *>(out + (int64_t)m * a.K + k0 + 16 * c + 4 * (ln >> 4)) = t;
    }
  }
}

// dX = the sum of the S partials (split order), in the output kind; one
// thread per 4 outputs (K % 256 == 0, so a row holds whole groups of 4).
// Eight partials are loaded before any is added, so a thread waits for one
// memory round trip per eight splits, not one per split.
__global__ __launch_bounds__(256) void skinny_dx_sum(const v4i *__restrict__ part, Out o, int64_t M, int64_t K,
                                                     int32_t S) {
  const int64_t n4 = M * K / 4, kq = K / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    v4i t = v4i{0, 0, 0, 0};
    for (int32_t s0 = 0; s0 < S; s0 += 8) {
      v4i p[8];
      // unconditional loads (past S: the last split again, added as 0), so
      // no branch separates them
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = part[(int64_t)(s0 + u < S ? s0 + u : S - 1) * n4 + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) t += s0 + u < S ? p[u] : v4i{0, 0, 0, 0};
    }
    const int64_t row = i / kq, col = 4 * (i % kq);
    const float rsc = row_scale(o, row);
    if (o.vec) {
      put4(o, K, row, col, t, rsc);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) put1(o, K, row, col + k, t[k], rsc);
    }
  }
}

template <int OP, class T, bool FAST>
hipError_t launch_t(const Args &a, hipStream_t stream) {
  hipLaunchKernelGGL((tgemm_kernel<OP, T, FAST>), dim3(a.tiles), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int OP, class T>
hipError_t launch_f(const Args &a, bool fast, hipStream_t stream) {
  return fast ? launch_t<OP, T, true>(a, stream) : launch_t<OP, T, false>(a, stream);
}


// Kernel per product, tile and load path:
//   tiled  tgemm_kernel: every case but the next
//   split  tgemm_split: dW, and dX with at most 256 tiles, on the 128 x 144
//          tile with a contraction of 8 steps or more
//   stream tgemm_stream: large forward and dX outputs (stream_plan)
//   skinny tgemm_skinny: forward with at most 32 rows (skinny_plan)
// (A variant that loads the int8 operand of the forward and dX straight into
// MFMA registers, without LDS, measured no faster in the three-product step
// on MI355X and was left out.)
enum KernelId { KTILED = 0, KSPLIT = 2, KSTREAM = 3, KSKINNY = 4 };

// The machine the plans are made for: compute units (one persistent
// workgroup each) and XCDs (workgroup b runs on XCD b % xcds, each XCD with
// its own L2).  The calls query the current device once and keep the answer;
// the host-only plan query takes MI355X's values unless given others.
struct Machine {
  int32_t cus, xcds;
};
constexpr Machine kMI355X = {256, 8};

bool machine_ok(const Machine &mc) { return mc.cus >= 1 && mc.xcds >= 1 && mc.cus % mc.xcds == 0; }

int query_machine(Machine *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TGEMM_ERR_HIP;
  constexpr int kMaxDev = 64;
  static std::atomic<uint64_t> cache[kMaxDev];
  uint64_t v = dev < kMaxDev ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return TGEMM_ERR_HIP;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1 ||
        cus % xcds != 0)
      xcds = 1;
    v = ((uint64_t)(uint32_t)cus << 32) | (uint32_t)xcds;
    if (dev < kMaxDev) cache[dev].store(v, std::memory_order_relaxed);
  }
  out->cus = (int32_t)(v >> 32);
  out->xcds = (int32_t)(uint32_t)v;
  return TGEMM_OK;
}


// The streaming kernels (forward, dX): apply when the contraction is a whole
// number of steps, the operands are aligned for their 16- and 4-byte loads
// (dX: packed columns in whole dwords, K % 16 == 0), their 32-bit offsets
// cannot overflow, and the output has enough tiles for a full persistent grid.

struct StreamPlan {
  bool ok;
  int32_t bn, tiles_r, tiles_c, tiles, grid, lds;
};

StreamPlan stream_plan(int op, int64_t M, int64_t N, int64_t K, uintptr_t qalign, uintptr_t walign,
                       const Machine &mc) {
  StreamPlan sp{};
  if (op == DW || qalign % 16 != 0 || walign % 4 != 0) return sp;
  const Shape s = shape_of(op, M, N, K);
  if (s.L % BK != 0 || (op == DX && K % 16 != 0)) return sp;
  if (M > INT32_MAX / s.L || N > INT32_MAX / (K / 4) || s.R > INT32_MAX / s.Cc) return sp;
  sp.bn = op == FWD ? fs::Geo<FWD>::BN : fs::Geo<DX>::BN;
  sp.lds = op == FWD ? fs::Geo<FWD>::kLds : fs::Geo<DX>::kLds;
  const int64_t tr = ceil_div(s.R, fs::BM), tc = ceil_div(s.Cc, sp.bn);
  if (tr * tc < mc.cus || !machine_ok(mc)) return sp;
  sp.ok = true;
  sp.tiles_r = (int32_t)tr;
  sp.tiles_c = (int32_t)tc;
  sp.tiles = (int32_t)(tr * tc);
  sp.grid = mc.cus;
  return sp;
}

// The skinny forward: at most 32 rows, K % 64 == 0 (whole 64-steps, packed
// rows in whole 16-byte pieces), 16-byte aligned A and Wpacked.  Column
// blocks of 64, 32 or 16: the widest that still gives 128 workgroups or more
// (A is re-read by every workgroup, so wider blocks read fewer bytes).  A in
// whole lines through LDS above 8 rows (at 1 row it measured 5% slower, at
// 16 and more 13-20% faster).
struct SkinnyPlan {
  bool ok, al;
  int32_t mf, nb, grid, lds;
};

SkinnyPlan skinny_plan(int op, int64_t M, int64_t N, int64_t K, uintptr_t qalign, uintptr_t walign,
                       const Machine &mc) {
  SkinnyPlan kp{};
  if (op != FWD || M > 32 || K % 64 != 0 || qalign % 16 != 0 || walign % 16 != 0) return kp;
  if (N > INT32_MAX - 64 || K > INT32_MAX) return kp;
  kp.mf = M > 16 ? 2 : 1;
  const int64_t half = mc.cus / 2 > 0 ? mc.cus / 2 : 1;   // workgroups wanted, at least
  kp.nb = N >= half * 64 ? 4 : N >= half * 32 ? 2 : 1;
  kp.al = M > 8;
  kp.grid = (int32_t)ceil_div(N, 16 * kp.nb);
  const int32_t red = sk::kWaves * 16 * kp.mf * (4 * kp.nb + 1) * 16;
  const int32_t tiles = kp.al ? sk::kWaves * 16 * kp.mf * 256 : 0;
  kp.lds = red > tiles ? red : tiles;
  kp.ok = true;
  return kp;
}

// The skinny dX: at most 32 rows, N % 64 == 0 (whole contraction steps),
// K % 16 == 0, 16-byte aligned dC, and Wpacked aligned for the per-row
// loads.  Column blocks of 64 (K % 64 == 0 and 128 or more of them) or 16.
SkinnyPlan skinny_dx_plan(int op, int64_t M, int64_t N, int64_t K, uintptr_t qalign, uintptr_t walign,
                          const Machine &mc) {
  SkinnyPlan kp{};
  if (op != DX || M > 32 || N % 64 != 0 || K % 16 != 0 || qalign % 16 != 0) return kp;
  if (N > INT32_MAX || K > INT32_MAX - 64) return kp;
  kp.mf = M > 16 ? 2 : 1;
  kp.nb = (K % 64 == 0 && K / 64 >= mc.cus / 2) ? 4 : 1;
  if (walign % (4 * kp.nb) != 0) return kp;
  kp.al = false;
  kp.grid = (int32_t)(K / (16 * kp.nb));
  const int32_t red = sk::kWaves * 16 * kp.mf * (4 * kp.nb + 1) * 16;
  const int32_t tiles = sk::kWaves * (kp.nb == 4 ? RowLayout<64>::kBytes : RowLayout<16>::kBytes);
  kp.lds = red > tiles ? red : tiles;
  kp.ok = true;
  return kp;
}

// The split skinny dX (with a workspace): the skinny dX's rows, N % 64 == 0,
// K % 256 == 0, 16-byte aligned dC and Wpacked; S = ceil(256 / (K / 256))
// splits, so the grid fills the CUs once, at least two (K / 256 >= 256
// column blocks fill the chip without a split, and the one-pass kernel runs)
// and each wave with at least one step of every split (N / 64 >= 8 S).
struct SplitDxPlan {
  bool ok;
  int32_t mf, blocks, S, grid;
  int64_t bytes;      // workspace: S partial sums of M x K int32
};
SplitDxPlan skinny_dx_split_plan(int op, int64_t M, int64_t N, int64_t K, uintptr_t qalign, uintptr_t walign,
                                 const Machine &mc) {
  SplitDxPlan xp{};
  if (op != DX || M > 32 || N % 64 != 0 || K % sxs::kBK != 0 || qalign % 16 != 0 || walign % 16 != 0)
    return xp;
  if (N > INT32_MAX || K > INT32_MAX - 64) return xp;
  const int64_t blocks = K / sxs::kBK, nsteps = N / 64;
  const int64_t S = (mc.cus + blocks - 1) / blocks;
  if (S < 2 || nsteps < sk::kWaves * S) return xp;
  xp.mf = M > 16 ? 2 : 1;
  xp.blocks = (int32_t)blocks;
  xp.S = (int32_t)S;
  xp.grid = (int32_t)(blocks * S);
  xp.bytes = S * M * K * 4;
  xp.ok = true;
  return xp;
}

template <int MF, int NB>
void launch_skinny_dx(const XArgs &xa, int grid, hipStream_t stream) {
  static_assert(SkxLds<MF, NB>::kTile == RowLayout<16 * NB>::kBytes, "plan LDS");
  hipLaunchKernelGGL((tgemm_skinny_dx<MF, NB>), dim3(grid), dim3(sk::kNT), 0, stream, xa);
}

template <int MF, int NB, bool AL>
void launch_skinny(const KArgs &ka, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((tgemm_skinny<MF, NB, AL>), dim3(grid), dim3(sk::kNT), 0, stream, ka);
}

// the contraction split between two halves of a workgroup: dW on the
// 128 x 144 tile, and dX on that tile when its tiles do not fill the CUs;
// at least 8 steps
int pick_kernel(int op, int tile, int64_t L, int64_t tiles, const Machine &mc) {
  if (op == DW && tile == TW && L >= 8 * BK) return KSPLIT;
  if (op == DX && tile == TW && L >= 8 * BK && tiles <= mc.cus) return KSPLIT;
  return KTILED;
}

template <int OP>
int lds_of_kernel(int kernel, int tile) {
  if (kernel == KSPLIT) {
    typedef typename Tiles<OP>::W T;
    typedef StageBytes<OP, T> SB;
    const int stages = 4 * (SB::Q + SB::P), red = T::FM * T::FN * kThreads * 16;
    return stages > red ? stages : red;
  }
  return lds_of_tile<OP>(tile);
}

int kernel_lds(int op, int kernel, int tile) {
  return op == FWD ? lds_of_kernel<FWD>(kernel, tile)
         : op == DX ? lds_of_kernel<DX>(kernel, tile)
                    : lds_of_kernel<DW>(kernel, tile);
}

template <int OP>
hipError_t launch_op(const Args &a, int kernel, int tile, bool fast, hipStream_t stream) {
  if constexpr (OP == DW || OP == DX) {
    if (kernel == KSPLIT) {
      typedef typename Tiles<OP>::W T;
      if (fast)
        hipLaunchKernelGGL((tgemm_split<OP, T, true>), dim3(a.tiles), dim3(2 * kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((tgemm_split<OP, T, false>), dim3(a.tiles), dim3(2 * kThreads), 0, stream, a);
      return hipGetLastError();
    }
  }
  switch (tile) {
    case TL: return launch_f<OP, typename Tiles<OP>::L>(a, fast, stream);
    case TW: return launch_f<OP, typename Tiles<OP>::W>(a, fast, stream);
    default: return launch_f<OP, typename Tiles<OP>::S>(a, fast, stream);
  }
}

// out: the output buffer, elements of `kind`; rs, cs, cscal: the scales of
// the scaled kinds (rs per output row; cs per output column, or null and
// cscal for every column)
int run(int op, const int8_t *q, const void *p, void *out, int kind, const float *rs, const float *cs,
        float cscal, int64_t M, int64_t N, int64_t K, hipStream_t stream, void *ws = nullptr,
        int64_t ws_bytes = 0) {
  const int st = check_dims(op, M, N, K);
  if (st != TGEMM_OK) return st;
  const Shape s = shape_of(op, M, N, K);

  // operand byte sizes, for the overlap check
  const int64_t qbytes = op == DX ? M * N : M * K;
  const int64_t pbytes = op == DW ? M * N : N * (K / 4);
  const int64_t esz = kind == OUT_BF16 ? 2 : 4;
  const int64_t obytes = s.R * s.Cc * esz;
  if (overlaps(out, obytes, q, qbytes) || overlaps(out, obytes, p, pbytes)) return TGEMM_ERR_ALIAS;
  if (kind != OUT_I32 &&
      (overlaps(out, obytes, rs, s.R * 4) || (cs && overlaps(out, obytes, cs, s.Cc * 4))))
    return TGEMM_ERR_ALIAS;
  if (ws && ws_bytes > 0 &&
      (overlaps(ws, ws_bytes, q, qbytes) || overlaps(ws, ws_bytes, p, pbytes) ||
       overlaps(ws, ws_bytes, out, obytes) || (kind != OUT_I32 && overlaps(ws, ws_bytes, rs, s.R * 4))))
    return TGEMM_ERR_ALIAS;
  Machine mc;
  if (query_machine(&mc) != TGEMM_OK) return TGEMM_ERR_HIP;
  Out o;
  o.ptr = out;
  o.rs = rs;
  o.cs = cs;
  o.cscal = cscal;
  o.kind = kind;
  o.vec = (s.Cc % 4 == 0 && aligned(out, 4 * esz)) ? 1 : 0;
  o.vec8 = (kind == OUT_BF16 && s.Cc % 8 == 0 && aligned(out, 16)) ? 1 : 0;

  const int tile = pick_tile_for(op, s, mc.cus);
  const TileInfo &ti = kTileInfo[tile];
  Args a;
  a.q = q;
  a.p = p;
  a.o = o;
  a.R = s.R;
  a.Cc = s.Cc;
  a.L = s.L;
  a.ldq = op == DX ? N : K;
  a.ldp = op == DW ? N : K / 4;
  a.tiles_c = (int32_t)ceil_div(s.Cc, ti.bn);
  a.tiles = (int32_t)(ceil_div(s.R, ti.bm) * a.tiles_c);
  a.band_cols = pick_band_cols(op, M, N, K, a.tiles_c, mc.xcds);
  a.xcds = mc.xcds;
  const bool fast = fast_ok(op, M, N, K, align_of(q), align_of(p));

  {
    const SkinnyPlan kp = skinny_plan(op, M, N, K, align_of(q), align_of(p), mc);
    if (kp.ok) {
      KArgs ka;
      ka.xcds = mc.xcds;
      ka.A = q;
      ka.Wp = static_cast<const uint8_t *>(p);
      ka.o = o;
      ka.M = (int32_t)M;
      ka.N = (int32_t)N;
      ka.K = (int32_t)K;
      ka.nfull = (int32_t)(K / sk::SK);
      ka.vq = (int32_t)(K % sk::SK / BK);
      const int sel = 100 * kp.mf + 10 * kp.nb + (kp.al ? 1 : 0);
      switch (sel) {
        case 110: launch_skinny<1, 1, false>(ka, kp.grid, stream); break;
        case 120: launch_skinny<1, 2, false>(ka, kp.grid, stream); break;
        case 140: launch_skinny<1, 4, false>(ka, kp.grid, stream); break;
        case 111: launch_skinny<1, 1, true>(ka, kp.grid, stream); break;
        case 121: launch_skinny<1, 2, true>(ka, kp.grid, stream); break;
        case 141: launch_skinny<1, 4, true>(ka, kp.grid, stream); break;
        case 211: launch_skinny<2, 1, true>(ka, kp.grid, stream); break;
        case 221: launch_skinny<2, 2, true>(ka, kp.grid, stream); break;
        default: launch_skinny<2, 4, true>(ka, kp.grid, stream); break;
      }
      static_assert(SkLds<2, 4, true>::kBytes == 8 * 32 * 17 * 16 && SkLds<1, 1, true>::kBytes == 8 * 16 * 256,
                    "plan LDS");
      return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
    }
  }
  {
    const SplitDxPlan xp = skinny_dx_split_plan(op, M, N, K, align_of(q), align_of(p), mc);
    if (xp.ok && ws && ws_bytes >= xp.bytes && aligned(ws, 16)) {
      XArgs xa;
      xa.xcds = mc.xcds;
      xa.dC = q;
      xa.Wp = static_cast<const uint8_t *>(p);
      xa.o = o;
      xa.M = (int32_t)M;
      xa.N = (int32_t)N;
      xa.K = (int32_t)K;
      xa.nsteps = (int32_t)(N / BK);
      int32_t *part = static_cast<int32_t *>(ws);
      if (xp.mf == 1)
        hipLaunchKernelGGL((tgemm_skinny_dx_split<1>), dim3(xp.grid), dim3(sk::kNT), 0, stream, xa, part, xp.S);
      else
        hipLaunchKernelGGL((tgemm_skinny_dx_split<2>), dim3(xp.grid), dim3(sk::kNT), 0, stream, xa, part, xp.S);
      if (hipGetLastError() != hipSuccess) return TGEMM_ERR_HIP;
      const int64_t groups = ceil_div(M * K / 4, 256);
      hipLaunchKernelGGL(skinny_dx_sum, dim3((uint32_t)(groups < 2048 ? groups : 2048)), dim3(256), 0, stream,
                         reinterpret_cast<const v4i *>(part), o, M, K, xp.S);
      return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
    }
  }
  {
    const SkinnyPlan kp = skinny_dx_plan(op, M, N, K, align_of(q), align_of(p), mc);
    if (kp.ok) {
      XArgs xa;
      xa.xcds = mc.xcds;
      xa.dC = q;
      xa.Wp = static_cast<const uint8_t *>(p);
      xa.o = o;
      xa.M = (int32_t)M;
      xa.N = (int32_t)N;
      xa.K = (int32_t)K;
      xa.nsteps = (int32_t)(N / BK);
      if (kp.mf == 1)
        kp.nb == 4 ? launch_skinny_dx<1, 4>(xa, kp.grid, stream) : launch_skinny_dx<1, 1>(xa, kp.grid, stream);
      else
        kp.nb == 4 ? launch_skinny_dx<2, 4>(xa, kp.grid, stream) : launch_skinny_dx<2, 1>(xa, kp.grid, stream);
      return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
    }
  }
  {
    const StreamPlan sp = stream_plan(op, M, N, K, align_of(q), align_of(p), mc);
    if (sp.ok) {
      SArgs sa;
      sa.xcds = mc.xcds;
      sa.Q = q;
      sa.Wp = static_cast<const uint8_t *>(p);
      sa.o = o;
      sa.R = (int32_t)s.R;
      sa.Cc = (int32_t)s.Cc;
      sa.L = (int32_t)s.L;
      sa.ldq = (int32_t)s.L;
      sa.kb = (int32_t)(K / 4);
      sa.tiles_c = sp.tiles_c;
      sa.tiles = sp.tiles;
      sa.nk = (int32_t)(s.L / BK);
      if (op == FWD)
        hipLaunchKernelGGL(tgemm_stream<FWD>, dim3(sp.grid), dim3(fs::kNT), 0, stream, sa);
      else
        hipLaunchKernelGGL(tgemm_stream<DX>, dim3(sp.grid), dim3(fs::kNT), 0, stream, sa);
      return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
    }
  }

  const int kernel = pick_kernel(op, tile, s.L, a.tiles, mc);
  hipError_t e;
  if (op == FWD)
    e = launch_op<FWD>(a, kernel, tile, fast, stream);
  else if (op == DX)
    e = launch_op<DX>(a, kernel, tile, fast, stream);
  else
    e = launch_op<DW>(a, kernel, tile, fast, stream);
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}

// Static scratch of ternary_gemm_s8_dx_noalloc: the split dX's partial sums
// for callers that cannot allocate.  Each device holds its own copy from the
// library's load until the process ends.  Host code never uses this name as
// an address: scratch_of() looks the device address up once per device.
constexpr int64_t kScratchBytes = TGEMM_STATIC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 16-byte vectors");
static __device__ __align__(256) int32_t scratch[kScratchBytes / 4];

// the current device's address of `scratch` (hipGetSymbolAddress with the
// device current, once per device)
int scratch_of(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TGEMM_ERR_HIP;
  constexpr int kMaxDev = 64;
  static std::atomic<void *> cache[kMaxDev];
  void *ptr = dev < kMaxDev ? cache[dev].load(std::memory_order_acquire) : nullptr;
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TGEMM_ERR_HIP;
    if (dev < kMaxDev) cache[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return TGEMM_OK;
}

}  // namespace

extern "C" {

int ternary_gemm_s8(const int8_t *A, const uint8_t *Wpacked, int32_t *C, int64_t M, int64_t N,
                    int64_t K, hipStream_t stream) {
  if (!A || !Wpacked || !C) return TGEMM_ERR_NULL;
  return run(FWD, A, Wpacked, C, OUT_I32, nullptr, nullptr, 0.f, M, N, K, stream);
}

int ternary_gemm_s8_dx(const int8_t *dC, const uint8_t *Wpacked, int32_t *dX, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  if (!dC || !Wpacked || !dX) return TGEMM_ERR_NULL;
  return run(DX, dC, Wpacked, dX, OUT_I32, nullptr, nullptr, 0.f, M, N, K, stream);
}

int ternary_gemm_s8_dw(const int8_t *A, const int8_t *dC, int32_t *dW, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
  if (!A || !dC || !dW) return TGEMM_ERR_NULL;
  return run(DW, A, dC, dW, OUT_I32, nullptr, nullptr, 0.f, M, N, K, stream);
}

int ternary_gemm_s8_scaled(const int8_t *A, const uint8_t *Wpacked, const float *a_row_scale,
                           float w_scale, void *Y, int out_kind, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream) {
  if (!A || !Wpacked || !a_row_scale || !Y) return TGEMM_ERR_NULL;
  if (out_kind != TGEMM_OUT_F32 && out_kind != TGEMM_OUT_BF16) return TGEMM_ERR_KIND;
  return run(FWD, A, Wpacked, Y, out_kind, a_row_scale, nullptr, w_scale, M, N, K, stream);
}

int ternary_gemm_s8_dx_scaled(const int8_t *dC, const uint8_t *Wpacked, const float *dc_row_scale,
                              float w_scale, void *dX, int out_kind, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream) {
  if (!dC || !Wpacked || !dc_row_scale || !dX) return TGEMM_ERR_NULL;
  if (out_kind != TGEMM_OUT_F32 && out_kind != TGEMM_OUT_BF16) return TGEMM_ERR_KIND;
  return run(DX, dC, Wpacked, dX, out_kind, dc_row_scale, nullptr, w_scale, M, N, K, stream);
}

int ternary_gemm_dx_workspace(int64_t M, int64_t N, int64_t K, int64_t align, int64_t *bytes) {
  if (!bytes) return TGEMM_ERR_NULL;
  const int st = check_dims(DX, M, N, K);
  if (st != TGEMM_OK) return st;
  const uintptr_t al = align > 0 ? (uintptr_t)align : 1;
  // the machine the calls will run on: the current device, else MI355X
  Machine mc = kMI355X;
  if (query_machine(&mc) != TGEMM_OK) mc = kMI355X;
  const SplitDxPlan xp = skinny_dx_split_plan(DX, M, N, K, al, al, mc);
  *bytes = xp.ok ? xp.bytes : 0;
  return TGEMM_OK;
}

int ternary_gemm_s8_dx_ws(const int8_t *dC, const uint8_t *Wpacked, int32_t *dX, int64_t M, int64_t N,
                          int64_t K, void *workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (!dC || !Wpacked || !dX) return TGEMM_ERR_NULL;
  if (workspace_bytes < 0) return TGEMM_ERR_DIM;
  return run(DX, dC, Wpacked, dX, OUT_I32, nullptr, nullptr, 0.f, M, N, K, stream, workspace, workspace_bytes);
}

int ternary_gemm_s8_dx_noalloc(const int8_t *dC, const uint8_t *Wpacked, int32_t *dX, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream) {
  if (!dC || !Wpacked || !dX) return TGEMM_ERR_NULL;
  const int st = check_dims(DX, M, N, K);
  if (st != TGEMM_OK) return st;
  Machine mc;
  if (query_machine(&mc) != TGEMM_OK) return TGEMM_ERR_HIP;
  const SplitDxPlan xp = skinny_dx_split_plan(DX, M, N, K, align_of(dC), align_of(Wpacked), mc);
  if (!xp.ok) return run(DX, dC, Wpacked, dX, OUT_I32, nullptr, nullptr, 0.f, M, N, K, stream);
  if (xp.bytes > kScratchBytes) return TGEMM_ERR_SCRATCH;
  void *ws = nullptr;
  const int sst = scratch_of(&ws);
  if (sst != TGEMM_OK) return sst;
  return run(DX, dC, Wpacked, dX, OUT_I32, nullptr, nullptr, 0.f, M, N, K, stream, ws, kScratchBytes);
}

int ternary_gemm_s8_dx_scaled_ws(const int8_t *dC, const uint8_t *Wpacked, const float *dc_row_scale,
                                 float w_scale, void *dX, int out_kind, int64_t M, int64_t N, int64_t K,
                                 void *workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (!dC || !Wpacked || !dc_row_scale || !dX) return TGEMM_ERR_NULL;
  if (out_kind != TGEMM_OUT_F32 && out_kind != TGEMM_OUT_BF16) return TGEMM_ERR_KIND;
  if (workspace_bytes < 0) return TGEMM_ERR_DIM;
  return run(DX, dC, Wpacked, dX, out_kind, dc_row_scale, nullptr, w_scale, M, N, K, stream, workspace,
             workspace_bytes);
}

int ternary_gemm_s8_dw_scaled(const int8_t *A, const int8_t *dC, const float *a_col_scale,
                              const float *dc_col_scale, void *dW, int out_kind, int64_t M, int64_t N,
                              int64_t K, hipStream_t stream) {
  if (!A || !dC || !a_col_scale || !dc_col_scale || !dW) return TGEMM_ERR_NULL;
  if (out_kind != TGEMM_OUT_F32 && out_kind != TGEMM_OUT_BF16) return TGEMM_ERR_KIND;
  return run(DW, A, dC, dW, out_kind, a_col_scale, dc_col_scale, 1.f, M, N, K, stream);
}

const char *ternary_gemm_status_str(int status) {
  switch (status) {
    case TGEMM_OK: return "ok";
    case TGEMM_ERR_NULL: return "a required pointer is NULL";
    case TGEMM_ERR_DIM: return "a dimension is < 1 or a size does not fit";
    case TGEMM_ERR_PACK: return "the packed dimension K is not a multiple of 4";
    case TGEMM_ERR_BOUND: return "the contraction is longer than the exact-int32 bound";
    case TGEMM_ERR_ALIAS: return "the output overlaps an input";
    case TGEMM_ERR_HIP: return "the HIP runtime reported an error at launch";
    case TGEMM_ERR_KIND: return "the output kind is not TGEMM_OUT_F32 or TGEMM_OUT_BF16";
    case TGEMM_ERR_SCRATCH: return "the split needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int ternary_gemm_machine(int32_t *cus, int32_t *xcds) {
  if (!cus || !xcds) return TGEMM_ERR_NULL;
  Machine mc;
  const int st = query_machine(&mc);
  if (st != TGEMM_OK) return st;
  *cus = mc.cus;
  *xcds = mc.xcds;
  return TGEMM_OK;
}

int ternary_gemm_plan_on(int op, int64_t M, int64_t N, int64_t K, int64_t align, int32_t cus, int32_t xcds,
                         tgemm_plan *plan) {
  if (!plan) return TGEMM_ERR_NULL;
  const Machine mc = {cus, xcds};
  if (!machine_ok(mc)) return TGEMM_ERR_DIM;
  const int st = check_dims(op, M, N, K);
  if (st != TGEMM_OK) return st;
  const Shape s = shape_of(op, M, N, K);
  const uintptr_t al = align > 0 ? (uintptr_t)align : 1;
  memset(plan, 0, sizeof(*plan));
  plan->out_rows = s.R;
  plan->out_cols = s.Cc;
  plan->contraction = s.L;
  plan->fast_path = fast_ok(op, M, N, K, al, al) ? 1 : 0;
  plan->xcds = mc.xcds;
  {
    SkinnyPlan kp = skinny_plan(op, M, N, K, al, al, mc);
    if (!kp.ok) kp = skinny_dx_plan(op, M, N, K, al, al, mc);
    if (kp.ok) {
      plan->tile_rows = 16 * kp.mf;
      plan->tile_cols = 16 * kp.nb;
      plan->tiles = kp.grid;
      plan->workgroups = kp.grid;
      plan->tiles_per_workgroup = 1;
      plan->band_cols = kp.grid;
      plan->kernel = KSKINNY;
      plan->threads_per_workgroup = sk::kNT;
      plan->lds_bytes = kp.lds;
      return TGEMM_OK;
    }
  }
  {
    const StreamPlan sp = stream_plan(op, M, N, K, al, al, mc);
    if (sp.ok) {
      plan->tile_rows = fs::BM;
      plan->tile_cols = sp.bn;
      plan->tiles = sp.tiles;
      plan->workgroups = sp.grid;
      plan->tiles_per_workgroup = ceil_div(ceil_div(sp.tiles, mc.xcds), sp.grid / mc.xcds);
      plan->band_cols = sp.tiles_c;
      plan->kernel = KSTREAM;
      plan->threads_per_workgroup = fs::kNT;
      plan->lds_bytes = sp.lds + fs::BM * 4;   // stages + the tile's row scales
      return TGEMM_OK;
    }
  }
  const int tile = pick_tile_for(op, s, mc.cus);
  const TileInfo &ti = kTileInfo[tile];
  plan->tile_rows = ti.bm;
  plan->tile_cols = ti.bn;
  plan->tiles = ceil_div(s.R, ti.bm) * ceil_div(s.Cc, ti.bn);
  plan->workgroups = plan->tiles;
  plan->tiles_per_workgroup = 1;
  plan->band_cols = pick_band_cols(op, M, N, K, (int32_t)ceil_div(s.Cc, ti.bn), mc.xcds);
  plan->kernel = pick_kernel(op, tile, s.L, plan->tiles, mc);
  plan->threads_per_workgroup = plan->kernel == KSPLIT ? 2 * kThreads : kThreads;
  plan->lds_bytes = kernel_lds(op, plan->kernel, tile);
  return TGEMM_OK;
}

int ternary_gemm_plan(int op, int64_t M, int64_t N, int64_t K, int64_t align, tgemm_plan *plan) {
  return ternary_gemm_plan_on(op, M, N, K, align, kMI355X.cus, kMI355X.xcds, plan);
}

int ternary_gemm_tile_of(const tgemm_plan *plan, int64_t workgroup, int64_t iteration, int64_t *row0,
                         int64_t *col0) {
  if (!plan || !row0 || !col0) return TGEMM_ERR_NULL;
  if (workgroup < 0 || workgroup >= plan->workgroups || iteration < 0 ||
      iteration >= plan->tiles_per_workgroup || plan->tiles > INT32_MAX || plan->tile_rows < 1 ||
      plan->tile_cols < 1 || plan->xcds < 1)
    return TGEMM_ERR_DIM;
  const int32_t tiles_c = (int32_t)ceil_div(plan->out_cols, plan->tile_cols);
  const int32_t tiles = (int32_t)plan->tiles, xcds = plan->xcds;
  int32_t tr, tc;
  if (plan->kernel == KSTREAM) {
    // the kernels' own order: one contiguous run of row-major tile positions
    // per XCD; workgroup b (XCD b % xcds) takes every nx-th position of its
    // run, starting at b / xcds
    if (plan->workgroups % xcds != 0) return TGEMM_ERR_DIM;
    const int32_t nx = (int32_t)plan->workgroups / xcds, xcd = (int32_t)(workgroup % xcds);
    const int32_t j = (int32_t)(workgroup / xcds);
    const int32_t qx = tiles / xcds, rx = tiles % xcds;
    const int32_t start = xcd * qx + (xcd < rx ? xcd : rx);
    const int32_t cnt = qx + (xcd < rx ? 1 : 0);
    const int64_t pos = j + iteration * nx;
    if (pos >= cnt) return TGEMM_ERR_DIM;
    tr = (int32_t)((start + pos) / tiles_c);
    tc = (int32_t)((start + pos) % tiles_c);
  } else if (plan->kernel == KSKINNY) {
    // all rows; the column block in the XCD-contiguous order
    if (iteration != 0) return TGEMM_ERR_DIM;
    tr = 0;
    tc = xcd_tile((int32_t)workgroup, tiles, xcds);
  } else {
    if (iteration != 0) return TGEMM_ERR_DIM;
    tile_rc(xcd_tile((int32_t)workgroup, tiles, xcds), tiles / tiles_c, tiles_c, plan->band_cols, &tr, &tc);
  }
  *row0 = (int64_t)tr * plan->tile_rows;
  *col0 = (int64_t)tc * plan->tile_cols;
  return TGEMM_OK;
}

}  // extern "C"
