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
//   product   O      R   Cc  L   Q operand (rows of O)   P operand (cols of O)
//   forward   C      M   N   K   A[m][.]       copied    W(., n) decoded from Wpacked
//   dX        dX     M   K   N   dC[m][.]      copied    W(k, .) decoded + transposed
//   dW        dW     K   N   M   A[.][k]     transposed  dC[.][n]    transposed
//
// A workgroup of 4 waves owns a BM x BN tile of O.  Per step of 64 along the
// contraction it stages a BM x 64 Q tile and a BN x 64 P tile into LDS as s8,
// contraction-contiguous rows with an 80-byte pitch, then each wave runs
// v_mfma_i32_16x16x64_i8 over its sub-tile with int32 accumulators held in
// registers for the whole contraction.  The 2-bit codes are decoded once per
// global->LDS tile load, not per MFMA [P10425 "What this adds"].  The next
// step's global loads are issued before the current step's MFMAs and written
// to the other LDS buffer after them (two LDS stages, one barrier per step);
// the pages name this double buffering with a 64-wide step as their next
// lever [P10425 "What this says"].
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
// PR body, "k <= 131071"].  The contraction is reduced serially inside one
// workgroup: no split of it, no atomics, identical bits on every call.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "ternary_gemm.h"

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int BK = 64;         // contraction per step (one 16x16x64 MFMA)
constexpr int LP = BK + 16;    // LDS row pitch: 80 B, so 8 consecutive rows
                               // read at one 16-B column hit 8 distinct
                               // 16-B bank groups (80*r mod 128 distinct)

// Byte c of this word is the int8 weight of code c: 00, 01, FF, 00, i.e.
// (c & 1) - ((c >> 1) & 1) [P10425 "What this adds"; P10855 PR body].
constexpr uint32_t kCodeTable = 0x00FF0100u;

enum Op { FWD = 0, DX = 1, DW = 2 };

struct Args {
  const int8_t *q;    // Q source
  const void *p;      // P source (Wpacked for FWD/DX, dC for DW)
  int32_t *out;
  int64_t R, Cc, L;   // output rows, output cols, contraction length
  int64_t ldq, ldp;   // row strides (bytes) of the Q and P sources
  int32_t tiles_c;    // column tiles
  int32_t tiles;      // total tiles (= workgroups)
  int32_t vec_out;    // Cc % 4 == 0 and out 16-B aligned: 16-B stores
};

// ---------------------------------------------------------------------------
// Workgroup -> tile order.  The hardware hands workgroup ids to the eight
// XCDs round-robin (id % 8), and each XCD has its own L2.  The remap gives
// each XCD a contiguous range of tile ids; tile ids run along the output
// columns first, so the tiles an XCD runs together share the same Q rows and
// read them from its L2 instead of HBM.  A bijection on [0, tiles).
// ---------------------------------------------------------------------------
__host__ __device__ inline int32_t xcd_tile(int32_t wg, int32_t tiles) {
  const int32_t q = tiles / 8, r = tiles % 8;
  const int32_t x = wg % 8, j = wg / 8;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// ---------------------------------------------------------------------------
// Code decode.  spread4 moves the four 2-bit codes of a byte into the low
// bits of four bytes; v_perm_b32 then uses each byte as a selector into
// kCodeTable, turning four codes into four int8 weights in one instruction.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t spread4(uint32_t b) {
  uint32_t t = b | (b << 6);        // codes 0,1 -> bits 0-1, 8-9
  t = t | (t << 12);                // codes 2,3 -> bits 16-17, 24-25
  return t & 0x03030303u;
}

__device__ __forceinline__ uint32_t weights4(uint32_t sel) {
  // v_perm_b32(src0=0, src1=table): selector values 0..3 pick bytes of src1
  return __builtin_amdgcn_perm(0u, kCodeTable, sel);
}

// 16 codes of one packed dword (code i at bits 2i) -> 16 int8 weights, in order
__device__ __forceinline__ v4i decode16(uint32_t x) {
  v4i w;
  w[0] = (int32_t)weights4(spread4(x & 0xFFu));
  w[1] = (int32_t)weights4(spread4((x >> 8) & 0xFFu));
  w[2] = (int32_t)weights4(spread4((x >> 16) & 0xFFu));
  w[3] = (int32_t)weights4(spread4(x >> 24));
  return w;
}

// 4x4 byte transpose: out[j] byte r = in[r] byte j
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t a_lo = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
  const uint32_t a_hi = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
  const uint32_t b_lo = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t b_hi = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

// ---------------------------------------------------------------------------
// Stagers.  load() issues the global reads of one step into registers;
// store() writes them (decoded / transposed) into an LDS tile of BT rows of
// LP bytes.  Contraction positions >= L are written as 0, so a ragged last
// step contributes nothing.  Rows beyond the output are clamped to the last
// valid row (in bounds, computed, never stored).
// ---------------------------------------------------------------------------

// Rows of an int8 matrix whose rows are contraction-contiguous (A or dC as
// the Q operand): chunk = 16 bytes, 4 chunks per row per step.
template <int BT, bool FAST>
struct CopyStage {
  static constexpr int kPer = BT * 4 / kThreads;
  static_assert(kPer >= 1 && BT * 4 % kThreads == 0, "tile too small");
  v4i r[kPer];

  __device__ __forceinline__ void load(const int8_t *src, int64_t ld, int64_t nrows,
                                       int64_t L, int64_t t0, int64_t c0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = i * kThreads + tid;
      const int row = id >> 2, cc = id & 3;
      const int64_t gr = t0 + row < nrows ? t0 + row : nrows - 1;
      const int64_t gc = c0 + cc * 16;
      const int8_t *s = src + gr * ld + gc;
      if (FAST) {  // L % 16 == 0 and 16-B aligned rows: a chunk is all in or all out
        r[i] = gc < L ? *reinterpret_cast<const v4i *>(s) : v4i{0, 0, 0, 0};
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < 16; ++b)
          if (gc + b < L) w[b >> 2] |= (uint32_t)(uint8_t)s[b] << (8 * (b & 3));
        r[i] = v4i{(int32_t)w[0], (int32_t)w[1], (int32_t)w[2], (int32_t)w[3]};
      }
    }
  }

  __device__ __forceinline__ void store(int8_t *lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = i * kThreads + tid;
      *reinterpret_cast<v4i *>(lds + (id >> 2) * LP + (id & 3) * 16) = r[i];
    }
  }
};

// Stored ternary weights as the P operand of the forward product: row n of
// Wpacked holds the codes of column n along K, so a step's 64 codes of a row
// are 16 contiguous bytes = 4 dwords.  Decoded once here, one 16-B LDS store
// per dword.
template <int BT, bool FAST>
struct DecodeStage {
  static constexpr int kPer = BT * 4 / kThreads;
  static_assert(kPer >= 1 && BT * 4 % kThreads == 0, "tile too small");
  uint32_t r[kPer];

  __device__ __forceinline__ void load(const uint8_t *wp, int64_t ld, int64_t nrows,
                                       int64_t L, int64_t t0, int64_t c0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = i * kThreads + tid;
      const int row = id >> 2, uc = id & 3;
      const int64_t gr = t0 + row < nrows ? t0 + row : nrows - 1;
      const int64_t gk = c0 + uc * 16;  // first code of this dword
      const uint8_t *s = wp + gr * ld + (gk >> 2);
      if (FAST) {  // L % 16 == 0, 4-B aligned rows
        r[i] = gk < L ? *reinterpret_cast<const uint32_t *>(s) : 0u;
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (gk + 4 * b < L) w |= (uint32_t)s[b] << (8 * b);
        r[i] = w;
      }
    }
  }

  __device__ __forceinline__ void store(int8_t *lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = i * kThreads + tid;
      *reinterpret_cast<v4i *>(lds + (id >> 2) * LP + (id & 3) * 16) = decode16(r[i]);
    }
  }
};

// Stored ternary weights as the P operand of dX: LDS row = output column k,
// contraction along n, but Wpacked rows run along k.  A unit is one packed
// byte column (4 consecutive k) over 16 consecutive n: 16 byte loads, then for
// each of the 4 codes of a byte, the 16 weights along n go out as one 16-B LDS
// store.  Units: (BT/4 byte columns) x (4 groups of 16 n) = BT; threads
// tid < BT take one each.
template <int BT>
struct DecodeTStage {
  static_assert(BT <= kThreads, "tile too large");
  uint32_t b[16];

  __device__ __forceinline__ void load(const uint8_t *wp, int64_t ld, int64_t kbytes,
                                       int64_t L, int64_t t0, int64_t c0, int tid) {
    if (tid >= BT) return;
    const int bc = tid % (BT / 4), nc = tid / (BT / 4);
    const int64_t gb = (t0 >> 2) + bc;  // packed byte column (k / 4)
    const bool colok = gb < kbytes;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t n = c0 + nc * 16 + r;
      b[r] = (colok && n < L) ? (uint32_t)wp[n * ld + gb] : 0u;
    }
  }

  __device__ __forceinline__ void store(int8_t *lds, int tid) const {
    if (tid >= BT) return;
    const int bc = tid % (BT / 4), nc = tid / (BT / 4);
    uint32_t x[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      x[g] = b[4 * g] | (b[4 * g + 1] << 8) | (b[4 * g + 2] << 16) | (b[4 * g + 3] << 24);
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // code j of each byte = column k = 4*bc + j
      v4i w;
#pragma unroll
      for (int g = 0; g < 4; ++g) w[g] = (int32_t)weights4((x[g] >> (2 * j)) & 0x03030303u);
      *reinterpret_cast<v4i *>(lds + (4 * bc + j) * LP + nc * 16) = w;
    }
  }
};

// An int8 matrix whose rows run along the contraction index's *other* side
// (A[m][k] and dC[m][n] for dW): LDS row = output index o, contraction m.  A
// unit is 4 consecutive o over 16 consecutive m: 16 dword loads (or guarded
// bytes), 4x4 byte transposes, then 4 16-B LDS stores.  Units: (BT/4) x 4 =
// BT; threads tid < BT take one each.
template <int BT, bool FAST>
struct TCopyStage {
  static_assert(BT <= kThreads, "tile too large");
  uint32_t r[16];

  __device__ __forceinline__ void load(const int8_t *src, int64_t ld, int64_t nout,
                                       int64_t L, int64_t t0, int64_t c0, int tid) {
    if (tid >= BT) return;
    const int oq = tid % (BT / 4), mc = tid / (BT / 4);
    const int64_t o = t0 + 4 * oq;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t m = c0 + mc * 16 + i;
      const int8_t *s = src + m * ld + o;
      if (FAST) {  // nout % 4 == 0, 4-B aligned rows
        r[i] = (m < L && o < nout) ? *reinterpret_cast<const uint32_t *>(s) : 0u;
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
          if (m < L && o + bb < nout) w |= (uint32_t)(uint8_t)s[bb] << (8 * bb);
        r[i] = w;
      }
    }
  }

  __device__ __forceinline__ void store(int8_t *lds, int tid) const {
    if (tid >= BT) return;
    const int oq = tid % (BT / 4), mc = tid / (BT / 4);
    uint32_t t[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g) transpose4x4(&r[4 * g], t[g]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i w{(int32_t)t[0][j], (int32_t)t[1][j], (int32_t)t[2][j], (int32_t)t[3][j]};
      *reinterpret_cast<v4i *>(lds + (4 * oq + j) * LP + mc * 16) = w;
    }
  }
};

// ---------------------------------------------------------------------------
// Tile shapes: BM x BN outputs per workgroup, 2 x 2 waves.
// ---------------------------------------------------------------------------
template <int BM_, int BN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = 2, WN = 2;
  static constexpr int TM = BM / WM, TN = BN / WN;  // per wave
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 blocks per wave
  static constexpr int kLds = 2 * (BM + BN) * LP;
};

template <int OP, class T, bool FAST>
struct Stages;

template <class T, bool FAST>
struct Stages<FWD, T, FAST> {
  CopyStage<T::BM, FAST> q;
  DecodeStage<T::BN, FAST> p;
  __device__ __forceinline__ void load(const Args &a, int64_t q0, int64_t p0, int64_t c0, int tid) {
    q.load(a.q, a.ldq, a.R, a.L, q0, c0, tid);
    p.load(static_cast<const uint8_t *>(a.p), a.ldp, a.Cc, a.L, p0, c0, tid);
  }
};

template <class T, bool FAST>
struct Stages<DX, T, FAST> {
  CopyStage<T::BM, FAST> q;
  DecodeTStage<T::BN> p;
  __device__ __forceinline__ void load(const Args &a, int64_t q0, int64_t p0, int64_t c0, int tid) {
    q.load(a.q, a.ldq, a.R, a.L, q0, c0, tid);
    p.load(static_cast<const uint8_t *>(a.p), a.ldp, a.Cc >> 2, a.L, p0, c0, tid);
  }
};

template <class T, bool FAST>
struct Stages<DW, T, FAST> {
  TCopyStage<T::BM, FAST> q;
  TCopyStage<T::BN, FAST> p;
  __device__ __forceinline__ void load(const Args &a, int64_t q0, int64_t p0, int64_t c0, int tid) {
    q.load(a.q, a.ldq, a.R, a.L, q0, c0, tid);
    p.load(static_cast<const int8_t *>(a.p), a.ldp, a.Cc, a.L, p0, c0, tid);
  }
};

template <int OP, class T, bool FAST>
__global__ __launch_bounds__(kThreads) void tgemm_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) int8_t smem[T::kLds];
  int8_t *const sq = smem;                    // [2][BM][LP]
  int8_t *const sp = smem + 2 * T::BM * LP;   // [2][BN][LP]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;

  const int32_t tile = xcd_tile((int32_t)blockIdx.x, a.tiles);
  const int64_t q0 = (int64_t)(tile / a.tiles_c) * T::BM;
  const int64_t p0 = (int64_t)(tile % a.tiles_c) * T::BN;

  v4i acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  Stages<OP, T, FAST> st;
  const int32_t nk = (int32_t)((a.L + BK - 1) / BK);

  st.load(a, q0, p0, 0, tid);
  st.q.store(sq, tid);
  st.p.store(sp, tid);
  __syncthreads();

  // fragment addresses: row (lane % 16) of each 16-row block, 16-B chunk lane / 16
  const int frag = (lane & 15) * LP + (lane >> 4) * 16;
  const int qoff = wm * T::TM * LP + frag;
  const int poff = wn * T::TN * LP + frag;

  for (int32_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) st.load(a, q0, p0, (int64_t)(kt + 1) * BK, tid);

    const int8_t *qb = sq + cur * T::BM * LP + qoff;
    const int8_t *pb = sp + cur * T::BN * LP + poff;
    v4i fq[T::FM], fp[T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i) fq[i] = *reinterpret_cast<const v4i *>(qb + i * 16 * LP);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) fp[j] = *reinterpret_cast<const v4i *>(pb + j * 16 * LP);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fp[j], fq[i], acc[i][j], 0, 0, 0);

    if (more) {
      st.q.store(sq + (cur ^ 1) * T::BM * LP, tid);
      st.p.store(sp + (cur ^ 1) * T::BN * LP, tid);
    }
    __syncthreads();
  }

  // epilogue: lane holds O[row][col .. col+3] of each 16x16 block
  const int64_t rbase = q0 + wm * T::TM + (lane & 15);
  const int64_t cbase = p0 + wn * T::TN + (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int64_t row = rbase + i * 16;
    if (row >= a.R) continue;
    int32_t *orow = a.out + row * a.Cc;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int64_t col = cbase + j * 16;
      if (a.vec_out && col + 3 < a.Cc) {
        *reinterpret_cast<v4i *>(orow + col) = acc[i][j];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < a.Cc) orow[col + e] = acc[i][j][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: validation, planning, launch.
// ---------------------------------------------------------------------------

typedef Tile<256, 128> TileL;
typedef Tile<128, 128> TileM;
typedef Tile<64, 64> TileS;

enum TileId { TL = 0, TM_ = 1, TS = 2 };

struct Shape {
  int64_t R, Cc, L;
};

Shape shape_of(int op, int64_t M, int64_t N, int64_t K) {
  if (op == FWD) return {M, N, K};
  if (op == DX) return {M, K, N};
  return {K, N, M};
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

void tile_dims(int t, int *bm, int *bn) {
  if (t == TL) { *bm = TileL::BM; *bn = TileL::BN; }
  else if (t == TM_) { *bm = TileM::BM; *bn = TileM::BN; }
  else { *bm = TileS::BM; *bn = TileS::BN; }
}

// Largest tile that still gives every CU (256 of them) work: big tiles read
// fewer operand bytes per MAC from LDS; small ones fill the chip on small
// outputs.
int pick_tile(const Shape &s) {
  const int64_t cus = 256;
  for (int t = TL; t <= TS; ++t) {
    int bm, bn;
    tile_dims(t, &bm, &bn);
    if (ceil_div(s.R, bm) * ceil_div(s.Cc, bn) >= 2 * cus) return t;
  }
  return TS;
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
  if (!mul_ok(M, K, &t) || !mul_ok(M, N, &t) || !mul_ok(K, N, &t)) return TGEMM_ERR_DIM;
  if (!mul_ok(M, N, &t) || !mul_ok(t, 4, &t) || !mul_ok(M, K, &t) || !mul_ok(t, 4, &t) ||
      !mul_ok(K, N, &t) || !mul_ok(t, 4, &t))
    return TGEMM_ERR_DIM;
  if (op != DW && K % 4 != 0) return TGEMM_ERR_PACK;
  const Shape s = shape_of(op, M, N, K);
  const int64_t bound = op == DW ? TGEMM_INT8_MAX_CONTRACTION : TGEMM_TERNARY_MAX_CONTRACTION;
  if (s.L > bound) return TGEMM_ERR_BOUND;
  // smallest tile must keep the workgroup count within a 1-D grid
  if (ceil_div(s.R, TileS::BM) * ceil_div(s.Cc, TileS::BN) > INT32_MAX) return TGEMM_ERR_DIM;
  return TGEMM_OK;
}

bool fast_ok(int op, int64_t M, int64_t N, int64_t K, uintptr_t qalign, uintptr_t palign) {
  (void)M;
  if (op == FWD) return K % 16 == 0 && qalign % 16 == 0 && palign % 4 == 0;
  if (op == DX) return N % 16 == 0 && qalign % 16 == 0;
  return K % 4 == 0 && N % 4 == 0 && qalign % 4 == 0 && palign % 4 == 0;
}

uintptr_t align_of(const void *p) {
  const uintptr_t v = (uintptr_t)p;
  return v ? (v & (~v + 1)) : ((uintptr_t)1 << 20);
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

template <int OP>
hipError_t launch_op(const Args &a, int tile, bool fast, hipStream_t stream) {
  if (tile == TL) return launch_f<OP, TileL>(a, fast, stream);
  if (tile == TM_) return launch_f<OP, TileM>(a, fast, stream);
  return launch_f<OP, TileS>(a, fast, stream);
}

int run(int op, const int8_t *q, const void *p, int32_t *out, int64_t M, int64_t N, int64_t K,
        hipStream_t stream) {
  const int st = check_dims(op, M, N, K);
  if (st != TGEMM_OK) return st;
  const Shape s = shape_of(op, M, N, K);

  // operand byte sizes, for the overlap check
  const int64_t qbytes = op == DX ? M * N : M * K;
  const int64_t pbytes = op == DW ? M * N : N * (K / 4);
  const int64_t obytes = s.R * s.Cc * 4;
  if (overlaps(out, obytes, q, qbytes) || overlaps(out, obytes, p, pbytes)) return TGEMM_ERR_ALIAS;

  const int tile = pick_tile(s);
  int bm, bn;
  tile_dims(tile, &bm, &bn);
  Args a;
  a.q = q;
  a.p = p;
  a.out = out;
  a.R = s.R;
  a.Cc = s.Cc;
  a.L = s.L;
  a.ldq = op == DX ? N : K;
  a.ldp = op == DW ? N : K / 4;
  a.tiles_c = (int32_t)ceil_div(s.Cc, bn);
  a.tiles = (int32_t)(ceil_div(s.R, bm) * a.tiles_c);
  a.vec_out = (s.Cc % 4 == 0 && aligned(out, 16)) ? 1 : 0;
  const bool fast = fast_ok(op, M, N, K, align_of(q), align_of(p));

  hipError_t e;
  if (op == FWD) e = launch_op<FWD>(a, tile, fast, stream);
  else if (op == DX) e = launch_op<DX>(a, tile, fast, stream);
  else e = launch_op<DW>(a, tile, fast, stream);
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}

}  // namespace

extern "C" {

int ternary_gemm_s8(const int8_t *A, const uint8_t *Wpacked, int32_t *C, int64_t M, int64_t N,
                    int64_t K, hipStream_t stream) {
  if (!A || !Wpacked || !C) return TGEMM_ERR_NULL;
  return run(FWD, A, Wpacked, C, M, N, K, stream);
}

int ternary_gemm_s8_dx(const int8_t *dC, const uint8_t *Wpacked, int32_t *dX, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  if (!dC || !Wpacked || !dX) return TGEMM_ERR_NULL;
  return run(DX, dC, Wpacked, dX, M, N, K, stream);
}

int ternary_gemm_s8_dw(const int8_t *A, const int8_t *dC, int32_t *dW, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
  if (!A || !dC || !dW) return TGEMM_ERR_NULL;
  return run(DW, A, dC, dW, M, N, K, stream);
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
    default: return "unknown status";
  }
}

int ternary_gemm_plan(int op, int64_t M, int64_t N, int64_t K, int64_t align, tgemm_plan *plan) {
  if (!plan) return TGEMM_ERR_NULL;
  const int st = check_dims(op, M, N, K);
  if (st != TGEMM_OK) return st;
  const Shape s = shape_of(op, M, N, K);
  const int tile = pick_tile(s);
  int bm, bn;
  tile_dims(tile, &bm, &bn);
  memset(plan, 0, sizeof(*plan));
  plan->out_rows = s.R;
  plan->out_cols = s.Cc;
  plan->contraction = s.L;
  plan->tile_rows = bm;
  plan->tile_cols = bn;
  plan->workgroups = ceil_div(s.R, bm) * ceil_div(s.Cc, bn);
  plan->threads_per_workgroup = kThreads;
  plan->lds_bytes = 2 * (bm + bn) * LP;
  const uintptr_t al = align > 0 ? (uintptr_t)align : 1;
  plan->fast_path = fast_ok(op, M, N, K, al, al) ? 1 : 0;
  return TGEMM_OK;
}

int ternary_gemm_tile_of_block(const tgemm_plan *plan, int64_t block, int64_t *row0,
                               int64_t *col0) {
  if (!plan || !row0 || !col0) return TGEMM_ERR_NULL;
  if (block < 0 || block >= plan->workgroups || plan->workgroups > INT32_MAX) return TGEMM_ERR_DIM;
  const int64_t tiles_c = ceil_div(plan->out_cols, plan->tile_cols);
  const int32_t t = xcd_tile((int32_t)block, (int32_t)plan->workgroups);
  *row0 = (int64_t)(t / tiles_c) * plan->tile_rows;
  *col0 = (int64_t)(t % tiles_c) * plan->tile_cols;
  return TGEMM_OK;
}

}  // extern "C"
