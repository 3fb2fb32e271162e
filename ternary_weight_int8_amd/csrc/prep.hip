// prep.hip -- gfx950 kernels for the two steps before the product, part of
// libternary_gemm.so (ABI in include/ternary_gemm.h):
//
//   packing   the trainer's int8 ternary weights Wt[N][K] (row n: output
//             column n, as a linear layer stores them) into the stored
//             format Wpacked[N][K/4]: 2-bit codes, four per byte along K, the
//             first in the low bits; code 1 for w > 0, 2 for w < 0, 0 for 0
//             (the code table of [P10425 "What this adds"]; the pages leave
//             wiring the trainer to it for later [P10855 PR body]);
//   quantizing activations X[R][C] (float32 or bfloat16) to int8 with one
//             scale per row (the forward's A, dX's dC) or per column (dW's X
//             and dY) [P10855 PR body, "the scales the host must use"]:
//                 s = max|x| / 127,   q = clamp(rint(x / s), -127, 127)
//             (q = 0 where s == 0), each step in IEEE single precision,
//             rounded to nearest even.
//
// Both are streaming passes bound by HBM bandwidth: the packer reads N K
// bytes and writes N K / 4; the quantizer reads X once from HBM (the per-row
// kernel's second pass over a row hits the caches) and writes R C bytes.
// Sources (cited by page title and section):
//   [P10425] t27 pull request #10425, "t27c PTX backend: ternary x int8 GEMM
//            kernel emitted by a .t27 spec (int8 mma.sync), ptx-run glue".
//   [P10855] t27 pull request #10855, "spec(igla): hslm_bwd_ptx -- HSLM
//            backward dX and dW as int8 tensor-core PTX written by t27".

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ternary_gemm.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint16_t v8h __attribute__((ext_vector_type(8)));

bool overlap(const void *a, int64_t an, const void *b, int64_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)bn && y < x + (uintptr_t)an;
}
bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

// ---------------------------------------------------------------------------
// Packing.  Codes of four int8 weights held in one dword, gathered into one
// byte: per byte, neg = its sign bit and nz = (byte != 0) (the low seven
// bits plus 0x7F carry into bit 7 exactly when one of them is set, and never
// into the next byte); the code is nz & !neg for 1, neg for 2; then the
// codes of bytes 1, 2, 3 move down to bits 2, 4, 6.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t codes_of4(uint32_t v) {
  const uint32_t neg = (v >> 7) & 0x01010101u;
  const uint32_t nz = ((((v & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | v) >> 7) & 0x01010101u;
  const uint32_t c = (nz & ~neg) | (neg << 1);
  return (c | (c >> 6) | (c >> 12) | (c >> 18)) & 0xFFu;
}

// Stored byte i holds the codes of input bytes 4i .. 4i + 3 (rows are
// contiguous and K % 4 == 0, so the row structure needs no index work).
// Vector kernel: each thread takes 64 input bytes (four 16-byte loads) and
// writes 16; grid-stride over the whole chunks.
__global__ __launch_bounds__(256) void pack_vec(const v4u *__restrict__ in, v4u *__restrict__ out, int64_t chunks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += stride) {
    v4u o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4u x = in[4 * c + j];
      o[j] = codes_of4(x[0]) | (codes_of4(x[1]) << 8) | (codes_of4(x[2]) << 16) | (codes_of4(x[3]) << 24);
    }
    out[c] = o;
  }
}

// Byte kernel (any alignment, and the tail of the vector kernel): each
// thread takes four input bytes and writes one.
__global__ __launch_bounds__(256) void pack_bytes(const int8_t *__restrict__ in, uint8_t *__restrict__ out,
                                                  int64_t first, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < first + count; i += stride) {
    const uint32_t v = (uint32_t)(uint8_t)in[4 * i] | ((uint32_t)(uint8_t)in[4 * i + 1] << 8) |
                       ((uint32_t)(uint8_t)in[4 * i + 2] << 16) | ((uint32_t)(uint8_t)in[4 * i + 3] << 24);
    out[i] = (uint8_t)codes_of4(v);
  }
}

// ---------------------------------------------------------------------------
// Quantizing.  Inputs are float32, or bfloat16 bit patterns widened exactly
// (bits << 16).  Inputs must be finite.
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ float widen(T v);
template <>
__device__ __forceinline__ float widen<float>(float v) { return v; }
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ int8_t quant1(float x, float s) {
  if (!(s > 0.f)) return 0;
  const float r = rintf(__fdiv_rn(x, s));
  return (int8_t)(r > 127.f ? 127.f : (r < -127.f ? -127.f : r));
}

// eight consecutive inputs as floats (16 bytes of bf16, 32 of float32)
__device__ __forceinline__ void load8(const float *p, float (&v)[8]) {
  const v4f a = *reinterpret_cast<const v4f *>(p), b = *reinterpret_cast<const v4f *>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
__device__ __forceinline__ void load8(const uint16_t *p, float (&v)[8]) {
  const v8h a = *reinterpret_cast<const v8h *>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = widen<uint16_t>(a[i]);
}

__device__ __forceinline__ uint2 pack8(const float (&v)[8], float s) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= (uint32_t)(uint8_t)quant1(v[i], s) << (8 * i);
    hi |= (uint32_t)(uint8_t)quant1(v[4 + i], s) << (8 * i);
  }
  return make_uint2(lo, hi);
}

constexpr int kQT = 256;   // threads per workgroup of the quantizer kernels

// Per row, rows of at most 512 V elements on the vector path: one wave per
// row (four per workgroup, grid-stride over rows), lane l holding units
// l, l + 64, ... (8 elements each) in registers; max|x| across the wave with
// xor shuffles, then q from the registers.  No LDS, no barrier.
template <class T, int V>
__global__ __launch_bounds__(256) void quant_rows_wave(const T *__restrict__ X, int8_t *__restrict__ Q,
                                                       float *__restrict__ S, int64_t R, int64_t C) {
  const int lane = threadIdx.x & 63;
  const int64_t nu = C / 8;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < R; row += (int64_t)gridDim.x * 4) {
    const T *x = X + row * C;
    float v[V][8];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t u = lane + 64 * j;
      if (u < nu) {
        load8(x + 8 * u, v[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float s = __fdiv_rn(m, 127.f);
    if (lane == 0) S[row] = s;
    int8_t *q = Q + row * C;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t u = lane + 64 * j;
      if (u < nu) *reinterpret_cast<uint2 *>(q + 8 * u) = pack8(v[j], s);
    }
  }
}

// Per row: one workgroup per row (grid-stride over rows).  Pass 1 takes
// max|x| over the row (per thread, then across the wave with xor shuffles,
// then across the four waves in LDS); s = max / 127; pass 2 reads the row
// again (from the caches) and writes q.  vec: C % 8 == 0 and the bases
// aligned for 8-element loads and 8-byte stores.
template <class T>
__global__ __launch_bounds__(kQT) void quant_rows(const T *__restrict__ X, int8_t *__restrict__ Q,
                                                  float *__restrict__ S, int64_t R, int64_t C, int vec) {
  __shared__ float part[kQT / 64];
  const int t = threadIdx.x;
  for (int64_t row = blockIdx.x; row < R; row += gridDim.x) {
    const T *x = X + row * C;
    int8_t *q = Q + row * C;
    float m = 0.f;
    if (vec) {
      for (int64_t u = t; u < C / 8; u += kQT) {
        float v[8];
        load8(x + 8 * u, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
      }
    } else {
      for (int64_t i = t; i < C; i += kQT) m = fmaxf(m, fabsf(widen<T>(x[i])));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((t & 63) == 0) part[t >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    __syncthreads();   // part is reused by the next row
    const float s = __fdiv_rn(m, 127.f);
    if (t == 0) S[row] = s;
    if (vec) {
      for (int64_t u = t; u < C / 8; u += kQT) {
        float v[8];
        load8(x + 8 * u, v);
        *reinterpret_cast<uint2 *>(q + 8 * u) = pack8(v, s);
      }
    } else {
      for (int64_t i = t; i < C; i += kQT) q[i] = quant1(widen<T>(x[i]), s);
    }
  }
}

// Per column.  A workgroup (four waves) takes a run of kRun rows and 512
// columns, lane l columns 8 l .. 8 l + 7 of the block, wave w rows w, w + 4,
// ... of the run; the four waves' maxima meet in LDS.  Each run's maxima go
// to a partial row P[run][col] (float32), and a second kernel takes the max
// over the runs (in run order; max is exact) and writes s = max / 127.  P
// lives in Q's memory: ceil(R / kRun) x C floats take at most R x C bytes,
// and the last kernel, which reads X and s and writes q, overwrites it.  With
// a single run the first kernel writes s itself.  If Q is not 4-byte
// aligned, the runs instead raise S[col] with an integer atomic max on the
// float's bits (s >= +0, whose bit patterns order like their values, and
// rounding max / 127 to nearest is monotone, so this gives the same s in any
// order), after S is zeroed.
constexpr int kRun = 64;      // rows per workgroup of the column kernels
constexpr int kBatch = 8;     // loads issued together per thread
constexpr int kColBlk = 512;  // columns per workgroup of the column kernels

template <class T>
__device__ __forceinline__ void load8_cols(const T *row, int64_t c0, int64_t C, bool vec, float (&v)[8]) {
  if (vec) {
    load8(row + c0, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = c0 + i < C ? widen<T>(row[c0 + i]) : 0.f;
  }
}

__global__ __launch_bounds__(kQT) void fill_zero(float *S, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kQT + threadIdx.x;
  if (i < n) S[i] = 0.f;
}

// mode 0: write the run's maxima to P; 1: write s (single run); 2: atomic max into S
template <class T>
__global__ __launch_bounds__(kQT) void col_max(const T *__restrict__ X, float *__restrict__ P, float *__restrict__ S,
                                               int64_t R, int64_t C, int vec, int mode) {
  __shared__ float part[4][kColBlk];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kColBlk + 8 * lane;
  const int64_t r0 = (int64_t)blockIdx.y * kRun;
  const int64_t r1 = r0 + kRun < R ? r0 + kRun : R;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < C)
    // eight rows per batch, their loads issued together; rows past the run
    // repeat the run's last row (the max does not change)
    for (int64_t rb = r0 + w; rb < r1; rb += 4 * kBatch) {
      float v[kBatch][8];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int64_t r = rb + 4 * k < r1 ? rb + 4 * k : r1 - 1;
        load8_cols(X + r * C, c0, C, vec, v[k]);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[k][i]));
    }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[w][8 * lane + i] = m[i];
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x + kQT * h;
    const int64_t col = (int64_t)blockIdx.x * kColBlk + c;
    if (col >= C) continue;
    const float mx = fmaxf(fmaxf(part[0][c], part[1][c]), fmaxf(part[2][c], part[3][c]));
    if (mode == 0) {
      P[blockIdx.y * C + col] = mx;
    } else {
      const float s = __fdiv_rn(mx, 127.f);
      if (mode == 1) S[col] = s;
      else if (s > 0.f) atomicMax(reinterpret_cast<int *>(S + col), __float_as_int(s));
    }
  }
}

// max over the runs' partial rows: a workgroup takes 16 columns, its 16
// run-groups of 16 threads each take every 16th run, and meet in LDS
__global__ __launch_bounds__(kQT) void col_reduce(const float *__restrict__ P, float *__restrict__ S, int64_t runs,
                                                  int64_t C) {
  __shared__ float part[16][16];
  const int c = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int64_t col = (int64_t)blockIdx.x * 16 + c;
  float m = 0.f;
  if (col < C)
    for (int64_t rb = g; rb < runs; rb += 16 * kBatch) {
      float t[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int64_t r = rb + 16 * k < runs ? rb + 16 * k : runs - 1;
        t[k] = P[r * C + col];
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) m = fmaxf(m, t[k]);
    }
  part[g][c] = m;
  __syncthreads();
  if (g == 0 && col < C) {
#pragma unroll
    for (int j = 1; j < 16; ++j) m = fmaxf(m, part[j][c]);
    S[col] = __fdiv_rn(m, 127.f);
  }
}

// q from X and s: a wave takes kQRows consecutive rows of the block's 512
// columns, loading the 8 column scales of each lane once and all its rows'
// inputs together, so one memory round trip serves the wave; many short
// waves then hide the latency, as in the row kernel.  Row groups are
// grid-strided past the grid's y limit.
constexpr int kQRows = 4;                       // rows per wave of col_quant
constexpr int kQGroup = 4 * kQRows;             // rows per workgroup of col_quant

template <class T>
__global__ __launch_bounds__(kQT) void col_quant(const T *__restrict__ X, const float *__restrict__ S,
                                                 int8_t *__restrict__ Q, int64_t R, int64_t C, int vec) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kColBlk + 8 * lane;
  if (c0 >= C) return;
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = c0 + i < C ? S[c0 + i] : 0.f;
  const int64_t groups = (R + kQGroup - 1) / kQGroup;
  for (int64_t gy = blockIdx.y; gy < groups; gy += gridDim.y) {
    const int64_t r0 = gy * kQGroup + (int64_t)w * kQRows;
    if (r0 >= R) break;
    float v[kQRows][8];
#pragma unroll
    for (int k = 0; k < kQRows; ++k) {
      const int64_t r = r0 + k < R ? r0 + k : R - 1;
      load8_cols(X + r * C, c0, C, vec, v[k]);
    }
#pragma unroll
    for (int k = 0; k < kQRows; ++k) {
      if (r0 + k >= R) break;
      int8_t *q = Q + (r0 + k) * C + c0;
      if (vec) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo |= (uint32_t)(uint8_t)quant1(v[k][i], s[i]) << (8 * i);
          hi |= (uint32_t)(uint8_t)quant1(v[k][4 + i], s[4 + i]) << (8 * i);
        }
        *reinterpret_cast<uint2 *>(q) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c0 + i < C) q[i] = quant1(v[k][i], s[i]);
      }
    }
  }
}

constexpr int kGridCap = 8 * 1024;   // workgroups of the packer's grid-stride kernels

int prep_check(const void *X, int kind, const void *Q, const void *S, int64_t R, int64_t C, int64_t ns) {
  if (!X || !Q || !S) return TGEMM_ERR_NULL;
  if (kind != TGEMM_IN_F32 && kind != TGEMM_IN_BF16) return TGEMM_ERR_KIND;
  if (R < 1 || C < 1 || R > INT64_MAX / C / 4) return TGEMM_ERR_DIM;
  const int64_t xb = R * C * (kind == TGEMM_IN_F32 ? 4 : 2);
  if (overlap(Q, R * C, X, xb) || overlap(S, 4 * ns, X, xb) || overlap(S, 4 * ns, Q, R * C))
    return TGEMM_ERR_ALIAS;
  return TGEMM_OK;
}

}  // namespace

extern "C" {

int ternary_pack_weights(const int8_t *Wt, uint8_t *Wpacked, int64_t N, int64_t K, hipStream_t stream) {
  if (!Wt || !Wpacked) return TGEMM_ERR_NULL;
  if (N < 1 || K < 1 || N > INT64_MAX / K) return TGEMM_ERR_DIM;
  if (K % 4 != 0) return TGEMM_ERR_PACK;
  const int64_t outb = N * (K / 4);
  if (overlap(Wpacked, outb, Wt, N * K)) return TGEMM_ERR_ALIAS;
  int64_t done = 0;
  if (aligned(Wt, 16) && aligned(Wpacked, 16)) {
    const int64_t chunks = outb / 16;   // 64 input bytes -> 16 stored bytes
    if (chunks > 0) {
      const int64_t g = (chunks + 255) / 256;
      hipLaunchKernelGGL(pack_vec, dim3((unsigned)(g < kGridCap ? g : kGridCap)), dim3(256), 0, stream,
                         reinterpret_cast<const v4u *>(Wt), reinterpret_cast<v4u *>(Wpacked), chunks);
      done = 16 * chunks;
    }
  }
  if (done < outb) {
    const int64_t rest = outb - done, g = (rest + 255) / 256;
    hipLaunchKernelGGL(pack_bytes, dim3((unsigned)(g < kGridCap ? g : kGridCap)), dim3(256), 0, stream, Wt,
                       Wpacked, done, rest);
  }
  return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}

int ternary_quantize_rows(const void *X, int in_kind, int8_t *Q, float *scale, int64_t R, int64_t C,
                          hipStream_t stream) {
  const int st = prep_check(X, in_kind, Q, scale, R, C, R);
  if (st != TGEMM_OK) return st;
  const int esz = in_kind == TGEMM_IN_F32 ? 4 : 2;
  const int vec = (C % 8 == 0 && aligned(X, 8 * esz > 16 ? 16 : 8 * esz) && aligned(Q, 8)) ? 1 : 0;
  const int64_t nu = C / 8;
  if (vec && nu <= 64 * 8) {
    // one wave per row, the row in registers: V units of 8 per lane
    const int64_t gw = (R + 3) / 4;
    const dim3 g((unsigned)(gw < 65536 * 8 ? gw : 65536 * 8));
    const int V = nu <= 64 ? 1 : nu <= 128 ? 2 : nu <= 256 ? 4 : 8;
#define QRW(TY, VV) hipLaunchKernelGGL((quant_rows_wave<TY, VV>), g, dim3(256), 0, stream, static_cast<const TY *>(X), Q, scale, R, C)
    if (in_kind == TGEMM_IN_F32) {
      if (V == 1) QRW(float, 1); else if (V == 2) QRW(float, 2); else if (V == 4) QRW(float, 4); else QRW(float, 8);
    } else {
      if (V == 1) QRW(uint16_t, 1); else if (V == 2) QRW(uint16_t, 2); else if (V == 4) QRW(uint16_t, 4); else QRW(uint16_t, 8);
    }
#undef QRW
    return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
  }
  const unsigned g = (unsigned)(R < 65536 * 32 ? R : 65536 * 32);
  if (in_kind == TGEMM_IN_F32)
    hipLaunchKernelGGL(quant_rows<float>, dim3(g), dim3(kQT), 0, stream, static_cast<const float *>(X), Q, scale,
                       R, C, vec);
  else
    hipLaunchKernelGGL(quant_rows<uint16_t>, dim3(g), dim3(kQT), 0, stream, static_cast<const uint16_t *>(X), Q,
                       scale, R, C, vec);
  return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}

int ternary_quantize_cols(const void *X, int in_kind, int8_t *Q, float *scale, int64_t R, int64_t C,
                          hipStream_t stream) {
  const int st = prep_check(X, in_kind, Q, scale, R, C, C);
  if (st != TGEMM_OK) return st;
  const int esz = in_kind == TGEMM_IN_F32 ? 4 : 2;
  const int vec = (C % 8 == 0 && aligned(X, 8 * esz > 16 ? 16 : 8 * esz) && aligned(Q, 8)) ? 1 : 0;
  const int64_t gx = (C + kColBlk - 1) / kColBlk, runs = (R + kRun - 1) / kRun;
  if (gx > INT32_MAX || runs > 65535) return TGEMM_ERR_DIM;
  const dim3 grid((unsigned)gx, (unsigned)runs);
  // partial maxima in Q's memory (runs * C floats <= R * C bytes) when Q is 4-byte aligned
  const int mode = runs == 1 ? 1 : aligned(Q, 4) ? 0 : 2;
  float *P = reinterpret_cast<float *>(Q);
  if (mode == 2) {
    const int64_t gz = (C + kQT - 1) / kQT;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)gz), dim3(kQT), 0, stream, scale, C);
  }
  if (in_kind == TGEMM_IN_F32)
    hipLaunchKernelGGL(col_max<float>, grid, dim3(kQT), 0, stream, static_cast<const float *>(X), P, scale, R, C,
                       vec, mode);
  else
    hipLaunchKernelGGL(col_max<uint16_t>, grid, dim3(kQT), 0, stream, static_cast<const uint16_t *>(X), P, scale, R,
                       C, vec, mode);
  if (mode == 0)
    hipLaunchKernelGGL(col_reduce, dim3((unsigned)((C + 15) / 16)), dim3(kQT), 0, stream, P, scale, runs, C);
  const int64_t qgroups = (R + kQGroup - 1) / kQGroup;
  const dim3 qgrid((unsigned)gx, (unsigned)(qgroups < 65535 ? qgroups : 65535));
  if (in_kind == TGEMM_IN_F32)
    hipLaunchKernelGGL(col_quant<float>, qgrid, dim3(kQT), 0, stream, static_cast<const float *>(X), scale, Q, R,
                       C, vec);
  else
    hipLaunchKernelGGL(col_quant<uint16_t>, qgrid, dim3(kQT), 0, stream, static_cast<const uint16_t *>(X), scale,
                       Q, R, C, vec);
  return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}

}  // extern "C"
