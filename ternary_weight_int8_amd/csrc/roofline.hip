// roofline.hip -- measurement probes for bench.py (not part of the GEMM
// library): a write-only pass over an int32 buffer, the HBM store floor for
// an output of a given size, and loops of int8 MFMAs with nothing else in
// the instruction stream, the matrix-core rate the GEMM kernels can reach.
// Built into libtgemm_roofline.so beside libternary_gemm.so.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v16i __attribute__((ext_vector_type(16)));

namespace {

constexpr int kFillThreads = 256;
constexpr int kMfmaThreads = 512;   // 8 waves per CU: two per SIMD
constexpr int kAcc16 = 8;           // independent accumulators per wave
constexpr int kAcc32 = 4;

// dst[i] = value for i < n4 16-byte vectors, grid-stride, one 16-byte store
// per lane per pass
__global__ __launch_bounds__(kFillThreads) void probe_fill(v4i *dst, int64_t n4, int32_t value) {
  const v4i v = {value, value, value, value};
  for (int64_t i = (int64_t)blockIdx.x * kFillThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kFillThreads)
    dst[i] = v;
}

// iters x kAcc16 v_mfma_i32_16x16x64_i8 per wave, independent accumulators
__global__ __attribute__((amdgpu_flat_work_group_size(kMfmaThreads, kMfmaThreads), amdgpu_waves_per_eu(2, 2)))
void probe_mfma16(int32_t *out, int32_t iters) {
  const int32_t t = (int32_t)threadIdx.x;
  const v4i a = {t, 1, 2, 3}, b = {3, 2, 1, t};
  v4i acc[kAcc16];
#pragma unroll
  for (int j = 0; j < kAcc16; ++j) acc[j] = v4i{j, 0, 0, 0};
  for (int32_t it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < kAcc16; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < kAcc16; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * kMfmaThreads + t] = s;
}

// iters x kAcc32 v_mfma_i32_32x32x32_i8 per wave, independent accumulators
__global__ __attribute__((amdgpu_flat_work_group_size(kMfmaThreads, kMfmaThreads), amdgpu_waves_per_eu(2, 2)))
void probe_mfma32(int32_t *out, int32_t iters) {
  const int32_t t = (int32_t)threadIdx.x;
  const v4i a = {t, 1, 2, 3}, b = {3, 2, 1, t};
  v16i acc[kAcc32];
#pragma unroll
  for (int j = 0; j < kAcc32; ++j) acc[j] = v16i{};
  for (int32_t it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < kAcc32; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < kAcc32; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(int64_t)blockIdx.x * kMfmaThreads + t] = s;
}

}  // namespace

extern "C" {

// Fill n int32 (n % 4 == 0, dst 16-byte aligned) with `value` on `stream`.
// Returns 0, or -1 for bad arguments, -2 for a launch error.
int tgemm_roofline_fill(int32_t *dst, int64_t n, int32_t value, hipStream_t stream) {
  if (!dst || n <= 0 || n % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return -1;
  hipLaunchKernelGGL(probe_fill, dim3(2048), dim3(kFillThreads), 0, stream, reinterpret_cast<v4i *>(dst), n / 4,
                     value);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// One workgroup of 8 waves per CU runs `iters` rounds of MFMAs of `shape`
// (16: 16x16x64, 32: 32x32x32) on `stream`; out must hold cus * 512 int32.
// *macs receives the multiply-accumulates the launch performs.  Returns 0,
// -1 for bad arguments, -2 for a HIP error.
int tgemm_roofline_mfma(int32_t *out, int32_t shape, int32_t iters, int32_t cus, int64_t *macs,
                        hipStream_t stream) {
  if (!out || !macs || iters <= 0 || cus <= 0 || (shape != 16 && shape != 32)) return -1;
  const int64_t waves = (int64_t)cus * (kMfmaThreads / 64);
  if (shape == 16) {
    hipLaunchKernelGGL(probe_mfma16, dim3(cus), dim3(kMfmaThreads), 0, stream, out, iters);
    *macs = waves * iters * kAcc16 * (16 * 16 * 64);
  } else {
    hipLaunchKernelGGL(probe_mfma32, dim3(cus), dim3(kMfmaThreads), 0, stream, out, iters);
    *macs = waves * iters * kAcc32 * (32 * 32 * 32);
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
