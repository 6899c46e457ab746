// Measured peaks of one MI355X, for the roofline lines of the benchmark:
// a streaming device copy (the HBM rate a kernel that only moves bytes
// reaches) and loops of independent matrix-core instructions of each kind
// the scan uses (the matrix rate a kernel that only multiplies reaches).
// Built as its own library (libssd_peaks.so); the scan's library does not
// use it.  C entry points:
//
//   int ssd_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t s)
//       dst[0 .. bytes) = src[0 .. bytes); bytes a multiple of 16, both
//       pointers 16-byte aligned.  Returns 0, or -1 for bad arguments, -5 for
//       a launch failure.
//   int ssd_peak_mfma(float* sink, int kind, int workgroups, int iters,
//                     hipStream_t s)
//       `workgroups` workgroups of four waves; every wave runs `iters` rounds
//       of eight independent products of kind `kind` (0: fp32 32x32x2, 1:
//       bf16 32x32x16, 2: bf16 16x16x32, 3: fp32 16x16x4), then
//       writes one float per lane to sink[workgroups * 256] (so nothing is
//       optimised away).  Returns 0, -1 or -5 as above.
//   double ssd_peak_mfma_flops(int kind, int workgroups, int iters)
//       the flops such a launch performs (2 m n k per product).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

enum Kind { kF32_32x32x2 = 0, kBF16_32x32x16 = 1, kBF16_16x16x32 = 2, kF32_16x16x4 = 3 };

typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

// Grid-stride copy, four 16-byte loads in flight per thread before their
// stores (one at a time leaves too few bytes in flight to cover the memory
// latency), then the remainder one by one.
__global__ __launch_bounds__(256) void copy_kernel(const u4v* __restrict__ src,
                                                   u4v* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u4v v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[k], dst + i + k * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Eight independent accumulators per wave (with eight waves per SIMD, far
// more products in flight than a matrix core's issue latency needs; twelve
// or sixteen 16 x 16 tiles made the compiler copy accumulators inside the
// loop).  Every accumulator element is summed at the end so that all of them
// stay live.
template <int K>
constexpr int kAccs = 8;

template <int K>
__device__ __forceinline__ void mfma_step(f16v& acc, float fa, float fb, bf8v a, bf8v b) {
  if constexpr (K == kF32_32x32x2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa, fb, acc, 0, 0, 0);
  else
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
template <int K>
__device__ __forceinline__ void mfma_step(f4v& acc, float fa, float fb, bf8v a, bf8v b) {
  if constexpr (K == kF32_16x16x4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, acc, 0, 0, 0);
  else
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

template <int K>
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ sink, int iters) {
  using Acc = typename std::conditional<K == kF32_32x32x2 || K == kBF16_32x32x16, f16v,
                                        f4v>::type;
  constexpr int NA = kAccs<K>;
  const int lane = threadIdx.x & 63;
  const float fa = 1.0f + 1e-3f * lane, fb = 1.0f - 1e-3f * lane;
  bf8v a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(fa + e);
    b[e] = (__bf16)(fb - e);
  }
  // distinct starting values, so that no two accumulators hold the same
  // computation (the compiler would merge them)
  Acc acc[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    acc[j] = Acc{};
    acc[j][0] = (float)(j + 1) * fa;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NA; ++j) mfma_step<K>(acc[j], fa, fb, a, b);
  }
  float total = 0.0f;
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int e = 0; e < (int)(sizeof(Acc) / sizeof(float)); ++e) total += acc[j][e];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = total;
}

double flops_per_product(int kind) {
  switch (kind) {
    case kF32_32x32x2: return 2.0 * 32 * 32 * 2;
    case kBF16_32x32x16: return 2.0 * 32 * 32 * 16;
    case kBF16_16x16x32: return 2.0 * 16 * 16 * 32;
    case kF32_16x16x4: return 2.0 * 16 * 16 * 4;
    default: return 0.0;
  }
}

}  // namespace

extern "C" {

int ssd_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  if (!src || !dst || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(dst) % 16)
    return -1;
  if (bytes == 0) return 0;
  const int64_t n = (int64_t)(bytes / 16);
  // eight workgroups of 256 threads per compute unit, each thread a
  // grid-stride loop of 16-byte accesses
  const unsigned grid = 256u * 8u;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, s, static_cast<const u4v*>(src),
                     static_cast<u4v*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int ssd_peak_mfma(float* sink, int kind, int workgroups, int iters, hipStream_t s) {
  if (!sink || workgroups <= 0 || iters <= 0 || flops_per_product(kind) == 0.0) return -1;
  const dim3 grid((unsigned)workgroups), block(256);
  switch (kind) {
    case kF32_32x32x2:
      hipLaunchKernelGGL(mfma_kernel<kF32_32x32x2>, grid, block, 0, s, sink, iters);
      break;
    case kBF16_32x32x16:
      hipLaunchKernelGGL(mfma_kernel<kBF16_32x32x16>, grid, block, 0, s, sink, iters);
      break;
    case kBF16_16x16x32:
      hipLaunchKernelGGL(mfma_kernel<kBF16_16x16x32>, grid, block, 0, s, sink, iters);
      break;
    default:
      hipLaunchKernelGGL(mfma_kernel<kF32_16x16x4>, grid, block, 0, s, sink, iters);
      break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

double ssd_peak_mfma_flops(int kind, int workgroups, int iters) {
  // four waves per workgroup, eight products per round
  return flops_per_product(kind) * 8.0 * 4.0 * (double)workgroups * (double)iters;
}

}  // extern "C"
