// Block-level prologue and epilogue around the scan, as mamba issue #647's
// repro calls them through mamba_split_conv1d_scan_combined (out_proj, a dense
// GEMM, is not part of this block).
//
// Prologue (conv_split_kernel): the packed in-projection zxbcdt holds, per
// token, [z (dim) | xBC (dim + 2 G N) | dt (H)] with xBC = [x | B | C].  xBC
// goes through a causal depthwise conv of width W (zeros before the first
// step, framework Conv1d orientation: weight[c][W-1] weighs the current step)
// plus bias, then SiLU, and lands in contiguous x [b,L,H,P], B and C
// [b,L,G,N] tensors of the input dtype; dt is copied out as [b,L,H].  z stays
// in zxbcdt: only the epilogue reads it.
//
// Epilogue (gated_rmsnorm_kernel): with y the scan's output (no gate) and
// g = y * silu(z), out = g / sqrt(mean(g^2) + eps) * weight, the mean over the
// whole width (norm_groups = 1) or over each of norm_groups equal slices
// (norm_before_gate=False); without a weight, out = g.  The page's printed
// outputs differ exactly by this choice: whole width in its python reference,
// per group in its fused kernel.
//
// Both kernels are bandwidth-bound streaming passes: the prologue reads each
// xBC element once (plus a W-1 step halo per time tile) and writes it once;
// the epilogue reads y and z and writes out once, the token's g held in LDS
// between the reduction and the scaling.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {
constexpr int kConvTT = 32;  // timesteps per prologue workgroup

// SiLU with the accurate exp and an IEEE division: the prologue is
// bandwidth-bound, and its result is rounded to the input dtype, so the fewer
// ulps it is off, the rarer a rounding lands on the neighbouring bf16 value.
__device__ __forceinline__ float silu_accurate(float v) { return v / (1.0f + expf(-v)); }

template <typename T>
__device__ __forceinline__ T from_f32(float v) {
  if constexpr (sizeof(T) == 2)
    return (T)f32_to_bf16_bits(v);
  else
    return v;
}
}  // namespace

// One thread per channel (consecutive lanes: consecutive channels, so every
// load and store of a wave is one contiguous run), kConvTT timesteps per
// workgroup with the last W-1 inputs in registers.  Channels past dim + 2GN
// are the dt columns: copied, no conv.
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_split_kernel(
    const T* __restrict__ zx, const float* __restrict__ cw, const float* __restrict__ cb,
    T* __restrict__ xo, T* __restrict__ bo, T* __restrict__ co, T* __restrict__ dto, int64_t L,
    int64_t dim, int64_t gn, int64_t H) {
  const int64_t nch = dim + 2 * gn;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.y * kConvTT, b = blockIdx.z;
  if (c >= nch + H) return;  // no barrier in this kernel
  const int64_t width = 2 * dim + 2 * gn + H;
  const T* src = zx + b * L * width + dim + c;  // column dim + c of row t: src[t * width]
  const int64_t t1 = t0 + kConvTT < L ? t0 + kConvTT : L;
  if (c >= nch) {  // dt column h = c - nch
    T* dst = dto + b * L * H + (c - nch);
    for (int64_t t = t0; t < t1; ++t) dst[t * H] = src[t * width];
    return;
  }
  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = cw[c * W + k];
  const float bias = cb ? cb[c] : 0.0f;
  float win[W];  // win[W-1] is the current step
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t t = t0 - (W - 1) + k;
    win[k] = t >= 0 ? to_f32(src[t * width]) : 0.0f;
  }
  T* dst;
  int64_t stride;
  if (c < dim) {
    dst = xo + b * L * dim + c;
    stride = dim;
  } else if (c < dim + gn) {
    dst = bo + b * L * gn + (c - dim);
    stride = gn;
  } else {
    dst = co + b * L * gn + (c - dim - gn);
    stride = gn;
  }
  for (int64_t t = t0; t < t1; ++t) {
    win[W - 1] = to_f32(src[t * width]);
    float acc = bias;
#pragma unroll
    for (int k = 0; k < W; ++k) acc += w[k] * win[k];
    dst[t * stride] = from_f32<T>(silu_accurate(acc));
#pragma unroll
    for (int k = 0; k < W - 1; ++k) win[k] = win[k + 1];
  }
}

// One workgroup per token: g = y * silu(z) into LDS, one wave per norm slice
// (looping) sums g^2, then every thread scales its channels.  y may be out
// (in place): the row is read completely before the first write.
template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(
    const T* y, const T* __restrict__ zx, const float* __restrict__ weight, float eps,
    T* out, int64_t dim, int64_t width, int norm_groups) {
  extern __shared__ float norm_lds[];  // dim floats of g, then norm_groups scales
  float* g_lds = norm_lds;
  float* inv_lds = norm_lds + dim;
  const int64_t row = blockIdx.x;  // b * L + t
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const T* yr = y + row * dim;
  const T* zr = zx + row * width;  // z = the first dim columns of the row
  for (int64_t c = tid; c < dim; c += 256) g_lds[c] = to_f32(yr[c]) * silu(to_f32(zr[c]));
  T* orow = out + row * dim;
  if (!weight) {
    __syncthreads();  // uniform: every thread takes this branch or none
    for (int64_t c = tid; c < dim; c += 256) orow[c] = from_f32<T>(g_lds[c]);
    return;
  }
  __syncthreads();
  const int64_t gs = dim / norm_groups;
  for (int k = wave; k < norm_groups; k += 256 / kWave) {
    float s = 0.0f;
    for (int64_t c = k * gs + lane; c < (k + 1) * gs; c += kWave) s += g_lds[c] * g_lds[c];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    if (lane == 0) inv_lds[k] = rsqrtf(s / (float)gs + eps);
  }
  __syncthreads();
  for (int64_t c = tid; c < dim; c += 256)
    orow[c] = from_f32<T>(g_lds[c] * inv_lds[c / gs] * weight[c]);
}

bool block_supported(int64_t dim, int norm_groups, int conv_width) {
  return conv_width >= 2 && conv_width <= 4 && dim <= kNormMaxDim && norm_groups >= 1 &&
         norm_groups <= kNormMaxGroups && dim % norm_groups == 0;
}

template <typename T>
static void launch_conv_t(const BlockProblem& q, hipStream_t s) {
  const int64_t dim = q.H * q.P, gn = q.G * q.N;
  const dim3 grid((unsigned)((dim + 2 * gn + q.H + 255) / 256), (unsigned)((q.L + kConvTT - 1) / kConvTT),
                  (unsigned)q.b);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, static_cast<const T*>(q.zxbcdt), q.conv_w,
                       q.conv_b, static_cast<T*>(q.x), static_cast<T*>(q.B), static_cast<T*>(q.C),
                       static_cast<T*>(q.dt), q.L, dim, gn, q.H);
  };
  switch (q.W) {
    case 2: go(conv_split_kernel<T, 2>); break;
    case 3: go(conv_split_kernel<T, 3>); break;
    case 4: go(conv_split_kernel<T, 4>); break;
  }
}

hipError_t launch_conv_split(const BlockProblem& q, hipStream_t s) {
  if (q.bf16)
    launch_conv_t<bf16_t>(q, s);
  else
    launch_conv_t<float>(q, s);
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const BlockProblem& q, hipStream_t s) {
  const int64_t dim = q.H * q.P, width = 2 * dim + 2 * q.G * q.N + q.H;
  const dim3 grid((unsigned)(q.b * q.L));
  const size_t lds = (size_t)(dim + q.norm_groups) * sizeof(float);
  if (q.bf16)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<bf16_t>), grid, dim3(256), lds, s,
                       static_cast<const bf16_t*>(q.y), static_cast<const bf16_t*>(q.zxbcdt),
                       q.norm_w, q.eps, static_cast<bf16_t*>(q.out), dim, width, q.norm_groups);
  else
    hipLaunchKernelGGL((gated_rmsnorm_kernel<float>), grid, dim3(256), lds, s,
                       static_cast<const float*>(q.y), static_cast<const float*>(q.zxbcdt),
                       q.norm_w, q.eps, static_cast<float*>(q.out), dim, width, q.norm_groups);
  return hipGetLastError();
}

}  // namespace ssd
