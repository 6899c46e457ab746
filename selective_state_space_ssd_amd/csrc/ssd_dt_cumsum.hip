// Stage 1: discretization step and its running sum inside each chunk.
//
//   dt_t = clamp(softplus(dt_raw_t + dt_bias_h), dt_min, dt_max)
//   cum_t = sum_{r = chunk start .. t} dt_r * A_h
//
// dt as a discretization input folded into the log-gate dt*A with a constant
// A per head: flash-linear-attention PR #49, its list of differences between
// the simple_gla and mamba2_ssd kernels.  dt_bias and dt_limit: the argument
// list of the repro script on mamba issue #647.
//
// One wave per (batch, chunk, head); lane l owns Q/64 consecutive timesteps,
// sums them serially, and a wave-wide inclusive scan of the lane totals gives
// each lane its offset.  Timesteps past the end of the sequence get dt = 0 and
// dA = 0, so the last cum of a ragged chunk equals the cum of its last step.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

// softplus(u) = log(1 + e^u) in a form that neither overflows nor cancels.
__device__ __forceinline__ float softplus(float u) {
  return fmaxf(u, 0.0f) + log1pf(expf(-fabsf(u)));
}

template <typename T, int Q>
__global__ __launch_bounds__(256) void dt_cumsum_kernel(const T* __restrict__ dt_raw,
                                                       const float* __restrict__ A,
                                                       const float* __restrict__ dt_bias,
                                                       float dt_min, float dt_max,
                                                       float* __restrict__ dt_out,
                                                       float* __restrict__ cum_out, int64_t L,
                                                       int64_t H, int64_t nc) {
  constexpr int E = Q / kWave;  // timesteps per lane
  const int lane = threadIdx.x % kWave;
  const int64_t h = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t c = blockIdx.y;
  const int64_t b = blockIdx.z;
  if (h >= H) return;  // whole wave leaves together

  const float a = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  float dtv[E], run[E];
  float total = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t t = c * Q + (int64_t)lane * E + i;
    float d = 0.0f;
    if (t < L) {
      d = softplus(ld1(dt_raw + (b * L + t) * H + h) + bias);
      // comparisons (not fminf/fmaxf) so that a NaN input stays NaN
      d = d < dt_min ? dt_min : d;
      d = d > dt_max ? dt_max : d;
    }
    dtv[i] = d;
    total += d * a;
    run[i] = total;
  }
  // inclusive scan of lane totals across the wave
  float incl = total;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  const float base = incl - total;
  const int64_t o = ((b * H + h) * nc + c) * Q + (int64_t)lane * E;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    dt_out[o + i] = dtv[i];
    cum_out[o + i] = base + run[i];
  }
}

template <typename T, int Q>
static void launch_q(const Problem& p, hipStream_t s) {
  dim3 grid((unsigned)((p.H + 3) / 4), (unsigned)p.nc, (unsigned)p.b);
  hipLaunchKernelGGL((dt_cumsum_kernel<T, Q>), grid, dim3(256), 0, s,
                     static_cast<const T*>(p.dt), p.A, p.dt_bias, p.dt_min, p.dt_max, p.ws_dt,
                     p.ws_cum, p.L, p.H, p.nc);
}

template <typename T>
static void launch_t(const Problem& p, hipStream_t s) {
  switch (p.Q) {
    case 64: launch_q<T, 64>(p, s); break;
    case 128: launch_q<T, 128>(p, s); break;
    case 256: launch_q<T, 256>(p, s); break;
  }
}

hipError_t launch_dt_cumsum(const Problem& p, hipStream_t stream) {
  if (p.bf16)
    launch_t<bf16_t>(p, stream);
  else
    launch_t<float>(p, stream);
  return hipGetLastError();
}

}  // namespace ssd
