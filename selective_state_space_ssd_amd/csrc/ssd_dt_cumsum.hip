// Stage 1 as its own kernel: dt and its in-chunk running sum for every
// (batch, chunk, head), one wave each.  Used with the general chunk-state
// kernel; the specialised chunk-state kernel computes the same values itself.
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {

template <typename T, int Q>
__global__ __launch_bounds__(256) void dt_cumsum_kernel(const T* __restrict__ dt_raw,
                                                       const float* __restrict__ A,
                                                       const float* __restrict__ dt_bias,
                                                       float dt_min, float dt_max,
                                                       float* __restrict__ ws_dt,
                                                       float* __restrict__ ws_cum, int64_t L,
                                                       int64_t H, int64_t nc) {
  const int64_t h = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t c = blockIdx.y;
  const int64_t b = blockIdx.z;
  if (h >= H) return;  // whole wave leaves together; no barrier follows
  float dtv[Q / kWave], cum[Q / kWave], last;
  wave_dt_cumsum<T, Q>(dt_raw, A[h], dt_bias ? dt_bias[h] : 0.0f, dt_min, dt_max, b, c, h, L, H,
                       nc, ws_dt, ws_cum, dtv, cum, &last);
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
