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

// Packed sequences (seq_idx): per chunk, the running count of sequence starts.
// A start is a step whose label differs from the previous step's (mamba issue
// #647's repro passes seq_idx to the chunked scan; the state does not flow
// across a start).  One wave per (batch, chunk); lane l owns steps
// l*E .. l*E+E-1 and a wave-wide inclusive scan adds the lanes' counts.  The
// kernels mask with these counts: steps s <= t of one chunk interact only if
// their counts are equal, the entering state reaches step t only if its count
// is 0, and a chunk whose last count is non-zero drops the carried state.
template <int Q>
__global__ __launch_bounds__(256) void seq_count_kernel(const int32_t* __restrict__ seq,
                                                       int32_t* __restrict__ ws_seg, int64_t L,
                                                       int64_t nc, int64_t nunits) {
  constexpr int E = Q / kWave;
  const int64_t u = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;  // b*nc + c
  if (u >= nunits) return;  // whole wave leaves together; no barrier follows
  const int64_t c = u % nc, b = u / nc;
  const int lane = threadIdx.x % kWave;
  int run[E];
  int total = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t t = c * Q + (int64_t)lane * E + i;
    if (t >= 1 && t < L) total += seq[b * L + t] != seq[b * L + t - 1];
    run[i] = total;
  }
  const int incl = wave_incl_sum(total);
  const int base = incl - total;
  int32_t* dst = ws_seg + u * Q + lane * E;
#pragma unroll
  for (int i = 0; i < E; ++i) dst[i] = base + run[i];
}

hipError_t launch_seq_count(const Problem& p, hipStream_t s) {
  const int64_t nunits = p.b * p.nc;
  const dim3 grid((unsigned)((nunits + 3) / 4));
  switch (p.Q) {
    case 64:
      hipLaunchKernelGGL((seq_count_kernel<64>), grid, dim3(256), 0, s, p.seq_idx, p.ws_seg, p.L,
                         p.nc, nunits);
      break;
    case 128:
      hipLaunchKernelGGL((seq_count_kernel<128>), grid, dim3(256), 0, s, p.seq_idx, p.ws_seg,
                         p.L, p.nc, nunits);
      break;
    case 256:
      hipLaunchKernelGGL((seq_count_kernel<256>), grid, dim3(256), 0, s, p.seq_idx, p.ws_seg,
                         p.L, p.nc, nunits);
      break;
  }
  return hipGetLastError();
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
