// Stage 2: each chunk's own contribution to the state,
//
//   S_c[p][n] = sum_{t in chunk c} x_t[p] * w_t * B_t[n],
//   w_t = exp(cum_last - cum_t) * dt_t,
//
// i.e. the recurrence run over the chunk alone from a zero state.  One
// workgroup (4 waves) per (batch, chunk, head); the [P x Q] x [Q x N] product
// runs on v_mfma_f32_16x16x4_f32 with fp32 accumulation.
//
// Operands go from global memory straight into the MFMA lane layout: the
// contraction index is time, and within one 4-deep MFMA step lane l handles
// timestep 4*k + l/16.  Rows of x and B are contiguous in p and n, so a lane
// reads MB consecutive x values and NB consecutive B values of its row; the
// p (n) index of a 16-wide MFMA block is therefore strided by MB (NB).
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

// Wave tiling of the P x N (64 x N) state: each wave owns MB x NB blocks of
// 16 x 16.  Waves split n first, then p.
template <int N>
struct StateTile {
  static constexpr int NB = N >= 128 ? 2 : 1;        // n-blocks per wave
  static constexpr int MB = (N / 16) / NB;            // p-blocks per wave (MB*NB = N/16)
  static constexpr int WN = N / (16 * NB);            // waves along n
  static constexpr int WP = 4 / WN;                   // waves along p
  static_assert(MB * NB * 4 == 4 * (N / 16), "tile");
  static_assert(WN * WP == 4 && MB * 16 * WP == 64, "P = 64 split");
};

template <typename T, int Q, int N>
__global__ __launch_bounds__(256) void chunk_state_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ ws_dt,
    const float* __restrict__ ws_cum, float* __restrict__ states, int64_t L, int64_t H,
    int64_t G, int64_t nc, int64_t nunits) {
  constexpr int P = 64;
  using Tl = StateTile<N>;
  constexpr int MB = Tl::MB, NB = Tl::NB, WP = Tl::WP;
  __shared__ float w_lds[Q];

  const int64_t u = xcd_remap(blockIdx.x, nunits);  // unit = ((b*nc + c)*H + h)
  const int64_t h = u % H;
  const int64_t c = (u / H) % nc;
  const int64_t b = u / (H * nc);
  const int64_t g = h / (H / G);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  const int64_t dc = ((b * H + h) * nc + c) * Q;  // dt / cum of this chunk
  if (tid < Q) {
    const float cum_last = ws_cum[dc + Q - 1];
    w_lds[tid] = __expf(cum_last - ws_cum[dc + tid]) * ws_dt[dc + tid];
  }
  __syncthreads();

  const int p0 = 16 * MB * (wave % WP);
  const int n0 = 16 * NB * (wave / WP);
  const int li = lane % 16, lk = lane / 16;
  f4 acc[MB][NB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int jn = 0; jn < NB; ++jn) acc[j][jn] = f4{0.f, 0.f, 0.f, 0.f};

  const int64_t t0 = c * Q;
  const T* xrow = x + ((b * L + t0) * H + h) * P + p0 + MB * li;
  const T* brow = Bm + ((b * L + t0) * G + g) * N + n0 + NB * li;
  const int64_t xstride = H * P, bstride = G * N;

#pragma unroll 4
  for (int k = 0; k < Q / 4; ++k) {
    const int q = 4 * k + lk;
    float xv[MB], bv[NB];
    if (t0 + q < L) {
      const T* xp = xrow + q * xstride;
      const T* bp = brow + q * bstride;
      if constexpr (MB == 4) {
        f4 v = ld4(xp);
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = v[j];
      } else {
#pragma unroll
        for (int j = 0; j < MB; ++j) xv[j] = ld1(xp + j);
      }
#pragma unroll
      for (int jn = 0; jn < NB; ++jn) bv[jn] = ld1(bp + jn);
    } else {
#pragma unroll
      for (int j = 0; j < MB; ++j) xv[j] = 0.f;
#pragma unroll
      for (int jn = 0; jn < NB; ++jn) bv[jn] = 0.f;
    }
    const float w = w_lds[q];
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int jn = 0; jn < NB; ++jn) acc[j][jn] = mfma16x16x4(xv[j] * w, bv[jn], acc[j][jn]);
  }

  // block (j, jn), register r: p = p0 + MB*(4*lk + r) + j, n = n0 + NB*li + jn
  float* dst = states + u * (int64_t)(P * N);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int p = p0 + MB * (4 * lk + r) + j;
#pragma unroll
      for (int jn = 0; jn < NB; ++jn) dst[p * N + n0 + NB * li + jn] = acc[j][jn][r];
    }
}

template <typename T, int Q, int N>
static void launch_qn(const Problem& p, hipStream_t s) {
  const int64_t nunits = p.b * p.nc * p.H;
  hipLaunchKernelGGL((chunk_state_kernel<T, Q, N>), dim3((unsigned)nunits), dim3(256), 0, s,
                     static_cast<const T*>(p.x), static_cast<const T*>(p.B), p.ws_dt, p.ws_cum,
                     p.ws_states, p.L, p.H, p.G, p.nc, nunits);
}

template <typename T, int Q>
static void launch_q(const Problem& p, hipStream_t s) {
  switch (p.N) {
    case 16: launch_qn<T, Q, 16>(p, s); break;
    case 32: launch_qn<T, Q, 32>(p, s); break;
    case 64: launch_qn<T, Q, 64>(p, s); break;
    case 128: launch_qn<T, Q, 128>(p, s); break;
  }
}

template <typename T>
static void launch_t(const Problem& p, hipStream_t s) {
  switch (p.Q) {
    case 64: launch_q<T, 64>(p, s); break;
    case 128: launch_q<T, 128>(p, s); break;
    case 256: launch_q<T, 256>(p, s); break;
  }
}

hipError_t launch_chunk_state(const Problem& p, hipStream_t stream) {
  if (p.bf16)
    launch_t<bf16_t>(p, stream);
  else
    launch_t<float>(p, stream);
  return hipGetLastError();
}

}  // namespace ssd
