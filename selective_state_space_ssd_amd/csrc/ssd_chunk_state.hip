// Stage 2: each chunk's own contribution to the state,
//
//   S_c[p][n] = sum_{t in chunk c} x_t[p] * w_t * B_t[n],
//   w_t = exp(cum_last - cum_t) * dt_t,
//
// i.e. the recurrence run over the chunk alone from a zero state, as a
// [P x Q] x [Q x N] product on the matrix cores with fp32 accumulation.  The
// contraction index is time.  Results go to the workspace in the tiled state
// layout (ssd_device.h).
//
// Packed sequences (seq_idx): only the steps of the chunk's last sequence
// reach the chunk's end state, so w_t = 0 for steps whose sequence-start count
// (ws_seg) differs from the chunk's last one.
//
// Two kernels:
//  * chunk_state_wave_kernel (N = 64 or 128): WPH waves per (chunk, head)
//    (two as launched), 4 waves (two heads) per workgroup: two workgroups
//    per compute unit in the same round measured 0.5 us faster than one of
//    four heads on batch 2 x 2048.  The first wave of a head
//    computes dt and the in-chunk cumsum (stage 1, fused here); then each wave
//    holds 32-column n-tiles of the state tile in accumulators of v_mfma_f32_32x32x2_f32
//    while it walks the chunk two timesteps per MFMA.  It computes
//    S^T = B^T (w x): lane l supplies B[t][32*nt + l%32] (A operand) and
//    w_t x[t][2*(l%32) + pt] (B operand) for timestep t = 2m + l/32, so x is
//    read as float2 and each register group of the result is four
//    consecutive n of one p -- one float4 of the tiled layout.
//  * chunk_state_kernel (any N): four waves per (chunk, head) on
//    v_mfma_f32_16x16x4_f32, after a separate stage-1 launch.
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {

// ---------------------------------------------------------------------------
// one wave per (chunk, head), stage 1 fused
// ---------------------------------------------------------------------------

template <typename T, int Q, int N, int WPH>
__global__ __launch_bounds__(256) void chunk_state_wave_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ dt_raw,
    const float* __restrict__ A, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    float* __restrict__ ws_dt, float* __restrict__ ws_cum, float* __restrict__ states,
    const int32_t* __restrict__ seg, int64_t L, int64_t H, int64_t G, int64_t nc, int64_t nunits) {
  // WPH waves per head, each owning NTW n-tiles (both p-halves); HPW heads per
  // workgroup of 4 waves
  constexpr int P = 64, NTN = N / 32, NTW = NTN / WPH, HPW = 4 / WPH, E = Q / kWave;
  static_assert((N == 64 || N == 128) && NTW >= 1 && NTW * WPH == NTN, "tile");
  __shared__ float w_lds[HPW][2][Q / 2];  // [head][t % 2][t / 2]

  const int64_t HQ = (H + HPW - 1) / HPW;
  const int64_t u = xcd_remap(blockIdx.x, nunits);  // ((b*nc + c)*HQ + hq)
  const int64_t hq = u % HQ, c = (u / HQ) % nc, b = u / (HQ * nc);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int slot = wave / WPH, half = wave % WPH;  // head within the workgroup, wave within the head
  const int64_t h = hq * HPW + slot;
  const bool active = h < H;

  // The ring's first loads are issued before the dt phase and its barrier,
  // whose latency they overlap.  A wave past the last head (H odd) reads
  // head H-1's rows and returns after the barrier.
  const int64_t ha = active ? h : H - 1;
  // 32-bit and wave-uniform (the B buffer resource needs a scalar base)
  const int64_t g = __builtin_amdgcn_readfirstlane((int)ha / (int)(H / G));
  const int i = lane % 32, kk = lane / 32;
  const int64_t t0 = c * Q;
  const float* wrow = w_lds[slot][kk];  // w of timesteps 2m + kk, m = 0 .. Q/2-1

  f16x acc[NTW][2];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) acc[nt][0] = acc[nt][1] = zero16();

  // Loads run PF steps ahead of the MFMAs through a ring of registers.  x and
  // B rows of the chunk are read through buffer resources that end after the
  // chunk's last row: rows past it (a ragged last chunk, and the refills past
  // the chunk's end) read as zero, which is their exact contribution (their
  // w is 0 too), so the loop has no clamp, select or branch.  Offsets are
  // 32-bit (a chunk spans < 2^32 bytes of x and of B).
  constexpr int PF = 8, KS = Q / 2;
  static_assert(KS % PF == 0, "ring");
  const int last = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
  const int64_t xs = H * P, bs = G * N;
  const auto xr = row_rsrc(x + ((b * L + t0) * H + ha) * P, (uint32_t)((last * xs + P) * sizeof(T)));
  const auto br_ = row_rsrc(Bm + ((b * L + t0) * G + g) * N,
                            (uint32_t)((last * bs + N) * sizeof(T)));
  const uint32_t xrow = (uint32_t)(xs * sizeof(T)), brow = (uint32_t)(bs * sizeof(T));
  // step m reads row t = 2m + kk: x at column 2i, B at columns 32 (NTW half + nt) + i
  const uint32_t xl = kk * xrow + 2 * i * sizeof(T);
  const uint32_t bl = kk * brow + (32 * NTW * half + i) * sizeof(T);
  f2 xr_[PF];
  float bq[PF][NTW];
#pragma unroll
  for (int d = 0; d < PF; ++d) {
    xr_[d] = bld2(xr, xl + 2 * d * xrow, T{});
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) bq[d][nt] = bld1(br_, bl + 2 * d * brow + 32 * nt * sizeof(T), T{});
  }
  if (active && half == 0) {
    float dtv[E], cum[E], cum_last;
    wave_dt_cumsum<T, Q>(dt_raw, A[h], dt_bias ? dt_bias[h] : 0.0f, dt_min, dt_max, b, c, h, L,
                         H, nc, ws_dt, ws_cum, dtv, cum, &cum_last);
    const int32_t* sc = seg ? seg + (b * nc + c) * Q : nullptr;
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int t = lane * E + k;
      const bool keep = !sc || sc[t] == sc[Q - 1];
      w_lds[slot][t & 1][t >> 1] = keep ? __expf(cum_last - cum[k]) * dtv[k] : 0.0f;
    }
  }
  __syncthreads();
  if (!active) return;  // after the only barrier

  for (int m0 = 0; m0 < KS; m0 += PF) {
    f4 wv[PF / 4];
#pragma unroll
    for (int k = 0; k < PF / 4; ++k) wv[k] = *reinterpret_cast<const f4*>(wrow + m0 + 4 * k);
    const uint32_t xn = xl + 2 * (m0 + PF) * xrow, bn = bl + 2 * (m0 + PF) * brow;
#pragma unroll
    for (int d = 0; d < PF; ++d) {
      const float w = wv[d / 4][d % 4];
      const float x0 = xr_[d][0] * w, x1 = xr_[d][1] * w;
      float bv[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) bv[nt] = bq[d][nt];
      // refill the slot for step m0 + d + PF (past the chunk: zeros, unused)
      xr_[d] = bld2(xr, xn + 2 * d * xrow, T{});
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) bq[d][nt] = bld1(br_, bn + 2 * d * brow + 32 * nt * sizeof(T), T{});
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        acc[nt][0] = mfma32x32x2(bv[nt], x0, acc[nt][0]);
        acc[nt][1] = mfma32x32x2(bv[nt], x1, acc[nt][1]);
      }
      // keep each step's loads and MFMAs in program order: the scheduler
      // would otherwise sink the refills next to their uses
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // register 4R+e of tile (nt, pt): n = 32*(NTW*half + nt) + 8*R + 4*kk + e, p = 2*i + pt
  float* dst = states + ((b * nc + c) * H + h) * (int64_t)(P * N);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        f4 v;
        v[0] = acc[nt][pt][4 * R];
        v[1] = acc[nt][pt][4 * R + 1];
        v[2] = acc[nt][pt][4 * R + 2];
        v[3] = acc[nt][pt][4 * R + 3];
        const int n = 32 * (NTW * half + nt) + 8 * R + 4 * kk;
        st4(dst + state_tile_offset(2 * i + pt, n, N), v);
      }
}

// ---------------------------------------------------------------------------
// general: four waves per (chunk, head)
// ---------------------------------------------------------------------------

// Wave tiling of the 64 x N state in 16 x 16 blocks: each wave owns MB x NB
// blocks; waves split n first, then p.  Lane l handles timestep 4k + l/16 of
// MFMA step k and reads MB consecutive x values and NB consecutive B values,
// so the p (n) index inside a block is strided by MB (NB).
template <int N>
struct StateTile {
  static constexpr int NB = N >= 128 ? 2 : 1;
  static constexpr int MB = (N / 16) / NB;
  static constexpr int WN = N / (16 * NB);
  static constexpr int WP = 4 / WN;
  static_assert(WN * WP == 4 && MB * 16 * WP == 64, "P = 64 split");
};

template <typename T, int Q, int N>
__global__ __launch_bounds__(256) void chunk_state_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ ws_dt,
    const float* __restrict__ ws_cum, float* __restrict__ states, const int32_t* __restrict__ seg,
    int64_t L, int64_t H, int64_t G, int64_t nc, int64_t nunits) {
  constexpr int P = 64;
  using Tl = StateTile<N>;
  constexpr int MB = Tl::MB, NB = Tl::NB, WP = Tl::WP;
  __shared__ float w_lds[Q];

  const int64_t u = xcd_remap(blockIdx.x, nunits);  // ((b*nc + c)*H + h)
  const int64_t h = u % H;
  const int64_t c = (u / H) % nc;
  const int64_t b = u / (H * nc);
  const int64_t g = h / (H / G);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  const int64_t dc = ((b * H + h) * nc + c) * Q;
  if (tid < Q) {
    const float cum_last = ws_cum[dc + Q - 1];
    const int32_t* sc = seg ? seg + (b * nc + c) * Q : nullptr;
    const bool keep = !sc || sc[tid] == sc[Q - 1];
    w_lds[tid] = keep ? __expf(cum_last - ws_cum[dc + tid]) * ws_dt[dc + tid] : 0.0f;
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
      for (int jn = 0; jn < NB; ++jn)
        dst[state_tile_offset(p, n0 + NB * li + jn, N)] = acc[j][jn][r];
    }
}

// ---------------------------------------------------------------------------

bool chunk_state_fuses_dt(const Problem& p) { return p.N == 64 || p.N == 128; }

template <typename T, int Q, int N>
static void launch_qn(const Problem& p, hipStream_t s) {
  if constexpr (N == 64 || N == 128) {
    // two waves per head: four (one n-tile each) double the waves in flight
    // but load every x row four times, and measured slower (48 vs 39 us on
    // batch 2 x seqlen 2048, 32 heads, dstate 128)
    constexpr int WPH = 2;
    const int64_t nunits = p.b * p.nc * ((p.H + (4 / WPH) - 1) / (4 / WPH));
    hipLaunchKernelGGL((chunk_state_wave_kernel<T, Q, N, WPH>), dim3((unsigned)nunits), dim3(256), 0,
                       s, static_cast<const T*>(p.x), static_cast<const T*>(p.B),
                       static_cast<const T*>(p.dt), p.A, p.dt_bias, p.dt_min, p.dt_max, p.ws_dt,
                       p.ws_cum, p.ws_states, p.ws_seg, p.L, p.H, p.G, p.nc, nunits);
  } else {
    const int64_t nunits = p.b * p.nc * p.H;
    hipLaunchKernelGGL((chunk_state_kernel<T, Q, N>), dim3((unsigned)nunits), dim3(256), 0, s,
                       static_cast<const T*>(p.x), static_cast<const T*>(p.B), p.ws_dt, p.ws_cum,
                       p.ws_states, p.ws_seg, p.L, p.H, p.G, p.nc, nunits);
  }
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
