// Stage 3: the state entering each chunk,
//
//   H_{-1} = initial state (or 0),  H_c = exp(cum_last_c) * H_{c-1} + S_c,
//
// written as states_in[c] = H_{c-1}; final = H_{nc-1}.  This is the
// associative scan over (decay, state) pairs whose identity is (1, 0) -- the
// same pairs the Mamba-1 scan keeps as intermediates (mamba issue #488, the
// prepended-state workaround that seeds them with (1, 0)).  It runs in fp32,
// sequentially over chunks and in parallel over (batch, head, p, n); each
// thread carries four consecutive state elements (one float4 of the tiled
// state layout) in registers and keeps four chunks of loads in flight.
// Packed sequences (seq_idx): a chunk in which a new sequence starts drops the
// carried state (decay 0); its own contribution S_c already holds only the
// steps of its last sequence.
//
// When the chunk scan that follows is the four-heads kernel, this launch also
// carries workgroups that form that kernel's causal 32 x 32 tiles of G^T =
// B C^T, once per (chunk, group), into the workspace.  They depend on the
// inputs alone; here their matrix work runs beside a pass that is bound by
// memory and leaves the matrix cores idle.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

// ---------------------------------------------------------------------------
// one tile of G^T = B C^T for the chunk scan, one wave
// ---------------------------------------------------------------------------

// Tile `job` = unit * NG + tau, unit = (b*nc + c)*G + g: G^T[s][t] = B_s . C_t
// for s in s-tile si, t in t-tile ti (tile_of), with rows past the sequence end
// taken as zero.  The same products in the same order as the chunk scan's own
// G phase (lane l supplies B[32 si + l%32][(N/2)(l/32) + k] and C[32 ti +
// l%32][...] for k = 0 .. N/2-1), so both give identical tiles; stored in
// register order (ssd_device.h).
template <typename T, int Q, int N>
__device__ __forceinline__ void gram_tile(const T* __restrict__ Bm, const T* __restrict__ Cm,
                                          float* __restrict__ gram, int64_t job, int64_t L,
                                          int64_t G, int64_t nc, int lane) {
  constexpr int NT = Q / 32, NG = NT * (NT + 1) / 2, KQ = N / 8;
  const int64_t unit = job / NG;
  const int tau = (int)(job - unit * NG);
  const int64_t g = unit % G, c = (unit / G) % nc, b = unit / (G * nc);
  int si = 0, ti = 0;
  tile_of<NT>(tau, &si, &ti);
  const int i = lane % 32, kk = lane / 32;
  const int64_t t0 = c * Q;
  const int last = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
  const int rs = 32 * si + i, rt = 32 * ti + i;
  // operands of rows past the end become +0 (a mask, not a branch)
  const uint32_t ms = rs <= last ? ~0u : 0u, mt = rt <= last ? ~0u : 0u;
  const T* bp = Bm + ((b * L + t0 + (rs < last ? rs : last)) * G + g) * N + (N / 2) * kk;
  const T* cp = Cm + ((b * L + t0 + (rt < last ? rt : last)) * G + g) * N + (N / 2) * kk;
  // every operand load at once (one memory latency per tile; the pass beside
  // it keeps the memory system busy, so a tile that waited batch by batch
  // would wait several times), then the 4 KQ products
  f16x acc = zero16();
  f4 bv[KQ], cv[KQ];
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    bv[q] = ld4(bp + 4 * q);
    cv[q] = ld4(cp + 4 * q);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
#pragma unroll
  for (int q = 0; q < KQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = mfma32x32x2(__uint_as_float(__float_as_uint(bv[q][e]) & ms),
                        __uint_as_float(__float_as_uint(cv[q][e]) & mt), acc);
  float* dst = gram + (unit * NG + tau) * 1024 + 4 * lane;
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    f4 v;
    v[0] = acc[4 * R];
    v[1] = acc[4 * R + 1];
    v[2] = acc[4 * R + 2];
    v[3] = acc[4 * R + 3];
    st4(dst + 256 * R, v);
  }
}


// Grid (N/16, H, gz + b): planes z < gz are G^T tiles (QG > 0), one per wave,
// numbered along x, y, z; the others pass states, one plane per batch row.
template <int N, typename T, int QG>
__global__ __launch_bounds__(256) void state_passing_kernel(
    const float* __restrict__ states, const float* __restrict__ ws_cum, const float* init,
    float* __restrict__ states_in, float* final_states, const int32_t* __restrict__ seg,
    int64_t H, int64_t nc, int64_t Q, const T* __restrict__ Bm, const T* __restrict__ Cm,
    float* __restrict__ gram, int64_t gz, int64_t gram_jobs, int64_t L, int64_t G) {
  constexpr int PN = 64 * N;
  constexpr int U = 16;  // chunks in flight
  if constexpr (QG > 0) {
    if (blockIdx.z < gz) {  // whole workgroup
      const int64_t job =
          (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 4 +
          threadIdx.x / kWave;
      if (job < gram_jobs) gram_tile<T, QG, N>(Bm, Cm, gram, job, L, G, nc, threadIdx.x % kWave);
      return;
    }
  }
  const int64_t h = blockIdx.y, b = blockIdx.z - gz;
  const int k = blockIdx.x * blockDim.x + threadIdx.x;  // float4 index in the tiled block
  if (k >= PN / 4) return;
  int p, n;
  state_tile_coords(k, N, &p, &n);
  // init and final_states may be the same buffer: each thread reads its four
  // elements of init before it writes the same four elements of final.
  f4 hs = init ? ld4(init + (b * H + h) * PN + p * N + n) : f4{0.f, 0.f, 0.f, 0.f};
  const float* cum = ws_cum + (b * H + h) * nc * Q + (Q - 1);
  const int64_t cstride = H * PN;
  const float* src = states + (b * nc * H + h) * PN + 4 * k;
  float* dst = states_in + (b * nc * H + h) * PN + 4 * k;
  for (int64_t c0 = 0; c0 < nc; c0 += U) {
    f4 s[U];
    float decay[U];
    bool carry[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (c0 + j < nc) {
        s[j] = ld4(src + (c0 + j) * cstride);
        carry[j] = !seg || seg[(b * nc + c0 + j) * Q + Q - 1] == 0;
        decay[j] = __expf(cum[(c0 + j) * Q]);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (c0 + j < nc) {
        st4(dst + (c0 + j) * cstride, hs);
        hs = carry[j] ? decay[j] * hs + s[j] : s[j];
      }
    }
  }
  if (final_states) st4(final_states + (b * H + h) * PN + p * N + n, hs);
}

int64_t gram_planes(int64_t b, int64_t nc, int64_t H, int64_t N, int64_t G, int64_t Q) {
  const int64_t jobs = b * nc * G * (gram_tile_floats(Q) / 1024);
  const int64_t per_plane = 4 * (N / 16) * H;  // waves in one (x, y) plane
  return (jobs + per_plane - 1) / per_plane;
}

template <int N, typename T, int QG>
static void launch_n(const Problem& p, hipStream_t s) {
  const int64_t gz = QG > 0 ? gram_planes(p.b, p.nc, p.H, N, p.G, QG) : 0;
  const int64_t jobs = QG > 0 ? p.b * p.nc * p.G * (gram_tile_floats(QG) / 1024) : 0;
  dim3 grid((unsigned)((64 * N / 4 + 255) / 256), (unsigned)p.H, (unsigned)(gz + p.b));
  hipLaunchKernelGGL((state_passing_kernel<N, T, QG>), grid, dim3(256), 0, s, p.ws_states,
                     p.ws_cum, p.init, p.ws_states_in, p.final_states, p.ws_seg, p.H, p.nc, p.Q,
                     static_cast<const T*>(p.B), static_cast<const T*>(p.C), p.ws_gram, gz, jobs,
                     p.L, p.G);
}

// the G^T tiles are formed here only for the shapes of the four-heads chunk
// scan: N 64/128 with Q 64/128 (bf16 inputs: Q 64)
template <int N>
static void launch_gram(const Problem& p, hipStream_t s) {
  if constexpr (N == 64 || N == 128) {
    if (p.ws_gram) {
      if (p.bf16) {
        if (p.Q == 64) return launch_n<N, bf16_t, 64>(p, s);
      } else {
        if (p.Q == 64) return launch_n<N, float, 64>(p, s);
        if (p.Q == 128) return launch_n<N, float, 128>(p, s);
      }
    }
  }
  launch_n<N, float, 0>(p, s);
}

hipError_t launch_state_passing(const Problem& p, hipStream_t stream) {
  switch (p.N) {
    case 16: launch_gram<16>(p, stream); break;
    case 32: launch_gram<32>(p, stream); break;
    case 64: launch_gram<64>(p, stream); break;
    case 128: launch_gram<128>(p, stream); break;
  }
  return hipGetLastError();
}

}  // namespace ssd
