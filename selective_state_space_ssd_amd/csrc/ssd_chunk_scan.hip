// Stage 4 (+5): outputs of one chunk, with the D-skip and z-gate epilogue.
//
//   Y[t][p] = exp(cum_t) * sum_n C_t[n] H_in[p][n]                  (state part)
//           + sum_{s <= t} (C_t . B_s) exp(cum_t - cum_s) dt_s x_s[p]  (in-chunk)
//   out[t][p] = (Y[t][p] + D_h x_t[p]) * silu(z_t[p])
//
// The in-chunk part is the masked "attention" form of the scan: query C,
// key B, value dt*x, decay mask exp(cum_t - cum_s) for s <= t, no 1/sqrt(d)
// scale, keys/queries shared by the heads of a group (flash-linear-attention
// PR #49, its list of differences between simple_gla and the mamba2_ssd
// kernel).  D skip and SiLU gate before any norm: mamba issue #647's repro
// script (norm_before_gate=False).
//
// One workgroup (4 waves) per (batch, chunk, head).  x of the chunk and the
// incoming state are staged in LDS; each wave owns whole 16-row t-blocks,
// paired (w, 7-w) so that every wave gets the same number of causal blocks.
// Per t-block, all on v_mfma_f32_16x16x4_f32:
//   1. acc  = C_tb . H_in^T                 (contraction over n)
//   2. acc *= exp(cum_t)
//   3. for each s-block sb <= tb:
//        G = B_sb . C_tb^T                 (contraction over n; G[s][t])
//        M = G * exp(cum_t - cum_s) * dt_s, zero where s > t
//        acc += M^T . x_sb                 (contraction over s)
//   4. out = (acc + D x) * silu(z), stored four p at a time.
// Only pairwise decays exp(cum_t - cum_s) with s <= t are formed, and they are
// at most 1, so nothing overflows however negative the running sums get.
//
// Lane layout: in the accumulator, register r of lane l holds row
// t = 16*tb + 4*(l/16) + r and column p = 4*(l%16) + j of p-block j, so a lane
// stores four consecutive p of one row.  The state is staged with its rows
// permuted (LDS row 16*j + i holds H_in row 4*i + j) so that the 16 lanes of a
// read hit 16 consecutive padded rows.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

template <typename T, int Q, int N>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ Dv, const T* __restrict__ z, const float* __restrict__ ws_dt,
    const float* __restrict__ ws_cum, const float* __restrict__ states_in, T* __restrict__ out,
    int64_t L, int64_t H, int64_t G, int64_t nc, int64_t nunits) {
  constexpr int P = 64;
  constexpr int NK = N / 4;      // MFMA k-steps over n (4 per step)
  constexpr int HS = N + 4;      // padded row stride of the staged state
  constexpr int NTB = Q / 16;    // t-blocks per chunk
  __shared__ float x_lds[Q * P];
  __shared__ float h_lds[P * HS];
  __shared__ float cum_lds[Q];
  __shared__ float dt_lds[Q];

  const int64_t u = xcd_remap(blockIdx.x, nunits);  // ((b*nc + c)*H + h)
  const int64_t h = u % H;
  const int64_t c = (u / H) % nc;
  const int64_t b = u / (H * nc);
  const int64_t g = h / (H / G);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int li = lane % 16, lk = lane / 16;
  const int64_t t0 = c * Q;
  const int64_t xstride = H * P, bstride = G * N;

  // ---- stage x, H_in, cum, dt --------------------------------------------------
  {
    const T* xs = x + ((b * L + t0) * H + h) * P;
#pragma unroll
    for (int i = 0; i < Q * P / 4 / 256; ++i) {
      const int e = (i * 256 + tid) * 4;
      const int row = e / P, col = e % P;
      f4 v = (t0 + row < L) ? ld4(xs + row * xstride + col) : f4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f4*>(&x_lds[row * P + col]) = v;
    }
    const float* hsrc = states_in + u * (int64_t)(P * N);
#pragma unroll
    for (int i = 0; i < P * N / 4 / 256; ++i) {
      const int e = (i * 256 + tid) * 4;
      const int p = e / N, n = e % N;
      const int prow = 16 * (p % 4) + p / 4;
      *reinterpret_cast<f4*>(&h_lds[prow * HS + n]) = ld4(hsrc + e);
    }
    const int64_t dc = ((b * H + h) * nc + c) * Q;
    if (tid < Q) {
      cum_lds[tid] = ws_cum[dc + tid];
      dt_lds[tid] = ws_dt[dc + tid];
    }
  }
  __syncthreads();

  const float Dh = Dv ? Dv[h] : 0.0f;
  const T* Cbase = Cm + ((b * L + t0) * G + g) * N + NK * lk;
  const T* Bbase = Bm + ((b * L + t0) * G + g) * N + NK * lk;

  for (int m = 0; m < (NTB + 7) / 8 * 2; ++m) {
    // t-blocks of this wave: (8k + w, 8k + 7 - w), or just w when NTB == 4
    int tb;
    if (NTB == 4) {
      if (m > 0) break;
      tb = wave;
    } else {
      tb = (m / 2) * 8 + ((m % 2) ? 7 - wave : wave);
    }

    // C rows of this t-block: lane row t = 16*tb + li, n = NK*lk + s
    float creg[NK];
    {
      const int trow = 16 * tb + li;
      const bool ok = t0 + trow < L;
      const T* cp = Cbase + trow * bstride;
#pragma unroll
      for (int s = 0; s < NK; s += 4) {
        f4 v = ok ? ld4(cp + s) : f4{0.f, 0.f, 0.f, 0.f};
        creg[s] = v[0];
        creg[s + 1] = v[1];
        creg[s + 2] = v[2];
        creg[s + 3] = v[3];
      }
    }

    // 1. state part
    f4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < NK; s4 += 4) {
      f4 hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hv[j] = *reinterpret_cast<const f4*>(&h_lds[(16 * j + li) * HS + NK * lk + s4]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16x16x4(creg[s4 + s], hv[j][s], acc[j]);
    }
    // 2. decay from the chunk start
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = __expf(cum_lds[16 * tb + 4 * lk + r]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j][r] *= e;
    }

    // 3. in-chunk part, causal s-blocks
    const int tcol = 16 * tb + li;
    const float cum_t = cum_lds[tcol];
    for (int sb = 0; sb <= tb; ++sb) {
      float breg[NK];
      {
        const int srow = 16 * sb + li;
        const bool ok = t0 + srow < L;
        const T* bp = Bbase + srow * bstride;
#pragma unroll
        for (int s = 0; s < NK; s += 4) {
          f4 v = ok ? ld4(bp + s) : f4{0.f, 0.f, 0.f, 0.f};
          breg[s] = v[0];
          breg[s + 1] = v[1];
          breg[s + 2] = v[2];
          breg[s + 3] = v[3];
        }
      }
      f4 gacc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NK; ++s) gacc = mfma16x16x4(breg[s], creg[s], gacc);
      // gacc[r] = C_t . B_s for s = 16*sb + 4*lk + r, t = tcol
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int srow = 16 * sb + 4 * lk + r;
        const float wgt = __expf(cum_t - cum_lds[srow]) * dt_lds[srow];
        const float mv = (srow <= tcol) ? gacc[r] * wgt : 0.0f;
        const f4 xv = *reinterpret_cast<const f4*>(&x_lds[srow * P + 4 * li]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16x16x4(mv, xv[j], acc[j]);
      }
    }

    // 4. epilogue: D skip, SiLU gate, store
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int trow = 16 * tb + 4 * lk + r;
      if (t0 + trow >= L) continue;
      const f4 xv = *reinterpret_cast<const f4*>(&x_lds[trow * P + 4 * li]);
      f4 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = acc[j][r] + Dh * xv[j];
      const int64_t o = ((b * L + t0 + trow) * H + h) * P + 4 * li;
      if (z) {
        const f4 zv = ld4(z + o);
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] *= silu(zv[j]);
      }
      st4(out + o, y);
    }
  }
}

template <typename T, int Q, int N>
static void launch_qn(const Problem& p, hipStream_t s) {
  const int64_t nunits = p.b * p.nc * p.H;
  hipLaunchKernelGGL((chunk_scan_kernel<T, Q, N>), dim3((unsigned)nunits), dim3(256), 0, s,
                     static_cast<const T*>(p.x), static_cast<const T*>(p.B),
                     static_cast<const T*>(p.C), p.D, static_cast<const T*>(p.z), p.ws_dt,
                     p.ws_cum, p.ws_states_in, static_cast<T*>(p.out), p.L, p.H, p.G, p.nc,
                     nunits);
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

hipError_t launch_chunk_scan(const Problem& p, hipStream_t stream) {
  if (p.bf16)
    launch_t<bf16_t>(p, stream);
  else
    launch_t<float>(p, stream);
  return hipGetLastError();
}

bool config_supported(int64_t P, int64_t N, int64_t Q) {
  return P == 64 && (N == 16 || N == 32 || N == 64 || N == 128) &&
         (Q == 64 || Q == 128 || Q == 256);
}

}  // namespace ssd
