// bf16 path: the chunk-state and chunk-scan stages on v_mfma_f32_32x32x16_bf16
// (fp32 accumulation), for bf16 inputs with chunk 128/256 and dstate 64/128.
//
// The scan's contractions over time need, per lane, eight consecutive
// timesteps of one column, while x and B are stored row-major (time is the
// row).  x tiles therefore go through LDS and are read back with the
// transposed LDS read (lds_tr_operand); B is transposed once per (chunk,
// group) by a small prep kernel into the workspace, so the chunk-state kernel
// reads B^T rows with plain 16-byte loads.  Contractions over n (C.H_in^T and
// C.B^T) read C, B and the state directly in operand layout.
//
// Operand precision: x, B, C are bf16 already and enter the matrix cores
// unchanged.  The operands formed on the fly -- the decay-weighted B^T of the
// chunk-state product, the fp32 state entering a chunk, and the decay-masked
// C.B^T values -- are each split into a hi and a lo bf16 part (split_bf16x8)
// and take two MFMAs, which keeps them to about 16 significant bits: with a
// single bf16 rounding of the entering state or of the masked C.B^T values,
// outputs of N(0,1) inputs at dstate 128 miss the bf16 bar of 2e-2 (1 + |y|)
// by up to 2x.  All sums are fp32 and the state passing stays fp32.
//
// Packed sequences (seq_idx): ws_seg masks the decay-weighted B^T (steps of
// the chunk's last sequence only), the state part (steps of the chunk's first
// sequence only) and the masked C.B^T (pairs of one sequence only).
#include "ssd_bf16_tiles.h"
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {
using namespace bf16t;


// ---------------------------------------------------------------------------
// prep: B^T of every (batch, chunk, group): [b, nc, G] blocks of N x Q bf16
// ---------------------------------------------------------------------------
template <int Q, int N>
__global__ __launch_bounds__(256) void transpose_b_kernel(const bf16_t* __restrict__ Bm,
                                                          bf16_t* __restrict__ bt, int64_t L,
                                                          int64_t G, int64_t nc) {
  __shared__ bf16_t tile[Q][N + 2];
  const int64_t g = blockIdx.x % G, c = (blockIdx.x / G) % nc, b = blockIdx.x / (G * nc);
  const int64_t t0 = c * Q;
  const int last = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
  const bf16_t* src = Bm + ((b * L + t0) * G + g) * N;
  const int tid = threadIdx.x;
  for (int e = tid * 8; e < Q * N; e += 256 * 8) {
    const int row = e / N, col = e % N;
    const int r = row < last ? row : last;
    uint4 v = *reinterpret_cast<const uint4*>(src + r * G * N + col);
    if (row > last) v = uint4{0u, 0u, 0u, 0u};
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[row][col + 2 * j] = (bf16_t)(wd[j] & 0xffffu);
      tile[row][col + 2 * j + 1] = (bf16_t)(wd[j] >> 16);
    }
  }
  __syncthreads();
  bf16_t* dst = bt + blockIdx.x * (int64_t)(N * Q);  // blockIdx.x == (b*nc + c)*G + g
  for (int e = tid * 8; e < Q * N; e += 256 * 8) {
    const int n = e / Q, t = e % Q;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[t + 2 * j][n] | ((uint32_t)tile[t + 2 * j + 1][n] << 16);
    *reinterpret_cast<uint4*>(dst + n * Q + t) = uint4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// chunk state: S^T = (B^T diag(w)) x for one (chunk, head) per workgroup, with
// w_t = exp(cum_last - cum_t) dt_t; the first wave computes dt and cum (stage
// 1) on the way.  The N/32 x 2 output tiles (n-tile, p-half) are split over
// the four waves: with N = 128 wave w owns n-tile w and both p-halves, with
// N = 64 it owns n-tile w/2 and p-half w%2.
// ---------------------------------------------------------------------------
template <int Q, int N>
__global__ __launch_bounds__(256) void chunk_state_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ bt, const bf16_t* __restrict__ dt_raw,
    const float* __restrict__ A, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    float* __restrict__ ws_dt, float* __restrict__ ws_cum, float* __restrict__ states,
    const int32_t* __restrict__ seg, int64_t L, int64_t H, int64_t G, int64_t nc, int64_t nunits) {
  static_assert(N == 64 || N == 128, "dstate 64 or 128");
  constexpr int NPT = N == 128 ? 2 : 1;  // p-halves per wave
  __shared__ bf16_t x_lds[Q * kXLD];
  __shared__ __align__(16) float w_lds[Q];

  const int64_t u = xcd_remap(blockIdx.x, nunits);  // ((b*nc + c)*H + h)
  const int64_t h = u % H, c = (u / H) % nc, b = u / (H * nc);
  const int64_t g = h / (H / G);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i = lane % 32, kk = lane / 32;
  const int64_t t0 = c * Q;
  const int last = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));

  if (wave == 0) {
    float dtv[Q / kWave], cum[Q / kWave], cum_last;
    wave_dt_cumsum<bf16_t, Q>(dt_raw, A[h], dt_bias ? dt_bias[h] : 0.0f, dt_min, dt_max, b, c, h,
                              L, H, nc, ws_dt, ws_cum, dtv, cum, &cum_last);
    // packed sequences: only the chunk's last sequence reaches its end state
    const int32_t* sc = seg ? seg + (b * nc + c) * Q : nullptr;
#pragma unroll
    for (int k = 0; k < Q / kWave; ++k) {
      const int t = lane * (Q / kWave) + k;
      const bool keep = !sc || sc[t] == sc[Q - 1];
      w_lds[t] = keep ? __expf(cum_last - cum[k]) * dtv[k] : 0.0f;
    }
  }
  stage_x_tile<Q>(x_lds, x + ((b * L + t0) * H + h) * kP, H * kP, last);
  __syncthreads();

  const int nt = N == 128 ? wave : wave / 2;
  const int pt0 = N == 128 ? 0 : wave % 2;
  // A operand rows: B^T[n = 32 nt + i][t = 16 ks + 8 kk + 0..7] (steps past the
  // end have w = 0)
  const bf16_t* arow = bt + ((b * nc + c) * G + g) * (int64_t)(N * Q) + (32 * nt + i) * Q + 8 * kk;
  f16x acc[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) acc[j] = zero16();
#pragma unroll 4
  for (int ks = 0; ks < Q / 16; ++ks) {
    const uint4 braw = *reinterpret_cast<const uint4*>(arow + 16 * ks);
    const f4 w0 = *reinterpret_cast<const f4*>(w_lds + 16 * ks + 8 * kk);
    const f4 w1 = *reinterpret_cast<const f4*>(w_lds + 16 * ks + 8 * kk + 4);
    const float av[8] = {bf16_lo(braw.x) * w0[0], bf16_hi(braw.x) * w0[1],
                         bf16_lo(braw.y) * w0[2], bf16_hi(braw.y) * w0[3],
                         bf16_lo(braw.z) * w1[0], bf16_hi(braw.z) * w1[1],
                         bf16_lo(braw.w) * w1[2], bf16_hi(braw.w) * w1[3]};
    s16x8 ahi, alo;
    split_bf16x8(av, ahi, alo);
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      // B operand: x[t = 16 ks + 8 kk + 0..7][p = 2 i + pt]
      const s16x8 bop =
          lds_tr_operand(x_lds, kXLD, 16 * ks + 8 * kk, 16 * ks + 8 * kk + 4, 32 * (pt0 + j));
      acc[j] = mfma32x32x16(ahi, bop, acc[j]);
      acc[j] = mfma32x32x16(alo, bop, acc[j]);
    }
  }
  // register 4R+e: n = 32 nt + 8 R + 4 kk + e, p = 2 i + pt (tiled state layout)
  float* dst = states + u * (int64_t)(kP * N);
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      f4 v;
      v[0] = acc[j][4 * R];
      v[1] = acc[j][4 * R + 1];
      v[2] = acc[j][4 * R + 2];
      v[3] = acc[j][4 * R + 3];
      st4(dst + state_tile_offset(2 * i + pt0 + j, 32 * nt + 8 * R + 4 * kk, N), v);
    }
  }
}

// ---------------------------------------------------------------------------
// chunk scan with the D-skip / z-gate epilogue, one (chunk, head) per
// workgroup.  Wave w owns t-tiles {w, NT-1-w} (NT = 8) or {w} (NT = 4).
// Per t-tile ti: acc = C_ti . H_in^T (then * exp(cum_t)); for each s-tile
// si <= ti: G^T = B_si . C_ti^T, masked and decayed (+ D on the diagonal),
// split into hi/lo bf16, times x_si from LDS; then the epilogue.
// ---------------------------------------------------------------------------
template <int Q, int N, bool GATE>
__global__ __launch_bounds__(256) void chunk_scan_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const float* __restrict__ Dv, const bf16_t* __restrict__ z, const float* __restrict__ ws_dt,
    const float* __restrict__ ws_cum, const float* __restrict__ states_in, bf16_t* __restrict__ out,
    const int32_t* __restrict__ seg, int64_t L, int64_t H, int64_t G, int64_t nc, int64_t nunits) {
  constexpr int NT = Q / 32, NS = NT / 4, KS = N / 16;
  static_assert(NT == 4 || NT == 8, "chunk 128 or 256");
  __shared__ bf16_t x_lds[Q * kXLD];
  __shared__ float cum_lds[Q];  // log2 units
  __shared__ float dt_lds[Q];
  __shared__ int32_t seg_lds[Q];  // sequence starts counted from the chunk start (0: no seq_idx)

  const int64_t u = xcd_remap(blockIdx.x, nunits);  // ((b*nc + c)*H + h)
  const int64_t h = u % H, c = (u / H) % nc, b = u / (H * nc);
  const int64_t g = h / (H / G);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i = lane % 32, kk = lane / 32;
  const int64_t t0 = c * Q;
  const int last = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
  const int64_t xs = H * kP, bs = G * N;

  stage_x_tile<Q>(x_lds, x + ((b * L + t0) * H + h) * kP, xs, last);
  {
    const int64_t dc = ((b * H + h) * nc + c) * Q;
    for (int t = tid; t < Q; t += 256) {
      cum_lds[t] = ws_cum[dc + t] * kLog2e;
      dt_lds[t] = ws_dt[dc + t];
      seg_lds[t] = seg ? seg[(b * nc + c) * Q + t] : 0;
    }
  }
  __syncthreads();

  const bf16_t* Cb = Cm + ((b * L + t0) * G + g) * N + 8 * kk;
  const bf16_t* Bb = Bm + ((b * L + t0) * G + g) * N + 8 * kk;
  const float* hs = states_in + u * (int64_t)(kP * N);
  const float Dh = Dv ? Dv[h] : 0.0f;

#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int ti = j == 0 ? wave : NT - 1 - wave;
    // C rows of this t-tile as operands: C[t = 32 ti + i][16 ks + 8 kk + 0..7]
    s16x8 creg[KS];
    {
      const int tr = 32 * ti + i;
      const int r = tr < last ? tr : last;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        creg[ks] = ld_bf16x8(Cb + r * bs + 16 * ks);
        if (tr > last) creg[ks] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    // 1. state part: acc = C . H_in^T, B operand H[p = 2 i + pt][16 ks + 8 kk + 0..7]
    f16x acc[2] = {zero16(), zero16()};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int n0 = 16 * ks + 8 * kk;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const f4 h0 = ld4(hs + state_tile_offset(2 * i + pt, n0, N));
        const f4 h1 = ld4(hs + state_tile_offset(2 * i + pt, n0 + 4, N));
        const float hv[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        s16x8 hhi, hlo;
        split_bf16x8(hv, hhi, hlo);
        acc[pt] = mfma32x32x16(creg[ks], hhi, acc[pt]);
        acc[pt] = mfma32x32x16(creg[ks], hlo, acc[pt]);
      }
    }
    // 2. decay from the chunk start, rows 32 ti + 8 (r/4) + 4 kk + r%4; with
    // packed sequences the entering state reaches only the first one
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = 32 * ti + 8 * (r / 4) + 4 * kk + (r % 4);
      const float e = seg_lds[tr] == 0 ? exp2f(cum_lds[tr]) : 0.0f;
      acc[0][r] *= e;
      acc[1][r] *= e;
    }
    // 3. in-chunk part (steps of different packed sequences do not interact)
    const float ct = cum_lds[32 * ti + i];
    const int kt = seg_lds[32 * ti + i];
    for (int si = 0; si <= ti; ++si) {
      f16x gt = zero16();
      {
        const int sr = 32 * si + i;
        const int r = sr < last ? sr : last;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s16x8 bv = ld_bf16x8(Bb + r * bs + 16 * ks);
          if (sr > last) bv = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
          gt = mfma32x32x16(bv, creg[ks], gt);  // G^T[s][t]
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float mv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * m + e;
          const int sl = 8 * (r / 4) + 4 * kk + (r % 4);  // s within the tile
          const int s = 32 * si + sl;
          float v = seg_lds[s] == kt ? gt[r] * exp2f(ct - cum_lds[s]) * dt_lds[s] : 0.0f;
          if (si == ti) v = (sl < i) ? v : (sl == i ? v + Dh : 0.0f);
          mv[e] = v;
        }
        s16x8 mhi, mlo;
        split_bf16x8(mv, mhi, mlo);
        const int r0 = 32 * si + 16 * m + 4 * kk;
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const s16x8 bop = lds_tr_operand(x_lds, kXLD, r0, r0 + 8, 32 * pt);
          acc[pt] = mfma32x32x16(mhi, bop, acc[pt]);
          acc[pt] = mfma32x32x16(mlo, bop, acc[pt]);
        }
      }
    }
    // 4. epilogue: z gate, bf16 store of p = 2 i, 2 i + 1
    bf16_t* oh = out + ((b * L + t0) * H + h) * kP + 2 * i;
    const bf16_t* zh = z + ((b * L + t0) * H + h) * kP + 2 * i;
    // z loads unconditional (rows clamped), so they are all in flight at once
    uint32_t zw[16];
    if constexpr (GATE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = 32 * ti + 8 * (r / 4) + 4 * kk + (r % 4);
        zw[r] = *reinterpret_cast<const uint32_t*>(zh + (tr < last ? tr : last) * xs);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = 32 * ti + 8 * (r / 4) + 4 * kk + (r % 4);
      f2 y;
      y[0] = acc[0][r];
      y[1] = acc[1][r];
      if constexpr (GATE) {
        y[0] *= silu(bf16_lo(zw[r]));
        y[1] *= silu(bf16_hi(zw[r]));
      }
      if (tr <= last) st2(oh + tr * xs, y);
    }
  }
}

// ---------------------------------------------------------------------------

bool use_bf16_kernels(const Problem& p) {
  return p.bf16 && (p.Q == 128 || p.Q == 256) && (p.N == 64 || p.N == 128);
}

template <int Q, int N>
static void launch_bf16_qn(const Problem& p, hipStream_t s, int stage) {
  const bf16_t* x = static_cast<const bf16_t*>(p.x);
  if (stage == 0) {
    const int64_t nblk = p.b * p.nc * p.G;
    hipLaunchKernelGGL((transpose_b_kernel<Q, N>), dim3((unsigned)nblk), dim3(256), 0, s,
                       static_cast<const bf16_t*>(p.B), p.ws_bt, p.L, p.G, p.nc);
  } else if (stage == 1) {
    const int64_t nunits = p.b * p.nc * p.H;
    hipLaunchKernelGGL((chunk_state_bf16_kernel<Q, N>), dim3((unsigned)nunits), dim3(256), 0, s, x,
                       p.ws_bt, static_cast<const bf16_t*>(p.dt), p.A, p.dt_bias, p.dt_min,
                       p.dt_max, p.ws_dt, p.ws_cum, p.ws_states, p.ws_seg, p.L, p.H, p.G, p.nc,
                       nunits);
  } else {
    const int64_t nunits = p.b * p.nc * p.H;
    if (p.z)
      hipLaunchKernelGGL((chunk_scan_bf16_kernel<Q, N, true>), dim3((unsigned)nunits), dim3(256),
                         0, s, x, static_cast<const bf16_t*>(p.B),
                         static_cast<const bf16_t*>(p.C), p.D, static_cast<const bf16_t*>(p.z),
                         p.ws_dt, p.ws_cum, p.ws_states_in, static_cast<bf16_t*>(p.out),
                         p.ws_seg, p.L, p.H, p.G, p.nc, nunits);
    else
      hipLaunchKernelGGL((chunk_scan_bf16_kernel<Q, N, false>), dim3((unsigned)nunits), dim3(256),
                         0, s, x, static_cast<const bf16_t*>(p.B),
                         static_cast<const bf16_t*>(p.C), p.D, static_cast<const bf16_t*>(p.z),
                         p.ws_dt, p.ws_cum, p.ws_states_in, static_cast<bf16_t*>(p.out),
                         p.ws_seg, p.L, p.H, p.G, p.nc, nunits);
  }
}

hipError_t launch_bf16_stage(const Problem& p, hipStream_t s, int stage) {
  switch (p.Q * 1000 + p.N) {
    case 128064: launch_bf16_qn<128, 64>(p, s, stage); break;
    case 128128: launch_bf16_qn<128, 128>(p, s, stage); break;
    case 256064: launch_bf16_qn<256, 64>(p, s, stage); break;
    case 256128: launch_bf16_qn<256, 128>(p, s, stage); break;
  }
  return hipGetLastError();
}

}  // namespace ssd
