// Backward of the scan (fp32): gradients of l = sum(dout * out) + sum(dfinal *
// final) with respect to x, dt_raw, A, B, C, D, z, dt_bias and the initial
// state.  The chunked form, with blocks of T = 64 steps (the gradient, like
// the forward result, does not depend on the block length):
//
// Inside a block, with cum_t the running sum of dt A from the block start,
// cl = cum_{T-1}, H_in the state entering the block, G the gradient of the
// state leaving it, dY = dout * silu(z) and
//     M[t][s] = exp(cum_t - cum_s) [s <= t],  K[t][s] = C_t . B_s,
//     R[t][s] = dY_t . x_s,  w_s = exp(cl - cum_s) dt_s,
// the forward pieces  Y = exp(cum) (C H_in^T) + (M o K) diag(dt) X + D X  and
// H_out = exp(cl) H_in + X^T diag(w) B  give
//     dX = D dY + (M o K diag(dt))^T dY + diag(w) B G^T
//     dB = diag(dt) (M o R)^T C + diag(w) X G
//     dC = diag(exp(cum)) dY H_in + (M o R) diag(dt) B
//     dH_in = dY^T diag(exp(cum)) C + exp(cl) G                 (state passing)
// and for the log-decays, with v[t][s] = M K R dt_s:
//     dcum_t += sum_s v[t][s] + exp(cum_t) dY_t . (H_in C_t)
//     dcum_s -= sum_t v[t][s] + w_s x_s . (G B_s)
//     dcum_cl += sum_s w_s x_s . (G B_s) + exp(cl) <G, H_in>
//     ddt_t = sum_{t'} M K R [t'][t] + exp(cl - cum_t) x_t . (G B_t)
//             + A sum_{t' >= t} dcum_t'        (cum_t = A * running sum of dt)
//     dA   += sum_t dt_t sum_{t' >= t} dcum_t'
// The pairs (t, s) that straddle blocks reach the gradients through H_in and
// G, which the reverse state passing provides: G_{c-1} = exp(cl_c) G_c + P_c
// with P_c = sum_t exp(cum_t) dY_t C_t^T, and dinit = G_{-1}.
//
// Kernels: the forward is re-run (64-step blocks) for dt, cum, the states
// entering each block and, with a gate, dY and dz (formed from the ungated y
// by the four-heads chunk scan's epilogue, else by gate_bwd_kernel); then
// bwd_state_scan_kernel (P_c and the reverse scan: G_c, dinit),
// block_bwd_kernel (dX, per-head dB and dC, ddt_raw, per-block dA and dD
// parts) and the reductions over heads, batch and blocks.  The products are
// on v_mfma_f32_16x16x4_f32 from LDS tiles; masks and decays are applied to
// the 64 x 64 in-block matrices in between.
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {
constexpr int kBT = 64;   // block length of the backward
// Row pitches of the LDS tiles (floats): multiples of 4, so that rows are
// read 16 bytes at a time.  64-wide tiles 72 (32 bytes past a multiple of 64
// bytes, at which 16-byte reads of 16 rows by four lane quarters measured
// free of bank conflicts); N-wide ones N + 4 (16 bytes past: the four lane
// quarters' 4-byte reads down a column, rows 4 apart, fall in distinct banks),
// since most of their reads go down columns.
constexpr int kXP = 72;
template <int N>
constexpr int kNP = N + 4;
constexpr int kBwdThreads = 512;  // block backward kernel: eight waves (sixteen measured the same)
// reverse state scan: up to 32 state columns, four waves per 16, per workgroup
template <int N>
constexpr int kScanThreads = 4 * ((N < 32 ? N : 32) / 16) * kWave;

// One 16 x 16 output tile of a wave on v_mfma_f32_16x16x4_f32: at each
// step lane l supplies a(l%16, k) and b(k, l%16) for its own k; register r of
// lane l holds the element (row 4 (l/16) + r, column l%16).
//
// The contraction runs in groups of 16: in the group from k0, the lanes of
// quarter g = l/16 take k = k0 + 4g + q at step q of four.  A lane's operands
// of a group are thus four consecutive k, which the accessors return as one
// f4: one 16-byte LDS read where they lie side by side (a row-major tile read
// along its rows), four 4-byte reads otherwise.
//
// NJ tiles of one 16-row strip at once: acc[j] += sum_k a(i, k) * b(j, k, c).
// The A value is shared by the NJ independent accumulators, so consecutive
// MFMAs never wait on each other.
template <int NJ, int K, typename FA, typename FB>
__device__ __forceinline__ void tiles16(FA a, FB b, f4 (&acc)[NJ]) {
  static_assert(K % 16 == 0, "contraction in groups of 16");
  const int lane = threadIdx.x % kWave, i = lane % 16, kq = 4 * (lane / 16);
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 16) {
    const f4 av = a(i, k0 + kq);
    f4 bv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) bv[j] = b(j, k0 + kq, i);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = mfma16x16x4(av[q], bv[j][q], acc[j]);
  }
}

// Operand accessors over LDS tiles of row pitch `pitch` floats: four
// consecutive k along row r (k and pitch multiples of 4), or down column c
// from row k.
__device__ __forceinline__ f4 along_row(const float* m, int pitch, int r, int k) {
  return *reinterpret_cast<const f4*>(m + r * pitch + k);
}
__device__ __forceinline__ f4 down_col(const float* m, int pitch, int k, int c) {
  return f4{m[k * pitch + c], m[(k + 1) * pitch + c], m[(k + 2) * pitch + c],
            m[(k + 3) * pitch + c]};
}
}  // namespace

// dY = dout * silu(z) (in place of y), dz = dout * y * silu'(z); launched
// only with a gate.  Four elements per thread.
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* __restrict__ dout,
                                                       const float* __restrict__ z, float* y_dy,
                                                       float* __restrict__ dz, int64_t n4) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= n4) return;
  const f4 d = ld4(dout + 4 * k);
  const f4 y = ld4(y_dy + 4 * k), zv = ld4(z + 4 * k);
  f4 dyv, dzv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float sg = 1.0f / (1.0f + expf(-zv[e]));
    dyv[e] = d[e] * zv[e] * sg;
    dzv[e] = d[e] * y[e] * sg * (1.0f + zv[e] * (1.0f - sg));
  }
  st4(y_dy + 4 * k, dyv);
  st4(dz + 4 * k, dzv);
}

// Gradient of the state leaving each block, by a reverse scan over the
// blocks: G_{nb-1} = dfinal (or 0), G_{c-1} = exp(cl_c) G_c + P_c with
// P_c = sum_t exp(cum_t) dY_t C_t^T over block c (cum the running sum of
// dt A inside the block, cl its last value); dinit = G_{-1}.  G_c is stored
// row-major [P][N] per block.
//
// One workgroup per (batch, head, NCOL state columns), four waves per 16
// columns; wave w holds the 16 x 16 tile (columns 16 (w % NS16) ..., rows
// 16 (w / NS16) ...) of G^T in registers.  P_c needs no carry, so the blocks
// go in groups of KD: a group's dY and C rows are staged into KD LDS buffers
// at once, the next group's rows are loaded into registers, and the KD
// products and updates of G run without waiting on memory (a wait for loads
// issued a whole group earlier, not one block earlier).  C is staged already
// scaled by exp(cum_t).  Rows past the sequence end, and blocks before the
// first, read as zero through empty buffer ranges; such blocks leave G as it
// is (exp(0) G + 0) and their stores are dropped.
template <int N>
__global__ __launch_bounds__(kScanThreads<N>) void bwd_state_scan_kernel(
    const float* __restrict__ dy, const float* __restrict__ Cm, const float* __restrict__ ws_cum,
    const float* dfinal, float* __restrict__ gst, float* dinit, int64_t L, int64_t H,
    int64_t G, int64_t nb) {
  constexpr int P = 64, T = kBT, NCOL = N < 32 ? N : 32, NS16 = NCOL / 16;
  constexpr int NT = kScanThreads<N>;
  constexpr int CS = NCOL == 32 ? 48 : 16, YS = 80;  // padded LDS row strides
  constexpr int QY = T * P / (4 * NT);               // dY float4 per thread
  constexpr int KD = 4;                              // blocks per group
  static_assert(T * NCOL == 4 * NT && T * P % (4 * NT) == 0, "staging");
  __shared__ __align__(16) float cl_[KD][T * CS];
  __shared__ __align__(16) float yl_[KD][T * YS];

  // blockIdx.x = ncs * (b H) + (b H index): the column slices of one head
  // are b H apart, on one XCD when b H is a multiple of 8
  const int64_t BH = (int64_t)gridDim.x / (N / NCOL);
  const int64_t bh = blockIdx.x % BH, ncs = blockIdx.x / BH;
  const int64_t b = bh / H, h = bh % H;
  const int64_t g = __builtin_amdgcn_readfirstlane((int)h / (int)(H / G));
  const int n0 = (int)ncs * NCOL;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ns = wave % NS16, pt = wave / NS16, i = lane % 16, kk = lane / 16;
  const uint32_t xrow = (uint32_t)(H * P * 4), brow = (uint32_t)(G * N * 4);
  const int64_t PN = (int64_t)P * N;

  // this thread's staging slots: C row tc, columns nc..nc+3; QY dY float4s
  const int tc = tid / (NCOL / 4), nc = 4 * (tid % (NCOL / 4));
  f4 cv[KD], yv[KD][QY];
  float cumv[KD], clv[KD];
  auto load = [&](int j, int64_t c) {  // block c < 0: nothing is read
    const int64_t t0 = c * T;
    const int last = (int)((L - 1 - t0) < (T - 1) ? (L - 1 - t0) : (T - 1));
    const uint32_t yb = c >= 0 ? (uint32_t)last * xrow + P * 4 : 0u;
    const uint32_t cb = c >= 0 ? (uint32_t)last * brow + NCOL * 4 : 0u;
    const auto yr = row_rsrc(dy + ((b * L + t0) * H + h) * P, yb);
    const auto cr = row_rsrc(Cm + ((b * L + t0) * G + g) * N + n0, cb);
    const auto ur = row_rsrc(ws_cum + (bh * nb + (c >= 0 ? c : 0)) * T, c >= 0 ? T * 4 : 0u);
#pragma unroll
    for (int q = 0; q < QY; ++q) {
      const int e = 4 * (q * NT + tid);
      yv[j][q] = bld4(yr, (uint32_t)(e / P) * xrow + (uint32_t)(e % P) * 4);
    }
    cv[j] = bld4(cr, (uint32_t)tc * brow + (uint32_t)nc * 4);
    cumv[j] = bld1(ur, (uint32_t)tc * 4, 0.0f);
    clv[j] = bld1(ur, (T - 1) * 4, 0.0f);
  };
  auto stage = [&](int j) {
    const float e = expf(cumv[j]);
#pragma unroll
    for (int c = 0; c < 4; ++c) cl_[j][tc * CS + nc + c] = e * cv[j][c];
#pragma unroll
    for (int q = 0; q < QY; ++q) {
      const int e4 = 4 * (q * NT + tid);
#pragma unroll
      for (int c = 0; c < 4; ++c) yl_[j][(e4 / P) * YS + e4 % P + c] = yv[j][q][c];
    }
  };

  // G^T tile: register r of lane (i, kk) is column n = n0 + 16 ns + 4 kk + r
  // of row p = 16 pt + i, i.e. four consecutive floats of the row-major block
  const int64_t toff = (int64_t)(16 * pt + i) * N + n0 + 16 * ns + 4 * kk;
  f4 gv = dfinal ? ld4(dfinal + bh * PN + toff) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KD; ++j) load(j, nb - 1 - j);
  for (int64_t c0 = nb - 1; c0 >= 0; c0 -= KD) {
#pragma unroll
    for (int j = 0; j < KD; ++j) stage(j);
    float ecl[KD];
#pragma unroll
    for (int j = 0; j < KD; ++j) ecl[j] = expf(clv[j]);
#pragma unroll
    for (int j = 0; j < KD; ++j) load(j, c0 - KD - j);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KD; ++j) {
      const int64_t c = c0 - j;
      const auto gr = row_rsrc(gst + ((b * nb + c) * H + h) * PN, c >= 0 ? (uint32_t)PN * 4 : 0u);
      bst4(gr, (uint32_t)toff * 4, gv);
      // P_c^T tile = sum_t (e_t C_t)[n] dY_t[p], two accumulators over t
      f4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      const float* ca = &cl_[j][16 * ns + i];
      const float* yb = &yl_[j][16 * pt + i];
#pragma unroll
      for (int k = 0; k < T; k += 8) {
        a0 = mfma16x16x4(ca[(k + kk) * CS], yb[(k + kk) * YS], a0);
        a1 = mfma16x16x4(ca[(k + 4 + kk) * CS], yb[(k + 4 + kk) * YS], a1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) gv[r] = ecl[j] * gv[r] + (a0[r] + a1[r]);
    }
    __syncthreads();  // the buffers are rewritten by the next group
  }
  if (dinit) st4(dinit + bh * PN + toff, gv);
}

// One workgroup (eight waves) per (batch, block, up to four heads of one
// group).  Everything the products read is staged in one LDS buffer with
// 16-byte global loads, regions reused as they die (floats, for N = 128; rows
// padded to the pitches above; B and C once, the rest per head):
//   [0, 4608)       x [64][72]                 | then H_in [64][132] over
//   [4608, 9216)    V^T [64][72]               |   x and V (dC phase)
//   [9216, 13824)   W [64][72]                 G [64][132] over V and W
//   [13824, 18432)  dY [64][72]                  (first phase)
//   [18432, 26880)  B [64][132]
//   [26880, 35328)  C [64][132]
// Phases per head: the products with G (G.B for dX, X.G for dB, x . (G B))
// with G in LDS, kept in registers; R, and with K = C B^T (formed once per
// workgroup, in registers) V and W in place of G; dX and dB;
// H_in over x and V, then dC and dY_t . (H_in C_t); the decay gradients.
template <int N, int HPW>
__global__ __launch_bounds__(kBwdThreads) void block_bwd_kernel(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ Cm,
    const float* __restrict__ dt_raw, const float* __restrict__ dt_bias, float dt_min,
    float dt_max, const float* __restrict__ A, const float* __restrict__ Dv,
    const float* __restrict__ ws_dt, const float* __restrict__ ws_cum,
    const float* __restrict__ states_in, const float* __restrict__ gst,
    const float* __restrict__ dy, float* __restrict__ dx, float* __restrict__ dBh,
    float* __restrict__ dCh, float* __restrict__ ddt_raw, float* __restrict__ dA_p,
    float* __restrict__ dD_p, int64_t L, int64_t H, int64_t G, int64_t nb) {
  constexpr int P = 64, T = kBT, NJ = N / 16, NS = kNP<N>;
  // NW waves: wave w takes the 16-row strip w % 4 of every product and
  // column group w / 4 of its column tiles (several waves per SIMD hide each
  // other's LDS and memory latency; with four waves, one per SIMD, they did
  // not).  N-wide products with fewer column tiles than groups are done by
  // the first groups.
  constexpr int NW = kBwdThreads / kWave, NTH = kBwdThreads;
  constexpr int NCG = NW / 4;                      // column groups
  constexpr int NJ4 = 4 / NCG;                     // 64-wide column tiles per wave
  constexpr int NJW = NJ >= NCG ? NJ / NCG : 1;    // N-wide column tiles per wave
  constexpr int OX = 0, OV = T * kXP, OW = OV + T * kXP, OY = OW + T * kXP, OB = OY + T * kXP,
                OC = OB + T * NS;
  static_assert(P * NS <= OY - OV && P * NS <= OW - OX && kXP % 4 == 0 && NS % 4 == 0,
                "LDS map");
  __shared__ __align__(16) float lds[OC + T * NS];
  float* const xs_ = lds + OX;   // x[t][p]      pitch kXP
  float* const vm = lds + OV;    // V^T[s][t]    pitch kXP
  float* const wm = lds + OW;    // W[t][s]      pitch kXP
  float* const ys_ = lds + OY;   // dY[t][p]     pitch kXP
  float* const bs_ = lds + OB;   // B[t][n]      pitch NS
  float* const cs_ = lds + OC;   // C[t][n]      pitch NS
  float* const gs_ = lds + OV;   // G[p][n]      pitch NS (first phase)
  float* const hs_ = lds + OX;   // H_in[p][n]   pitch NS (dC phase)
  __shared__ __align__(16) float cum_l[T], dt_l[T];
  __shared__ float ecum[T], wdt[T];  // exp(cum_t); w_t = exp(cl - cum_t) dt_t
  // per-half row sums and per-strip column sums, added in a fixed order
  __shared__ float rowv[NCG][T], xgb[NCG][T], yod[NCG][T], red[2 * NW];
  __shared__ float colw[4][T], col0w[4][T];

  // HPW heads of one group per workgroup, one after the other: B and C are
  // staged once for all of them, and their dB and dC parts are summed in
  // registers, so one part per HPW heads goes to memory (the group sum then
  // reads H/HPW parts per step instead of H).
  const int64_t HQ = H / HPW;
  const int64_t uq = blockIdx.x;  // (b * nb + blk) * HQ + hq
  const int64_t hq = uq % HQ, blk = (uq / HQ) % nb, b = uq / (HQ * nb);
  // 32-bit and wave-uniform: the B and C buffer resources need a scalar base
  const int64_t g = __builtin_amdgcn_readfirstlane((int)(hq * HPW) / (int)(H / G)), t0 = blk * T;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int strip = wave & 3, colh = wave >> 2;  // row strip, column group
  const int i = lane % 16, kk = lane / 16;
  const int64_t PN = (int64_t)P * N;
  const int last = (int)((L - 1 - t0) < (T - 1) ? (L - 1 - t0) : (T - 1));

  // Rows of this block (a head's x, dY and dX; the group's B and C; the dB
  // and dC parts of the HPW heads) through buffer resources that end after
  // row `last`: rows past it read as zero and the gradient stores there are
  // dropped, with 32-bit offsets and no clamps, selects or branches.
  const uint32_t xrow = (uint32_t)(H * P * 4), brow = (uint32_t)(G * N * 4);
  const uint32_t prow = (uint32_t)(HQ * N * 4);  // dB / dC parts, one per HPW heads
  const int64_t bo = ((b * L + t0) * G + g) * N, po = ((b * L + t0) * HQ + hq) * N;
  const uint32_t xbytes = (uint32_t)last * xrow + P * 4, bbytes = (uint32_t)last * brow + N * 4;
  const uint32_t pbytes = (uint32_t)last * prow + N * 4;
  // float4 per thread (the last may be partial for N = 16: guarded)
  constexpr int QX = T * P / (4 * NTH), QB = (T * N / 4 + NTH - 1) / NTH, QG = QB;
  static_assert(T * P % (4 * NTH) == 0 && T == P, "staging");

  // ---- stage B and C once (rows past the end are zero) -----------------------
  {
    const auto br = row_rsrc(Bm + bo, bbytes), cr = row_rsrc(Cm + bo, bbytes);
    f4 bv[QB], cv[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int e = 4 * (q * NTH + tid), t = e / N, n = e % N;
      const uint32_t o = (uint32_t)t * brow + (uint32_t)n * 4;
      if (e < T * N) {
        bv[q] = bld4(br, o);
        cv[q] = bld4(cr, o);
      }
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int e = 4 * (q * NTH + tid), t = e / N, n = e % N;
      if (e < T * N) {
        *reinterpret_cast<f4*>(bs_ + t * NS + n) = bv[q];
        *reinterpret_cast<f4*>(cs_ + t * NS + n) = cv[q];
      }
    }
  }

  // Column tiles of this wave: 64-wide products (over p or s) tiles
  // NJ4 colh ...; N-wide ones NJW tiles from jn (none for the later column
  // groups when N has fewer tiles than groups).
  const int j4 = NJ4 * colh, jn = colh * NJW;
  const bool hasn = jn < NJ;  // wave-uniform
  f4 dbacc[NJW], dcacc[NJW];  // dB and dC parts summed over the HPW heads
#pragma unroll
  for (int j = 0; j < NJW; ++j) dbacc[j] = dcacc[j] = f4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  // K = C B^T is the same for every head of the group: formed once, kept in
  // registers (rows t in [16 strip, 16 strip + 16), this wave's s tiles).
  f4 kall[NJ4];
  tiles16<NJ4, N>([&](int r, int k) { return along_row(cs_, NS, 16 * strip + r, k); },
                  [&](int j, int k, int c) { return along_row(bs_, NS, 16 * (j4 + j) + c, k); },
                  kall);

  for (int hk = 0; hk < HPW; ++hk) {
  const int64_t h = hq * HPW + hk;
  const int64_t u = (b * nb + blk) * H + h;  // this head's block
  const float* hin = states_in + u * PN;  // tiled layout
  const float* gc = gst + u * PN;         // row-major [P][N]
  const int64_t xo = ((b * L + t0) * H + h) * P;

  // ---- stage x, dY, G, cum, dt of this head (rows past the end are zero) -----
  {
    const auto xr = row_rsrc(x + xo, xbytes), yr = row_rsrc(dy + xo, xbytes);
    f4 xv[QX], yv[QX], gv[QG];
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int e = 4 * (q * NTH + tid), t = e / P, p = e % P;
      const uint32_t o = (uint32_t)t * xrow + (uint32_t)p * 4;
      xv[q] = bld4(xr, o);
      yv[q] = bld4(yr, o);
    }
#pragma unroll
    for (int q = 0; q < QG; ++q)
      if (4 * (q * NTH + tid) < P * N) gv[q] = ld4(gc + 4 * (q * NTH + tid));
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int e = 4 * (q * NTH + tid), t = e / P, p = e % P;
      *reinterpret_cast<f4*>(xs_ + t * kXP + p) = xv[q];
      *reinterpret_cast<f4*>(ys_ + t * kXP + p) = yv[q];
    }
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const int e = 4 * (q * NTH + tid), p = e / N, n = e % N;
      if (e < P * N) *reinterpret_cast<f4*>(gs_ + p * NS + n) = gv[q];
    }
  }
  if (tid < T) {
    const int64_t o = ((b * H + h) * nb + blk) * T + tid;
    const float c = ws_cum[o], d = ws_dt[o];
    cum_l[tid] = c;
    dt_l[tid] = d;
    ecum[tid] = expf(c);
    wdt[tid] = expf(ws_cum[o - tid + T - 1] - c) * d;
  }
  __syncthreads();
  const float cl = cum_l[T - 1];
  const float Dh = Dv ? Dv[h] : 0.0f;

  // Sums over a row of a wave's 16 x 64 strip (16 lanes x 4 tiles) or a column
  // (4 lane groups x 4 registers x 4 waves) are taken in a fixed order: lane
  // moves within the wave (DPP and row swaps, no LDS), then the per-wave parts
  // in wave order, so the gradients are identical from run to run.
  auto sum16 = [](float v) { return row_sum16(v); };  // over the 16 lanes of a row group
  auto sum4g = [](float v) { return rows_sum4(v); };  // over the four 16-lane groups

  // ---- products with G: GB[s][p] = B_s . G_p (dX), XG[s][n] = x_s^T G (dB) --
  // rows s in [16 strip, 16 strip + 16)
  f4 gball[NJ4], xgall[NJW];
  tiles16<NJ4, N>([&](int r, int k) { return along_row(bs_, NS, 16 * strip + r, k); },
                  [&](int j, int k, int c) { return along_row(gs_, NS, 16 * (j4 + j) + c, k); },
                  gball);
  if (hasn)
    tiles16<NJW, P>([&](int r, int k) { return along_row(xs_, kXP, 16 * strip + r, k); },
                    [&](int j, int k, int c) { return down_col(gs_, NS, k, 16 * (jn + j) + c); },
                    xgall);
  {
    float xsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xsum[r] += xs_[(16 * strip + 4 * kk + r) * kXP + 16 * (j4 + j) + i] * gball[j][r];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = sum16(xsum[r]);
      if (i == 0) xgb[colh][16 * strip + 4 * kk + r] = v;
    }
  }
  __syncthreads();  // G is dead: V and W take its place

  // ---- R = dY X^T; masks, decays and the dcum sums with K --------------------
  // rows t in [16 strip, 16 strip + 16), this wave's column tiles of s
  float rsum[4] = {0.f, 0.f, 0.f, 0.f};
  f4 rall[NJ4];
  tiles16<NJ4, P>([&](int r, int k) { return along_row(ys_, kXP, 16 * strip + r, k); },
                  [&](int j, int k, int c) { return along_row(xs_, kXP, 16 * (j4 + j) + c, k); },
                  rall);
#pragma unroll
  for (int j = 0; j < NJ4; ++j) {
    const f4 kacc = kall[j], racc = rall[j];
    const int s = 16 * (j4 + j) + i;
    float cs = 0.0f, cs0 = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * strip + 4 * kk + r;
      const float m = s <= t ? __expf(cum_l[t] - cum_l[s]) : 0.0f;
      const float v0 = m * kacc[r] * racc[r];
      const float v = v0 * dt_l[s];
      vm[s * kXP + t] = m * kacc[r] * dt_l[s];
      wm[t * kXP + s] = m * racc[r];
      rsum[r] += v;
      cs += v;
      cs0 += v0;
    }
    cs = sum4g(cs);
    cs0 = sum4g(cs0);
    if (kk == 0) {
      colw[strip][s] = cs;
      col0w[strip][s] = cs0;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float v = sum16(rsum[r]);
    if (i == 0) rowv[colh][16 * strip + 4 * kk + r] = v;
  }
  __syncthreads();

  // ---- dX = D dY + V^T dY + diag(w) GB;  dB = diag(dt) W^T C + diag(w) XG ----
  {
    const auto dxr = row_rsrc(dx + xo, xbytes);
    f4 vall[NJ4];
    tiles16<NJ4, T>([&](int r, int k) { return along_row(vm, kXP, 16 * strip + r, k); },
                    [&](int j, int k, int c) { return down_col(ys_, kXP, k, 16 * (j4 + j) + c); },
                    vall);
#pragma unroll
    for (int j = 0; j < NJ4; ++j) {
      const int p = 16 * (j4 + j) + i;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 16 * strip + 4 * kk + r;
        bst1(dxr, (uint32_t)s * xrow + (uint32_t)p * 4,
             Dh * ys_[s * kXP + p] + vall[j][r] + wdt[s] * gball[j][r]);
      }
    }
    if (hasn) {
    f4 a1[NJW];
    tiles16<NJW, T>([&](int r, int k) { return down_col(wm, kXP, k, 16 * strip + r); },
                    [&](int j, int k, int c) { return down_col(cs_, NS, k, 16 * (jn + j) + c); },
                    a1);
#pragma unroll
    for (int j = 0; j < NJW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 16 * strip + 4 * kk + r;
        dbacc[j][r] += dt_l[s] * a1[j][r] + wdt[s] * xgall[j][r];
      }
    }
  }
  float dd = 0.0f;  // dY . x over the block
  for (int e = tid; e < T * P; e += NTH) dd += ys_[(e / P) * kXP + e % P] * xs_[(e / P) * kXP + e % P];
  __syncthreads();  // x and V are dead: H_in takes their place

  // ---- H_in into LDS, with <G, H_in> on the way ------------------------------
  float gh = 0.0f;
  {
    constexpr int QH = (P * N / 4 + NTH - 1) / NTH;
    f4 hv[QH], gv2[QH];
#pragma unroll
    for (int q = 0; q < QH; ++q) {
      const int k4 = q * NTH + tid;  // float4 index in the tiled block
      if (k4 >= P * N / 4) break;
      int p, n;
      state_tile_coords(k4, N, &p, &n);
      hv[q] = ld4(hin + 4 * k4);
      gv2[q] = ld4(gc + p * N + n);
    }
#pragma unroll
    for (int q = 0; q < QH; ++q) {
      if (q * NTH + tid >= P * N / 4) break;
      int p, n;
      state_tile_coords(q * NTH + tid, N, &p, &n);
      *reinterpret_cast<f4*>(hs_ + p * NS + n) = hv[q];
#pragma unroll
      for (int c = 0; c < 4; ++c) gh += hv[q][c] * gv2[q][c];
    }
  }
  __syncthreads();

  // ---- dC = diag(exp(cum)) dY H_in + W diag(dt) B; dY_t . (H_in C_t) ----------
  float ysum[4] = {0.f, 0.f, 0.f, 0.f};
  if (hasn) {
    f4 a1[NJW], a2[NJW];
    tiles16<NJW, P>([&](int r, int k) { return along_row(ys_, kXP, 16 * strip + r, k); },
                    [&](int j, int k, int c) { return down_col(hs_, NS, k, 16 * (jn + j) + c); },
                    a1);
    tiles16<NJW, T>(
        [&](int r, int k) { return along_row(wm, kXP, 16 * strip + r, k) * along_row(dt_l, 0, 0, k); },
        [&](int j, int k, int c) { return down_col(bs_, NS, k, 16 * (jn + j) + c); }, a2);
#pragma unroll
    for (int j = 0; j < NJW; ++j) {
      const int n = 16 * (jn + j) + i;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * strip + 4 * kk + r;
        const float e = ecum[t] * a1[j][r];
        dcacc[j][r] += e + a2[j][r];
        ysum[r] += e * cs_[t * NS + n];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {  // zero partials from a wave without N tiles
    const float v = sum16(ysum[r]);
    if (i == 0) yod[colh][16 * strip + 4 * kk + r] = v;
  }

  // ---- <G, H_in> and dY . x across the workgroup ------------------------------
  gh = wave_sum(gh);
  dd = wave_sum(dd);
  if (lane == 0) {
    red[wave] = gh;
    red[NW + wave] = dd;
  }
  __syncthreads();

  // ---- dcum, its reverse running sum, ddt_raw, the dA and dD parts -----------
  if (wave == 0) {
    const int t = lane;
    float xg = 0.0f, rv = 0.0f, yo = 0.0f;
#pragma unroll
    for (int q = 0; q < NCG; ++q) {
      xg += xgb[q][t];
      rv += rowv[q][t];
      yo += yod[q][t];
    }
    const float us = wdt[t] * xg;
    const float usum = wave_sum(us);
    float ghs = 0.0f, dds = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      ghs += red[w];
      dds += red[NW + w];
    }
    const float colv = colw[0][t] + colw[1][t] + colw[2][t] + colw[3][t];
    const float col0 = col0w[0][t] + col0w[1][t] + col0w[2][t] + col0w[3][t];
    float dc = rv + yo - colv - us;
    if (t == T - 1) dc += usum + __expf(cl) * ghs;
    // suffix sum over t: the prefix sum of the lanes in reverse order
    const float rc = wave_reverse(wave_incl_sum(wave_reverse(dc)));
    const float Ah = A[h];
    const float ddt = col0 + __expf(cl - cum_l[t]) * xg + Ah * rc;
    const float da = wave_sum(dt_l[t] * rc);
    if (t <= last) {
      const int64_t o = (b * L + t0 + t) * H + h;
      const float uu = dt_raw[o] + (dt_bias ? dt_bias[h] : 0.0f);
      const float sp = softplus(uu);
      const bool pass = sp >= dt_min && sp <= dt_max;
      ddt_raw[o] = pass ? ddt * fast_rcp(1.0f + __expf(-uu)) : 0.0f;
    }
    if (t == 0) {
      dA_p[u] = da;
      dD_p[u] = dds;
    }
  }
  __syncthreads();  // every LDS region of this head is read before the next
  }

  // ---- dB and dC parts of the HPW heads ---------------------------------------
  if (hasn) {
    const auto dbr = row_rsrc(dBh + po, pbytes), dcr = row_rsrc(dCh + po, pbytes);
#pragma unroll
    for (int j = 0; j < NJW; ++j) {
      const int n = 16 * (jn + j) + i;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t o = (uint32_t)(16 * strip + 4 * kk + r) * prow + (uint32_t)n * 4;
        bst1(dbr, o, dbacc[j][r]);
        bst1(dcr, o, dcacc[j][r]);
      }
    }
  }
}

// dB and dC: sum the parts (one per HPW heads, HQ = H / HPW per step) over the
// heads of each group.
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float* __restrict__ dBh,
                                                            const float* __restrict__ dCh,
                                                            float* __restrict__ dB,
                                                            float* __restrict__ dC, int64_t n,
                                                            int64_t HQ, int64_t G, int64_t N) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;  // ((b*L + t) * G + g) * N + c
  if (k >= n) return;
  const int64_t c = k % N, g = (k / N) % G, bt = k / (N * G);
  const int64_t ppg = HQ / G;  // parts per group
  float sb = 0.0f, sc = 0.0f;
  for (int64_t j = 0; j < ppg; ++j) {
    const int64_t o = (bt * HQ + g * ppg + j) * N + c;
    sb += dBh[o];
    sc += dCh[o];
  }
  dB[k] = sb;
  dC[k] = sc;
}

// dA, dD, ddt_bias: one workgroup per head, fixed summation order.  1024
// threads, so each walks few rows of the [b L, H] and [b nb, H] parts.
constexpr int kHeadSumThreads = 1024;
__global__ __launch_bounds__(kHeadSumThreads) void bwd_head_sum_kernel(
    const float* __restrict__ dA_p, const float* __restrict__ dD_p,
    const float* __restrict__ ddt_raw, float* __restrict__ dA, float* dD, float* ddt_bias,
    int64_t b, int64_t L, int64_t H, int64_t nb) {
  constexpr int NW = kHeadSumThreads / kWave;
  __shared__ float red[3][NW];
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  float sa = 0.0f, sd = 0.0f, sbias = 0.0f;
  for (int64_t k = tid; k < b * nb; k += kHeadSumThreads) {
    sa += dA_p[k * H + h];
    sd += dD_p[k * H + h];
  }
  for (int64_t k = tid; k < b * L; k += kHeadSumThreads) sbias += ddt_raw[k * H + h];
  sa = wave_sum(sa);
  sd = wave_sum(sd);
  sbias = wave_sum(sbias);
  if (lane == 0) {
    red[0][wave] = sa;
    red[1][wave] = sd;
    red[2][wave] = sbias;
  }
  __syncthreads();
  if (tid == 0) {
    float ta = 0.0f, td = 0.0f, tb = 0.0f;
    for (int w = 0; w < NW; ++w) {
      ta += red[0][w];
      td += red[1][w];
      tb += red[2][w];
    }
    dA[h] = ta;
    if (dD) dD[h] = td;
    if (ddt_bias) ddt_bias[h] = tb;
  }
}

int64_t bwd_blocks(int64_t L) { return (L + kBT - 1) / kBT; }

// Heads of one group per block workgroup: 8 when that still fills the
// compute units (one round of batch x blocks x H/8 workgroups), else 4, 2 or
// 1, as the heads per group divide.
static int bwd_heads_per_workgroup(int64_t H, int64_t G, int64_t bnb) {
  const int64_t hpg = H / G;
  if (hpg % 8 == 0 && bnb * (H / 8) >= kChainCUs) return 8;
  return hpg % 4 == 0 ? 4 : hpg % 2 == 0 ? 2 : 1;
}

// The reverse state scan over nb blocks (nb = 0: dinit = dfinal, or 0).
template <int N>
static void launch_state_scan(const BwdProblem& q, hipStream_t s, int64_t nb) {
  const Problem& p = q.fwd;
  constexpr int NCOL = N < 32 ? N : 32, NT = kScanThreads<N>;
  hipLaunchKernelGGL((bwd_state_scan_kernel<N>), dim3((unsigned)(N / NCOL * p.b * p.H)),
                     dim3(NT), 0, s, q.dy, static_cast<const float*>(p.C), p.ws_cum, q.dfinal,
                     q.gst, q.dinit, p.L, p.H, p.G, nb);
}

template <int N>
static void launch_bwd_n(const BwdProblem& q, hipStream_t s) {
  const Problem& p = q.fwd;
  const int64_t units = p.b * p.nc * p.H;
  launch_state_scan<N>(q, s, p.nc);
  const int hpw = bwd_heads_per_workgroup(p.H, p.G, p.b * p.nc);
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)(units / hpw)), dim3(kBwdThreads), 0, s,
                       static_cast<const float*>(p.x), static_cast<const float*>(p.B),
                       static_cast<const float*>(p.C), static_cast<const float*>(p.dt), p.dt_bias,
                       p.dt_min, p.dt_max, p.A, p.D, p.ws_dt, p.ws_cum, p.ws_states_in, q.gst,
                       q.dy, q.dx, q.dBh, q.dCh, q.ddt, q.dA_p, q.dD_p, p.L, p.H, p.G, p.nc);
  };
  if (hpw == 8)
    launch(block_bwd_kernel<N, 8>);
  else if (hpw == 4)
    launch(block_bwd_kernel<N, 4>);
  else if (hpw == 2)
    launch(block_bwd_kernel<N, 2>);
  else
    launch(block_bwd_kernel<N, 1>);
}

hipError_t launch_bwd(const BwdProblem& q, hipStream_t s) {
  const Problem& p = q.fwd;
  if (p.L > 0) {
    const int64_t nx4 = p.b * p.L * p.H * p.P / 4;
    // without a gate dY is dout, which q.dy then points at; dy_formed: the
    // re-run's chunk scan has written dY and dz already
    if (p.z && !q.dy_formed)
      hipLaunchKernelGGL(gate_bwd_kernel, dim3((unsigned)((nx4 + 255) / 256)), dim3(256), 0, s,
                         q.dout, static_cast<const float*>(p.z), q.dy, q.dz, nx4);
    switch (p.N) {
      case 16: launch_bwd_n<16>(q, s); break;
      case 32: launch_bwd_n<32>(q, s); break;
      case 64: launch_bwd_n<64>(q, s); break;
      case 128: launch_bwd_n<128>(q, s); break;
    }
    const int64_t nbc = p.b * p.L * p.G * p.N;
    hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0,
                       s, q.dBh, q.dCh, q.dB, q.dC, nbc,
                       p.H / bwd_heads_per_workgroup(p.H, p.G, p.b * p.nc),
                       p.G, p.N);
  } else if (q.dinit) {  // no steps: the initial state's gradient is dfinal (or 0)
    switch (p.N) {
      case 16: launch_state_scan<16>(q, s, 0); break;
      case 32: launch_state_scan<32>(q, s, 0); break;
      case 64: launch_state_scan<64>(q, s, 0); break;
      case 128: launch_state_scan<128>(q, s, 0); break;
    }
  }
  hipLaunchKernelGGL(bwd_head_sum_kernel, dim3((unsigned)p.H), dim3(kHeadSumThreads), 0, s,
                     q.dA_p, q.dD_p, q.ddt, q.dA, q.dD, q.ddt_bias, p.b, p.L, p.H, p.nc);
  return hipGetLastError();
}

// ---- bf16 <-> fp32 for the backward of bf16 inputs --------------------------
// The backward of bf16 inputs widens them to fp32 (exactly), runs the fp32
// kernels and rounds the gradients of the bf16 tensors to bf16 (nearest
// even).  One launch converts every tensor of a list (a launch per tensor left
// each small one's start-up and drain exposed): thread piece p takes eight
// elements of the tensor whose range of pieces holds p; 16-byte accesses when
// both pointers of that tensor are 16-byte aligned, element by element
// otherwise and in its tail.

__device__ __forceinline__ int conv_entry(const ConvList& cl, int64_t piece) {
  int k = 0;
  while (k + 1 < cl.count && piece >= cl.start[k + 1]) ++k;
  return k;
}

__global__ __launch_bounds__(256) void widen_bf16_kernel(const ConvList cl) {
  const int64_t piece = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (piece >= cl.start[cl.count]) return;
  const int k = conv_entry(cl, piece);
  const bf16_t* __restrict__ src = static_cast<const bf16_t*>(cl.src[k]);
  float* __restrict__ dst = static_cast<float*>(cl.dst[k]);
  const int64_t n = cl.n[k], i = (piece - cl.start[k]) * 8;
  if (cl.vec[k] && i + 8 <= n) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    f4 a, b;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      a[2 * j] = bf16_lo(w[j]);
      a[2 * j + 1] = bf16_hi(w[j]);
      b[2 * j] = bf16_lo(w[j + 2]);
      b[2 * j + 1] = bf16_hi(w[j + 2]);
    }
    st4(dst + i, a);
    st4(dst + i + 4, b);
  } else {
    for (int64_t e = i; e < n && e < i + 8; ++e) dst[e] = to_f32(src[e]);
  }
}

__global__ __launch_bounds__(256) void narrow_bf16_kernel(const ConvList cl) {
  const int64_t piece = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (piece >= cl.start[cl.count]) return;
  const int k = conv_entry(cl, piece);
  const float* __restrict__ src = static_cast<const float*>(cl.src[k]);
  bf16_t* __restrict__ dst = static_cast<bf16_t*>(cl.dst[k]);
  const int64_t n = cl.n[k], i = (piece - cl.start[k]) * 8;
  if (cl.vec[k] && i + 8 <= n) {
    const f4 a = ld4(src + i), b = ld4(src + i + 4);
    uint4 v;
    v.x = f32_to_bf16_bits(a[0]) | (f32_to_bf16_bits(a[1]) << 16);
    v.y = f32_to_bf16_bits(a[2]) | (f32_to_bf16_bits(a[3]) << 16);
    v.z = f32_to_bf16_bits(b[0]) | (f32_to_bf16_bits(b[1]) << 16);
    v.w = f32_to_bf16_bits(b[2]) | (f32_to_bf16_bits(b[3]) << 16);
    *reinterpret_cast<uint4*>(dst + i) = v;
  } else {
    for (int64_t e = i; e < n && e < i + 8; ++e) dst[e] = (bf16_t)f32_to_bf16_bits(src[e]);
  }
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Fill the piece ranges of a list; false when it is empty.
static bool conv_prepare(ConvList& cl) {
  cl.start[0] = 0;
  for (int k = 0; k < cl.count; ++k) {
    cl.vec[k] = aligned16(cl.src[k]) && aligned16(cl.dst[k]);
    cl.start[k + 1] = cl.start[k] + (cl.n[k] + 7) / 8;
  }
  return cl.count > 0 && cl.start[cl.count] > 0;
}

hipError_t launch_widen_bf16(ConvList cl, hipStream_t s) {
  if (!conv_prepare(cl)) return hipSuccess;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3((unsigned)((cl.start[cl.count] + 255) / 256)),
                     dim3(256), 0, s, cl);
  return hipGetLastError();
}

hipError_t launch_narrow_bf16(ConvList cl, hipStream_t s) {
  if (!conv_prepare(cl)) return hipSuccess;
  hipLaunchKernelGGL(narrow_bf16_kernel, dim3((unsigned)((cl.start[cl.count] + 255) / 256)),
                     dim3(256), 0, s, cl);
  return hipGetLastError();
}

}  // namespace ssd
