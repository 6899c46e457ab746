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
// Packed sequences (seq_idx): with k_t the count of sequence starts from the
// chunk start to t (ws_seg), the state part keeps rows with k_t = 0 and the
// in-chunk part keeps pairs with k_s = k_t (no start in (s, t]).
//
// Lane layout: in the accumulator, register r of lane l holds row
// t = 16*tb + 4*(l/16) + r and column p = 4*(l%16) + j of p-block j, so a lane
// stores four consecutive p of one row.  The state is staged with its rows
// permuted (LDS row 16*j + i holds H_in row 4*i + j) so that the 16 lanes of a
// read hit 16 consecutive padded rows.
#include "ssd_device.h"
#include "ssd_kernels.h"
#include <type_traits>

namespace ssd {

template <typename T, int Q, int N>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ Dv, const T* __restrict__ z, const float* __restrict__ ws_dt,
    const float* __restrict__ ws_cum, const float* __restrict__ states_in, T* __restrict__ out,
    const int32_t* __restrict__ seg, int64_t L, int64_t H, int64_t G, int64_t nc, int64_t nunits) {
  constexpr int P = 64;
  constexpr int NK = N / 4;      // MFMA k-steps over n (4 per step)
  constexpr int HS = N + 4;      // padded row stride of the staged state
  constexpr int NTB = Q / 16;    // t-blocks per chunk
  __shared__ float x_lds[Q * P];
  __shared__ float h_lds[P * HS];
  __shared__ float cum_lds[Q];
  __shared__ float dt_lds[Q];
  __shared__ int32_t seg_lds[Q];  // 0 everywhere without seq_idx

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
      const int k = i * 256 + tid;  // float4 index in the tiled state layout
      int p, n;
      state_tile_coords(k, N, &p, &n);
      const int prow = 16 * (p % 4) + p / 4;
      *reinterpret_cast<f4*>(&h_lds[prow * HS + n]) = ld4(hsrc + 4 * k);
    }
    const int64_t dc = ((b * H + h) * nc + c) * Q;
    if (tid < Q) {
      cum_lds[tid] = ws_cum[dc + tid];
      dt_lds[tid] = ws_dt[dc + tid];
      seg_lds[tid] = seg ? seg[(b * nc + c) * Q + tid] : 0;
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
      const int tr = 16 * tb + 4 * lk + r;
      const float e = seg_lds[tr] == 0 ? __expf(cum_lds[tr]) : 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j][r] *= e;
    }

    // 3. in-chunk part, causal s-blocks
    const int tcol = 16 * tb + li;
    const float cum_t = cum_lds[tcol];
    const int k_t = seg_lds[tcol];
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
        const float mv = (srow <= tcol && seg_lds[srow] == k_t) ? gacc[r] * wgt : 0.0f;
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

// ---------------------------------------------------------------------------
// Four heads of one group per workgroup, two waves per head (Q = 64 or 128,
// N = 64 or 128, nheads / ngroups a multiple of 4).
//
// The group's C tile of the chunk is staged in LDS once, and so are the
// causal 32 x 32 tiles of G^T = B C^T (G[t][s] = C_t . B_s), shared by the
// four heads, in register order.  With PRE they come from the workspace,
// formed once per (chunk, group) by the chunk-state launch; otherwise B is
// staged too and the eight waves form them on v_mfma_f32_32x32x2_f32 first.
// Each wave then holds half of its head's
// Q x 64 output in accumulators (t-tiles {h, Q/32-1-h} of wave half h, x 2
// p-tiles of 32 x 32, so both halves do the same causal work):
//   1. acc = C . H_in^T        (A: C rows from LDS; B: H_in, tiled layout,
//                               one coalesced float4 per lane per 4 k-steps)
//   2. acc *= exp(cum_t)
//   3. per s-tile si: acc[ti] += (G^T tile * exp(cum_t - cum_s) * dt_s,
//      causal) . x  for ti >= si; t-tile si is then complete and goes
//      through the D-skip / z-gate epilogue at once.
// The D skip is folded into the diagonal of the masked matrix (M[t][t] += D),
// so x is read once, as the B operand of step 3; its rows for the next s-tile
// stream into a rolling register buffer while the current s-tile computes.
// Lane l covers p = 2*(l%32) + pj of p-tile pj and, in the accumulator,
// rows 8*(r/4) + 4*(l/32) + r%4 of register r, so every store is one float2
// per lane, two full 256-byte rows per instruction.
// ---------------------------------------------------------------------------

// ZT: the type of z (and, in the gate gradient epilogue, of dout and dz).
template <typename T, int Q, int N, bool GATE, bool PRE, bool GB = false, typename ZT = T>
__global__ __launch_bounds__(512) void chunk_scan_group_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ Dv, const ZT* __restrict__ z, const float* __restrict__ ws_dt,
    const float* __restrict__ ws_cum, const float* __restrict__ states_in,
    const float* __restrict__ gram, T* __restrict__ out,
    const int32_t* __restrict__ seg, int64_t L, int64_t H, int64_t G, int64_t nc, int64_t nunits,
    const ZT* __restrict__ gd, ZT* __restrict__ gdz) {
  constexpr int P = 64, NT = Q / 32, CS = N + 4, NG = NT * (NT + 1) / 2, KQ = N / 8;
  static_assert(!(GB && GATE), "the gate gradient epilogue takes the ungated y");
  // byte offsets of the ZT tensors: those of the T tensors over kZS
  constexpr uint32_t kZS = sizeof(T) / sizeof(ZT);
  static_assert(kZS == 1 || (kZS == 2 && sizeof(T) == 4), "z type");
  constexpr int NW = 8;                   // waves: two per head
  constexpr int GW = (NG + NW - 1) / NW;  // G tiles per wave, at most
  constexpr int NS = NT / 2;              // t-tiles per wave
  // B tile, then the G^T tiles; only the tiles when they are read in
  constexpr int BGS = (!PRE && Q * CS > NG * 1024) ? Q * CS : NG * 1024;
  constexpr int HR = 3;                   // ring of state loads: two steps ahead
  constexpr float kLog2e = 1.4426950408889634f;
  static_assert((Q == 64 || Q == 128) && (N == 64 || N == 128), "tile");
  __shared__ float c_lds[Q * CS];
  __shared__ float bg_lds[BGS];
  __shared__ float cum_lds[4][Q];  // running sums in log2 units (cum * log2 e)
  __shared__ float dt_lds[4][Q];
  // u_s = 2^(cum_e - cum_s) dt_s, e = last step of s's 32-step tile (<= dt_s);
  // 0 when a packed sequence starts in (s, e]
  __shared__ __align__(16) float u_lds[4][Q];
  __shared__ __align__(16) int32_t seg_lds[Q];  // sequence starts from the chunk start (0: no seq_idx)

  const int64_t HQ = H / 4;
  const int64_t u = xcd_remap(blockIdx.x, nunits);  // ((b*nc + c)*HQ + hq)
  const int64_t hq = u % HQ, c = (u / HQ) % nc, b = u / (HQ * nc);
  const int64_t h0 = 4 * hq;
  const int64_t g = h0 / (H / G);
  const int tid = threadIdx.x, lane = tid % kWave;
  // wave-uniform (the buffer resources below and the per-wave branches need it)
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int slot = wave >> 1, half = wave & 1;
  const int i = lane % 32, kk = lane / 32;
  const int64_t h = h0 + slot;
  const int64_t t0 = c * Q;
  const int64_t xs = H * P;
  // last real row of this chunk, clamped to the chunk (rows past it are padding)
  const int last = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
  // t-tiles of this wave: {half, NT-1-half} (NT = 4) or {half} (NT = 2); equal
  // causal work for both halves when NT = 4
  auto own = [&](int j) { return j == 0 ? half : NT - 1 - half; };
  const int smax = own(NS - 1) > own(0) ? own(NS - 1) : own(0);  // last s-tile needed

  // ---- 0. stage C (and B, or the G^T tiles), cum, dt ---------------------------
  // Every global load of the set-up -- the tiles, the step tables and this
  // wave's first per-head operands -- is issued before the first LDS write,
  // so the set-up waits for one memory latency rather than one per group of
  // loads.
  constexpr int KC = Q * N / (4 * 64 * NW);             // float4 per thread per tile
  constexpr int KG = (NG * 256 + 64 * NW - 1) / (64 * NW);  // float4 of G^T per thread
  const T* cs = Cm + ((b * L + t0) * G + g) * N;
  const T* bs = Bm + ((b * L + t0) * G + g) * N;
  const int64_t rs = G * N;
  f4 cst[KC], bst[PRE ? 1 : KC], gst[PRE ? KG : 1];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int e = (k * 64 * NW + tid) * 4;
    const int row = e / N, col = e % N;
    const int r = row < last ? row : last;
    cst[k] = ld4(cs + r * rs + col);
    if constexpr (!PRE) bst[k] = ld4(bs + r * rs + col);
  }
  if constexpr (PRE) {
    const float* gs = gram + ((b * nc + c) * G + g) * (int64_t)(NG * 1024);
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int q = k * 64 * NW + tid;
      if (q < NG * 256) gst[k] = ld4(gs + 4 * q);
    }
  }
  // step tables: step t of head slot w per thread (4 Q <= 512 threads)
  const int32_t* sc = seg ? seg + (b * nc + c) * Q : nullptr;
  const int tw = tid / Q, tt = tid % Q;
  const bool tab = tid < 4 * Q;
  float cum_a = 0.f, dt_a = 0.f, cend_a = 0.f;
  int32_t seg_a = 0, seg_e = 0;
  if (tab) {
    const int64_t o = ((b * H + h0 + tw) * nc + c) * Q + tt;
    cum_a = ws_cum[o];
    dt_a = ws_dt[o];
    cend_a = ws_cum[o - tt + (tt | 31)];
    if (sc) {
      seg_a = sc[tt];
      seg_e = sc[tt | 31];
    }
  }

  // ---- first per-head loads, in flight during the set-up (and the shared G
  // phase) --------------------------------------------------------------------
  // x, z and out rows of this head in the chunk through buffer resources that
  // end after row `last`: padding rows read as zero and are never written
  const int64_t hoff = ((b * L + t0) * H + h) * P;
  const uint32_t rowb = (uint32_t)(xs * sizeof(T));  // bytes from one step to the next
  const uint32_t nbytes = (uint32_t)((last * xs + P) * sizeof(T));
  const auto xr = row_rsrc(x + hoff, nbytes);
  const auto zr = row_rsrc(GATE || GB ? static_cast<const void*>(z + hoff)
                                      : static_cast<const void*>(x + hoff),
                           nbytes / kZS);  // read only when GATE or GB
  const auto orr = row_rsrc(out + hoff, nbytes);
  // gate gradient epilogue: dout in, dz out (same rows)
  const auto dr = row_rsrc(GB ? static_cast<const void*>(gd + hoff)
                              : static_cast<const void*>(x + hoff),
                           nbytes / kZS);
  const auto dzr = row_rsrc(GB ? static_cast<const void*>(gdz + hoff)
                               : static_cast<const void*>(out + hoff),
                            nbytes / kZS);
  const uint32_t lane_b = (uint32_t)((4 * kk * xs + 2 * i) * sizeof(T));  // row 4 kk, column 2 i
  const float* hs = states_in + ((b * nc + c) * H + h) * (int64_t)(P * N) + 4 * lane;
  f4 hv[HR][2];
#pragma unroll
  for (int q = 0; q < HR - 1; ++q) {
    hv[q][0] = ld4(hs + (2 * q) * 256);
    hv[q][1] = ld4(hs + (2 * q + 1) * 256);
  }
  // x rows of s-tile si held by this lane: 32*si + 8*(m/4) + 4*kk + m%4.  One
  // rolling buffer: slots 4R..4R+3 are refilled with the next s-tile's rows as
  // soon as the MFMAs of step R have consumed them.  Padding rows read as zero.
  f2 xv[16];
  auto load_x = [&](int si, int R) {
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[4 * R + e] = bld2(xr, lane_b + (32 * si + 8 * R + e) * rowb, T{});
  };
  // z rows of the t-tile this wave emits next (its first owned tile now; the
  // second one is loaded as soon as the first has been emitted)
  f2 zv[16];
  auto load_z = [&](int ti) {
#pragma unroll
    for (int m = 0; m < 16; ++m)
      zv[m] = bld2(zr, (lane_b + (32 * ti + 8 * (m / 4) + m % 4) * rowb) / kZS, ZT{});
  };
  f2 dv[GB ? 16 : 1];  // dout rows of that t-tile (gate gradient epilogue)
  auto load_d = [&](int ti) {
#pragma unroll
    for (int m = 0; m < (GB ? 16 : 1); ++m)
      dv[m] = bld2(dr, (lane_b + (32 * ti + 8 * (m / 4) + m % 4) * rowb) / kZS, ZT{});
  };
  __builtin_amdgcn_sched_barrier(0);  // every set-up load is issued above

#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int e = (k * 64 * NW + tid) * 4;
    const int row = e / N, col = e % N;
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f4*>(&c_lds[row * CS + col]) = row > last ? zero : cst[k];
    if constexpr (!PRE) *reinterpret_cast<f4*>(&bg_lds[row * CS + col]) = row > last ? zero : bst[k];
  }
  if constexpr (PRE) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int q = k * 64 * NW + tid;
      if (q < NG * 256) *reinterpret_cast<f4*>(&bg_lds[4 * q]) = gst[k];
    }
  }
  if (tab) {
    const float cum2 = cum_a * kLog2e, cend2 = cend_a * kLog2e;
    cum_lds[tw][tt] = cum2;
    dt_lds[tw][tt] = dt_a;
    u_lds[tw][tt] = seg_a == seg_e ? fast_exp2(cend2 - cum2) * dt_a : 0.0f;
    if (tw == 0) seg_lds[tt] = seg_a;
  }
  __syncthreads();
  // x of the first s-tile and z of the first t-tile stream in under the
  // state part, which is bound by the matrix cores
#pragma unroll
  for (int R = 0; R < 4; ++R) load_x(0, R);
  if constexpr (GATE || GB) load_z(own(0));
  if constexpr (GB) load_d(own(0));

  // ---- 1. causal tiles of G^T = B C^T, shared by the four heads ---------------
  if constexpr (!PRE) {
  f16x gt[GW];
#pragma unroll
  for (int k = 0; k < GW; ++k) {
    gt[k] = zero16();
    const int tau = wave + NW * k;
    if (tau < NG) {
      int si = 0, ti = 0;
      tile_of<NT>(tau, &si, &ti);
      const float* ap = &bg_lds[(32 * si + i) * CS + (N / 2) * kk];
      const float* bp = &c_lds[(32 * ti + i) * CS + (N / 2) * kk];
#pragma unroll 4
      for (int q = 0; q < KQ; ++q) {
        const f4 av = *reinterpret_cast<const f4*>(ap + 4 * q);
        const f4 bv = *reinterpret_cast<const f4*>(bp + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) gt[k] = mfma32x32x2(av[e], bv[e], gt[k]);
      }
    }
  }
  __syncthreads();  // every read of the B tile is done
#pragma unroll
  for (int k = 0; k < GW; ++k) {
    const int tau = wave + NW * k;
    if (tau < NG) {
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        f4 v;
        v[0] = gt[k][4 * R];
        v[1] = gt[k][4 * R + 1];
        v[2] = gt[k][4 * R + 2];
        v[3] = gt[k][4 * R + 3];
        *reinterpret_cast<f4*>(&bg_lds[((tau * 4 + R) * 64 + lane) * 4]) = v;
      }
    }
  }
  __syncthreads();
  }

  const float* cumw = cum_lds[slot];
  const float* dtw = dt_lds[slot];
  const float* uw = u_lds[slot];
  // cum_t (log2 units) and exp(cum_t) of this lane's A-operand row; with
  // packed sequences the entering state reaches only the chunk's first one
  float ct[NS], ect[NS];
  int kt[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    ct[j] = cumw[32 * own(j) + i];
    kt[j] = seg_lds[32 * own(j) + i];
    ect[j] = kt[j] == 0 ? fast_exp2(ct[j]) : 0.0f;
  }

  // ---- 2. state part: acc = (exp(cum_t) C) . H_in^T ---------------------------
  f16x acc[NS][2];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j][0] = acc[j][1] = zero16();
  auto load_c = [&](int q, f4 (&cv)[NS]) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      cv[j] = *reinterpret_cast<const f4*>(&c_lds[(32 * own(j) + i) * CS + (N / 2) * kk + 4 * q]);
  };
  f4 cnext[NS];
  load_c(0, cnext);
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    const int rs = q % HR;
    if (q + HR - 1 < KQ) {
      const int nq = q + HR - 1, ns = nq % HR;
      hv[ns][0] = ld4(hs + (2 * nq) * 256);
      hv[ns][1] = ld4(hs + (2 * nq + 1) * 256);
    }
    f4 cv[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) cv[j] = cnext[j] * ect[j];
    if (q + 1 < KQ) load_c(q + 1, cnext);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        acc[j][0] = mfma32x32x2(cv[j][e], hv[rs][0][e], acc[j][0]);
        acc[j][1] = mfma32x32x2(cv[j][e], hv[rs][1][e], acc[j][1]);
      }
  }

  // ---- 3. in-chunk part per s-tile, then the epilogue of t-tile si ------------
  // The D skip rides on the diagonal of the decay-masked matrix: M[t][t] gets
  // + D_h, so the epilogue needs no x.  The four masked values of step R+1 are
  // computed while the MFMAs of step R run.
  const float Dh = Dv ? Dv[h] : 0.0f;
#pragma unroll
  for (int si = 0; si < NT; ++si) {
    if (si > smax) break;  // uniform per wave
    // masked values mv[j][e] of step R: G^T(s, t) * 2^(ct - cs) * dt_s, causal on
    // the diagonal tile, plus D at s == t.  Below the diagonal the decay is
    // split at the s-tile's last step e: 2^(ct - ce) * u_s, both factors <= 1,
    // so one exp per lane and tile; the diagonal tile keeps the direct form.
    // A start in (s, t] is one in (s, e] or in (e, t] (e = 32 si + 31 lies
    // between them), so the packed-sequence mask splits like the decay: u_s
    // carries the first half, rs the second.
    float rs[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j)
      rs[j] = kt[j] == seg_lds[32 * si + 31] ? fast_exp2(ct[j] - cumw[32 * si + 31]) : 0.0f;
    auto masked = [&](int R, float (&mv)[NS][4]) {
      const f4 cs4 = *reinterpret_cast<const f4*>(&cumw[32 * si + 8 * R + 4 * kk]);
      const f4 ds4 = *reinterpret_cast<const f4*>(&dtw[32 * si + 8 * R + 4 * kk]);
      const f4 us4 = *reinterpret_cast<const f4*>(&uw[32 * si + 8 * R + 4 * kk]);
      const int4 ks4 = *reinterpret_cast<const int4*>(&seg_lds[32 * si + 8 * R + 4 * kk]);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int ti = own(j) >= si ? own(j) : si;  // tiles below si are not used
        const f4 gv = *reinterpret_cast<const f4*>(
            &bg_lds[(((ti * (ti + 1) / 2 + si) * 4 + R) * 64 + lane) * 4]);
        if (own(j) == si) {  // uniform
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = gv[e] * fast_exp2(ct[j] - cs4[e]) * ds4[e];
            const int sl = 8 * R + 4 * kk + e;  // s within the tile
            const int ks = e == 0 ? ks4.x : e == 1 ? ks4.y : e == 2 ? ks4.z : ks4.w;
            mv[j][e] = (sl < i) ? (ks == kt[j] ? v : 0.0f) : (sl == i ? v + Dh : 0.0f);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[j][e] = gv[e] * rs[j] * us4[e];
        }
      }
    };
    float mcur[NS][4], mnext[NS][4];
    masked(0, mcur);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      float x0[4], x1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x0[e] = xv[4 * R + e][0];
        x1[e] = xv[4 * R + e][1];
      }
      if (si + 1 <= smax) load_x(si + 1, R);  // refill the slots just read
      if (R + 1 < 4) masked(R + 1, mnext);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if (own(j) < si) continue;  // uniform
          acc[j][0] = mfma32x32x2(mcur[j][e], x0[e], acc[j][0]);
          acc[j][1] = mfma32x32x2(mcur[j][e], x1[e], acc[j][1]);
        }
      if (R + 1 < 4) {
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) mcur[j][e] = mnext[j][e];
      }
    }
    // epilogue of t-tile si if this wave owns it: rows 32*si + 8*(r/4) + 4*kk + r%4
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (own(j) != si) continue;  // uniform
      auto emit = [&](int r) {
        f2 y;
        y[0] = acc[j][0][r];
        y[1] = acc[j][1][r];
        // rows past `last` fall outside the buffer and are dropped
        const uint32_t off = lane_b + (32 * si + 8 * (r / 4) + r % 4) * rowb;
        if constexpr (GB) {
          // dY = dout silu(z), dz = dout y sigmoid(z) (1 + z (1 - sigmoid(z)))
          f2 dyv, dzv;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float zz = zv[r][e], d = dv[r][e];
            const float sg = fast_rcp(1.0f + fast_exp2(-zz * kLog2e));
            dyv[e] = d * zz * sg;
            dzv[e] = d * y[e] * sg * (1.0f + zz * (1.0f - sg));
          }
          bst2(orr, off, dyv, T{});
          bst2(dzr, off / kZS, dzv, ZT{});
        } else {
          if constexpr (GATE) {
            y[0] *= silu(zv[r][0]);
            y[1] *= silu(zv[r][1]);
          }
          bst2(orr, off, y, T{});
        }
      };
#pragma unroll
      for (int r = 0; r < 16; ++r) emit(r);
      if constexpr (GATE || GB) {
        if (j + 1 < NS) load_z(own(j + 1));
      }
      if constexpr (GB) {
        if (j + 1 < NS) load_d(own(j + 1));
      }
    }
  }
}

// True when the four-heads-per-workgroup kernel handles this problem.
static bool use_group_kernel(const Problem& p) {
  return (p.Q == 64 || p.Q == 128) && (p.N == 64 || p.N == 128) && ((p.H / p.G) % 4 == 0);
}

bool use_group_scan(int64_t H, int64_t N, int64_t G, int64_t Q, bool bf16) {
  // bf16 inputs at chunk 128/256 take the bf16 matrix-core kernels instead
  const bool bf16_kernels = bf16 && (Q == 128 || Q == 256) && (N == 64 || N == 128);
  return (Q == 64 || Q == 128) && (N == 64 || N == 128) && (H / G) % 4 == 0 && !bf16_kernels;
}

bool use_gram(int64_t H, int64_t N, int64_t G, int64_t Q, bool bf16) {
  return use_group_scan(H, N, G, Q, bf16) && H / G >= 8;
}

int64_t gram_tile_floats(int64_t Q) {
  const int64_t nt = Q / 32;
  return nt * (nt + 1) / 2 * 1024;
}

template <typename T, int Q, int N, bool GATE, bool PRE, bool GB = false, typename ZT = T>
static void launch_group(const Problem& p, hipStream_t s, int64_t nunits) {
  hipLaunchKernelGGL((chunk_scan_group_kernel<T, Q, N, GATE, PRE, GB, ZT>), dim3((unsigned)nunits),
                     dim3(512), 0, s, static_cast<const T*>(p.x), static_cast<const T*>(p.B),
                     static_cast<const T*>(p.C), p.D, static_cast<const ZT*>(p.z), p.ws_dt,
                     p.ws_cum, p.ws_states_in, p.ws_gram, static_cast<T*>(p.out), p.ws_seg, p.L,
                     p.H, p.G, p.nc, nunits,
                     static_cast<const ZT*>(p.gate_dout), static_cast<ZT*>(p.gate_dz));
}

template <typename T, int Q, int N>
static void launch_qn(const Problem& p, hipStream_t s) {
  if constexpr ((Q == 64 || Q == 128) && (N == 64 || N == 128)) {
    if (use_group_kernel(p)) {
      const int64_t nunits = p.b * p.nc * (p.H / 4);
      if constexpr (std::is_same<T, float>::value && Q == 64) {
        if (p.gate_dout) {  // the backward's re-run: the gate gradient epilogue
          if (p.gate_bf16) launch_group<T, Q, N, false, false, true, bf16_t>(p, s, nunits);
          else launch_group<T, Q, N, false, false, true>(p, s, nunits);
          return;
        }
      }
      if (p.ws_gram) {
        if (p.z) launch_group<T, Q, N, true, true>(p, s, nunits);
        else launch_group<T, Q, N, false, true>(p, s, nunits);
      } else {
        if (p.z) launch_group<T, Q, N, true, false>(p, s, nunits);
        else launch_group<T, Q, N, false, false>(p, s, nunits);
      }
      return;
    }
  }
  const int64_t nunits = p.b * p.nc * p.H;
  hipLaunchKernelGGL((chunk_scan_kernel<T, Q, N>), dim3((unsigned)nunits), dim3(256), 0, s,
                     static_cast<const T*>(p.x), static_cast<const T*>(p.B),
                     static_cast<const T*>(p.C), p.D, static_cast<const T*>(p.z), p.ws_dt,
                     p.ws_cum, p.ws_states_in, static_cast<T*>(p.out), p.ws_seg, p.L, p.H, p.G,
                     p.nc, nunits);
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
