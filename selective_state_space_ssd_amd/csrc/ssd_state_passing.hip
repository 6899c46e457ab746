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
#include <type_traits>

#include "ssd_dt.h"
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
// register order (ssd_device.h).  The operands are loaded in NB batches (one
// memory latency per batch; NB > 1 where registers are short).
template <typename T, int Q, int N, int NB = 1>
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
  static_assert(KQ % NB == 0, "batches");
  constexpr int KB = KQ / NB;
  f16x acc = zero16();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f4 bv[KB], cv[KB];
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      bv[q] = ld4(bp + 4 * (nb * KB + q));
      cv[q] = ld4(cp + 4 * (nb * KB + q));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
#pragma unroll
    for (int q = 0; q < KB; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = mfma32x32x2(__uint_as_float(__float_as_uint(bv[q][e]) & ms),
                          __uint_as_float(__float_as_uint(cv[q][e]) & mt), acc);
  }
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

// ---------------------------------------------------------------------------
// stages 2 and 3 in one pass
// ---------------------------------------------------------------------------

// For fp32 inputs with few chunks per sequence, one workgroup per (batch,
// head, SL = 32 or 64 state columns) walks the chunks in order: it forms each chunk's
// contribution S_c on the matrix cores (as stage 2) and folds it into the
// state it carries in registers (as above), so the chunk states never go
// through memory and the two launches become one.  The walk is sequential in
// c, but the S_c products are independent and the fold is four fmas per
// lane, so the matrix work of the chunks follows back to back; the
// parallelism is batch x heads x N/32 workgroups instead of also x chunks,
// which is why the pass is chosen only when that fills the machine.
//
// Eight waves; wave w holds SL/32 16 x 16 tiles (state columns 16 (SL/32
// (w % 2) + j) of the slice, rows 16 (w / 2); with two, they share the x
// operand) of S^T = B^T diag(w) X on v_mfma_f32_16x16x4_f32:
// lane (i, g = l/16) supplies B[t][n] and w_t x[t][p] for t = k0 + 4g + q at
// step q of each group of 16 steps (its four rows of the chunk's LDS tiles),
// and register r holds column n = 4g + r of row p = i, i.e. four consecutive
// n of one p: one float4 of the tiled state layout.  A chunk's x rows and the
// slice's B rows are staged in LDS (row pitches 68 and 36 floats: the four
// lane quarters read rows four apart, which land in distinct banks); the rows
// of the chunk after next are loaded into a second register set while the
// current one computes, so each load has two chunks' time to arrive.  64
// columns are taken when 32 would need two rounds of workgroups: half the
// workgroups, and fewer LDS and L1 bytes per product.
// dt, the running sums and w_t of every chunk are formed first (a wave per
// chunk, the slice-0 workgroup also writing them for the chunk scan) and kept
// in LDS, and the staged x rows are scaled by w_t on the way in.  The chunk
// scan's G^T tiles are formed by the same workgroups, a wave per tile, while
// their first loads are in flight.  Packed sequences as in stages 2 and 3:
// w_t = 0 for the steps of a chunk's earlier sequences, and a chunk in which
// a sequence starts drops the carried state (its decay taken as 0).
constexpr int kScanChunksMax = 32;

template <int Q, int N, int SL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void state_scan_kernel(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ dt_raw,
    const float* __restrict__ A, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* init, float* __restrict__ ws_dt, float* __restrict__ ws_cum,
    float* __restrict__ states_in, float* final_states, int64_t L, int64_t H, int64_t G,
    int64_t nc, int64_t nscan, const float* __restrict__ Cm, float* __restrict__ gram,
    int64_t gram_jobs, const int32_t* __restrict__ seg) {
  constexpr int P = 64, NT = 512, XP = 68, BP = SL + 4, E = Q / kWave, NTW = SL / 32;
  constexpr int QX = Q * P / (4 * NT), QB = Q * SL / (4 * NT);
  static_assert(QX >= 1 && QB >= 1 && Q * P % (4 * NT) == 0 && Q * SL % (4 * NT) == 0 &&
                (SL == 32 || SL == 64), "staging");
  __shared__ __align__(16) float xs[Q * XP];                // w_t x[t][p] of the chunk
  __shared__ __align__(16) float bs[Q * BP];                // B[t][n] of the slice
  __shared__ __align__(16) float wl[kScanChunksMax * Q];    // w_t of every chunk
  __shared__ float dec[kScanChunksMax];                     // exp(cum_last) of every chunk

  // the slices of one head are b H workgroups apart: on one XCD (sharing the
  // x rows in its L2) when b H is a multiple of 8
  const int64_t BH = nscan / (N / SL);
  const int64_t bh = blockIdx.x % BH, sl = blockIdx.x / BH;
  const int64_t b = bh / H, h = bh % H;
  // 32-bit and wave-uniform: the B buffer resource needs a scalar base
  const int64_t g = __builtin_amdgcn_readfirstlane((int)h / (int)(H / G));
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i = lane % 16, kq = 4 * (lane / 16);
  const int nl = 16 * NTW * (wave & 1), p0 = 16 * (wave >> 1);  // first tile in the slice
  const int n = SL * (int)sl + nl + kq, p = p0 + i;  // this lane's first float4 of the state
  constexpr int64_t PN = (int64_t)P * N;

  const uint32_t xrow = (uint32_t)(H * P * 4), brow = (uint32_t)(G * N * 4);
  // rows past the sequence end read as zero (their w is zero too); chunks
  // past the last are not read
  auto load = [&](int64_t c, f4 (&xv)[QX], f4 (&bv)[QB]) {
    if (c >= nc) return;
    const int64_t t0 = c * Q;
    const uint32_t last = (uint32_t)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
    const auto xr = row_rsrc(x + ((b * L + t0) * H + h) * P, last * xrow + P * 4);
    const auto br = row_rsrc(Bm + ((b * L + t0) * G + g) * N + SL * sl, last * brow + SL * 4);
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int e = 4 * (q * NT + tid);
      xv[q] = bld4(xr, (uint32_t)(e / P) * xrow + (uint32_t)(e % P) * 4);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int e = 4 * (q * NT + tid);
      bv[q] = bld4(br, (uint32_t)(e / SL) * brow + (uint32_t)(e % SL) * 4);
    }
  };
  // init and final_states may be the same buffer: each lane reads its four
  // elements of init before it writes the same four of final.  Loaded first:
  // the prologue's wait then covers it, and the loop never waits on it (a
  // load still in flight at the loop would make every chunk wait for all).
  f4 hs[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
    hs[j] = init ? ld4(init + bh * PN + p * N + n + 16 * j) : f4{0.f, 0.f, 0.f, 0.f};
  f4 xa[QX], ba[QB], xb[QX], bb[QB];  // register sets of even and odd chunks
  load(0, xa, ba);
  load(1, xb, bb);

  // the chunk scan's G^T tiles, a wave per tile, while those loads are in
  // flight: tile j goes to workgroup j % nscan, wave j / nscan
  for (int64_t job = (int64_t)wave * nscan + blockIdx.x; job < gram_jobs;
       job += (NT / kWave) * nscan)
    gram_tile<float, Q, N, N / 64>(Bm, Cm, gram, job, L, G, nc, lane);

  // dt, running sums (stored once, by the slice-0 workgroup) and w_t, a wave
  // per chunk
  {
    constexpr int CW = kScanChunksMax / (NT / kWave);  // chunks per wave, at most
    const float a = A[h], bias = dt_bias ? dt_bias[h] : 0.0f;
    float raw[CW][E];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int64_t c = wave + (NT / kWave) * j;
      if (c < nc) wave_dt_load<float, Q>(dt_raw, b, c, h, L, H, raw[j]);
    }
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int64_t c = wave + (NT / kWave) * j;
      if (c < nc) {
        float dtv[E], cum[E], cl;
        wave_dt_scan<Q>(raw[j], a, bias, dt_min, dt_max, b, c, h, L, H, nc,
                        sl == 0 ? ws_dt : nullptr, ws_cum, dtv, cum, &cl);
        const int32_t* sc = seg ? seg + (b * nc + c) * Q : nullptr;
        const int32_t slast = sc ? sc[Q - 1] : 0;
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const bool keep = !sc || sc[lane * E + k] == slast;
          wl[c * Q + lane * E + k] = keep ? __expf(cl - cum[k]) * dtv[k] : 0.0f;
        }
        if (lane == 0) dec[c] = slast == 0 ? __expf(cl) : 0.0f;
      }
    }
  }

  __syncthreads();  // every w_t is in LDS before the first staging scales by it
  float* const sbase = states_in + (b * nc * H + h) * PN;
  const int64_t cstride = H * PN;
  // chunk c: stage its rows from their register set (x scaled by w_t), load
  // chunk c + 2 into that set, then form S_c and fold it in
  auto step = [&](int64_t c, f4 (&xv)[QX], f4 (&bv)[QB]) {
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int e = 4 * (q * NT + tid);
      const float w = wl[c * Q + e / P];
      f4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = w * xv[q][k];
      *reinterpret_cast<f4*>(xs + (e / P) * XP + e % P) = v;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int e = 4 * (q * NT + tid);
      *reinterpret_cast<f4*>(bs + (e / SL) * BP + e % SL) = bv[q];
    }
    __syncthreads();  // chunk c staged
    load(c + 2, xv, bv);
    // the operands of the chunk's first half read, then its second half's,
    // whose reads run under the first half's products; four accumulators,
    // one per step of a group, so that consecutive MFMAs are independent
    constexpr int NGR = Q / 16, HG = NGR / 2;
    f4 bq[NTW][NGR], xq[NGR];
    auto read = [&](int gr) {
      const int k = 16 * gr + kq;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int cn = nl + 16 * j + i;
        bq[j][gr] = f4{bs[k * BP + cn], bs[(k + 1) * BP + cn], bs[(k + 2) * BP + cn],
                       bs[(k + 3) * BP + cn]};
      }
      xq[gr] = f4{xs[k * XP + p], xs[(k + 1) * XP + p], xs[(k + 2) * XP + p],
                  xs[(k + 3) * XP + p]};
    };
    f4 acc[NTW][4];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[j][q] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gr = 0; gr < HG; ++gr) read(gr);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gr = HG; gr < NGR; ++gr) read(gr);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gr = 0; gr < HG; ++gr)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[j][q] = mfma16x16x4(bq[j][gr][q], xq[gr][q], acc[j][q]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gr = HG; gr < NGR; ++gr)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[j][q] = mfma16x16x4(bq[j][gr][q], xq[gr][q], acc[j][q]);
    const float d = dec[c];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      st4(sbase + c * cstride + state_tile_offset(p, n + 16 * j, N), hs[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hs[j][e] = d * hs[j][e] + ((acc[j][0][e] + acc[j][1][e]) + (acc[j][2][e] + acc[j][3][e]));
    }
    __syncthreads();  // chunk c's tiles are read before the next is staged
  };
  for (int64_t c = 0; c < nc; c += 2) {
    step(c, xa, ba);
    if (c + 1 < nc) step(c + 1, xb, bb);
  }
  if (final_states) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) st4(final_states + bh * PN + p * N + n + 16 * j, hs[j]);
  }
}

// Chosen when its workgroups fill the compute units in one round (at least
// half of them), with 32-column slices, or else with 64: two rounds of
// 32-column workgroups measured no faster than the two launches (batch 4 x
// 2048, 32 heads: 630 vs 635 us for four calls), and a quarter of the
// machine would leave the per-chunk work to few units.  Returns the slice
// width, 0 when the pass is not taken.
int state_scan_slice(bool bf16, bool varlen, int64_t b, int64_t L, int64_t H, int64_t N,
                     int64_t Q) {
  (void)varlen;  // packed sequences are handled as in stages 2 and 3
  if (bf16 || !(N == 64 || N == 128) || !(Q == 64 || Q == 128) || L < 1) return 0;
  if ((L + Q - 1) / Q > kScanChunksMax) return 0;
  for (int sl : {32, 64}) {
    const int64_t nscan = b * H * (N / sl);
    if (2 * nscan >= kChainCUs && nscan <= kChainCUs) return sl;
  }
  return 0;
}

bool use_state_scan(bool bf16, bool varlen, int64_t b, int64_t L, int64_t H, int64_t N,
                    int64_t Q) {
  return state_scan_slice(bf16, varlen, b, L, H, N, Q) != 0;
}

template <int Q, int N, int SL>
static void launch_scan_qn(const Problem& p, hipStream_t s) {
  const int64_t nscan = p.b * p.H * (N / SL);
  const int64_t jobs = p.ws_gram ? p.b * p.nc * p.G * (gram_tile_floats(Q) / 1024) : 0;
  hipLaunchKernelGGL((state_scan_kernel<Q, N, SL>), dim3((unsigned)nscan), dim3(512), 0, s,
                     static_cast<const float*>(p.x), static_cast<const float*>(p.B),
                     static_cast<const float*>(p.dt), p.A, p.dt_bias, p.dt_min, p.dt_max, p.init,
                     p.ws_dt, p.ws_cum, p.ws_states_in, p.final_states, p.L, p.H, p.G, p.nc,
                     nscan, static_cast<const float*>(p.C), p.ws_gram, jobs, p.ws_seg);
}

hipError_t launch_state_scan(const Problem& p, hipStream_t stream) {
  const bool wide = state_scan_slice(p.bf16, p.seq_idx != nullptr, p.b, p.L, p.H, p.N, p.Q) == 64;
  auto go = [&](auto q, auto n) {
    constexpr int Q = decltype(q)::value, N = decltype(n)::value;
    if (wide) launch_scan_qn<Q, N, 64>(p, stream);
    else launch_scan_qn<Q, N, 32>(p, stream);
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  if (p.Q == 64) {
    if (p.N == 64) go(I64{}, I64{});
    else go(I64{}, I128{});
  } else {
    if (p.N == 64) go(I128{}, I64{});
    else go(I128{}, I128{});
  }
  return hipGetLastError();
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
