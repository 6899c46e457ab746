// Chain bf16 scan: one workgroup carries two heads of one group through the
// whole sequence, block after block, with the running state in registers.
//
// The chunked form of the scan (the state-space-duality pages: a chunk's
// output is its own masked C.B^T part plus C times the state entering it,
// and the state leaving it is the decayed entering state plus the chunk's
// own B^T.(decay*dt*x) part) needs, per 128-step block and head, inputs x,
// B, C, z (B and C shared by the heads of a group) and the entering state.
// Here the state never leaves the compute unit: wave w of a head holds rows
// p = 16w .. 16w+15 of the head's P x N fp32 state for the whole run, so no
// state crosses memory and no workgroup waits on another.  Latency is hidden
// by loading block c+1's x, B, C (and dt) into registers while block c is
// computed, and z at the start of the block whose epilogue needs it.
//
// Per block (t0 = 128 c, 16-step tiles i = 0..7, lanes (g, m) = (l/16, l%16)):
//   stage    the prefetched B, C, x tiles into LDS; wave 0 of each head
//            computes dt = clamp(softplus(dt_raw + dt_bias)), the running
//            sum cum of dt*A, and the per-step factors below into LDS;
//   in-block wave w of a head takes t-tiles {w, 7-w} (nine 16 x 16 tiles of
//            C.B^T each, so the four waves do equal work):
//              Y^T[p][t] += x^T[p][s] M^T[s][t],  M^T = G^T o decay,
//              G^T[s][t] = B[s] . C[t]   (16x16x32 bf16 MFMAs),
//            with decay(s, t) = exp(cum_t - cum_s) dt_s (s <= t) and D on
//            the diagonal.  Below the tile holding t the decay is split at
//            the step r = 16 i - 1 before the tile: exp(cum_r - cum_s) dt_s
//            (a table over (i, s)) times exp(cum_t - cum_r), both <= 1,
//            the second applied once to the accumulated tiles;
//   C.H      wave w: Y^T[p][t] (its 16 p, every t) = H[p][n] C^T[n][t],
//            scaled by exp(cum_t) in the epilogue;
//   state    H = exp(cum_last) H + B^T (w o x), w_t = exp(cum_last - cum_t)
//            dt_t, accumulated by the MFMAs straight into H's registers;
//   epilogue the in-block and C.H parts meet in LDS (they are owned by
//            different waves), then z gate and 16-byte stores.
//
// Operands formed on the fly (w o x, the state, the masked C.B^T values) are
// split into hi/lo bf16 pairs, as in the other bf16 kernels; x, B, C enter
// the matrix cores as they are.
//
// Packed sequences (seq_idx): wave 0 counts the sequence starts k_t from the
// block start; w_t needs k_t = k_last, the carried state needs k_last = 0,
// exp(cum_t) of the C.H part needs k_t = 0, and a pair (s, t) needs
// k_s = k_t -- split at r like the decay, [k_s = k_r][k_r = k_t], since k
// never decreases within a block.
#include <type_traits>

#include "ssd_bf16_tiles.h"
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {
using namespace bf16t;

namespace {
constexpr int CQ = 128;       // timesteps per block
constexpr int CT = CQ / 16;   // 16-step tiles per block
constexpr int kPair = 2;      // heads per workgroup
constexpr int kChainThreads = 256 * kPair;

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].  Lane l = 16 g + m
// supplies row m of A and column m of B at the eight contraction slots
// (g, 0..7); register r of the result is D[4 g + r][m].  Only the pairing of
// A's and B's slots matters, so each product below names its own slot order.
__device__ __forceinline__ f4 mfma16(s16x8 a, s16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// LDS row pitches, chosen so that every access of an unrolled loop is one
// per-lane base plus an immediate offset, and free of bank conflicts
// (measured with the LDS conflict counter, access pattern by pattern):
//  * transposed reads, where the two lane groups served together read rows
//    r0 + 0..3 and r0 + 4..7 (32 bytes each): conflict-free at pitches of
//    160 and 352 bytes, while groups 8 rows apart conflict at any pitch --
//    so every transposed read here takes its slots from rows 4 apart;
//  * B (read both ways): 352 bytes at N = 128, 160 at N = 64;
//  * C (row reads only: 16 rows of 16 or 8 bytes at one column): 304 / 144;
//  * x (transposed reads only): 160 bytes;
//  * fp32 output tiles (64 floats): 272 bytes, 16 rows of 16 bytes distinct.
template <int N>
struct Pitch {
  static constexpr int kB = N == 128 ? 176 : 80;   // elements
  static constexpr int kC = N == 128 ? 152 : 72;
};
constexpr int kXP = 80;   // x tile pitch, elements
constexpr int kYP = 68;   // output tile pitch, floats

__device__ __forceinline__ s16x4 tr4(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
__device__ __forceinline__ s16x8 cat8(s16x4 a, s16x4 b) {
  s16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}
// Transposed read (lane 16 g + m): rows r0 + 0..3 of column c0 + m of a tile
// with row pitch `ld`, r0 per lane group.  In each group of 16 lanes, lane
// 4a + e receives element e of the 8-byte words read by lanes a, a+4, a+8,
// a+12; lane m therefore reads row r0 + m/4 at column c0 + 4 (m%4).
__device__ __forceinline__ s16x4 tr_rows(const bf16_t* t, int ld, int r0, int c0, int m) {
  return tr4(t + (r0 + (m >> 2)) * ld + c0 + 4 * (m & 3));
}

// 16 bytes at a per-lane 32-bit byte offset into a buffer resource (zero past
// its end, ssd_device.h).
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float fexp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fsilu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + fexp2(-v * kLog2e));
}

// LDS layout (bytes).  The staging tiles and the two fp32 output tiles per
// head share one region (the tiles are dead once the output is formed).
template <int N>
struct ChainLds {
  static constexpr int kB = 0;
  static constexpr int kC = kB + CQ * Pitch<N>::kB * 2;
  static constexpr int kX = kC + CQ * Pitch<N>::kC * 2;      // kPair x [CQ][kXP] bf16
  static constexpr int kStageEnd = kX + kPair * CQ * kXP * 2;
  static constexpr int kYBytes = kPair * 2 * CQ * kYP * 4;   // per head: in-block, then C.H
  static constexpr int kU = kStageEnd > kYBytes ? kStageEnd : kYBytes;
  // per head: cum2, dt, w, et, ett (fp32), kseq (int), v[CT][CQ] (fp32)
  static constexpr int kTabFloats = 6 * CQ + CT * CQ;
  static constexpr int kTab = kU;
  static constexpr int kDl = kTab + kPair * kTabFloats * 4;
  static constexpr int kBytes = kDl + 16;
};
}  // namespace

// Workgroup wi = (segment, pair) with the pairs fastest (the pairs of a group
// stay contiguous, so they share an XCD).  A segment is a range of `span`
// blocks (unsegmented: one segment of all blocks).  Segment 0 starts from
// initial_states (or zero); segment s > 0 from initial_states folded with the
// local end states E_u and decays D_u of the units 0 .. s * units_per_seg - 1
// (seg_states [b, H, nunits] blocks of P x N floats, row-major [p][n], and
// seg_decay [b, H, nunits], written by the unit-state kernel before): H =
// D_u H + E_u in unit order.  The outputs of the segment's blocks are written;
// the last segment writes final_states.
template <int N, bool GATE, bool VARLEN>
__global__ __launch_bounds__(kChainThreads) void chain_scan_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const bf16_t* __restrict__ dt_raw, const float* __restrict__ A,
    const float* __restrict__ dt_bias, float dt_min, float dt_max, const float* __restrict__ Dv,
    const bf16_t* __restrict__ z, bf16_t* __restrict__ out, const float* __restrict__ init,
    float* __restrict__ final_states, const int32_t* __restrict__ seq, int64_t L, int64_t H,
    int64_t G, int64_t nblk, int64_t nwg, int64_t npairs, int64_t span,
    const float* __restrict__ seg_states, const float* __restrict__ seg_decay, int64_t nunits,
    int64_t units_per_seg) {
  static_assert(N == 64 || N == 128, "dstate 64 or 128");
  // without packed sequences every start count is zero: the compiler drops
  // the counts, their compares and their table
  if constexpr (!VARLEN) seq = nullptr;
  constexpr int KN = N / 32;                   // contraction steps over n
  constexpr int NT = N / 16;                   // 16-row n tiles of the state
  constexpr int PB = CQ * N / 8 / kChainThreads;  // 16-byte pieces of a B (C) tile per thread
  constexpr int PX = CQ * kP / 8 / 256;        // ... of an x (z, out) tile per thread of a head
  using Lay = ChainLds<N>;
  __shared__ __align__(16) char lds[Lay::kBytes];

  // lane indices; refreshed from an opaque copy of threadIdx.x at every block
  // (see the top of the block loop)
  int tid = threadIdx.x & (kChainThreads - 1), th = tid & 255, lane = tid & 63, g = lane >> 4,
      m = lane & 15;
  const int hd = __builtin_amdgcn_readfirstlane(tid >> 8);         // head of the pair (per wave)
  const int wt = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);   // wave within the head
  // workgroup -> (batch, head pair) in 32-bit scalar arithmetic (64-bit
  // division runs on the vector unit and would leave every address derived
  // from it in vector registers); the head pairs of a group share an XCD
  const int wi = (int)xcd_remap(blockIdx.x, nwg);
  const int piece = __builtin_amdgcn_readfirstlane(wi / (int)npairs);  // the segment
  const int pair = __builtin_amdgcn_readfirstlane(wi % (int)npairs);
  const int hp = (int)H / kPair;
  const int64_t b = __builtin_amdgcn_readfirstlane(pair / hp);
  const int64_t h = __builtin_amdgcn_readfirstlane(kPair * (pair % hp) + hd);
  const int64_t c_begin = (int64_t)piece * span;
  const int64_t c_end = c_begin + span < nblk ? c_begin + span : nblk;
  const int64_t grp = __builtin_amdgcn_readfirstlane((int)h / ((int)H / (int)G));
  const int64_t xs = H * kP, bs = G * N;
  const uint32_t xrow = (uint32_t)(xs * 2), brow = (uint32_t)(bs * 2);  // row pitches, bytes

  bf16_t* Bl = reinterpret_cast<bf16_t*>(lds + Lay::kB);
  bf16_t* Cl = reinterpret_cast<bf16_t*>(lds + Lay::kC);
  bf16_t* Xl = reinterpret_cast<bf16_t*>(lds + Lay::kX) + hd * CQ * kXP;
  float* yin = reinterpret_cast<float*>(lds) + hd * 2 * CQ * kYP;
  float* ych = yin + CQ * kYP;
  constexpr int BP = Pitch<N>::kB, CP = Pitch<N>::kC;
  float* tab = reinterpret_cast<float*>(lds + Lay::kTab) + hd * Lay::kTabFloats;
  float* cum2_l = tab;             // cum_t log2(e)
  float* dt_l = tab + CQ;          // dt_t
  float* w_l = tab + 2 * CQ;       // exp(cum_last - cum_t) dt_t        [k_t = k_last]
  float* et_l = tab + 3 * CQ;      // exp(cum_t)                        [k_t = 0]
  float* ett_l = tab + 4 * CQ;     // exp(cum_t - cum_r(t))             [k_t = k_r]
  int* k_l = reinterpret_cast<int*>(tab + 5 * CQ);  // sequence starts since the block start
  float* v_l = tab + 6 * CQ;       // v[i][s] = exp(cum_r(i) - cum_s) dt_s [k_s = k_r], s < 16 i
  float* dl_l = reinterpret_cast<float*>(lds + Lay::kDl);

  const float Ah = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const float Dh = Dv ? Dv[h] : 0.0f;
  const int pme = 16 * wt + m;  // this lane's state row

  // running state: Hs[j][r] = H[p = 16 wt + m][n = 16 j + 4 g + r]
  f4 Hs[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
    Hs[j] = init ? ld4(init + ((b * H + h) * kP + pme) * N + 16 * j + 4 * g) : zero4();
  {
    // a later segment: fold in the end states of the units before it
    const int64_t ubase = (b * H + h) * nunits;
    const int64_t nfold = (int64_t)piece * units_per_seg;
    // two units per step, so that both units' loads are in flight together
    int64_t u = 0;
    for (; u + 2 <= nfold; u += 2) {
      const float d0 = seg_decay[ubase + u], d1 = seg_decay[ubase + u + 1];
      const float* E0 = seg_states + ((ubase + u) * kP + pme) * N + 4 * g;
      const float* E1 = E0 + kP * N;
      f4 e0[NT], e1[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        e0[j] = ld4(E0 + 16 * j);
        e1[j] = ld4(E1 + 16 * j);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) Hs[j] = (Hs[j] * d0 + e0[j]) * d1 + e1[j];
    }
    if (u < nfold) {
      const float du = seg_decay[ubase + u];
      const float* E = seg_states + ((ubase + u) * kP + pme) * N + 4 * g;
#pragma unroll
      for (int j = 0; j < NT; ++j) Hs[j] = Hs[j] * du + ld4(E + 16 * j);
    }
  }

  // ---- prefetch registers: the next block's B, C and x tiles ----
  uint4 pb[PB], pc[PB], px[PX];
  bf16_t pdt[2] = {0, 0};
  // Rows of a block go through buffer resources that end after the block's
  // last row: rows past the sequence end read as zero (and the epilogue's
  // stores there are dropped), with no clamp, mask or branch.
  auto prefetch = [&](int64_t c) {
    const int64_t t0 = c * CQ;
    const uint32_t last = (uint32_t)((L - 1 - t0) < (CQ - 1) ? (L - 1 - t0) : (CQ - 1));
    const uint32_t nb = last * brow + N * 2;
    const auto brs = row_rsrc(Bm + ((b * L + t0) * G + grp) * N, nb);
    const auto crs = row_rsrc(Cm + ((b * L + t0) * G + grp) * N, nb);
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int e = k * kChainThreads + tid;
      const int row = e / (N / 8), col = (e % (N / 8)) * 8;
      const uint32_t o = (uint32_t)row * brow + (uint32_t)col * 2;
      pb[k] = bld16(brs, o);
      pc[k] = bld16(crs, o);
    }
    const auto xrs = row_rsrc(x + ((b * L + t0) * H + h) * kP, last * xrow + kP * 2);
#pragma unroll
    for (int k = 0; k < PX; ++k) {
      const int e = k * 256 + th;
      const int row = e / 8, col = (e % 8) * 8;
      px[k] = bld16(xrs, (uint32_t)row * xrow + (uint32_t)col * 2);
    }
  };
  // dt_raw of block c (lane l: steps 2l, 2l+1), loaded where it is used: held
  // across a block it would be spilled, and the wait for a spilled value
  // would also wait for every load issued before it
  auto load_dt = [&](int64_t c) {
    const int64_t t0 = c * CQ;
    const int last = (int)((L - 1 - t0) < (CQ - 1) ? (L - 1 - t0) : (CQ - 1));
    const bf16_t* dsrc = dt_raw + (b * L + t0) * H + h;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 2 * lane + k;
      pdt[k] = *reinterpret_cast<const bf16_t*>(reinterpret_cast<const char*>(dsrc) +
                                                (uint32_t)(r < last ? r : last) * (uint32_t)(H * 2));
    }
  };

  // dt, its running sum and the per-step factors of block c into the tables.
  // Every wave of the head runs the scan over the block's 128 steps (lane l:
  // steps 2l, 2l+1; steps past the end get dt = 0); the exponentials are
  // shared out between the four waves.
  auto tables = [&](int64_t c) {
    const int64_t t0 = c * CQ;
    float dv[2], cum[2], run = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float d = 0.0f;
      if (t0 + 2 * lane + k < L) {
        d = softplus(to_f32(pdt[k]) + bias);
        d = d < dt_min ? dt_min : d;  // comparisons keep a NaN a NaN
        d = d > dt_max ? dt_max : d;
      }
      dv[k] = d;
      run += d * Ah;
      cum[k] = run;
    }
    const float incl = wave_incl_sum(run);
    const float base = incl - run;
    cum[0] += base;
    cum[1] += base;
    const float cum_last = wave_read(incl, kWave - 1);
    int ks[2] = {0, 0};
    if (seq) {
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int64_t t = t0 + 2 * lane + k;
        if (t >= 1 && t < L) cnt += seq[b * L + t] != seq[b * L + t - 1];
        ks[k] = cnt;
      }
      const int ic = wave_incl_sum(cnt);
      ks[0] += ic - cnt;
      ks[1] += ic - cnt;
    }
    const int klast = wave_read(ks[1], kWave - 1);
    // reference step r = 16 i - 1 of this lane's tile i = lane / 8 (tile 0 has none)
    const int ti = lane >> 3;
    const int rsrc = ti > 0 ? 8 * ti - 1 : 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = 2 * lane + k;
      if (wt == 0) {
        cum2_l[t] = cum[k] * kLog2e;
        dt_l[t] = dv[k];
        if constexpr (VARLEN) k_l[t] = ks[k];
        w_l[t] = ks[k] == klast ? __expf(cum_last - cum[k]) * dv[k] : 0.0f;
      } else if (wt == 1) {
        et_l[t] = ks[k] == 0 ? __expf(cum[k]) : 0.0f;
      } else if (wt == 2) {
        const float cref = __shfl(cum[1], rsrc, kWave);
        const int kref = __shfl(ks[1], rsrc, kWave);
        ett_l[t] = ti == 0 ? 1.0f : (ks[k] == kref ? __expf(cum[k] - cref) : 0.0f);
      }
    }
    // v rows: 1, 2 (wave 0), 3, 4 (wave 1), 5 (wave 2), 6, 7 (wave 3)
#pragma unroll
    for (int i = 1; i < CT; ++i) {
      const int owner = i <= 2 ? 0 : i <= 4 ? 1 : i == 5 ? 2 : 3;
      if (owner != wt) continue;
      const float ci = wave_read(cum[1], 8 * i - 1);
      const int ki = wave_read(ks[1], 8 * i - 1);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int sv = 2 * lane + k;
        if (sv < 16 * i) v_l[i * CQ + sv] = ks[k] == ki ? __expf(ci - cum[k]) * dv[k] : 0.0f;
      }
    }
    // a start inside the block drops the carried state (marked by -1)
    if (wt == 0 && lane == 0) dl_l[hd] = klast == 0 ? __expf(cum_last) : -1.0f;
  };

  // ---- state: H = exp(cum_last) H + B^T (w o x); slots t = 32 kt + 4 g + j
  // (j < 4) and 32 kt + 16 + 4 g + j - 4 ----
  auto state_update = [&]() {
    const float dlv = dl_l[hd];
    const float dl = dlv < 0.0f ? 0.0f : dlv;
#pragma unroll
    for (int j = 0; j < NT; ++j) Hs[j] *= dl;
    // x rows and w of step group kt + 1 are read while group kt is multiplied
    s16x4 xa, xb;
    f4 w0, w1;
    auto read_xw = [&](int kt) {
      const int r0 = 32 * kt + 4 * g, r1 = r0 + 16;
      xa = tr_rows(Xl, kXP, r0, 16 * wt, m);
      xb = tr_rows(Xl, kXP, r1, 16 * wt, m);
      w0 = *reinterpret_cast<const f4*>(w_l + r0);
      w1 = *reinterpret_cast<const f4*>(w_l + r1);
    };
    read_xw(0);
#pragma unroll
    for (int kt = 0; kt < CQ / 32; ++kt) {
      const int r0 = 32 * kt + 4 * g, r1 = r0 + 16;
      const float xw[8] = {to_f32((bf16_t)xa[0]) * w0[0], to_f32((bf16_t)xa[1]) * w0[1],
                           to_f32((bf16_t)xa[2]) * w0[2], to_f32((bf16_t)xa[3]) * w0[3],
                           to_f32((bf16_t)xb[0]) * w1[0], to_f32((bf16_t)xb[1]) * w1[1],
                           to_f32((bf16_t)xb[2]) * w1[2], to_f32((bf16_t)xb[3]) * w1[3]};
      s16x8 whi, wlo;
      split_bf16x8(xw, whi, wlo);
      if (kt + 1 < CQ / 32) read_xw(kt + 1);
#pragma unroll
      for (int j0 = 0; j0 < NT; j0 += 4) {  // four n-tiles at a time, as in C.H
        s16x8 bops[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          bops[q] = cat8(tr_rows(Bl, BP, r0, 16 * (j0 + q), m),
                         tr_rows(Bl, BP, r1, 16 * (j0 + q), m));
#pragma unroll
        for (int q = 0; q < 4; ++q) Hs[j0 + q] = mfma16(bops[q], whi, Hs[j0 + q]);
#pragma unroll
        for (int q = 0; q < 4; ++q) Hs[j0 + q] = mfma16(bops[q], wlo, Hs[j0 + q]);
      }
    }
  };

  prefetch(c_begin);
  load_dt(c_begin);
  tables(c_begin);

  for (int64_t c = c_begin; c < c_end; ++c) {
    // A fresh, opaque copy of the lane index each block: per-lane offsets are
    // then recomputed where they are used (a few integer ops) instead of
    // dozens of them being held in registers across the whole loop.
    {
      int t = threadIdx.x;
      asm volatile("" : "+v"(t));
      // (masked, so that index arithmetic on it is known non-negative)
      tid = t & (kChainThreads - 1); th = t & 255; lane = t & 63; g = lane >> 4; m = lane & 15;
    }
    const int64_t t0 = c * CQ;
    const int last = (int)((L - 1 - t0) < (CQ - 1) ? (L - 1 - t0) : (CQ - 1));

    // ---- stage: tiles into LDS (rows past the end arrived as zeros) ----
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int e = k * kChainThreads + tid;
      const int row = e / (N / 8), col = (e % (N / 8)) * 8;
      *reinterpret_cast<uint4*>(Bl + row * BP + col) = pb[k];
      *reinterpret_cast<uint4*>(Cl + row * CP + col) = pc[k];
    }
#pragma unroll
    for (int k = 0; k < PX; ++k) {
      const int e = k * 256 + th;
      const int row = e / 8, col = (e % 8) * 8;
      *reinterpret_cast<uint4*>(Xl + row * kXP + col) = px[k];
    }
    __syncthreads();

    // ---- next block's tiles in flight ----
    if (c + 1 < c_end) prefetch(c + 1);
    // ---- in-block part: t-tiles wt and 7 - wt of this head ----
    // G^T slots (g, j): n = 32 kn + 8 g + j.  Y^T slots (g, j): s = 32 cc +
    // 4 g + j (j < 4) and 32 cc + 16 + 4 g + j - 4, the rows of the two
    // G^T tiles that lane holds.
    // (two calls with their own accumulators: a loop over the tiles would
    // index the accumulators dynamically and put them in scratch memory)
    // (the tile's parity is a compile-time argument: one of the two tiles is
    // even, the other odd, and only an odd tile's diagonal chunk holds a tile
    // wholly below the diagonal)
    auto in_block = [&](const int i, f4 (&acc)[4], auto odd) {
      const int t = 16 * i + m;
      s16x8 cop[KN];
#pragma unroll
      for (int kn = 0; kn < KN; ++kn) cop[kn] = ld_bf16x8(Cl + t * CP + 32 * kn + 8 * g);
      const float ct2 = cum2_l[t];
      const int kt = VARLEN ? k_l[t] : 0;
      const int cl = i >> 1;  // the chunk of 32 s holding the diagonal tile
      // G^T tiles of chunk cc: s-tiles 2 cc and 2 cc + 1 (rows of the staged
      // block; the second is not used when the first holds the diagonal of
      // an even t-tile).  Both tiles' B rows are read first, so the reads are
      // in flight together: formed only when used, the second tile's reads
      // moved behind the branch and each waited alone before its product.
      auto gtiles = [&](const int cc, f4& g0, f4& g1) {
        const int s0r = 32 * cc + m, s1r = s0r + 16;
        s16x8 b0[KN], b1[KN];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) b0[kn] = ld_bf16x8(Bl + s0r * BP + 32 * kn + 8 * g);
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) b1[kn] = ld_bf16x8(Bl + s1r * BP + 32 * kn + 8 * g);
        g0 = zero4();
        g1 = zero4();
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          g0 = mfma16(b0[kn], cop[kn], g0);
          g1 = mfma16(b1[kn], cop[kn], g1);
        }
      };
      // the masked values of chunk cc times x into acc (the first product of
      // the tile starts from zero: a constant operand of the MFMA instead of
      // zeroed registers)
      auto product = [&](const int cc, const float (&mv)[8], auto first) {
        const int sa = 32 * cc + 4 * g, sb = sa + 16;
        s16x8 mhi, mlo;
        split_bf16x8(mv, mhi, mlo);
        s16x8 xo[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          xo[pt] = cat8(tr_rows(Xl, kXP, sa, 16 * pt, m), tr_rows(Xl, kXP, sb, 16 * pt, m));
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          acc[pt] = mfma16(xo[pt], mhi, decltype(first)::value ? zero4() : acc[pt]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma16(xo[pt], mlo, acc[pt]);
      };
      // chunks below the diagonal one (both s-tiles below t's tile): the
      // tabulated factors exp(cum_r - cum_s) dt_s [k_s = k_r]; the next
      // chunk's products run on the matrix cores under this chunk's masking
      f4 g0, g1;
      constexpr bool kOdd = decltype(odd)::value;
      gtiles(0, g0, g1);
      auto below = [&](const int cc, auto first) {
        f4 n0, n1;
        gtiles(cc + 1, n0, n1);
        const int sa = 32 * cc + 4 * g, sb = sa + 16;
        const f4 v0 = *reinterpret_cast<const f4*>(v_l + i * CQ + sa);
        const f4 v1 = *reinterpret_cast<const f4*>(v_l + i * CQ + sb);
        float mv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mv[r] = g0[r] * v0[r];
          mv[4 + r] = g1[r] * v1[r];
        }
        product(cc, mv, first);
        g0 = n0;
        g1 = n1;
      };
      // the diagonal chunk: the tiles so far carried exp(cum_r - cum_s), so
      // add exp(cum_t - cum_r)
      const float e = ett_l[t];
      // the diagonal s-tile itself: the direct decay, [k_s = k_t] below the
      // diagonal, D on it, zero above -- selects on flags computed without
      // branches (a short-circuit form became a branch per element)
      auto diagonal = [&](const f4& gd, const int sd, float* o) {
        const f4 cs = *reinterpret_cast<const f4*>(cum2_l + sd);
        const f4 ds = *reinterpret_cast<const f4*>(dt_l + sd);
        int4 kd = int4{0, 0, 0, 0};
        if constexpr (VARLEN) kd = *reinterpret_cast<const int4*>(k_l + sd);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ks = r == 0 ? kd.x : r == 1 ? kd.y : r == 2 ? kd.z : kd.w;
          const float v = gd[r] * fexp2(ct2 - cs[r]) * ds[r];
          const bool on = sd + r == t;
          const bool keep = ((sd + r < t) & (ks == kt)) | on;
          o[r] = keep ? (on ? v + Dh : v) : 0.0f;
        }
      };
      auto last = [&](auto first) {
        const int sa = 32 * cl + 4 * g, sb = sa + 16;
        float mv[8];
        if constexpr (kOdd) {
          // s-tile i - 1 lies wholly below t's tile: the tabulated factor
          // exp(cum_r - cum_s) dt_s [k_s = k_r] times exp(cum_t - cum_r), as
          // in the chunks before; then the diagonal tile
          const f4 v0 = *reinterpret_cast<const f4*>(v_l + i * CQ + sa);
#pragma unroll
          for (int r = 0; r < 4; ++r) mv[r] = g0[r] * v0[r] * e;
          diagonal(g1, sb, mv + 4);
        } else {
          diagonal(g0, sa, mv);
#pragma unroll
          for (int r = 4; r < 8; ++r) mv[r] = 0.0f;
        }
        product(cl, mv, first);
      };
      // the first chunk's product starts the accumulators (peeled)
      if (cl > 0) {
        below(0, std::true_type{});
        for (int cc = 1; cc < cl; ++cc) below(cc, std::false_type{});
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] *= e;
        last(std::false_type{});
      } else {
        last(std::true_type{});
      }
    };
    f4 ya0[4], ya1[4];
    const int ie = (wt & 1) ? CT - 1 - wt : wt, io = CT - 1 - ie;  // even and odd tile
    in_block(ie, ya0, std::false_type{});
    in_block(io, ya1, std::true_type{});

    // ---- C.H: rows p = 16 wt + 4 g + r of every t; slots n = 32 kn + 4 g + j
    // (j < 4) and 32 kn + 16 + 4 g + j - 4: the lane's own state registers ----
    f4 ch[CT];
#pragma unroll
    for (int i = 0; i < CT; ++i) ch[i] = zero4();
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) {
      const float hv[8] = {Hs[2 * kn][0], Hs[2 * kn][1], Hs[2 * kn][2], Hs[2 * kn][3],
                           Hs[2 * kn + 1][0], Hs[2 * kn + 1][1], Hs[2 * kn + 1][2],
                           Hs[2 * kn + 1][3]};
      s16x8 hhi, hlo;
      split_bf16x8(hv, hhi, hlo);
      // four tiles at a time: their operands first, then four independent
      // products per half (reading, hi and lo tile by tile makes one long
      // latency chain)
#pragma unroll
      for (int i0 = 0; i0 < CT; i0 += 4) {
        s16x8 cops[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = 16 * (i0 + q) + m;
          cops[q] = cat8(*reinterpret_cast<const s16x4*>(Cl + t * CP + 32 * kn + 4 * g),
                         *reinterpret_cast<const s16x4*>(Cl + t * CP + 32 * kn + 16 + 4 * g));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) ch[i0 + q] = mfma16(hhi, cops[q], ch[i0 + q]);
#pragma unroll
        for (int q = 0; q < 4; ++q) ch[i0 + q] = mfma16(hlo, cops[q], ch[i0 + q]);
      }
    }

    state_update();
    __syncthreads();  // staging tiles dead: the output tiles take their space

    // The next block's dt, then this block's z, are loaded here, once the
    // output registers are free (held from earlier, they would be spilled, and
    // the wait for a spilled value waits for every load issued before it); the
    // barrier and the table work cover their latency.
    if (c + 1 < c_end) load_dt(c + 1);
    // x, z and out rows of this head in the block: the same range
    const uint32_t nxb = (uint32_t)last * xrow + kP * 2;
    uint4 zr[PX];
    if constexpr (GATE) {
      const auto zrs = row_rsrc(z + ((b * L + t0) * H + h) * kP, nxb);
#pragma unroll
      for (int k = 0; k < PX; ++k) {
        const int e = k * 256 + th;
        const int row = e / 8, col = (e % 8) * 8;
        zr[k] = bld16(zrs, (uint32_t)row * xrow + (uint32_t)col * 2);
      }
    }

    // ---- both output parts into LDS ----
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      *reinterpret_cast<f4*>(yin + (16 * ie + m) * kYP + 16 * pt + 4 * g) = ya0[pt];
      *reinterpret_cast<f4*>(yin + (16 * io + m) * kYP + 16 * pt + 4 * g) = ya1[pt];
    }
#pragma unroll
    for (int i = 0; i < CT; ++i)
      *reinterpret_cast<f4*>(ych + (16 * i + m) * kYP + 16 * wt + 4 * g) = ch[i];
    __syncthreads();

    // exp(cum_t) of the epilogue's steps, read before the tables are refilled
    // (the epilogue applies it: one fma per output instead of a multiply per
    // C.H value)
    float etr[PX];
#pragma unroll
    for (int k = 0; k < PX; ++k) etr[k] = et_l[(k * 256 + th) / 8];
    // the tables are free until the next staging: fill them for block c + 1
    if (c + 1 < c_end) tables(c + 1);

    // ---- epilogue: 8 consecutive p of one step per thread piece ----
    const auto ors = row_rsrc(out + ((b * L + t0) * H + h) * kP, nxb);
#pragma unroll
    for (int k = 0; k < PX; ++k) {
      const int e = k * 256 + th;
      const int row = e / 8, col = (e % 8) * 8;
      const f4 y0 = *reinterpret_cast<const f4*>(yin + row * kYP + col) +
                    *reinterpret_cast<const f4*>(ych + row * kYP + col) * etr[k];
      const f4 y1 = *reinterpret_cast<const f4*>(yin + row * kYP + col + 4) +
                    *reinterpret_cast<const f4*>(ych + row * kYP + col + 4) * etr[k];
      float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      if constexpr (GATE) {
        const uint32_t zw[4] = {zr[k].x, zr[k].y, zr[k].z, zr[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          yv[2 * q] *= fsilu(bf16_lo(zw[q]));
          yv[2 * q + 1] *= fsilu(bf16_hi(zw[q]));
        }
      }
      // rows past the end fall outside the resource and are dropped
      const uint4 o = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]),
                       pack_bf16x2(yv[4], yv[5]), pack_bf16x2(yv[6], yv[7])};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, o),
                                             ors, (uint32_t)row * xrow + (uint32_t)col * 2, 0, 0);
    }
    __syncthreads();  // the output tiles are read before the next staging
  }

  if (final_states && c_end == nblk) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
      st4(final_states + ((b * H + h) * kP + pme) * N + 16 * j + 4 * g, Hs[j]);
  }
}

// ---------------------------------------------------------------------------

bool use_chain_bf16(const Problem& p) {
  return p.bf16 && p.P == kP && (p.N == 64 || p.N == 128) && p.G > 0 && p.H % p.G == 0 &&
         (p.H / p.G) % kPair == 0;
}

int64_t chain_workgroups(int64_t b, int64_t H) { return b * H / kPair; }

bool chain_fills_machine(int64_t b, int64_t H) {
  const int64_t n = chain_workgroups(b, H), rounds = (n + kChainCUs - 1) / kChainCUs;
  return n > 0 && 4 * n >= 3 * kChainCUs * rounds;
}

ChainPlan chain_plan(int64_t b, int64_t L, int64_t H, bool force) {
  ChainPlan pl;
  const int64_t npairs = chain_workgroups(b, H), nblk = (L + CQ - 1) / CQ;
  pl.nseg = 1;
  pl.span = nblk;
  if (npairs <= 0 || nblk < 2) return pl;
  // segments: as many as fill one round of the compute units (at most one
  // per block); by default when the workgroups fill the round at least 3/4,
  // or from 8 blocks on at least half of it (below that, the fused path).
  // Segments of one or two blocks measured faster than the fused per-head
  // kernel in both cases, slower with 4 blocks filling half the round.
  int64_t nseg = kChainCUs / npairs;
  if (force) {
    nseg = nseg < 2 ? 2 : nseg;
  } else {
    nseg = nseg < nblk ? nseg : nblk;
    const bool full = 4 * npairs * nseg >= 3 * kChainCUs;
    const bool half_long = nblk >= 8 && 2 * npairs * nseg >= kChainCUs;
    if (nseg < 2 || !(full || half_long)) return pl;
  }
  nseg = nseg < nblk ? nseg : nblk;
  const int64_t span = (nblk + nseg - 1) / nseg;
  pl.nseg = (nblk + span - 1) / span;
  if (pl.nseg < 2) return pl;
  pl.span = span;
  // units of the unit-state pass (one workgroup per pair of heads and unit,
  // two resident per CU): halve the span while it stays even and above 8
  // blocks and the pass has fewer than four workgroups per CU, so that its
  // last, partly filled round is at most a third of it
  int64_t unit = span;
  while (unit % 2 == 0 && unit > 8 && npairs * (pl.nseg - 1) * (span / unit) < 4 * kChainCUs)
    unit /= 2;
  pl.unit = unit;
  pl.nunits = (pl.nseg - 1) * (span / unit);
  return pl;
}

template <int N>
static void launch_chain_n(const Problem& p, hipStream_t s) {
  const int64_t nblk = (p.L + CQ - 1) / CQ, npairs = chain_workgroups(p.b, p.H);
  const auto* xb = static_cast<const bf16_t*>(p.x);
  const auto* Bb = static_cast<const bf16_t*>(p.B);
  const auto* Cb = static_cast<const bf16_t*>(p.C);
  const auto* db = static_cast<const bf16_t*>(p.dt);
  const auto* zb = static_cast<const bf16_t*>(p.z);
  auto* ob = static_cast<bf16_t*>(p.out);
  const ChainPlan& pl = p.chain;
  const int64_t nwg = npairs * pl.nseg;
  const int64_t ups = pl.nseg > 1 ? pl.span / pl.unit : 0;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(kChainThreads), 0, s, xb, Bb, Cb, db,
                       p.A, p.dt_bias, p.dt_min, p.dt_max, p.D, zb, ob, p.init, p.final_states,
                       p.seq_idx, p.L, p.H, p.G, nblk, nwg, npairs, pl.span, p.cs_states,
                       p.cs_decay, pl.nunits, ups);
  };
  if (p.seq_idx) {
    if (p.z) go(chain_scan_bf16_kernel<N, true, true>);
    else go(chain_scan_bf16_kernel<N, false, true>);
  } else {
    if (p.z) go(chain_scan_bf16_kernel<N, true, false>);
    else go(chain_scan_bf16_kernel<N, false, false>);
  }
}

hipError_t launch_chain_bf16(const Problem& p, hipStream_t s, int pass) {
  if (p.L <= 0 || p.b <= 0) return hipSuccess;
  if (pass == 0) return p.chain.nseg < 2 ? hipSuccess : launch_unit_state_bf16(p, s);
  if (p.N == 128)
    launch_chain_n<128>(p, s);
  else
    launch_chain_n<64>(p, s);
  return hipGetLastError();
}

}  // namespace ssd
