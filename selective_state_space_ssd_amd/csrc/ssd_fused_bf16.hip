// Fused bf16 scan: all stages of the chunked scan in one kernel, with the
// state handed from chunk to chunk through a two-slot ring in memory.
//
// One workgroup handles one block of 128 timesteps of one (batch, head)
// "chain".  Everything that does not depend on the state entering the block
// runs first: dt and its running sum (stage 1), the block's own state
// contribution S = B^T diag(w) x with w_t = exp(cum_last - cum_t) dt_t
// (stage 2), and the in-block output (C B^T o L) x with the D skip on the
// diagonal (the diagonal part of stage 4).  Then the workgroup waits for the
// entering state H_in of its chain, copies it to LDS, publishes the leaving
// state exp(cum_last) H_in + S for the next block (stage 3, one link of the
// inter-chunk recurrence), and finishes the output with C H_in^T scaled by
// exp(cum_t) and the z gate (stage 5).  The states never make a round trip
// through HBM: each chain's ring is 64 KB and stays in the caches.
//
// The block length is 128 whatever chunk size the caller names: the chunked
// form gives the same result for any block length up to rounding, and 128
// keeps the LDS footprint at two workgroups per CU and the causal C B^T
// work per token at half that of 256.
//
// Ordering: a workgroup takes a ticket from a per-class counter when it
// starts and handles the block that ticket names, block-major, so the block
// it waits for always belongs to a workgroup that started earlier (resident
// or finished).  No workgroup can wait on one that has not started, whatever
// order the hardware dispatches in.  Classes (blockIdx % 8) partition the
// chains group by group, so the heads that share B and C run on the same XCD
// when workgroups are dealt round-robin to the XCDs.  The wait is bounded:
// past the limit the workgroup records an error word and carries on.
//
// Packed sequences (seq_idx): wave 0 counts the sequence starts k_t from the
// block's first step to t alongside dt; the masks ride on the per-step
// factors already held in LDS -- w_t (only the block's last sequence reaches
// its end state), u_s and the per-lane decay of an s-tile (pairs of one
// sequence; k is monotone in t, so [k_s = k_t] = [k_s = k_e][k_e = k_t] for
// the tile's last step e), exp(cum_t) (only the first sequence sees the
// entering state) -- plus a compare on the diagonal tile, and a block with a
// start drops the carried state.
//
// Operand precision as in the staged bf16 kernels: x, B, C enter the matrix
// cores as they are; the decay-weighted B^T, the entering state and the
// decay-masked C B^T values are split into hi/lo bf16 pairs.
#include "ssd_bf16_tiles.h"
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {
using namespace bf16t;

namespace {
constexpr int FQ = 128;           // timesteps per block
constexpr int FNT = FQ / 32;      // t-tiles per block
constexpr int kClasses = 8;

// The B tile sits in LDS unpadded (N bf16 per row) with its 16-byte chunks
// XOR-swizzled by row, so that both the row reads of C.B^T (lanes on
// consecutive rows) and the transposed reads of the state product (lanes on
// four rows, two chunks) land on distinct banks.
template <int N>
__device__ __forceinline__ int bswz(int r) {
  if constexpr (N == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}
template <int N>
__device__ __forceinline__ int b_off(int r, int col) {  // element offset of (r, col)
  return r * N + ((((col >> 3) ^ bswz<N>(r))) << 3) + (col & 7);
}

// Transposed read of the swizzled B tile (see lds_tr4): lane l receives
// B[r0 + 0..3][c0 + l%32].
template <int N>
__device__ __forceinline__ s16x4 b_tr4(const bf16_t* lds, int r0, int c0) {
  const int lane = threadIdx.x % 64;
  const int m = lane % 16, half = (lane / 16) % 2;
  const bf16_t* p = lds + b_off<N>(r0 + m / 4, c0 + 16 * half + 4 * (m % 4));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
template <int N>
__device__ __forceinline__ s16x8 b_tr_operand(const bf16_t* lds, int r0, int r1, int c0) {
  const s16x4 a = b_tr4<N>(lds, r0, c0), b = b_tr4<N>(lds, r1, c0);
  s16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// The x tile sits in LDS unpadded (64 bf16 per row, columns permuted as in
// stage_x_tile) with 16-byte chunk j of row r at j ^ (r & 2): the four rows of
// a transposed read then land on distinct banks.
__device__ __forceinline__ int x_off(int r, int col) {
  return r * kP + ((((col >> 3) ^ (r & 2))) << 3) + (col & 7);
}
__device__ __forceinline__ s16x4 x_tr4(const bf16_t* lds, int r0, int c0) {
  const int lane = threadIdx.x % 64;
  const int m = lane % 16, half = (lane / 16) % 2;
  const bf16_t* p = lds + x_off(r0 + m / 4, c0 + 16 * half + 4 * (m % 4));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
// B operand from the x tile: lane l gets x rows {r0 + 0..3} and {r1 + 0..3} of
// LDS column c0 + l%32.
__device__ __forceinline__ s16x8 x_tr_operand(const bf16_t* lds, int r0, int r1, int c0) {
  const s16x4 a = x_tr4(lds, r0, c0), b = x_tr4(lds, r1, c0);
  s16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// 2^x with v_exp_f32 (results below the normal range flush to zero).
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
// z * sigmoid(z) with v_exp_f32 and v_rcp_f32.
__device__ __forceinline__ float fsilu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + fexp2(-z * 1.4426950408889634f));
}

// Four fp32 stored with device (agent) scope (cache policy sc1) in one
// 16-byte buffer store: written through to the memory side rather than held
// in this XCD's L2.  `slot` is wave-uniform; `byte_off` < slot_bytes.
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ void st4_agent(float* slot, int slot_bytes, int byte_off, f4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(slot, 0, slot_bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                         r, byte_off, 0, kCachePolicySc1);
}

// 16 bytes read with system-scope coherence (sc0 sc1): past this CU's L1 and
// this XCD's L2, from the memory side where the producer's write-through
// stores landed.  Reading the entering state this way replaces an agent-scope
// acquire, which would invalidate the whole L2 of the XCD (the B, C and x
// tiles other workgroups there are about to reuse) on every hand-off.
constexpr int kCachePolicySc0 = 1;
__device__ __forceinline__ f4 ld4_agent(const float* slot, int slot_bytes, int byte_off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(slot), 0, slot_bytes, 0x00020000);
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0,
                                                                      kCachePolicySc0 | kCachePolicySc1));
}

// s_waitcnt vmcnt(0): this wave's vector memory operations, stores included,
// have completed (gfx9 encoding: vmcnt 0, expcnt and lgkmcnt at their maxima).
__device__ __forceinline__ void wait_vmem_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
struct FusedLds {
  static constexpr int kX = FQ * kP;              // x tile (bf16, swizzled)
  static constexpr int kB = FQ * N;               // B tile (bf16)
  static constexpr int kH = kP * N * 2;           // entering state, hi/lo bf16
  static constexpr int kY = FQ * kP * 2;          // output tile, fp32
  static constexpr int kBH = kB > kH ? (kB > kY ? kB : kY) : (kH > kY ? kH : kY);
};
}  // namespace

// Zeroes the tickets and flags of one call, writes each chain's entering
// state (initial_states or zero) into ring slot 0 in the tiled layout and
// marks block 0 of every chain ready.
template <int N>
__global__ __launch_bounds__(256) void fused_prep_kernel(const float* __restrict__ init,
                                                         float* __restrict__ ring,
                                                         unsigned* __restrict__ flags,
                                                         unsigned* __restrict__ ctl, int64_t nchain,
                                                         int64_t nblk) {
  const int64_t chain = blockIdx.x;
  const int tid = threadIdx.x;
  float* slot = ring + chain * 2 * (kP * N);
  for (int e = tid; e < kP * N / 4; e += 256) {
    // tiled float4 index e -> (p, n0): e = (q*2 + p%2)*64 + 32*k + p/2
    const int lane = e % 64, pj = (e / 64) % 2, q = e / 128;
    const int p = 2 * (lane % 32) + pj, n0 = (N / 2) * (lane / 32) + 4 * q;
    f4 v = init ? ld4(init + (chain * kP + p) * N + n0) : f4{0.f, 0.f, 0.f, 0.f};
    st4(slot + 4 * e, v);
  }
  for (int64_t c = tid; c < nblk; c += 256) flags[chain * nblk + c] = c == 0 ? 1u : 0u;
  if (chain == 0 && tid < kClasses + 1) ctl[tid] = 0u;  // tickets, then the error word
}

template <int N, bool GATE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void fused_scan_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const bf16_t* __restrict__ dt_raw, const float* __restrict__ A,
    const float* __restrict__ dt_bias, float dt_min, float dt_max, const float* __restrict__ Dv,
    const bf16_t* __restrict__ z, bf16_t* __restrict__ out, float* __restrict__ final_states,
    float* __restrict__ ring, unsigned* __restrict__ flags, unsigned* __restrict__ ctl,
    const int32_t* __restrict__ seq, int64_t L, int64_t H, int64_t G, int64_t nblk,
    int64_t nchain, int nclass, unsigned spin_limit) {
  static_assert(N == 64 || N == 128, "dstate 64 or 128");
  constexpr int KS = N / 16;                // k-steps over n
  constexpr int NPT = N == 128 ? 2 : 1;     // p-halves of the block state per wave
  using Lds = FusedLds<N>;
  __shared__ __align__(16) bf16_t x_lds[Lds::kX];
  __shared__ __align__(16) bf16_t bh_lds[Lds::kBH];  // B tile, then the entering state (hi/lo)
  __shared__ __align__(16) float cum2_lds[FQ];        // running sum of dt*A, log2 units
  __shared__ __align__(16) float dt_lds[FQ];
  __shared__ __align__(16) float w_lds[FQ];           // exp(cum_last - cum_t) dt_t
  __shared__ __align__(16) float u_lds[FQ];           // exp(cum_end(tile of s) - cum_s) dt_s
  __shared__ __align__(16) float et_lds[FQ];          // exp(cum_t)
  __shared__ __align__(16) int32_t kseq_lds[FQ];      // sequence starts from the block start
  __shared__ float dlast_lds;
  __shared__ unsigned ticket_lds;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i = lane % 32, kk = lane / 32;

  // ---- which block: ticket order within this workgroup's class ----
  const int cls = (int)(blockIdx.x % (unsigned)nclass);
  if (tid == 0) ticket_lds = atomicAdd(&ctl[cls], 1u);
  __syncthreads();
  const int64_t tk = __builtin_amdgcn_readfirstlane(ticket_lds);  // uniform: scalar index math
  const int64_t cpc = nchain / nclass;  // chains per class
  const int64_t c = tk / cpc, jj = tk % cpc;
  const int64_t hpg = H / G;
  const int64_t gg = (jj / hpg) * nclass + cls;  // b*G + g
  const int64_t b = gg / G, g = gg % G, h = g * hpg + jj % hpg;
  const int64_t chain = b * H + h;
  const int64_t t0 = c * FQ;
  const int last = (int)((L - 1 - t0) < (FQ - 1) ? (L - 1 - t0) : (FQ - 1));
  const int64_t xs = H * kP, bs = G * N;

  // ---- phase A: everything that does not need the entering state ----
  XTile<FQ> xt;
  RowTile<FQ, N> bt;
  load_x_tile<FQ>(xt, x + ((b * L + t0) * H + h) * kP, xs, last);
  load_rows<FQ, N>(bt, Bm + ((b * L + t0) * G + g) * N, bs, last);
  if (wave == 0) {
    constexpr int E = FQ / kWave;
    static_assert(E == 2, "two timesteps per lane");
    float dtv[E], cum[E], cum_last;
    wave_dt_cumsum<bf16_t, FQ>(dt_raw, A[h], dt_bias ? dt_bias[h] : 0.0f, dt_min, dt_max, b, c, h,
                               L, H, nblk, nullptr, nullptr, dtv, cum, &cum_last);
    // lane l holds t = 2l, 2l + 1; the last step of its 32-step tile is lane 16 (l/16) + 15
    const float cend = __shfl(cum[1], 16 * (lane / 16) + 15, kWave);
    // packed sequences: running count of starts over the block (0 without seq)
    int ks[E] = {0, 0};
    if (seq) {
      int run = 0;
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const int64_t tt = t0 + lane * E + k;
        if (tt >= 1 && tt < L) run += seq[b * L + tt] != seq[b * L + tt - 1];
        ks[k] = run;
      }
      const int incl = wave_incl_sum(run);
#pragma unroll
      for (int k = 0; k < E; ++k) ks[k] += incl - run;
    }
    const int kend = __shfl(ks[1], 16 * (lane / 16) + 15, kWave);
    const int klast = wave_read(ks[1], kWave - 1);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int t = lane * E + k;
      cum2_lds[t] = cum[k] * kLog2e;
      dt_lds[t] = dtv[k];
      w_lds[t] = ks[k] == klast ? __expf(cum_last - cum[k]) * dtv[k] : 0.0f;
      u_lds[t] = ks[k] == kend ? __expf(cend - cum[k]) * dtv[k] : 0.0f;
      et_lds[t] = ks[k] == 0 ? __expf(cum[k]) : 0.0f;
      kseq_lds[t] = ks[k];
    }
    // a start inside the block drops the carried state (marked by -1)
    if (lane == 0) dlast_lds = klast == 0 ? __expf(cum_last) : -1.0f;
  }
#pragma unroll
  for (int k = 0; k < XTile<FQ>::ITER; ++k) {  // x tile, permuted columns, swizzled chunks
    const int e = (k * 256 + tid) * 8;
    const int row = e / kP, col = e % kP;
    const uint4 v = xt.v[k];
    const uint32_t m = row > last ? 0u : 0xffffffffu;
    const uint2 even = {((v.x & 0xffffu) | (v.y << 16)) & m, ((v.z & 0xffffu) | (v.w << 16)) & m};
    const uint2 odd = {((v.x >> 16) | (v.y & 0xffff0000u)) & m, ((v.z >> 16) | (v.w & 0xffff0000u)) & m};
    *reinterpret_cast<uint2*>(x_lds + x_off(row, col / 2)) = even;
    *reinterpret_cast<uint2*>(x_lds + x_off(row, 32 + col / 2)) = odd;
  }
#pragma unroll
  for (int k = 0; k < RowTile<FQ, N>::ITER; ++k) {  // B tile, swizzled chunks
    const int e = k * 256 + tid;
    const int row = e / (N / 8), chunk = e % (N / 8);
    *reinterpret_cast<uint4*>(bh_lds + row * N + ((chunk ^ bswz<N>(row)) << 3)) =
        row > last ? uint4{0u, 0u, 0u, 0u} : bt.v[k];
  }
  __syncthreads();

  // in-block output: wave w owns p-half pt = w%2 of t-tiles {3 - w/2, w/2};
  // each (t-tile, s-tile <= t-tile) product G^T = B_s C_t^T is formed by the
  // two waves of that t-tile (one per p-half).  Contraction index n of lane
  // (i, kk) at step ks: (N/2) kk + 8 ks + 0..7, the same in C.H_in^T below.
  // Decay of an s-tile below the diagonal, split at the tile's last step e:
  // exp(cum_t - cum_s) dt_s = exp(cum_t - cum_e) * u_s, both factors <= 1.
  const int ypt = wave % 2, ya = wave / 2;
  const int ti0 = FNT - 1 - ya, ti1 = ya;
  const bf16_t* Cb = Cm + ((b * L + t0) * G + g) * N + (N / 2) * kk;
  const float Dh = Dv ? Dv[h] : 0.0f;
  f16x yacc[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ti = jt == 0 ? ti0 : ti1;
    s16x8 creg[KS];
    {
      const int tr = 32 * ti + i;
      const int r = tr < last ? tr : last;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        creg[ks] = ld_bf16x8(Cb + r * bs + 8 * ks);
        if (tr > last) creg[ks] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    const float ct = cum2_lds[32 * ti + i];
    const int kt = kseq_lds[32 * ti + i];
    f16x acc = zero16();
    for (int si = 0; si <= ti; ++si) {
      f16x gt = zero16();
      const int brw = 32 * si + i;
      const bf16_t* brow = bh_lds + brw * N;
      const int bsw = bswz<N>(brw);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)  // B[s][(N/2) kk + 8 ks + 0..7]: chunk (N/16) kk + ks
        gt = mfma32x32x16(ld_bf16x8(brow + ((((N / 16) * kk + ks) ^ bsw) << 3)), creg[ks], gt);
      // register r: s = 32 si + 8 (r/4) + 4 kk + r%4, t = 32 ti + i
      float mv[16];
      if (si < ti) {
        const float rs = kt == kseq_lds[32 * si + 31] ? fexp2(ct - cum2_lds[32 * si + 31]) : 0.0f;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const f4 u = *reinterpret_cast<const f4*>(u_lds + 32 * si + 8 * R + 4 * kk);
#pragma unroll
          for (int q = 0; q < 4; ++q) mv[4 * R + q] = gt[4 * R + q] * rs * u[q];
        }
      } else {
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const f4 cs = *reinterpret_cast<const f4*>(cum2_lds + 32 * si + 8 * R + 4 * kk);
          const f4 ds = *reinterpret_cast<const f4*>(dt_lds + 32 * si + 8 * R + 4 * kk);
          const int4 k4 = *reinterpret_cast<const int4*>(kseq_lds + 32 * si + 8 * R + 4 * kk);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int sl = 8 * R + 4 * kk + q;
            const int kq = q == 0 ? k4.x : q == 1 ? k4.y : q == 2 ? k4.z : k4.w;
            const float v = gt[4 * R + q] * fexp2(ct - cs[q]) * ds[q];
            mv[4 * R + q] = sl < i ? (kq == kt ? v : 0.0f) : (sl == i ? v + Dh : 0.0f);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float mm[8] = {mv[8 * m], mv[8 * m + 1], mv[8 * m + 2], mv[8 * m + 3],
                             mv[8 * m + 4], mv[8 * m + 5], mv[8 * m + 6], mv[8 * m + 7]};
        s16x8 mhi, mlo;
        split_bf16x8(mm, mhi, mlo);
        const int r0 = 32 * si + 16 * m + 4 * kk;
        const s16x8 bop = x_tr_operand(x_lds, r0, r0 + 8, 32 * ypt);
        acc = mfma32x32x16(mhi, bop, acc);
        acc = mfma32x32x16(mlo, bop, acc);
      }
    }
    yacc[jt] = acc;
  }

  // block state contribution S^T[n][p] = sum_t B[t][n] w_t x[t][p]; wave w
  // owns n-tile w (N = 128, both p-halves) or n-tile w/2, p-half w%2 (N = 64)
  const int snt = N == 128 ? wave : wave / 2;
  const int spt0 = N == 128 ? 0 : wave % 2;
  f16x sacc[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) sacc[j] = zero16();
#pragma unroll 2
  for (int ks = 0; ks < FQ / 16; ++ks) {
    const int r0 = 16 * ks + 8 * kk;
    const s16x8 braw = b_tr_operand<N>(bh_lds, r0, r0 + 4, 32 * snt);
    const f4 w0 = *reinterpret_cast<const f4*>(w_lds + r0);
    const f4 w1 = *reinterpret_cast<const f4*>(w_lds + r0 + 4);
    const uint4 bw = __builtin_bit_cast(uint4, braw);
    const float av[8] = {bf16_lo(bw.x) * w0[0], bf16_hi(bw.x) * w0[1], bf16_lo(bw.y) * w0[2],
                         bf16_hi(bw.y) * w0[3], bf16_lo(bw.z) * w1[0], bf16_hi(bw.z) * w1[1],
                         bf16_lo(bw.w) * w1[2], bf16_hi(bw.w) * w1[3]};
    s16x8 ahi, alo;
    split_bf16x8(av, ahi, alo);
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const s16x8 bop = x_tr_operand(x_lds, r0, r0 + 4, 32 * (spt0 + j));
      sacc[j] = mfma32x32x16(ahi, bop, sacc[j]);
      sacc[j] = mfma32x32x16(alo, bop, sacc[j]);
    }
  }

  // ---- phase B: the entering state ----
  __syncthreads();  // B tile no longer read; its space takes the state
  if (tid == 0) {
    const unsigned* f = flags + chain * nblk + c;
    unsigned spins = 0;
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > spin_limit) {
        atomicOr(&ctl[kClasses], 1u);
        break;
      }
    }
  }
  // the barrier orders every wave's state loads after thread 0 saw the flag;
  // the loads themselves bypass the caches (ld4_agent)
  __syncthreads();

  // Each thread loads the entering state at the elements of its own S tiles,
  // publishes exp(cum_last) H_in + S there, and leaves H_in split into hi/lo
  // bf16 in LDS in the operand order of C.H_in^T:
  //   hsplit[half][(ks*2 + pt)*64 + lane] = 8 bf16 of H[2 (lane%32) + pt][(N/2)(lane/32) + 8 ks + 0..7]
  const float* hin = ring + (chain * 2 + (c & 1)) * (kP * N);
  f4 hreg[NPT][4];
#pragma unroll
  for (int j = 0; j < NPT; ++j)
#pragma unroll
    for (int R = 0; R < 4; ++R)
      hreg[j][R] = ld4_agent(hin, kP * N * 4,
                             4 * state_tile_offset(2 * i + spt0 + j, 32 * snt + 8 * R + 4 * kk, N));
  // C rows 64..127 of the block (t-tiles 2 and 3, i.e. ti0 of every wave;
  // ti1's rows are still in creg) go to the x tile's space, swizzled like the
  // B tile; loads now, LDS stores after the state update
  constexpr int CITER = (FQ / 2) * N / 8 / 256;
  uint4 cv[CITER];
  {
    const bf16_t* src = Cm + ((b * L + t0) * G + g) * N;
#pragma unroll
    for (int k = 0; k < CITER; ++k) {
      const int e = k * 256 + tid;
      const int row = FQ / 2 + e / (N / 8), chunk = e % (N / 8);
      cv[k] = *reinterpret_cast<const uint4*>(src + (row < last ? row : last) * bs + chunk * 8);
    }
  }
  {
    const float dl = dlast_lds;
    const bool more = c + 1 < nblk;
    float* hout = ring + (chain * 2 + ((c + 1) & 1)) * (kP * N);
    uint2* hs_hi = reinterpret_cast<uint2*>(bh_lds);
    uint2* hs_lo = hs_hi + KS * 2 * 64 * 2;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int p = 2 * i + spt0 + j;
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const int n0 = 32 * snt + 8 * R + 4 * kk;
        const f4 hv = hreg[j][R];
        f4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dl < 0.0f ? sacc[j][4 * R + e] : dl * hv[e] + sacc[j][4 * R + e];
        if (more)
          st4_agent(hout, kP * N * 4, 4 * state_tile_offset(p, n0, N), v);
        else if (final_states)
          st4(final_states + (chain * kP + p) * N + n0, v);
        // operand slot of (p, n0..n0+3): ks = (n0 % (N/2)) / 8, reader lane
        // 32 (n0 / (N/2)) + i, half 4-element piece kk of the 8
        const int rks = (n0 % (N / 2)) / 8, rlane = 32 * (n0 / (N / 2)) + i;
        const int slot = ((rks * 2 + (spt0 + j)) * 64 + rlane) * 2 + kk;
        const uint32_t h01 = pack_bf16x2(hv[0], hv[1]), h23 = pack_bf16x2(hv[2], hv[3]);
        hs_hi[slot] = uint2{h01, h23};
        hs_lo[slot] = uint2{pack_bf16x2(hv[0] - bf16_lo(h01), hv[1] - bf16_hi(h01)),
                            pack_bf16x2(hv[2] - bf16_lo(h23), hv[3] - bf16_hi(h23))};
      }
    }
    // the state went out with device-scope stores (written through to the
    // memory side); waiting for them to complete makes them visible to any
    // XCD that invalidates its caches, as the consumer does after the flag
#pragma unroll
    for (int k = 0; k < CITER; ++k) {
      const int e = k * 256 + tid;
      const int row = e / (N / 8), chunk = e % (N / 8);
      *reinterpret_cast<uint4*>(x_lds + b_off<N>(row, chunk * 8)) =
          FQ / 2 + row > last ? uint4{0u, 0u, 0u, 0u} : cv[k];
    }
    if (more) wait_vmem_stores();
    __syncthreads();  // state published by every wave; H_in split and C rows in LDS
    if (more && tid == 0)
      __hip_atomic_store(flags + chain * nblk + c + 1, 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // C rows of t-tile ti1 (rows 0..63 are not in LDS)
  s16x8 creg[KS];
  {
    const int tr = 32 * ti1 + i;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) creg[ks] = ld_bf16x8(Cb + (tr < last ? tr : last) * bs + 8 * ks);
  }
  // C H_in^T, decayed from the block start, plus the in-block part
  const uint4* hs_hi4 = reinterpret_cast<const uint4*>(bh_lds);
  const uint4* hs_lo4 = hs_hi4 + KS * 2 * 64;
  float ysum[2][16];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {  // ti0 first: its C rows are in LDS already
    const int ti = jt == 0 ? ti0 : ti1;
    const int tr = 32 * ti + i;
    f16x acc = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // C[32 ti + i][(N/2) kk + 8 ks + 0..7]: registers (ti1) or the LDS copy (ti0)
      s16x8 ca = creg[ks];
      if (jt == 0)
        ca = ld_bf16x8(x_lds + b_off<N>(32 * ti - FQ / 2 + i, (N / 2) * kk + 8 * ks));
      const s16x8 cvv = tr > last ? s16x8{0, 0, 0, 0, 0, 0, 0, 0} : ca;
      const s16x8 hhi = __builtin_bit_cast(s16x8, hs_hi4[(ks * 2 + ypt) * 64 + lane]);
      const s16x8 hlo = __builtin_bit_cast(s16x8, hs_lo4[(ks * 2 + ypt) * 64 + lane]);
      acc = mfma32x32x16(cvv, hhi, acc);
      acc = mfma32x32x16(cvv, hlo, acc);
    }
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const f4 et = *reinterpret_cast<const f4*>(et_lds + 32 * ti + 8 * R + 4 * kk);
#pragma unroll
      for (int q = 0; q < 4; ++q) ysum[jt][4 * R + q] = yacc[jt][4 * R + q] + acc[4 * R + q] * et[q];
    }
  }
  // z for the coalesced epilogue: thread piece k covers row (k*256 + tid)/8,
  // columns 8 ((k*256 + tid) % 8) + 0..7 (rows clamped to the sequence)
  constexpr int EP = FQ * kP / 8 / 256;
  uint4 zv[EP];
  if constexpr (GATE) {
#pragma unroll
    for (int k = 0; k < EP; ++k) {
      const int e = k * 256 + tid, row = e / 8, col = (e % 8) * 8;
      zv[k] = *reinterpret_cast<const uint4*>(
          z + ((b * L + t0 + (row < last ? row : last)) * H + h) * kP + col);
    }
  }
  // epilogue through LDS: the fp32 output tile [t][p], then z gate and
  // 16-byte stores of eight consecutive p per thread
  __syncthreads();  // every wave is done with the state split
  float* y_lds = reinterpret_cast<float*>(bh_lds);
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ti = jt == 0 ? ti0 : ti1;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int tl = 32 * ti + 8 * (rr / 4) + 4 * kk + (rr % 4);
      y_lds[tl * kP + 2 * i + ypt] = ysum[jt][rr];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < EP; ++k) {
    const int e = k * 256 + tid, row = e / 8, col = (e % 8) * 8;
    const f4 y0 = *reinterpret_cast<const f4*>(y_lds + row * kP + col);
    const f4 y1 = *reinterpret_cast<const f4*>(y_lds + row * kP + col + 4);
    float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    if constexpr (GATE) {
      const uint32_t zw[4] = {zv[k].x, zv[k].y, zv[k].z, zv[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        yv[2 * q] *= fsilu(bf16_lo(zw[q]));
        yv[2 * q + 1] *= fsilu(bf16_hi(zw[q]));
      }
    }
    if (row <= last) {
      const uint4 o = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]),
                       pack_bf16x2(yv[4], yv[5]), pack_bf16x2(yv[6], yv[7])};
      *reinterpret_cast<uint4*>(out + ((b * L + t0 + row) * H + h) * kP + col) = o;
    }
  }
}

// ---------------------------------------------------------------------------

// Local end states of units of consecutive 128-step blocks, for the
// segmented chain path: one workgroup per (unit, batch, pair of heads of one
// group), the state recurrence alone run over the unit's blocks from a zero
// state,
//   E = sum over the unit's blocks c of P_c B_c^T (w_c o x_c),
//   w_t = exp(cum_last - cum_t) dt_t,  P_c = the product of exp(cum_last) of
//   the unit's blocks after c,
// on 32x32x16 bf16 MFMAs with E in the accumulators.  The blocks are taken
// last to first, so that P_c is a running product folded into w (one
// multiply per step, where scaling the accumulators by each block's decay
// would cost one per state element).  The pair shares the B tile; wave w
// takes head w/2 and p = 32 (w%2) .. 32 (w%2) + 31 over all n, so B^T enters
// the matrix cores as it is and only w o x (the smaller operand) is split
// into hi/lo bf16.  Rows go through buffer resources ending at the block's
// last row (rows past the sequence end load as zero).  The next block's
// tiles load while the current one is multiplied.  Outputs: E row-major
// [p][n] at seg_states[((b H + h) nunits + u) P N] and D = the product of the
// unit's exp(cum_last) (0 where a sequence starts inside a block: the
// carried state does not survive it) at seg_decay[(b H + h) nunits + u].
// Workgroups are numbered with the pairs fastest, so the pairs of a group
// (which read the same B rows) stay on one XCD.
template <int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void unit_state_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ dt_raw,
    const float* __restrict__ A, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const int32_t* __restrict__ seq, int64_t L, int64_t H, int64_t G, int64_t nblk, int64_t unit,
    int64_t nunits, int64_t npairs, int64_t nwg, float* __restrict__ seg_states,
    float* __restrict__ seg_decay) {
  static_assert(N == 64 || N == 128, "dstate 64 or 128");
  constexpr int NJ = N / 32;                // n-tiles of 32
  constexpr int XI = FQ * kP / 8 / 256;     // 16-byte pieces of one head's x tile per thread
  constexpr int BI = FQ * N / 8 / 256;      // ... of the B tile
  __shared__ __align__(16) bf16_t x_lds[2][FQ * kP];
  __shared__ __align__(16) bf16_t b_lds[FQ * N];
  __shared__ __align__(16) float w_lds[2][FQ];

  const int tid = threadIdx.x & 255, lane = tid % kWave, wave = tid / kWave;
  const int i = lane % 32, kk = lane / 32;
  const int hd = wave / 2, pt = wave % 2;  // head of the pair, half of p
  const int wi = (int)xcd_remap(blockIdx.x, nwg);
  const int64_t u = __builtin_amdgcn_readfirstlane(wi / (int)npairs);
  const int pair = __builtin_amdgcn_readfirstlane(wi % (int)npairs);
  const int hp = (int)H / 2;
  const int64_t b = __builtin_amdgcn_readfirstlane(pair / hp);
  const int64_t h0 = __builtin_amdgcn_readfirstlane(2 * (pair % hp));
  const int64_t h = h0 + hd;
  const int64_t g = __builtin_amdgcn_readfirstlane((int)h0 / ((int)H / (int)G));
  const int64_t c0 = u * unit, c1 = c0 + unit < nblk ? c0 + unit : nblk;
  const int64_t xs = H * kP, bs = G * N;
  const uint32_t xrow = (uint32_t)(xs * 2), brow = (uint32_t)(bs * 2);  // row pitches, bytes

  f16x sacc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) sacc[j] = zero16();
  float P = 1.0f;  // decay of the blocks already taken (kept by the pt == 0 waves)

  // tiles in flight: both heads' x (pieces k < XI: head 0, else head 1) and
  // the shared B tile
  uint4 xv[2 * XI], bv[BI];
  auto load = [&](int64_t c) {
    const int64_t t0 = c * FQ;
    const uint32_t last = (uint32_t)((L - 1 - t0) < (FQ - 1) ? (L - 1 - t0) : (FQ - 1));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const auto xr = row_rsrc(x + ((b * L + t0) * H + h0 + q) * kP, last * xrow + kP * 2);
#pragma unroll
      for (int k = 0; k < XI; ++k) {
        const uint32_t e = (uint32_t)(k * 256 + tid) * 8;
        xv[q * XI + k] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, (e / kP) * xrow + (e % kP) * 2, 0, 0));
      }
    }
    const auto br = row_rsrc(Bm + ((b * L + t0) * G + g) * N, last * brow + N * 2);
#pragma unroll
    for (int k = 0; k < BI; ++k) {
      const uint32_t e = (uint32_t)(k * 256 + tid);
      bv[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            br, (e / (N / 8)) * brow + (e % (N / 8)) * 16, 0, 0));
    }
  };
  load(c1 - 1);
  for (int64_t c = c1 - 1; c >= c0; --c) {
    const int64_t t0 = c * FQ;
    if (pt == 0) {  // one wave per head: dt, its running sum, w scaled by P
      constexpr int E = FQ / kWave;
      float dtv[E], cum[E], cum_last;
      wave_dt_cumsum<bf16_t, FQ>(dt_raw, A[h], dt_bias ? dt_bias[h] : 0.0f, dt_min, dt_max, b, c,
                                 h, L, H, nblk, nullptr, nullptr, dtv, cum, &cum_last);
      int ks[E] = {0, 0};
      if (seq) {
        int run = 0;
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const int64_t tt = t0 + lane * E + k;
          if (tt >= 1 && tt < L) run += seq[b * L + tt] != seq[b * L + tt - 1];
          ks[k] = run;
        }
        const int incl = wave_incl_sum(run);
#pragma unroll
        for (int k = 0; k < E; ++k) ks[k] += incl - run;
      }
      const int klast = wave_read(ks[E - 1], kWave - 1);
#pragma unroll
      for (int k = 0; k < E; ++k)
        w_lds[hd][lane * E + k] = ks[k] == klast ? __expf(cum_last - cum[k]) * dtv[k] * P : 0.0f;
      P *= klast == 0 ? __expf(cum_last) : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {  // x tiles, swizzled chunks
#pragma unroll
      for (int k = 0; k < XI; ++k) {
        const int e = (k * 256 + tid) * 8;
        *reinterpret_cast<uint4*>(x_lds[q] + x_off(e / kP, e % kP)) = xv[q * XI + k];
      }
    }
#pragma unroll
    for (int k = 0; k < BI; ++k) {  // B tile, swizzled chunks
      const int e = k * 256 + tid;
      const int row = e / (N / 8), chunk = e % (N / 8);
      *reinterpret_cast<uint4*>(b_lds + row * N + ((chunk ^ bswz<N>(row)) << 3)) = bv[k];
    }
    __syncthreads();
    if (c > c0) load(c - 1);  // the next tiles in flight under this block's products
    // x rows and w of step group ks + 1 are read while group ks is multiplied
    uint4 xw;
    f4 w0, w1;
    auto read_xw = [&](int ks) {
      const int r0 = 16 * ks + 8 * kk;
      xw = __builtin_bit_cast(uint4, x_tr_operand(x_lds[hd], r0, r0 + 4, 32 * pt));
      w0 = *reinterpret_cast<const f4*>(w_lds[hd] + r0);
      w1 = *reinterpret_cast<const f4*>(w_lds[hd] + r0 + 4);
    };
    read_xw(0);
#pragma unroll 2
    for (int ks = 0; ks < FQ / 16; ++ks) {
      const int r0 = 16 * ks + 8 * kk;
      // w o x at t = r0 + 0..7, p = 32 pt + i, split hi/lo
      const float xv8[8] = {bf16_lo(xw.x) * w0[0], bf16_hi(xw.x) * w0[1], bf16_lo(xw.y) * w0[2],
                            bf16_hi(xw.y) * w0[3], bf16_lo(xw.z) * w1[0], bf16_hi(xw.z) * w1[1],
                            bf16_lo(xw.w) * w1[2], bf16_hi(xw.w) * w1[3]};
      // every n-tile's B operand read before the products (read next to its
      // product, each read waits alone); the hi products of all tiles, then
      // the lo ones, so that consecutive MFMAs are independent
      s16x8 bop[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bop[j] = b_tr_operand<N>(b_lds, r0, r0 + 4, 32 * j);
      s16x8 xhi, xlo;
      split_bf16x8(xv8, xhi, xlo);
      if (ks + 1 < FQ / 16) read_xw(ks + 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) sacc[j] = mfma32x32x16(bop[j], xhi, sacc[j]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) sacc[j] = mfma32x32x16(bop[j], xlo, sacc[j]);
    }
    __syncthreads();  // tiles and w read before the next block is staged
  }
  // sacc[j][4 R + e] holds E at p = 32 pt + i, n = 32 j + 8 R + 4 kk + e
  const int64_t slot = (b * H + h) * nunits + u;
  const int p = 32 * pt + i;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const int n0 = 32 * j + 8 * R + 4 * kk;
      st4(seg_states + (slot * kP + p) * N + n0,
          f4{sacc[j][4 * R], sacc[j][4 * R + 1], sacc[j][4 * R + 2], sacc[j][4 * R + 3]});
    }
  }
  if (pt == 0 && lane == 0) seg_decay[slot] = P;
}

template <int N>
static void launch_unit_state_n(const Problem& p, hipStream_t s) {
  const int64_t nblk = fused_blocks(p.L), npairs = p.b * p.H / 2, nwg = npairs * p.chain.nunits;
  hipLaunchKernelGGL((unit_state_bf16_kernel<N>), dim3((unsigned)nwg), dim3(256), 0, s,
                     static_cast<const bf16_t*>(p.x), static_cast<const bf16_t*>(p.B),
                     static_cast<const bf16_t*>(p.dt), p.A, p.dt_bias, p.dt_min, p.dt_max,
                     p.seq_idx, p.L, p.H, p.G, nblk, p.chain.unit, p.chain.nunits, npairs, nwg,
                     p.cs_states, p.cs_decay);
}

hipError_t launch_unit_state_bf16(const Problem& p, hipStream_t s) {
  if (p.chain.nunits <= 0 || p.L <= 0 || p.b <= 0) return hipSuccess;
  if (p.N == 128)
    launch_unit_state_n<128>(p, s);
  else
    launch_unit_state_n<64>(p, s);
  return hipGetLastError();
}

bool use_fused_bf16(const Problem& p) {
  return p.bf16 && p.P == kP && (p.N == 64 || p.N == 128);
}

int64_t fused_blocks(int64_t L) { return (L + FQ - 1) / FQ; }

int fused_classes(int64_t b, int64_t G) { return (b * G) % kClasses == 0 ? kClasses : 1; }

template <int N>
static void launch_fused_n(const Problem& p, hipStream_t s, int stage) {
  const int64_t nblk = fused_blocks(p.L), nchain = p.b * p.H;
  if (stage == 0) {
    hipLaunchKernelGGL((fused_prep_kernel<N>), dim3((unsigned)nchain), dim3(256), 0, s, p.init,
                       p.fs_ring, p.fs_flags, p.fs_ctl, nchain, nblk);
    return;
  }
  const int nclass = fused_classes(p.b, p.G);
  const unsigned spin_limit = 1u << 22;
  const dim3 grid((unsigned)(nchain * nblk));
  const auto* xb = static_cast<const bf16_t*>(p.x);
  const auto* Bb = static_cast<const bf16_t*>(p.B);
  const auto* Cb = static_cast<const bf16_t*>(p.C);
  const auto* db = static_cast<const bf16_t*>(p.dt);
  const auto* zb = static_cast<const bf16_t*>(p.z);
  auto* ob = static_cast<bf16_t*>(p.out);
  if (p.z)
    hipLaunchKernelGGL((fused_scan_bf16_kernel<N, true>), grid, dim3(256), 0, s, xb, Bb, Cb, db,
                       p.A, p.dt_bias, p.dt_min, p.dt_max, p.D, zb, ob, p.final_states, p.fs_ring,
                       p.fs_flags, p.fs_ctl, p.seq_idx, p.L, p.H, p.G, nblk, nchain, nclass,
                       spin_limit);
  else
    hipLaunchKernelGGL((fused_scan_bf16_kernel<N, false>), grid, dim3(256), 0, s, xb, Bb, Cb, db,
                       p.A, p.dt_bias, p.dt_min, p.dt_max, p.D, zb, ob, p.final_states, p.fs_ring,
                       p.fs_flags, p.fs_ctl, p.seq_idx, p.L, p.H, p.G, nblk, nchain, nclass,
                       spin_limit);
}

hipError_t launch_fused_bf16(const Problem& p, hipStream_t s, int stage) {
  // the group kernel runs only when asked for: on the measured workloads the
  // per-head kernel is faster (its workgroups hide each other's latency); it
  // does not take packed sequences
  const bool group = stage == 1 && p.fused_kind == 2 && !p.seq_idx;
  if (group) return launch_fused_group_bf16(p, s);
  if (p.N == 128)
    launch_fused_n<128>(p, s, stage);
  else
    launch_fused_n<64>(p, s, stage);
  return hipGetLastError();
}

}  // namespace ssd
