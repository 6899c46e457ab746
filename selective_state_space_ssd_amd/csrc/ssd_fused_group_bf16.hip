// Fused bf16 scan, group form: one workgroup per (128-step block, B/C group,
// set of up to 8 heads of that group).
//
// The heads of a group share B and C, so the workgroup stages the B tile and
// the C rows once and forms the causal products G^T = B_s C_t^T once, then
// walks its heads.  Per head it does what the per-head fused kernel does:
// dt and its running sum, the block's state contribution S, the in-block
// output (G o decay) x with the D skip, then -- once the entering state of
// that (batch, head) is published by the workgroup of the previous block --
// the leaving state, C H_in^T and the z gate.  The heads form a software
// pipeline: while head j's entering state is in flight, the state-free part
// of head j+1 is computed, so each memory round trip overlaps matrix work.
//
// Ordering and hand-off are those of the per-head fused kernel: tickets per
// class, block-major, a bounded wait on a per-(batch, head, block) flag, the
// state written with device-scope stores into a two-slot ring per (batch,
// head), flags set after the stores complete.
#include <type_traits>

#include "ssd_bf16_tiles.h"
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {
using namespace bf16t;

namespace {
constexpr int GQ = 128;        // timesteps per block
constexpr int GNT = GQ / 32;   // t-tiles per block
constexpr int kGClasses = 8;
constexpr int kMaxHeadsPerWg = 8;

template <int N>
__device__ __forceinline__ int gbswz(int r) {
  if constexpr (N == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}
template <int N>
__device__ __forceinline__ int gb_off(int r, int col) {
  return r * N + ((((col >> 3) ^ gbswz<N>(r))) << 3) + (col & 7);
}
template <int N>
__device__ __forceinline__ s16x4 gb_tr4(const bf16_t* lds, int r0, int c0) {
  const int lane = threadIdx.x % 64;
  const int m = lane % 16, half = (lane / 16) % 2;
  const bf16_t* p = lds + gb_off<N>(r0 + m / 4, c0 + 16 * half + 4 * (m % 4));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
template <int N>
__device__ __forceinline__ s16x8 gb_tr_operand(const bf16_t* lds, int r0, int r1, int c0) {
  const s16x4 a = gb_tr4<N>(lds, r0, c0), b = gb_tr4<N>(lds, r1, c0);
  s16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}
__device__ __forceinline__ float gexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float gsilu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + gexp2(-z * 1.4426950408889634f));
}
constexpr int kGSc1 = 16;  // cache policy: device scope
__device__ __forceinline__ void gst4_agent(float* slot, int slot_bytes, int byte_off, f4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(slot, 0, slot_bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                         r, byte_off, 0, kGSc1);
}
__device__ __forceinline__ void gwait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// x tile of one head, in flight: two 16-byte pieces per thread (512 threads)
struct GX {
  uint4 v[2];
};
__device__ __forceinline__ void gload_x(GX& t, const bf16_t* xs, int64_t stride, int last) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = (k * 512 + (int)threadIdx.x) * 8;
    const int row = e / kP, col = e % kP;
    t.v[k] = *reinterpret_cast<const uint4*>(xs + (row < last ? row : last) * stride + col);
  }
}
__device__ __forceinline__ void gstore_x(bf16_t* x_lds, const GX& t, int last) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = (k * 512 + (int)threadIdx.x) * 8;
    const int row = e / kP, col = e % kP;
    const uint4 v = t.v[k];
    const uint32_t m = row > last ? 0u : 0xffffffffu;
    uint2 even, odd;
    even.x = ((v.x & 0xffffu) | (v.y << 16)) & m;
    even.y = ((v.z & 0xffffu) | (v.w << 16)) & m;
    odd.x = ((v.x >> 16) | (v.y & 0xffff0000u)) & m;
    odd.y = ((v.z >> 16) | (v.w & 0xffff0000u)) & m;
    *reinterpret_cast<uint2*>(x_lds + row * kXLD + col / 2) = even;
    *reinterpret_cast<uint2*>(x_lds + row * kXLD + 32 + col / 2) = odd;
  }
}

// per-head scalars of one block, double-buffered across the head pipeline
struct GHeadLds {
  float cum2[GQ];  // running sum of dt*A, log2 units
  float dt[GQ];
  float w[GQ];     // exp(cum_last - cum_t) dt_t
  float u[GQ];     // exp(cum_end(tile of s) - cum_s) dt_s
  float dlast;     // exp(cum_last)
};
}  // namespace

template <int N, bool GATE>
__global__ __launch_bounds__(512) void fused_group_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const bf16_t* __restrict__ dt_raw, const float* __restrict__ A,
    const float* __restrict__ dt_bias, float dt_min, float dt_max, const float* __restrict__ Dv,
    const bf16_t* __restrict__ z, bf16_t* __restrict__ out, float* __restrict__ final_states,
    float* __restrict__ ring, unsigned* __restrict__ flags, unsigned* __restrict__ ctl, int64_t L,
    int64_t H, int64_t G, int64_t nblk, int64_t gpc, int nsub, int hs, int nclass,
    unsigned spin_limit) {
  static_assert(N == 64 || N == 128, "dstate 64 or 128");
  constexpr int KS = N / 16;
  __shared__ __align__(16) bf16_t x_lds[GQ * kXLD];
  __shared__ __align__(16) bf16_t b_lds[GQ * N];
  __shared__ __align__(16) float hy_lds[GQ * kP];  // entering state (hi/lo bf16), then output tile
  __shared__ __align__(16) GHeadLds hd[2];
  // G^T tiles (s-tile si <= t-tile ti) in MFMA register order: tile
  // ti (ti + 1) / 2 + si, float4 R of lane l at [tile][R][l]
  __shared__ __align__(16) f4 g_lds[GNT * (GNT + 1) / 2][4][64];
  __shared__ unsigned ticket_lds;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i = lane % 32, kk = lane / 32;

  // ---- which (block, group, head set): ticket order within the class ----
  const int cls = (int)(blockIdx.x % (unsigned)nclass);
  if (tid == 0) ticket_lds = atomicAdd(&ctl[cls], 1u);
  __syncthreads();
  const int64_t tk = __builtin_amdgcn_readfirstlane(ticket_lds);
  // tickets of a class, block-major: gpc groups (b*G + g = cls + nclass*k) times
  // nsub head sets per block index
  const int64_t per_c = gpc * nsub;
  const int64_t c = tk / per_c, r = tk % per_c;
  const int64_t gg = (r / nsub) * nclass + cls, sub = r % nsub;
  const int64_t b = gg / G, g = gg % G;
  const int64_t hpg = H / G;
  const int64_t h0 = g * hpg + sub * hs;
  const int64_t t0 = c * GQ;
  const int last = (int)((L - 1 - t0) < (GQ - 1) ? (L - 1 - t0) : (GQ - 1));
  const int64_t xs = H * kP, bs = G * N;
  const bool more = c + 1 < nblk;

  // wave roles: output t-tile yti, p-half ypt; state tile (snt, spt)
  const int yti = wave >> 1, ypt = wave & 1;
  const bool has_s = N == 128 || wave < 4;
  const int snt = wave >> 1, spt = wave & 1;

  // ---- prologue: B tile, C rows of this wave's t-tile, x and dt of head 0 ----
  constexpr int BITER = GQ * N / 8 / 512;
  uint4 bv[BITER];
  {
    const bf16_t* src = Bm + ((b * L + t0) * G + g) * N;
#pragma unroll
    for (int k = 0; k < BITER; ++k) {
      const int e = k * 512 + tid;
      const int row = e / (N / 8), chunk = e % (N / 8);
      bv[k] = *reinterpret_cast<const uint4*>(src + (row < last ? row : last) * bs + chunk * 8);
    }
  }
  s16x8 creg[KS];
  {
    const int tr = 32 * yti + i;
    const bf16_t* Cb = Cm + ((b * L + t0) * G + g) * N + (N / 2) * kk;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) creg[ks] = ld_bf16x8(Cb + (tr < last ? tr : last) * bs + 8 * ks);
    if (tr > last) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) creg[ks] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  GX xv;
  gload_x(xv, x + ((b * L + t0) * H + h0) * kP, xs, last);

  // dt / cum / w / u of head h into hd[buf] (wave 0)
  auto head_scalars = [&](int64_t h, int buf) {
    constexpr int E = GQ / kWave;
    float dtv[E], cum[E], cum_last;
    wave_dt_cumsum<bf16_t, GQ>(dt_raw, A[h], dt_bias ? dt_bias[h] : 0.0f, dt_min, dt_max, b, c, h,
                               L, H, nblk, nullptr, nullptr, dtv, cum, &cum_last);
    const float cend = __shfl(cum[1], 16 * (lane / 16) + 15, kWave);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int t = lane * E + k;
      hd[buf].cum2[t] = cum[k] * kLog2e;
      hd[buf].dt[t] = dtv[k];
      hd[buf].w[t] = __expf(cum_last - cum[k]) * dtv[k];
      hd[buf].u[t] = __expf(cend - cum[k]) * dtv[k];
    }
    if (lane == 0) hd[buf].dlast = __expf(cum_last);
  };
  if (wave == 0) head_scalars(h0, 0);
#pragma unroll
  for (int k = 0; k < BITER; ++k) {
    const int e = k * 512 + tid;
    const int row = e / (N / 8), chunk = e % (N / 8);
    *reinterpret_cast<uint4*>(b_lds + row * N + ((chunk ^ gbswz<N>(row)) << 3)) =
        row > last ? uint4{0u, 0u, 0u, 0u} : bv[k];
  }
  gstore_x(x_lds, xv, last);
  __syncthreads();

  // G^T[s][t] = B_s C_t^T for every s-tile si <= t-tile ti, once for all heads
  // (the p-half 0 wave of each t-tile); register r of lane (i, kk):
  // s = 32 si + 8 (r/4) + 4 kk + r%4, t = 32 ti + i
  if (ypt == 0) {
    for (int si = 0; si <= yti; ++si) {
      f16x gt = zero16();
      const int brw = 32 * si + i;
      const bf16_t* brow = b_lds + brw * N;
      const int bsw = gbswz<N>(brw);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        gt = mfma32x32x16(ld_bf16x8(brow + ((((N / 16) * kk + ks) ^ bsw) << 3)), creg[ks], gt);
      const int tix = yti * (yti + 1) / 2 + si;
#pragma unroll
      for (int R = 0; R < 4; ++R)
        g_lds[tix][R][lane] = f4{gt[4 * R], gt[4 * R + 1], gt[4 * R + 2], gt[4 * R + 3]};
    }
  }
  __syncthreads();

  const float* Dp = Dv;
  // the state-free part of one head: S (this wave's tile) and the in-block output
  auto head_a = [&](int64_t h, int buf, f16x& sacc, f16x& yacc) {
    const GHeadLds& s = hd[buf];
    sacc = zero16();
    if (has_s) {
#pragma unroll 2
      for (int ks = 0; ks < GQ / 16; ++ks) {
        const int r0 = 16 * ks + 8 * kk;
        const s16x8 braw = gb_tr_operand<N>(b_lds, r0, r0 + 4, 32 * snt);
        const f4 w0 = *reinterpret_cast<const f4*>(s.w + r0);
        const f4 w1 = *reinterpret_cast<const f4*>(s.w + r0 + 4);
        const uint4 bw = __builtin_bit_cast(uint4, braw);
        const float av[8] = {bf16_lo(bw.x) * w0[0], bf16_hi(bw.x) * w0[1], bf16_lo(bw.y) * w0[2],
                             bf16_hi(bw.y) * w0[3], bf16_lo(bw.z) * w1[0], bf16_hi(bw.z) * w1[1],
                             bf16_lo(bw.w) * w1[2], bf16_hi(bw.w) * w1[3]};
        s16x8 ahi, alo;
        split_bf16x8(av, ahi, alo);
        const s16x8 bop = lds_tr_operand(x_lds, kXLD, r0, r0 + 4, 32 * spt);
        sacc = mfma32x32x16(ahi, bop, sacc);
        sacc = mfma32x32x16(alo, bop, sacc);
      }
    }
    const float Dh = Dp ? Dp[h] : 0.0f;
    const float ct = s.cum2[32 * yti + i];
    yacc = zero16();
    for (int si = 0; si <= yti; ++si) {
      const int tix = yti * (yti + 1) / 2 + si;
      f16x gt;
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const f4 v = g_lds[tix][R][lane];
        gt[4 * R] = v[0]; gt[4 * R + 1] = v[1]; gt[4 * R + 2] = v[2]; gt[4 * R + 3] = v[3];
      }
      float mv[16];
      if (si < yti) {
        const float rs = gexp2(ct - s.cum2[32 * si + 31]);
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const f4 u = *reinterpret_cast<const f4*>(s.u + 32 * si + 8 * R + 4 * kk);
#pragma unroll
          for (int q = 0; q < 4; ++q) mv[4 * R + q] = gt[4 * R + q] * rs * u[q];
        }
      } else {
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const f4 cs = *reinterpret_cast<const f4*>(s.cum2 + 32 * si + 8 * R + 4 * kk);
          const f4 ds = *reinterpret_cast<const f4*>(s.dt + 32 * si + 8 * R + 4 * kk);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int sl = 8 * R + 4 * kk + q;
            const float v = gt[4 * R + q] * gexp2(ct - cs[q]) * ds[q];
            mv[4 * R + q] = sl < i ? v : (sl == i ? v + Dh : 0.0f);
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
        const s16x8 bop = lds_tr_operand(x_lds, kXLD, r0, r0 + 8, 32 * ypt);
        yacc = mfma32x32x16(mhi, bop, yacc);
        yacc = mfma32x32x16(mlo, bop, yacc);
      }
    }
  };

  f16x sacc0, yacc0, sacc1, yacc1;
  head_a(h0, 0, sacc0, yacc0);

  constexpr int EP = GQ * kP / 8 / 512;  // 16-byte output pieces per thread
  // one pipeline step: finish head j (scalars in hd[BUF], state parts in
  // sacc_j / yacc_j) and compute the state-free part of head j+1 into
  // sacc_n / yacc_n
  auto step = [&](auto bufc, int j, f16x& sacc_j, f16x& yacc_j, f16x& sacc_n, f16x& yacc_n) {
    constexpr int buf = decltype(bufc)::value;
    const int64_t h = h0 + j;
    const int64_t chain = b * H + h;
    // ---- wait for head j's entering state; start its loads ----
    __syncthreads();  // x tile and head scalars of the previous step are no longer read
    if (tid == 0) {
      const unsigned* f = flags + chain * nblk + c;
      unsigned spins = 0;
      while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > spin_limit) {
          atomicOr(&ctl[kGClasses], 1u);
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    const float* hin = ring + (chain * 2 + (c & 1)) * (kP * N);
    f4 hreg[4];
    if (has_s) {
#pragma unroll
      for (int R = 0; R < 4; ++R)
        hreg[R] = ld4(hin + state_tile_offset(2 * i + spt, 32 * snt + 8 * R + 4 * kk, N));
    }
    // ---- state-free part of head j+1 while those loads are in flight ----
    if (j + 1 < hs) {
      GX xn;
      gload_x(xn, x + ((b * L + t0) * H + h + 1) * kP, xs, last);
      if (wave == 0) head_scalars(h + 1, buf ^ 1);
      gstore_x(x_lds, xn, last);
      __syncthreads();
      head_a(h + 1, buf ^ 1, sacc_n, yacc_n);
    }
    uint4 zv[EP];
    if constexpr (GATE) {
#pragma unroll
      for (int k = 0; k < EP; ++k) {
        const int e = k * 512 + tid, row = e / 8, col = (e % 8) * 8;
        zv[k] = *reinterpret_cast<const uint4*>(
            z + ((b * L + t0 + (row < last ? row : last)) * H + h) * kP + col);
      }
    }
    // ---- leaving state of head j: publish it; entering state split into LDS ----
    {
      const float dl = hd[buf].dlast;
      float* hout = ring + (chain * 2 + ((c + 1) & 1)) * (kP * N);
      uint2* hs_hi = reinterpret_cast<uint2*>(hy_lds);
      uint2* hs_lo = hs_hi + KS * 2 * 64 * 2;
      if (has_s) {
        const int p = 2 * i + spt;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const int n0 = 32 * snt + 8 * R + 4 * kk;
          const f4 hv = hreg[R];
          f4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = dl * hv[e] + sacc_j[4 * R + e];
          if (more)
            gst4_agent(hout, kP * N * 4, 4 * state_tile_offset(p, n0, N), v);
          else if (final_states)
            st4(final_states + (chain * kP + p) * N + n0, v);
          const int rks = (n0 % (N / 2)) / 8, rlane = 32 * (n0 / (N / 2)) + i;
          const int slot = ((rks * 2 + spt) * 64 + rlane) * 2 + kk;
          const uint32_t h01 = pack_bf16x2(hv[0], hv[1]), h23 = pack_bf16x2(hv[2], hv[3]);
          hs_hi[slot] = uint2{h01, h23};
          hs_lo[slot] = uint2{pack_bf16x2(hv[0] - bf16_lo(h01), hv[1] - bf16_hi(h01)),
                              pack_bf16x2(hv[2] - bf16_lo(h23), hv[3] - bf16_hi(h23))};
        }
      }
    }
    __syncthreads();  // H_in split complete
    // ---- C H_in^T for this wave's tile, decayed, plus the in-block part ----
    float ysum[16];
    {
      const uint4* hs_hi4 = reinterpret_cast<const uint4*>(hy_lds);
      const uint4* hs_lo4 = hs_hi4 + KS * 2 * 64;
      f16x acc = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const s16x8 hhi = __builtin_bit_cast(s16x8, hs_hi4[(ks * 2 + ypt) * 64 + lane]);
        const s16x8 hlo = __builtin_bit_cast(s16x8, hs_lo4[(ks * 2 + ypt) * 64 + lane]);
        acc = mfma32x32x16(creg[ks], hhi, acc);
        acc = mfma32x32x16(creg[ks], hlo, acc);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int tl = 32 * yti + 8 * (rr / 4) + 4 * kk + (rr % 4);
        ysum[rr] = yacc_j[rr] + acc[rr] * gexp2(hd[buf].cum2[tl]);
      }
    }
    __syncthreads();  // every wave is done with the state split
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int tl = 32 * yti + 8 * (rr / 4) + 4 * kk + (rr % 4);
      hy_lds[tl * kP + 2 * i + ypt] = ysum[rr];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < EP; ++k) {
      const int e = k * 512 + tid, row = e / 8, col = (e % 8) * 8;
      const f4 y0 = *reinterpret_cast<const f4*>(hy_lds + row * kP + col);
      const f4 y1 = *reinterpret_cast<const f4*>(hy_lds + row * kP + col + 4);
      float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      if constexpr (GATE) {
        const uint32_t zw[4] = {zv[k].x, zv[k].y, zv[k].z, zv[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          yv[2 * q] *= gsilu(bf16_lo(zw[q]));
          yv[2 * q + 1] *= gsilu(bf16_hi(zw[q]));
        }
      }
      if (row <= last) {
        const uint4 o = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]),
                         pack_bf16x2(yv[4], yv[5]), pack_bf16x2(yv[6], yv[7])};
        *reinterpret_cast<uint4*>(out + ((b * L + t0 + row) * H + h) * kP + col) = o;
      }
    }
    // ---- head j's leaving state is out: tell the next block ----
    if (more) {
      gwait_vmem();
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(flags + chain * nblk + c + 1, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  for (int j = 0; j < hs; j += 2) {
    step(std::integral_constant<int, 0>{}, j, sacc0, yacc0, sacc1, yacc1);
    if (j + 1 < hs) step(std::integral_constant<int, 1>{}, j + 1, sacc1, yacc1, sacc0, yacc0);
  }
}

// ---------------------------------------------------------------------------

// Heads per workgroup: the largest divisor of heads-per-group up to 8.
int fused_group_heads(int64_t H, int64_t G) {
  const int64_t hpg = H / G;
  for (int hs = kMaxHeadsPerWg; hs > 1; --hs)
    if (hpg % hs == 0) return hs;
  return 1;
}

// Workgroups of the group kernel for this problem.
int64_t fused_group_units(const Problem& p) {
  const int64_t nblk = (p.L + GQ - 1) / GQ;
  return p.b * p.G * nblk * ((p.H / p.G) / fused_group_heads(p.H, p.G));
}

template <int N>
static void launch_group_n(const Problem& p, hipStream_t s) {
  const int64_t nblk = (p.L + GQ - 1) / GQ;
  const int hs = fused_group_heads(p.H, p.G);
  const int nsub = (int)((p.H / p.G) / hs);
  const int nclass = (p.b * p.G) % kGClasses == 0 ? kGClasses : 1;
  const int64_t gpc = p.b * p.G / nclass;
  const unsigned spin_limit = 1u << 22;
  const dim3 grid((unsigned)(p.b * p.G * nblk * nsub));
  const auto* xb = static_cast<const bf16_t*>(p.x);
  const auto* Bb = static_cast<const bf16_t*>(p.B);
  const auto* Cb = static_cast<const bf16_t*>(p.C);
  const auto* db = static_cast<const bf16_t*>(p.dt);
  const auto* zb = static_cast<const bf16_t*>(p.z);
  auto* ob = static_cast<bf16_t*>(p.out);
  if (p.z)
    hipLaunchKernelGGL((fused_group_bf16_kernel<N, true>), grid, dim3(512), 0, s, xb, Bb, Cb, db,
                       p.A, p.dt_bias, p.dt_min, p.dt_max, p.D, zb, ob, p.final_states, p.fs_ring,
                       p.fs_flags, p.fs_ctl, p.L, p.H, p.G, nblk, gpc, nsub, hs, nclass,
                       spin_limit);
  else
    hipLaunchKernelGGL((fused_group_bf16_kernel<N, false>), grid, dim3(512), 0, s, xb, Bb, Cb, db,
                       p.A, p.dt_bias, p.dt_min, p.dt_max, p.D, zb, ob, p.final_states, p.fs_ring,
                       p.fs_flags, p.fs_ctl, p.L, p.H, p.G, nblk, gpc, nsub, hs, nclass,
                       spin_limit);
}

hipError_t launch_fused_group_bf16(const Problem& p, hipStream_t s) {
  if (p.N == 128)
    launch_group_n<128>(p, s);
  else
    launch_group_n<64>(p, s);
  return hipGetLastError();
}

}  // namespace ssd
