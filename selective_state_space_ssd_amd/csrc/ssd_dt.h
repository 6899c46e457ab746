// Per-wave discretization step and in-chunk running sum (stage 1 of the scan),
// shared by the standalone dt/cumsum kernel and the chunk-state kernel that
// fuses it.
//
//   dt_t  = clamp(softplus(dt_raw_t + dt_bias_h), dt_min, dt_max)
//   cum_t = sum_{r = chunk start .. t} dt_r * A_h
//
// dt is a discretization input folded into the log-gate dt*A with A constant
// per head (flash-linear-attention PR #49, its list of differences between
// simple_gla and the mamba2_ssd kernel); dt_bias and dt_limit are arguments of
// the repro script on mamba issue #647.
#pragma once

#include "ssd_device.h"

namespace ssd {

// softplus(u) = log(1 + e^u) = max(u, 0) + log1p(e), e = exp(-|u|) in (0, 1],
// a form that neither overflows nor cancels.  log1p(e) by Goldberg's identity
// (D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, theorem 4): with w = 1 + e rounded,
// log1p(e) = log(w) * e / (w - 1), and e itself where w rounds to 1; the
// factor e / (w - 1) cancels the rounding of w.  exp, log and the reciprocal
// are the hardware's base-2 instructions.  Measured against the fp64 value
// over u in [-40, 20): within 1.9e-6 relative (the library's log1pf / expf
// form: 1.3e-7), for a tenth of the instructions.
__device__ __forceinline__ float softplus(float u) {
  constexpr float kLog2eF = 1.4426950408889634f, kLn2F = 0.6931471805599453f;
  const float e = __builtin_amdgcn_exp2f(-fabsf(u) * kLog2eF);
  const float w = 1.0f + e, d = w - 1.0f;
  const float l = d == 0.0f ? e : __builtin_amdgcn_logf(w) * kLn2F * (e * __builtin_amdgcn_rcpf(d));
  return fmaxf(u, 0.0f) + l;
}

// One wave computes dt and cum for the Q timesteps of chunk c of head h
// (batch b).  Lane l owns timesteps l*E .. l*E+E-1 (E = Q/64); it sums them
// serially and a wave-wide inclusive scan of the lane totals gives its offset.
// Steps past the sequence end get dt = 0 and dA = 0, so the chunk's last cum
// is the cum of its last real step.  Writes dt and cum to the workspace and
// returns them in dt_out / cum_out (the lane's E values) and the chunk's last
// cum in *cum_last.  ws_dt / ws_cum may be null (nothing stored).
//
// In two parts, so that a wave handling several chunks can issue every load
// first: wave_dt_load reads the lane's raw dt values (0 past the end), and
// wave_dt_scan forms the rest from them.
template <typename T, int Q>
__device__ __forceinline__ void wave_dt_load(const T* __restrict__ dt_raw, int64_t b, int64_t c,
                                             int64_t h, int64_t L, int64_t H,
                                             float (&raw)[Q / 64]) {
  constexpr int E = Q / kWave;
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t t = c * Q + (int64_t)lane * E + i;
    raw[i] = t < L ? ld1(dt_raw + (b * L + t) * H + h) : 0.0f;
  }
}

template <int Q>
__device__ __forceinline__ void wave_dt_scan(const float (&raw)[Q / 64], float a, float bias,
                                             float dt_min, float dt_max, int64_t b, int64_t c,
                                             int64_t h, int64_t L, int64_t H, int64_t nc,
                                             float* __restrict__ ws_dt,
                                             float* __restrict__ ws_cum, float (&dt_out)[Q / 64],
                                             float (&cum_out)[Q / 64], float* cum_last) {
  constexpr int E = Q / kWave;
  const int lane = threadIdx.x % kWave;
  float run[E];
  float total = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t t = c * Q + (int64_t)lane * E + i;
    float d = 0.0f;
    if (t < L) {
      d = softplus(raw[i] + bias);
      // comparisons (not fminf/fmaxf) so that a NaN input stays NaN
      d = d < dt_min ? dt_min : d;
      d = d > dt_max ? dt_max : d;
    }
    dt_out[i] = d;
    total += d * a;
    run[i] = total;
  }
  const float incl = wave_incl_sum(total);
  const float base = incl - total;
  *cum_last = wave_read(incl, kWave - 1);
  const int64_t o = ((b * H + h) * nc + c) * Q + (int64_t)lane * E;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    cum_out[i] = base + run[i];
    if (ws_dt) {
      ws_dt[o + i] = dt_out[i];
      ws_cum[o + i] = cum_out[i];
    }
  }
}

template <typename T, int Q>
__device__ __forceinline__ void wave_dt_cumsum(const T* __restrict__ dt_raw, float a, float bias,
                                               float dt_min, float dt_max, int64_t b, int64_t c,
                                               int64_t h, int64_t L, int64_t H, int64_t nc,
                                               float* __restrict__ ws_dt,
                                               float* __restrict__ ws_cum, float (&dt_out)[Q / 64],
                                               float (&cum_out)[Q / 64], float* cum_last) {
  float raw[Q / kWave];
  wave_dt_load<T, Q>(dt_raw, b, c, h, L, H, raw);
  wave_dt_scan<Q>(raw, a, bias, dt_min, dt_max, b, c, h, L, H, nc, ws_dt, ws_cum, dt_out,
                  cum_out, cum_last);
}

}  // namespace ssd
