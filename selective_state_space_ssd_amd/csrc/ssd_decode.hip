// Short sequences (decode / speculative verify): seqlen <= kDecodeMaxL steps
// of the recurrence continuing from initial_states, one workgroup per
// (batch, head), the state in registers from the first step to the last.
//
// The chunked form pays for its chunk machinery (dt/cumsum, chunk state, state
// passing, chunk scan, a workspace) on every call; for a handful of steps the
// work is the recurrence itself, bound by reading and writing the P x N fp32
// state once per call (mamba issue #488 uses the state hand-off for chunked
// prefill; serving one token at a time is the same hand-off with L = 1).
//
//   dt_t  = clamp(softplus(dt_raw_t + dt_bias_h), dt_min, dt_max)
//   h_t   = exp(dt_t A_h) h_{t-1} + dt_t x_t (outer) B_t
//   y_t   = C_t . h_t + D_h x_t,   out_t = y_t silu(z_t)
//
// Packed sequences (seq_idx): where the label changes between steps t-1 and
// t a new sequence starts and the state is reset to zero before step t.
//
// 256 threads: thread k owns row p = k / 4 and columns n in
// [(k % 4) N/4, (k % 4 + 1) N/4) of the state; the C . h_t reduction over n
// is four partial sums combined with two lane shuffles (the four threads of a
// row are consecutive lanes).  Each thread reads and writes only its own
// slice of the state, so final_states may be initial_states.
#include "ssd_dt.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {
constexpr int kDP = 64;  // headdim
}

template <typename T, int N>
__global__ __launch_bounds__(256) void decode_kernel(
    const T* __restrict__ x, const T* __restrict__ dt_raw, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dv,
    const T* __restrict__ z, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* init, T* __restrict__ out, float* fin, const int32_t* __restrict__ seq,
    int64_t L, int64_t H, int64_t G) {
  constexpr int NT = N / 4;  // state columns per thread
  const int64_t bh = blockIdx.x, b = bh / H, h = bh % H;
  const int64_t g = h / (H / G);
  const int tid = threadIdx.x, p = tid / 4, q = tid % 4;
  const int n0 = q * NT;

  float s[NT];
  const int64_t so = (bh * kDP + p) * N + n0;
  if (init) {
#pragma unroll
    for (int j = 0; j < NT; j += 4) {
      const f4 v = ld4(init + so + j);
      s[j] = v[0]; s[j + 1] = v[1]; s[j + 2] = v[2]; s[j + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NT; ++j) s[j] = 0.0f;
  }
  const float a_h = A[h], bias = dt_bias ? dt_bias[h] : 0.0f, Dh = Dv ? Dv[h] : 0.0f;

  for (int64_t t = 0; t < L; ++t) {
    if (seq && t > 0 && seq[b * L + t] != seq[b * L + t - 1]) {  // uniform per workgroup
#pragma unroll
      for (int j = 0; j < NT; ++j) s[j] = 0.0f;
    }
    float d = softplus(to_f32(dt_raw[(b * L + t) * H + h]) + bias);
    d = d < dt_min ? dt_min : d;  // comparisons, so that NaN stays NaN
    d = d > dt_max ? dt_max : d;
    const float a = __expf(d * a_h);
    const int64_t xo = ((b * L + t) * H + h) * kDP + p;
    const float xv = to_f32(x[xo]);
    const float u = d * xv;
    const T* Bt = Bm + ((b * L + t) * G + g) * N + n0;
    const T* Ct = Cm + ((b * L + t) * G + g) * N + n0;
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < NT; j += 4) {
      const f4 bv = ld4(Bt + j), cv = ld4(Ct + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[j + e] = a * s[j + e] + u * bv[e];
        y += s[j + e] * cv[e];
      }
    }
    y += __shfl_xor(y, 1, kWave);
    y += __shfl_xor(y, 2, kWave);
    if (q == 0) {
      y += Dh * xv;
      if (z) y *= silu(to_f32(z[xo]));
      if constexpr (sizeof(T) == 2)
        out[xo] = (T)f32_to_bf16_bits(y);
      else
        out[xo] = y;
    }
  }
  if (fin) {
#pragma unroll
    for (int j = 0; j < NT; j += 4) st4(fin + so + j, f4{s[j], s[j + 1], s[j + 2], s[j + 3]});
  }
}

bool use_decode(int64_t seqlen) { return seqlen <= kDecodeMaxL; }

template <typename T>
static void launch_decode_t(const Problem& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.b * p.H));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, static_cast<const T*>(p.x),
                       static_cast<const T*>(p.dt), p.A, static_cast<const T*>(p.B),
                       static_cast<const T*>(p.C), p.D, static_cast<const T*>(p.z), p.dt_bias,
                       p.dt_min, p.dt_max, p.init, static_cast<T*>(p.out), p.final_states,
                       p.seq_idx, p.L, p.H, p.G);
  };
  switch (p.N) {
    case 16: go(decode_kernel<T, 16>); break;
    case 32: go(decode_kernel<T, 32>); break;
    case 64: go(decode_kernel<T, 64>); break;
    case 128: go(decode_kernel<T, 128>); break;
  }
}

hipError_t launch_decode(const Problem& p, hipStream_t s) {
  if (p.bf16)
    launch_decode_t<bf16_t>(p, s);
  else
    launch_decode_t<float>(p, s);
  return hipGetLastError();
}

}  // namespace ssd
