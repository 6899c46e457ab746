// Block-level prologue and epilogue around the scan, as mamba issue #647's
// repro calls them through mamba_split_conv1d_scan_combined (out_proj, a dense
// GEMM, is not part of this block).
//
// Prologue (conv_split_kernel): the packed in-projection zxbcdt holds, per
// token, [z (dim) | xBC (dim + 2 G N) | dt (H)] with xBC = [x | B | C].  xBC
// goes through a causal depthwise conv of width W (zeros before the first
// step, framework Conv1d orientation: weight[c][W-1] weighs the current step)
// plus bias, then SiLU, and lands in contiguous x [b,L,H,P], B and C
// [b,L,G,N] tensors of the input dtype; dt is copied out as [b,L,H].  z stays
// in zxbcdt: only the epilogue reads it.
//
// Epilogue (gated_rmsnorm_kernel): with y the scan's output (no gate) and
// g = y * silu(z), out = g / sqrt(mean(g^2) + eps) * weight, the mean over the
// whole width (norm_groups = 1) or over each of norm_groups equal slices
// (norm_before_gate=False); without a weight, out = g.  The page's printed
// outputs differ exactly by this choice: whole width in its python reference,
// per group in its fused kernel.
//
// Both kernels are bandwidth-bound streaming passes: the prologue reads each
// xBC element once (plus a W-1 step halo per time tile) and writes it once;
// the epilogue reads y and z and writes out once, the token's g held in LDS
// between the reduction and the scaling.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {
constexpr int kConvTT = 32;  // timesteps per prologue workgroup

// SiLU with the accurate exp and an IEEE division: the prologue is
// bandwidth-bound, and its result is rounded to the input dtype, so the fewer
// ulps it is off, the rarer a rounding lands on the neighbouring bf16 value.
__device__ __forceinline__ float silu_accurate(float v) { return v / (1.0f + expf(-v)); }

// The bf16 activation of one conv output, as the exact value rounded to fp32
// and then to bf16 (nearest even both times).  The fp32 result act of
// conv = bias + sum_k w_k v_k (W fmas) and silu lies within
//   E = 1.1 W 2^-24 M + 5 2^-24 |act|,  M = |bias| + sum_k |w_k v_k|
// of the exact value (each fma rounds once; exp, the sum and the division
// add at most 5 units in the last place; silu's slope is below 1.1).  Its
// bf16 rounding can differ from the exact value's only when a bf16 rounding
// midpoint (low 16 bits 0x8000) lies within 2 E plus one fp32 unit of act:
// such rare values are recomputed in fp64, summed in the order
// sum_k w_k v_k + bias.  (Before this, about 700 of the 25 million values of
// a batch row of the 8 x 4096 block landed on the neighbouring bf16 value,
// and the gated norm turned those into 1.4e-2 of the output's 2e-2 bar.)
template <int W>
__device__ __forceinline__ uint32_t conv_silu_bf16(const float (&w)[W], const float* v, float bias,
                                                   float act, float mag) {
  const uint32_t u = __float_as_uint(act);
  const int ex = (int)((u >> 23) & 0xffu);
  if (ex == 0xff) return f32_to_bf16_bits(act);  // inf or NaN: as is
  if (ex > 23) {  // |act| >= 2^-103 (smaller ones take the fp64 path)
    const float ulp = __uint_as_float((uint32_t)(ex - 23) << 23);  // 2^(e - 23)
    const float err = 1.1f * W * 0x1p-24f * mag + 5.0f * 0x1p-24f * fabsf(act);
    const float k = (2.0f * err + ulp) / ulp + 2.0f;  // in fp32 units of act
    const int lo = (int)(u & 0xffffu);
    if (fabsf((float)(lo - 0x8000)) > k) return f32_to_bf16_bits(act);
  }
  double conv = 0.0;
#pragma unroll
  for (int i = 0; i < W; ++i) conv += (double)w[i] * (double)v[i];
  conv += (double)bias;
  const double ad = conv / (1.0 + exp(-conv));
  return f32_to_bf16_bits((float)ad);
}

template <typename T>
__device__ __forceinline__ T from_f32(float v) {
  if constexpr (sizeof(T) == 2)
    return (T)f32_to_bf16_bits(v);
  else
    return v;
}
}  // namespace

// One thread per channel (consecutive lanes: consecutive channels, so every
// load and store of a wave is one contiguous run), kConvTT timesteps per
// workgroup.  All kConvTT + W - 1 inputs of the tile are loaded first, from
// rows clamped into [0, L) and zeroed outside, so they are in flight together.
// Channels past dim + 2GN are the dt columns: copied, no conv.
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_split_kernel(
    const T* __restrict__ zx, const float* __restrict__ cw, const float* __restrict__ cb,
    T* __restrict__ xo, T* __restrict__ bo, T* __restrict__ co, T* __restrict__ dto, int64_t L,
    int64_t dim, int64_t gn, int64_t H) {
  constexpr int NV = kConvTT + W - 1;
  const int64_t nch = dim + 2 * gn;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.y * kConvTT, b = blockIdx.z;
  if (c >= nch + H) return;  // no barrier in this kernel
  const int64_t width = 2 * dim + 2 * gn + H;
  const T* src = zx + b * L * width + dim + c;  // column dim + c of row t: src[t * width]
  float v[NV];  // v[k]: step t0 - (W-1) + k
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int64_t t = t0 - (W - 1) + k;
    const int64_t tc = t < 0 ? 0 : (t < L ? t : L - 1);
    const float e = to_f32(src[tc * width]);
    v[k] = (t >= 0 && t < L) ? e : 0.0f;
  }
  T* dst;
  int64_t stride;
  if (c >= nch) {  // dt column h = c - nch: copied
    dst = dto + b * L * H + (c - nch);
#pragma unroll
    for (int j = 0; j < kConvTT; ++j)
      if (t0 + j < L) dst[(t0 + j) * H] = from_f32<T>(v[j + W - 1]);
    return;
  }
  if (c < dim) {
    dst = xo + b * L * dim + c;
    stride = dim;
  } else if (c < dim + gn) {
    dst = bo + b * L * gn + (c - dim);
    stride = gn;
  } else {
    dst = co + b * L * gn + (c - dim - gn);
    stride = gn;
  }
  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = cw[c * W + k];
  const float bias = cb ? cb[c] : 0.0f;
#pragma unroll
  for (int j = 0; j < kConvTT; ++j) {
    float acc = bias, mag = fabsf(bias);
#pragma unroll
    for (int k = 0; k < W; ++k) {
      acc = fmaf(w[k], v[j + k], acc);
      mag = fmaf(fabsf(w[k]), fabsf(v[j + k]), mag);
    }
    if (t0 + j < L) {
      if constexpr (sizeof(T) == 2)
        dst[(t0 + j) * stride] = (T)conv_silu_bf16<W>(w, v + j, bias, silu_accurate(acc), mag);
      else
        dst[(t0 + j) * stride] = silu_accurate(acc);
    }
  }
}

// One workgroup per token: g = y * silu(z) into LDS, one wave per norm slice
// (looping) sums g^2, then every thread scales its channels.  y may be out
// (in place): the row is read completely before the first write.  dim is a
// multiple of 64 (headdim 64), so y, out and weight rows take 4-element
// accesses; z does too when its rows are aligned (VZ).
template <typename T, bool VZ>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(
    const T* y, const T* __restrict__ zx, const float* __restrict__ weight, float eps,
    T* out, int64_t dim, int64_t width, int norm_groups) {
  extern __shared__ __align__(16) float norm_lds[];  // dim floats of g, then the scales
  f4* g4 = reinterpret_cast<f4*>(norm_lds);
  float* g_lds = norm_lds;
  float* inv_lds = norm_lds + dim;
  const int64_t row = blockIdx.x;  // b * L + t
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const T* yr = y + row * dim;
  const T* zr = zx + row * width;  // z = the first dim columns of the row
  for (int64_t c = 4 * tid; c < dim; c += 1024) {
    const f4 yv = ld4(yr + c);
    f4 zv;
    if constexpr (VZ) {
      zv = ld4(zr + c);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) zv[e] = to_f32(zr[c + e]);
    }
    f4 g;
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = yv[e] * silu(zv[e]);
    g4[c / 4] = g;
  }
  T* orow = out + row * dim;
  __syncthreads();
  if (!weight) {  // uniform: the gate alone
    for (int64_t c = 4 * tid; c < dim; c += 1024) st4(orow + c, g4[c / 4]);
    return;
  }
  const int64_t gs = dim / norm_groups;
  for (int k = wave; k < norm_groups; k += 256 / kWave) {
    float s = 0.0f;
    for (int64_t c = k * gs + lane; c < (k + 1) * gs; c += kWave) s += g_lds[c] * g_lds[c];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    if (lane == 0) inv_lds[k] = rsqrtf(s / (float)gs + eps);
  }
  __syncthreads();
  for (int64_t c = 4 * tid; c < dim; c += 1024) {
    const f4 g = g4[c / 4];
    const f4 wv = ld4(weight + c);
    const float inv = inv_lds[c / gs];  // the scale of all four when gs % 4 == 0
    f4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = g[e] * (gs % 4 == 0 ? inv : inv_lds[(c + e) / gs]) * wv[e];
    st4(orow + c, o);
  }
}

bool block_supported(int64_t dim, int norm_groups, int conv_width) {
  return conv_width >= 2 && conv_width <= 4 && dim <= kNormMaxDim && norm_groups >= 1 &&
         norm_groups <= kNormMaxGroups && dim % norm_groups == 0;
}

template <typename T>
static void launch_conv_t(const BlockProblem& q, hipStream_t s) {
  const int64_t dim = q.H * q.P, gn = q.G * q.N;
  const dim3 grid((unsigned)((dim + 2 * gn + q.H + 255) / 256), (unsigned)((q.L + kConvTT - 1) / kConvTT),
                  (unsigned)q.b);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, static_cast<const T*>(q.zxbcdt), q.conv_w,
                       q.conv_b, static_cast<T*>(q.x), static_cast<T*>(q.B), static_cast<T*>(q.C),
                       static_cast<T*>(q.dt), q.L, dim, gn, q.H);
  };
  switch (q.W) {
    case 2: go(conv_split_kernel<T, 2>); break;
    case 3: go(conv_split_kernel<T, 3>); break;
    case 4: go(conv_split_kernel<T, 4>); break;
  }
}

hipError_t launch_conv_split(const BlockProblem& q, hipStream_t s) {
  if (q.bf16)
    launch_conv_t<bf16_t>(q, s);
  else
    launch_conv_t<float>(q, s);
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const BlockProblem& q, hipStream_t s) {
  const int64_t dim = q.H * q.P, width = 2 * dim + 2 * q.G * q.N + q.H;
  const dim3 grid((unsigned)(q.b * q.L));
  const size_t lds = (size_t)(dim + q.norm_groups) * sizeof(float);
  const size_t es = q.bf16 ? 2 : 4;
  // z rows start every width elements from zxbcdt: 4-element loads need every
  // row start 4-element aligned (4 * es bytes)
  const bool vz = (width % 4 == 0) && (reinterpret_cast<uintptr_t>(q.zxbcdt) % (4 * es) == 0);
  auto go = [&](auto kern, auto tp) {
    using T = decltype(tp);
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, static_cast<const T*>(q.y),
                       static_cast<const T*>(q.zxbcdt), q.norm_w, q.eps, static_cast<T*>(q.out),
                       dim, width, q.norm_groups);
  };
  if (q.bf16) {
    if (vz)
      go(gated_rmsnorm_kernel<bf16_t, true>, bf16_t{});
    else
      go(gated_rmsnorm_kernel<bf16_t, false>, bf16_t{});
  } else {
    if (vz)
      go(gated_rmsnorm_kernel<float, true>, 0.0f);
    else
      go(gated_rmsnorm_kernel<float, false>, 0.0f);
  }
  return hipGetLastError();
}

}  // namespace ssd
