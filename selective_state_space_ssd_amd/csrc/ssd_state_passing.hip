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
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

template <int N>
__global__ __launch_bounds__(256) void state_passing_kernel(
    const float* __restrict__ states, const float* __restrict__ ws_cum, const float* init,
    float* __restrict__ states_in, float* final_states, const int32_t* __restrict__ seg,
    int64_t H, int64_t nc, int64_t Q) {
  constexpr int PN = 64 * N;
  constexpr int U = 4;  // chunks in flight
  const int64_t h = blockIdx.y, b = blockIdx.z;
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

template <int N>
static void launch_n(const Problem& p, hipStream_t s) {
  dim3 grid((unsigned)((64 * N / 4 + 255) / 256), (unsigned)p.H, (unsigned)p.b);
  hipLaunchKernelGGL((state_passing_kernel<N>), grid, dim3(256), 0, s, p.ws_states, p.ws_cum,
                     p.init, p.ws_states_in, p.final_states, p.ws_seg, p.H, p.nc, p.Q);
}

hipError_t launch_state_passing(const Problem& p, hipStream_t stream) {
  switch (p.N) {
    case 16: launch_n<16>(p, stream); break;
    case 32: launch_n<32>(p, stream); break;
    case 64: launch_n<64>(p, stream); break;
    case 128: launch_n<128>(p, stream); break;
  }
  return hipGetLastError();
}

}  // namespace ssd
