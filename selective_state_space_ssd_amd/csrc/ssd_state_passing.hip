// Stage 3: the state entering each chunk,
//
//   H_{-1} = initial state (or 0),  H_c = exp(cum_last_c) * H_{c-1} + S_c,
//
// written as states_in[c] = H_{c-1}; final = H_{nc-1}.  This is the
// associative scan over (decay, state) pairs whose identity is (1, 0) -- the
// same pairs the Mamba-1 scan keeps as intermediates (mamba issue #488, the
// prepended-state workaround that seeds them with (1, 0)).  It runs in fp32,
// sequentially over chunks and in parallel over (batch, head, p, n); each
// thread carries four consecutive state elements in registers.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

__global__ __launch_bounds__(256) void state_passing_kernel(
    const float* __restrict__ states, const float* __restrict__ ws_cum,
    const float* init, float* states_in, float* final_states, int64_t H, int64_t nc,
    int64_t Q, int64_t PN) {
  // init and final_states may be the same buffer: each thread reads its four
  // elements of init before it writes the same four elements of final.
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (e >= PN) return;
  f4 hs = init ? ld4(init + (b * H + h) * PN + e) : f4{0.f, 0.f, 0.f, 0.f};
  const float* cum = ws_cum + (b * H + h) * nc * Q + (Q - 1);
  const int64_t cstride = H * PN;
  const float* src = states + (b * nc * H + h) * PN + e;
  float* dst = states_in + (b * nc * H + h) * PN + e;
  for (int64_t c = 0; c < nc; ++c) {
    const float decay = __expf(cum[c * Q]);
    const f4 s = ld4(src + c * cstride);
    st4(dst + c * cstride, hs);
    hs = decay * hs + s;
  }
  if (final_states) st4(final_states + (b * H + h) * PN + e, hs);
}

hipError_t launch_state_passing(const Problem& p, hipStream_t stream) {
  const int64_t PN = p.P * p.N;
  dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)p.H, (unsigned)p.b);
  hipLaunchKernelGGL(state_passing_kernel, grid, dim3(256), 0, stream, p.ws_states, p.ws_cum,
                     p.init, p.ws_states_in, p.final_states, p.H, p.nc, p.Q, PN);
  return hipGetLastError();
}

}  // namespace ssd
