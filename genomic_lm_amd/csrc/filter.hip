// filter.hip -- standalone modal filter and the state-copy helper.
//
// h[c, t] = sum_n R[c, n] exp(lam[c, n] t): the modal (sum of real
// exponentials) form of the hcl long filter with fp32 log_poles / residues
// (Evo2-7B-262K model card, Architecture 'Training dtype' and Implementation
// Notes 'log_poles / residues kept in fp32').  exp is evaluated directly for
// every t: a long fp32 power recurrence p^t drifts by ~1e-3 over 2^18 steps.
#include "common.hpp"
#include "launch.hpp"

namespace hyena {

// CPX: lam and R are complex, (re, im) pairs, and h = Re sum_n R_n exp(lam_n t)
// (the complex-pole form of Evo 1's poles / residues, Evo1-1.5-7B-8K model
// card, Architecture).
template <bool CPX>
__global__ __launch_bounds__(256) void modal_filter_kernel(
    const float* __restrict__ lam, const float* __restrict__ res, int N, int L,
    float* __restrict__ h) {
  const int c = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= L) return;
  constexpr int W = CPX ? 2 : 1;
  const float* lc = lam + static_cast<int64_t>(c) * N * W;
  const float* rc = res + static_cast<int64_t>(c) * N * W;
  const float tf = static_cast<float>(t);
  float acc = 0.0f;
  for (int n = 0; n < N; ++n) {
    if constexpr (CPX) {
      const float2 e = cexp_at(cpx_mode(lc[2 * n], lc[2 * n + 1]), tf);
      acc = fmaf(rc[2 * n], e.x, fmaf(-rc[2 * n + 1], e.y, acc));
    } else {
      acc = fmaf(rc[n], expf(lc[n] * tf), acc);
    }
  }
  h[static_cast<int64_t>(c) * L + t] = acc;
}

hipError_t launch_modal_filter(const float* lam, const float* res, int D, int N, int L,
                               float* h, bool cpx, hipStream_t stream) {
  dim3 grid((L + 255) / 256, D);
  if (cpx)
    modal_filter_kernel<true><<<grid, 256, 0, stream>>>(lam, res, N, L, h);
  else
    modal_filter_kernel<false><<<grid, 256, 0, stream>>>(lam, res, N, L, h);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void state_copy_kernel(
    const float* __restrict__ src, float* dst, int64_t count) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < count) dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_state_copy(const float* state_in, float* state_out, int64_t count,
                             hipStream_t stream) {
  if (state_in == state_out) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  state_copy_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(state_in, state_out, count);
  return hipGetLastError();
}

}  // namespace hyena
