// decode.hip -- the operator continued from its per-layer caches.
//
// The hcl block's cache is its modal state, the hcm / hcs blocks' cache the
// window of their last K-1 inputs (Evo2-7B-262K model card, Implementation
// Notes, 'Custom cache'; Evo1-1.5-7B-8K model card, Implementation Notes,
// 'Cache subclass': FIR window + IIR modal state).
//
// modal_decode_kernel: one token per (b, c) row,
//     s_n <- p_n s_n + u,   y = x2 * sum_n R_n s_n + skip * u,   u = x1 v.
//
// fir_window_kernel: the first min(L, K-1) outputs of an FIR call that
// continues a sequence, i.e. those that reach back into the window, and the
// new window.  The rest of the outputs do not depend on the window and come
// from the ordinary FIR kernels, launched first on the same stream; this
// kernel then overwrites the outputs they computed with a zero history.
#include <type_traits>

#include "common.hpp"
#include "pow_pair.hpp"
#include "launch.hpp"

namespace hyena {

// One lane per (row, mode): a row's modes sit in a group of G = next power
// of two >= N lanes of one wave, so every load is coalesced across the group
// and the sum over modes is a butterfly of log2(G) lane exchanges.
// CPX: complex modes and state as (re, im) pairs; y = x2 Re sum_n R_n s_n + skip u.
template <typename IO, bool CPX>
__global__ __launch_bounds__(256) void modal_decode_kernel(
    const IO* __restrict__ x1, const IO* __restrict__ x2, const IO* __restrict__ v,
    const float* __restrict__ lam, const float* __restrict__ res, int N, int lgG,
    const float* __restrict__ skip, const float* state_in, float* state_out,
    IO* __restrict__ y, int D, int64_t rows) {
  const int G = 1 << lgG;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid >> lgG;
  const int n = static_cast<int>(gid & (G - 1));
  const bool live = row < rows && n < N;
  float part = 0.0f, u = 0.0f;
  int c = 0;
  if (row < rows) {
    c = static_cast<int>(row % D);
    u = Io<IO>::ld(x1, row) * Io<IO>::ld(v, row);
  }
  if (live) {
    const int64_t pi = static_cast<int64_t>(c) * N + n;
    const int64_t si = row * N + n;
    // read before write: state_out may be state_in
    if constexpr (CPX) {
      // the pole as hi + lo: decode steps compound its rounding (pow_pair.hpp)
      float2 pl;
      const float2 ph = cpow_pair(lam[2 * pi], lam[2 * pi + 1], 1.0f, pl);
      const float2 s0 = state_in ? make_float2(state_in[2 * si], state_in[2 * si + 1])
                                 : make_float2(0.0f, 0.0f);
      const float2 ps = cadd(cmul(ph, s0), cmul(pl, s0));
      const float2 s = make_float2(ps.x + u, ps.y);
      state_out[2 * si] = s.x;
      state_out[2 * si + 1] = s.y;
      part = fmaf(res[2 * pi], s.x, -res[2 * pi + 1] * s.y);
    } else {
      const float2 p = pow_pair(lam[pi], 1.0f);        // hi + lo (pow_pair.hpp)
      const float s0 = state_in ? state_in[si] : 0.0f;
      const float s = fmaf(p.x, s0, fmaf(p.y, s0, u));
      state_out[si] = s;
      part = res[pi] * s;
    }
  }
  // every lane of the wave takes part in the exchanges (groups never span
  // waves: G divides 64)
  for (int o = 1; o < G; o <<= 1) part += __shfl_xor(part, o);
  if (row < rows && n == 0) {
    const float sk = skip ? skip[c] : 0.0f;
    Io<IO>::st(y, row, fmaf(Io<IO>::ld(x2, row), part, sk * u));
  }
}

constexpr int FIRW_T = 128;

// One workgroup per row.  LDS: the taps, then e = [window, u[0:T0)],
// T0 = min(L, K-1).  Each of the T0 outputs is one wave's dot product (taps
// strided over the lanes, then a butterfly), so a decode step (T0 = 1) does
// not run K products on one lane.
template <typename IO>
__global__ __launch_bounds__(FIRW_T) void fir_window_kernel(
    const IO* __restrict__ x1, const IO* __restrict__ x2, const IO* __restrict__ v,
    const float* __restrict__ taps, int K, const float* __restrict__ skip,
    const float* win_in, float* win_out, IO* __restrict__ y, int D, int L) {
  extern __shared__ float smf[];
  const int W = K - 1;
  const int T0 = L < W ? L : W;
  float* w = smf;
  float* e = smf + K;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int c = static_cast<int>(row % D);
  const IO* x1r = x1 + row * L;
  const IO* x2r = x2 + row * L;
  const IO* vr = v + row * L;
  for (int k = tid; k < K; k += FIRW_T) w[k] = taps[static_cast<int64_t>(c) * K + k];
  for (int j = tid; j < W; j += FIRW_T) e[j] = win_in ? win_in[row * W + j] : 0.0f;
  for (int t = tid; t < T0; t += FIRW_T) e[W + t] = Io<IO>::ld(x1r, t) * Io<IO>::ld(vr, t);
  __syncthreads();                      // every read of win_in is done

  const float sk = skip ? skip[c] : 0.0f;
  for (int t = wave; t < T0; t += FIRW_T / 64) {
    float z = 0.0f;
    for (int k = lane; k < K; k += 64) z = fmaf(w[k], e[W + t - k], z);
    for (int o = 1; o < 64; o <<= 1) z += __shfl_xor(z, o);
    if (lane == 0) Io<IO>::st(y + row * L, t, fmaf(Io<IO>::ld(x2r, t), z, sk * e[W + t]));
  }
  // new window: entries L .. L+W-1 of [window, u]
  for (int j = tid; j < W; j += FIRW_T) {
    const int src = L + j;
    const float val = (src < W) ? e[src] : Io<IO>::ld(x1r, src - W) * Io<IO>::ld(vr, src - W);
    win_out[row * W + j] = val;
  }
}

hipError_t launch_modal_decode(const DecodeArgs& a) {
  const int64_t rows = static_cast<int64_t>(a.B) * a.D;
  int lgG = 0;
  while ((1 << lgG) < a.N) ++lgG;         // N <= 64: G <= 64 lanes
  const unsigned blocks = static_cast<unsigned>(((rows << lgG) + 255) / 256);
  auto go = [&](auto io_tag, auto cpx_tag) {
    using IO = decltype(io_tag);
    modal_decode_kernel<IO, decltype(cpx_tag)::value><<<blocks, 256, 0, a.stream>>>(
        static_cast<const IO*>(a.x1), static_cast<const IO*>(a.x2), static_cast<const IO*>(a.v),
        a.lam, a.res, a.N, lgG, a.skip, a.state_in, a.state_out, static_cast<IO*>(a.y), a.D, rows);
  };
  if (a.bf16) {
    if (a.cpx) go(bf16_t{}, std::true_type{}); else go(bf16_t{}, std::false_type{});
  } else {
    if (a.cpx) go(float{}, std::true_type{}); else go(float{}, std::false_type{});
  }
  return hipGetLastError();
}

hipError_t launch_fir_window(const FirArgs& a, const float* win_in, float* win_out) {
  // outputs that do not reach back into the window: the ordinary kernels
  if (a.L > a.K - 1) {
    const hipError_t e = launch_fir(a);
    if (e != hipSuccess) return e;
  }
  if (a.K == 1) return hipSuccess;      // no window
  const int W = a.K - 1;
  const int T0 = a.L < W ? a.L : W;
  const size_t shmem = static_cast<size_t>(a.K + W + T0) * sizeof(float);
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.D);
  if (a.bf16)
    fir_window_kernel<bf16_t><<<grid, FIRW_T, shmem, a.stream>>>(
        static_cast<const bf16_t*>(a.x1), static_cast<const bf16_t*>(a.x2),
        static_cast<const bf16_t*>(a.v), a.taps, a.K, a.skip, win_in, win_out,
        static_cast<bf16_t*>(a.y), a.D, a.L);
  else
    fir_window_kernel<float><<<grid, FIRW_T, shmem, a.stream>>>(
        static_cast<const float*>(a.x1), static_cast<const float*>(a.x2),
        static_cast<const float*>(a.v), a.taps, a.K, a.skip, win_in, win_out,
        static_cast<float*>(a.y), a.D, a.L);
  return hipGetLastError();
}

}  // namespace hyena
