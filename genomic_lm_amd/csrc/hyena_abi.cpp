// hyena_abi.cpp -- the extern "C" entry points declared in include/hyena.h.
//
// Host only: every argument is validated before anything is launched, then the
// call is routed to a kernel launcher (launch.hpp).  Nothing here allocates,
// prints, throws or synchronises.
#include "hyena.h"

#include <hip/hip_runtime.h>

#include <limits>

#include "launch.hpp"

namespace {

using hyena::aligned_to;

constexpr int64_t kMaxInt = std::numeric_limits<int>::max();

hyena_status_t from_hip(hipError_t e) { return e == hipSuccess ? HYENA_OK : HYENA_ERR_LAUNCH; }

bool valid_io(hyena_dtype_t io) { return io == HYENA_F32 || io == HYENA_BF16; }
size_t io_size(hyena_dtype_t io) { return io == HYENA_BF16 ? 2 : 4; }

// Common checks of the activation arguments.  Returns HYENA_OK, or the error;
// `empty` is set when there is no element to compute.
hyena_status_t check_acts(const void* x1, const void* x2, const void* v, const void* y,
                          int64_t B, int64_t D, int64_t L, hyena_dtype_t io, bool* empty) {
  if (!valid_io(io)) return HYENA_ERR_INVALID_ARG;
  if (B < 0 || D < 0 || L < 0) return HYENA_ERR_INVALID_ARG;
  *empty = (B == 0 || D == 0 || L == 0);
  if (B > kMaxInt || D > kMaxInt || L > kMaxInt || B * D > kMaxInt) return HYENA_ERR_UNSUPPORTED;
  if (!*empty && B * D > std::numeric_limits<int64_t>::max() / L) return HYENA_ERR_UNSUPPORTED;
  if (*empty) return HYENA_OK;
  if (!x1 || !x2 || !v || !y) return HYENA_ERR_INVALID_ARG;
  const size_t a = io_size(io);
  if (!aligned_to(x1, a) || !aligned_to(x2, a) || !aligned_to(v, a) || !aligned_to(y, a))
    return HYENA_ERR_INVALID_ARG;
  return HYENA_OK;
}

hyena_status_t check_modal(const float* lam, const float* res, int64_t N, const float* skip) {
  if (N < 1 || N > HYENA_MAX_MODES) return HYENA_ERR_INVALID_ARG;
  if (!lam || !res) return HYENA_ERR_INVALID_ARG;
  if (!aligned_to(lam, 4) || !aligned_to(res, 4) || (skip && !aligned_to(skip, 4)))
    return HYENA_ERR_INVALID_ARG;
  return HYENA_OK;
}

int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ---- validated implementations; the real- and complex-mode entry points
// share them (cpx: parameters and states as (re, im) pairs)

hyena_status_t modal_filter_impl(const float* log_poles, const float* residues, int64_t D,
                                 int64_t N, int64_t L, float* h, bool cpx, hipStream_t stream) {
  if (D < 0 || L < 0) return HYENA_ERR_INVALID_ARG;
  if (N < 1 || N > HYENA_MAX_MODES) return HYENA_ERR_INVALID_ARG;
  if (D == 0 || L == 0) return HYENA_OK;
  if (!log_poles || !residues || !h) return HYENA_ERR_INVALID_ARG;
  if (!aligned_to(log_poles, 4) || !aligned_to(residues, 4) || !aligned_to(h, 4))
    return HYENA_ERR_INVALID_ARG;
  if (D > 65535 || L > kMaxInt || D * L > std::numeric_limits<int64_t>::max() / 4)
    return HYENA_ERR_UNSUPPORTED;
  return from_hip(hyena::launch_modal_filter(log_poles, residues, static_cast<int>(D),
                                             static_cast<int>(N), static_cast<int>(L), h,
                                             cpx, stream));
}

hyena_status_t decode_impl(const void* x1, const void* x2, const void* v,
                           const float* log_poles, const float* residues, int64_t N,
                           const float* skip, const float* state_in, float* state_out,
                           void* y, int64_t B, int64_t D, hyena_dtype_t io, bool cpx,
                           hipStream_t stream) {
  bool empty = false;
  hyena_status_t st = check_acts(x1, x2, v, y, B, D, 1, io, &empty);
  if (st != HYENA_OK) return st;
  if (N < 1 || N > HYENA_MAX_MODES) return HYENA_ERR_INVALID_ARG;
  if (empty) return HYENA_OK;
  st = check_modal(log_poles, residues, N, skip);
  if (st != HYENA_OK) return st;
  if (!state_out || !aligned_to(state_out, 4) || (state_in && !aligned_to(state_in, 4)))
    return HYENA_ERR_INVALID_ARG;
  hyena::DecodeArgs a{x1, x2, v, log_poles, residues, static_cast<int>(N), skip, state_in,
                      state_out, y, static_cast<int>(B), static_cast<int>(D),
                      io == HYENA_BF16, stream, cpx};
  return from_hip(hyena::launch_modal_decode(a));
}

// noalloc: the workspace is the library's device scratch; rows then go
// through it in batches that fit it, and a row longer than it is refused.
hyena_status_t fftconv_impl(const void* x1, const void* x2, const void* v,
                            const float* log_poles, const float* residues, int64_t N,
                            const float* skip, void* y, int64_t B, int64_t D, int64_t L,
                            hyena_dtype_t io, void* workspace, size_t ws_bytes, bool cpx,
                            hipStream_t stream, bool noalloc = false) {
  bool empty = false;
  hyena_status_t st = check_acts(x1, x2, v, y, B, D, L, io, &empty);
  if (st != HYENA_OK) return st;
  if (N < 1 || N > HYENA_MAX_MODES) return HYENA_ERR_INVALID_ARG;
  if (!empty && next_pow2(2 * L) > HYENA_MAX_FFT_LEN) return HYENA_ERR_UNSUPPORTED;
  if (empty) return HYENA_OK;
  st = check_modal(log_poles, residues, N, skip);
  if (st != HYENA_OK) return st;
  size_t batch = 0;
  if (noalloc) {
    const hipError_t e = hyena::noalloc_scratch(&workspace, &ws_bytes);
    if (e != hipSuccess) return HYENA_ERR_LAUNCH;
    batch = ws_bytes;
  }
  hyena::FftconvArgs a{x1, x2, v, log_poles, residues, static_cast<int>(N), skip, y,
                       static_cast<int>(B), static_cast<int>(D), static_cast<int>(L),
                       io == HYENA_BF16, workspace, ws_bytes, stream, cpx, batch};
  const bool onchip = hyena::fftconv_onchip_S(L) != 0;
  const size_t need = onchip ? hyena::fftconv_onchip_workspace(B, D, L, batch)
                             : hyena::fftconv_large_workspace(B, D, L, batch);
  if (!onchip && need == 0) return HYENA_ERR_UNSUPPORTED;
  if (noalloc && need > ws_bytes) return HYENA_ERR_UNSUPPORTED;   // one row beyond the scratch
  if (need > 0 && (!workspace || ws_bytes < need || !aligned_to(workspace, 16)))
    return HYENA_ERR_WORKSPACE;
  return from_hip(onchip ? hyena::launch_fftconv_onchip(a) : hyena::launch_fftconv_large(a));
}

hyena_status_t chunk_impl(const void* x1, const void* x2, const void* v,
                          const float* log_poles, const float* residues, int64_t N,
                          const float* skip, const float* state_in, float* state_out,
                          void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                          hyena_dtype_t io, hyena_chunk_algo_t algo, bool cpx, hipStream_t stream) {
  if (algo != HYENA_CHUNK_AUTO && algo != HYENA_CHUNK_FFT && algo != HYENA_CHUNK_MFMA)
    return HYENA_ERR_INVALID_ARG;
  bool empty = false;
  hyena_status_t st = check_acts(x1, x2, v, y, B, D, L, io, &empty);
  if (L == 0 && B >= 0 && D >= 0 && valid_io(io)) {
    // no token: the state passes through unchanged
    if (C < 1 || N < 1 || N > HYENA_MAX_MODES) return HYENA_ERR_INVALID_ARG;
    if (B == 0 || D == 0) return HYENA_OK;
    if (!state_out || !aligned_to(state_out, 4) || (state_in && !aligned_to(state_in, 4)))
      return HYENA_ERR_INVALID_ARG;
    if (B * D > kMaxInt) return HYENA_ERR_UNSUPPORTED;
    return from_hip(hyena::launch_state_copy(state_in, state_out, B * D * N * (cpx ? 2 : 1),
                                             stream));
  }
  if (st != HYENA_OK) return st;
  if (C < 1) return HYENA_ERR_INVALID_ARG;
  if (N < 1 || N > HYENA_MAX_MODES) return HYENA_ERR_INVALID_ARG;
  if (empty) return HYENA_OK;
  st = check_modal(log_poles, residues, N, skip);
  if (st != HYENA_OK) return st;
  if (!state_out || !aligned_to(state_out, 4) || (state_in && !aligned_to(state_in, 4)))
    return HYENA_ERR_INVALID_ARG;
  const int64_t Ceff = C < L ? C : L;
  const int64_t slots = cpx ? 2 * N : N;      // real lanes of the MFMA kernel's scan
  hyena_chunk_algo_t use = algo;
  if (use == HYENA_CHUNK_AUTO) use = (slots <= 32) ? HYENA_CHUNK_MFMA : HYENA_CHUNK_FFT;
  if (use == HYENA_CHUNK_MFMA && slots > 32) return HYENA_ERR_UNSUPPORTED;
  if (use == HYENA_CHUNK_FFT && Ceff > HYENA_MAX_FFT_CHUNK) return HYENA_ERR_UNSUPPORTED;
  hyena::ChunkArgs a{x1, x2, v, log_poles, residues, static_cast<int>(N), skip, state_in,
                     state_out, y, static_cast<int>(B), static_cast<int>(D),
                     static_cast<int>(L), static_cast<int>(Ceff), io == HYENA_BF16,
                     stream, cpx};
  return from_hip(use == HYENA_CHUNK_MFMA ? hyena::launch_chunk_mfma(a) : hyena::launch_chunk_fft(a));
}

hyena_status_t chunk_tokmajor_impl(const void* xin, int32_t pos_x1, int32_t pos_x2,
                                   int32_t pos_v, const float* log_poles, const float* residues,
                                   int64_t N, const float* skip, const float* state_in,
                                   float* state_out, void* y, int64_t B, int64_t D, int64_t L,
                                   hyena_dtype_t io, hyena_chunk_algo_t algo, void* workspace,
                                   size_t ws_bytes, hipStream_t stream) {
  if (algo == HYENA_CHUNK_FFT) return HYENA_ERR_UNSUPPORTED;
  if (algo != HYENA_CHUNK_AUTO && algo != HYENA_CHUNK_MFMA && algo != HYENA_CHUNK_RECURRENCE)
    return HYENA_ERR_INVALID_ARG;
  if (!valid_io(io) || B < 0 || D < 0 || L < 0) return HYENA_ERR_INVALID_ARG;
  const bool perm = pos_x1 >= 0 && pos_x2 >= 0 && pos_v >= 0 && pos_x1 < 3 && pos_x2 < 3 &&
                    pos_v < 3 && pos_x1 != pos_x2 && pos_x1 != pos_v && pos_x2 != pos_v;
  if (!perm || N < 1 || N > HYENA_MAX_MODES) return HYENA_ERR_INVALID_ARG;
  if (B == 0 || D == 0) return HYENA_OK;
  if (B > 65535 || D > kMaxInt / 3 || L > kMaxInt - 1024 || B * D > kMaxInt)
    return HYENA_ERR_UNSUPPORTED;
  if (!state_out || !aligned_to(state_out, 4) || (state_in && !aligned_to(state_in, 4)))
    return HYENA_ERR_INVALID_ARG;
  if (L == 0)   // no token: the state passes through unchanged
    return from_hip(hyena::launch_state_copy(state_in, state_out, B * D * N, stream));
  if (B * D > std::numeric_limits<int64_t>::max() / (3 * L)) return HYENA_ERR_UNSUPPORTED;
  const size_t a = io_size(io);
  if (!xin || !y || !aligned_to(xin, a) || !aligned_to(y, a)) return HYENA_ERR_INVALID_ARG;
  hyena_status_t st = check_modal(log_poles, residues, N, skip);
  if (st != HYENA_OK) return st;
  hyena::TokmajorArgs args{xin, pos_x1, pos_x2, pos_v, log_poles, residues,
                           static_cast<int>(N), skip, state_in, state_out, y,
                           static_cast<int>(B), static_cast<int>(D), static_cast<int>(L),
                           io == HYENA_BF16, workspace, stream};
  const bool mfma = hyena::tokmajor_mfma_supported(args);
  if (algo == HYENA_CHUNK_MFMA && !mfma) return HYENA_ERR_UNSUPPORTED;
  if (algo == HYENA_CHUNK_MFMA || (algo == HYENA_CHUNK_AUTO && mfma && hyena::tokmajor_mfma_preferred(args)))
    return from_hip(hyena::launch_chunk_mfma_tokmajor(args));
  const size_t need = hyena::tokmajor_workspace(B, D, L, N, io == HYENA_BF16);
  if (need && (!workspace || ws_bytes < need || !aligned_to(workspace, 16)))
    return HYENA_ERR_WORKSPACE;
  return from_hip(hyena::launch_tokmajor(args));
}

hyena_status_t fir_tokmajor_impl(const void* xin, int32_t pos_x1, int32_t pos_x2, int32_t pos_v,
                                 const float* taps, int64_t K, const float* skip,
                                 const float* window_in, float* window_out, void* y, int64_t B,
                                 int64_t D, int64_t L, hyena_dtype_t io, hipStream_t stream) {
  if (!valid_io(io) || B < 0 || D < 0 || L < 0) return HYENA_ERR_INVALID_ARG;
  const bool perm = pos_x1 >= 0 && pos_x2 >= 0 && pos_v >= 0 && pos_x1 < 3 && pos_x2 < 3 &&
                    pos_v < 3 && pos_x1 != pos_x2 && pos_x1 != pos_v && pos_x2 != pos_v;
  if (!perm || K < 1) return HYENA_ERR_INVALID_ARG;
  if (K > HYENA_MAX_FIR_TAPS_TOKMAJOR) return HYENA_ERR_UNSUPPORTED;
  if (B == 0 || D == 0) return HYENA_OK;
  if (B > 65535 || D > kMaxInt / 3 || L > kMaxInt - 1024 || B * D > kMaxInt)
    return HYENA_ERR_UNSUPPORTED;
  if (L > 0 && B * D > std::numeric_limits<int64_t>::max() / (3 * L)) return HYENA_ERR_UNSUPPORTED;
  if (!taps || !aligned_to(taps, 4) || (skip && !aligned_to(skip, 4))) return HYENA_ERR_INVALID_ARG;
  if ((window_in && !aligned_to(window_in, 4)) || (window_out && !aligned_to(window_out, 4)))
    return HYENA_ERR_INVALID_ARG;
  const size_t a = io_size(io);
  if (L > 0 && (!xin || !y || !aligned_to(xin, a) || !aligned_to(y, a))) return HYENA_ERR_INVALID_ARG;
  if (L == 0 && (K == 1 || !window_out)) return HYENA_OK;
  hyena::TokmajorFirArgs args{xin, pos_x1, pos_x2, pos_v, taps, static_cast<int>(K), skip,
                              window_in, window_out, y, static_cast<int>(B),
                              static_cast<int>(D), static_cast<int>(L), io == HYENA_BF16,
                              stream};
  return from_hip(hyena::launch_tokmajor_fir(args));
}

}  // namespace

extern "C" {

int hyena_abi_version(void) { return HYENA_ABI_VERSION; }

const char* hyena_status_string(hyena_status_t status) {
  switch (status) {
    case HYENA_OK: return "HYENA_OK";
    case HYENA_ERR_INVALID_ARG: return "HYENA_ERR_INVALID_ARG: null, negative, misaligned or out-of-range argument";
    case HYENA_ERR_UNSUPPORTED: return "HYENA_ERR_UNSUPPORTED: shape beyond the limits of this build";
    case HYENA_ERR_WORKSPACE: return "HYENA_ERR_WORKSPACE: workspace missing or too small";
    case HYENA_ERR_LAUNCH: return "HYENA_ERR_LAUNCH: a HIP launch or runtime call failed";
  }
  return "HYENA_ERR_UNKNOWN";
}

hyena_status_t hyena_modal_filter(const float* log_poles, const float* residues, int64_t D,
                                  int64_t N, int64_t L, float* h, hipStream_t stream) {
  return modal_filter_impl(log_poles, residues, D, N, L, h, false, stream);
}

hyena_status_t hyena_fir_fwd(const void* x1, const void* x2, const void* v, const float* taps,
                             int64_t K, const float* skip, void* y, int64_t B, int64_t D,
                             int64_t L, hyena_dtype_t io, hipStream_t stream) {
  bool empty = false;
  hyena_status_t st = check_acts(x1, x2, v, y, B, D, L, io, &empty);
  if (st != HYENA_OK) return st;
  if (K < 1) return HYENA_ERR_INVALID_ARG;
  if (K > HYENA_MAX_FIR_TAPS) return HYENA_ERR_UNSUPPORTED;
  if (empty) return HYENA_OK;
  if (!taps || !aligned_to(taps, 4) || (skip && !aligned_to(skip, 4))) return HYENA_ERR_INVALID_ARG;
  if (B * D > 65535 && !(io == HYENA_BF16 && K <= 128)) return HYENA_ERR_UNSUPPORTED;   // grid.y
  hyena::FirArgs a{x1, x2, v, taps, static_cast<int>(K), skip, y, static_cast<int>(B),
                   static_cast<int>(D), static_cast<int>(L), io == HYENA_BF16, stream};
  return from_hip(hyena::launch_fir(a));
}

hyena_status_t hyena_fftconv_fwd(const void* x1, const void* x2, const void* v,
                                 const float* log_poles, const float* residues, int64_t N,
                                 const float* skip, void* y, int64_t B, int64_t D, int64_t L,
                                 hyena_dtype_t io, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  return fftconv_impl(x1, x2, v, log_poles, residues, N, skip, y, B, D, L, io, workspace,
                      ws_bytes, false, stream);
}

hyena_status_t hyena_fftconv_fwd_noalloc(const void* x1, const void* x2, const void* v,
                                         const float* log_poles, const float* residues,
                                         int64_t N, const float* skip, void* y, int64_t B,
                                         int64_t D, int64_t L, hyena_dtype_t io,
                                         hipStream_t stream) {
  return fftconv_impl(x1, x2, v, log_poles, residues, N, skip, y, B, D, L, io, nullptr, 0,
                      false, stream, true);
}

size_t hyena_fftconv_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N, hyena_dtype_t io) {
  (void)N;
  (void)io;
  if (B <= 0 || D <= 0 || L <= 0) return 0;
  if (hyena::fftconv_onchip_S(L) != 0) return hyena::fftconv_onchip_workspace(B, D, L);
  if (next_pow2(2 * L) > HYENA_MAX_FFT_LEN) return 0;
  return hyena::fftconv_large_workspace(B, D, L);
}

hyena_status_t hyena_chunk_fwd(const void* x1, const void* x2, const void* v,
                               const float* log_poles, const float* residues, int64_t N,
                               const float* skip, const float* state_in, float* state_out,
                               void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                               hyena_dtype_t io, hipStream_t stream) {
  return chunk_impl(x1, x2, v, log_poles, residues, N, skip, state_in, state_out, y, B, D, L,
                    C, io, HYENA_CHUNK_AUTO, false, stream);
}

hyena_status_t hyena_chunk_fwd_algo(const void* x1, const void* x2, const void* v,
                                    const float* log_poles, const float* residues, int64_t N,
                                    const float* skip, const float* state_in, float* state_out,
                                    void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                                    hyena_dtype_t io, hyena_chunk_algo_t algo,
                                    hipStream_t stream) {
  return chunk_impl(x1, x2, v, log_poles, residues, N, skip, state_in, state_out, y, B, D, L,
                    C, io, algo, false, stream);
}

hyena_status_t hyena_modal_decode(const void* x1, const void* x2, const void* v,
                                  const float* log_poles, const float* residues, int64_t N,
                                  const float* skip, const float* state_in, float* state_out,
                                  void* y, int64_t B, int64_t D, hyena_dtype_t io,
                                  hipStream_t stream) {
  return decode_impl(x1, x2, v, log_poles, residues, N, skip, state_in, state_out, y, B, D, io,
                     false, stream);
}

hyena_status_t hyena_fir_fwd_window(const void* x1, const void* x2, const void* v,
                                    const float* taps, int64_t K, const float* skip,
                                    const float* window_in, float* window_out, void* y,
                                    int64_t B, int64_t D, int64_t L, hyena_dtype_t io,
                                    hipStream_t stream) {
  bool empty = false;
  hyena_status_t st = check_acts(x1, x2, v, y, B, D, L, io, &empty);
  // L = 0 still moves the window over; only B = 0 or D = 0 is a no-op
  if (st != HYENA_OK) return st;
  if (K < 1) return HYENA_ERR_INVALID_ARG;
  if (K > HYENA_MAX_FIR_TAPS) return HYENA_ERR_UNSUPPORTED;
  if (B == 0 || D == 0) return HYENA_OK;
  if (empty && K == 1) return HYENA_OK;
  if (!taps || !aligned_to(taps, 4) || (skip && !aligned_to(skip, 4))) return HYENA_ERR_INVALID_ARG;
  if (K > 1 && (!window_out || !aligned_to(window_out, 4) || (window_in && !aligned_to(window_in, 4))))
    return HYENA_ERR_INVALID_ARG;
  if (L > K - 1 && B * D > 65535 && !(io == HYENA_BF16 && K <= 128)) return HYENA_ERR_UNSUPPORTED;
  hyena::FirArgs a{x1, x2, v, taps, static_cast<int>(K), skip, y, static_cast<int>(B),
                   static_cast<int>(D), static_cast<int>(L), io == HYENA_BF16, stream};
  return from_hip(hyena::launch_fir_window(a, window_in, window_out));
}

hyena_status_t hyena_modal_filter_cpx(const float* log_poles, const float* residues, int64_t D,
                                      int64_t N, int64_t L, float* h, hipStream_t stream) {
  return modal_filter_impl(log_poles, residues, D, N, L, h, true, stream);
}

hyena_status_t hyena_fftconv_fwd_cpx(const void* x1, const void* x2, const void* v,
                                     const float* log_poles, const float* residues, int64_t N,
                                     const float* skip, void* y, int64_t B, int64_t D, int64_t L,
                                     hyena_dtype_t io, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  return fftconv_impl(x1, x2, v, log_poles, residues, N, skip, y, B, D, L, io, workspace,
                      ws_bytes, true, stream);
}

hyena_status_t hyena_chunk_fwd_cpx(const void* x1, const void* x2, const void* v,
                                   const float* log_poles, const float* residues, int64_t N,
                                   const float* skip, const float* state_in, float* state_out,
                                   void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                                   hyena_dtype_t io, hipStream_t stream) {
  return chunk_impl(x1, x2, v, log_poles, residues, N, skip, state_in, state_out, y, B, D, L,
                    C, io, HYENA_CHUNK_AUTO, true, stream);
}

hyena_status_t hyena_chunk_fwd_cpx_algo(const void* x1, const void* x2, const void* v,
                                        const float* log_poles, const float* residues, int64_t N,
                                        const float* skip, const float* state_in,
                                        float* state_out, void* y, int64_t B, int64_t D,
                                        int64_t L, int64_t C, hyena_dtype_t io,
                                        hyena_chunk_algo_t algo, hipStream_t stream) {
  return chunk_impl(x1, x2, v, log_poles, residues, N, skip, state_in, state_out, y, B, D, L,
                    C, io, algo, true, stream);
}

hyena_status_t hyena_modal_decode_cpx(const void* x1, const void* x2, const void* v,
                                      const float* log_poles, const float* residues, int64_t N,
                                      const float* skip, const float* state_in, float* state_out,
                                      void* y, int64_t B, int64_t D, hyena_dtype_t io,
                                      hipStream_t stream) {
  return decode_impl(x1, x2, v, log_poles, residues, N, skip, state_in, state_out, y, B, D, io,
                     true, stream);
}

hyena_status_t hyena_chunk_fwd_tokmajor(const void* xin, int32_t pos_x1, int32_t pos_x2,
                                        int32_t pos_v, const float* log_poles,
                                        const float* residues, int64_t N, const float* skip,
                                        const float* state_in, float* state_out, void* y,
                                        int64_t B, int64_t D, int64_t L, hyena_dtype_t io,
                                        void* workspace, size_t ws_bytes, hipStream_t stream) {
  return chunk_tokmajor_impl(xin, pos_x1, pos_x2, pos_v, log_poles, residues, N, skip, state_in,
                             state_out, y, B, D, L, io, HYENA_CHUNK_AUTO, workspace, ws_bytes,
                             stream);
}

hyena_status_t hyena_chunk_fwd_tokmajor_algo(const void* xin, int32_t pos_x1, int32_t pos_x2,
                                             int32_t pos_v, const float* log_poles,
                                             const float* residues, int64_t N, const float* skip,
                                             const float* state_in, float* state_out, void* y,
                                             int64_t B, int64_t D, int64_t L, hyena_dtype_t io,
                                             hyena_chunk_algo_t algo, void* workspace,
                                             size_t ws_bytes, hipStream_t stream) {
  return chunk_tokmajor_impl(xin, pos_x1, pos_x2, pos_v, log_poles, residues, N, skip, state_in,
                             state_out, y, B, D, L, io, algo, workspace, ws_bytes, stream);
}

hyena_status_t hyena_fir_fwd_tokmajor(const void* xin, int32_t pos_x1, int32_t pos_x2,
                                      int32_t pos_v, const float* taps, int64_t K,
                                      const float* skip, const float* window_in,
                                      float* window_out, void* y, int64_t B, int64_t D, int64_t L,
                                      hyena_dtype_t io, hipStream_t stream) {
  return fir_tokmajor_impl(xin, pos_x1, pos_x2, pos_v, taps, K, skip, window_in, window_out, y,
                           B, D, L, io, stream);
}

size_t hyena_chunk_tokmajor_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N,
                                           hyena_dtype_t io) {
  if (!valid_io(io) || N < 1 || N > HYENA_MAX_MODES) return 0;
  if (B > 65535 || D > kMaxInt / 3 || L > kMaxInt - 1024 || B * D > kMaxInt) return 0;
  return hyena::tokmajor_workspace(B, D, L, N, io == HYENA_BF16);
}

}  // extern "C"
