// launch.hpp -- internal host-side interface between the C ABI (hyena_abi.cpp)
// and the kernel launchers in the .hip files.  Arguments arrive here already
// validated; launchers only pick a kernel variant and launch it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hyena {

inline bool aligned_to(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}
template <typename... Ps>
inline bool aligned_all(size_t a, Ps... ps) {
  return (aligned_to(ps, a) && ...);
}

struct FftconvArgs {
  const void* x1;
  const void* x2;
  const void* v;
  const float* lam;
  const float* res;
  int N;
  const float* skip;
  void* y;
  int B, D, L;
  bool bf16;
  void* workspace;
  size_t ws_bytes;
  hipStream_t stream;
  bool cpx = false;
  size_t batch_bytes = 0;   // workspace per batch of rows; 0: the default 1 GiB
};

struct FirArgs {
  const void* x1;
  const void* x2;
  const void* v;
  const float* taps;
  int K;
  const float* skip;
  void* y;
  int B, D, L;
  bool bf16;
  hipStream_t stream;
};

struct ChunkArgs {
  const void* x1;
  const void* x2;
  const void* v;
  const float* lam;
  const float* res;
  int N;
  const float* skip;
  const float* state_in;
  float* state_out;
  void* y;
  int B, D, L, C;
  bool bf16;
  hipStream_t stream;
  bool cpx = false;
};

struct DecodeArgs {
  const void* x1;
  const void* x2;
  const void* v;
  const float* lam;
  const float* res;
  int N;
  const float* skip;
  const float* state_in;
  float* state_out;
  void* y;
  int B, D;
  bool bf16;
  hipStream_t stream;
  bool cpx = false;
};

// Token-major input (B, L, 3D), channel c's x1, x2, v at columns 3c + pos_*;
// y (B, L, D).
struct TokmajorArgs {
  const void* xin;
  int pos_x1, pos_x2, pos_v;
  const float* lam;
  const float* res;
  int N;
  const float* skip;
  const float* state_in;
  float* state_out;
  void* y;
  int B, D, L;
  bool bf16;
  void* workspace;
  hipStream_t stream;
};

// Token-major explicit FIR: xin as above, taps (D, K), windows (B, D, K-1).
struct TokmajorFirArgs {
  const void* xin;
  int pos_x1, pos_x2, pos_v;
  const float* taps;
  int K;
  const float* skip;
  const float* win_in;
  float* win_out;
  void* y;
  int B, D, L;
  bool bf16;
  hipStream_t stream;
};

// cpx: complex modes, lam and res as (re, im) pairs (also in the structs below)
hipError_t launch_modal_filter(const float* lam, const float* res, int D, int N, int L,
                               float* h, bool cpx, hipStream_t stream);

hipError_t launch_fir(const FirArgs& a);        // picks the kernel below or the VALU one
hipError_t launch_fir_mfma(const FirArgs& a);   // bf16, K <= 128

// Sub-transform size S of the on-chip single-pass kernel for length L, or 0
// when L is too long for it (L > 32768).  From S = 4096 on (L > 4096) the
// parity halves are two launches that pass the even half's result through a
// workspace of fftconv_onchip_workspace bytes (0 below).
int fftconv_onchip_S(int64_t L);
size_t fftconv_onchip_workspace(int64_t B, int64_t D, int64_t L, size_t batch_bytes = 0);
hipError_t launch_fftconv_onchip(const FftconvArgs& a);

// The device scratch of hyena_fftconv_fwd_noalloc (noalloc.hip): its address
// on the current device, looked up on the first call per device and kept.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Multi-kernel single pass for L > 32768 through a caller workspace.
size_t fftconv_large_workspace(int64_t B, int64_t D, int64_t L, size_t batch_bytes = 0);
hipError_t launch_fftconv_large(const FftconvArgs& a);

hipError_t launch_chunk_fft(const ChunkArgs& a);
hipError_t launch_chunk_mfma(const ChunkArgs& a);
// The matrix-core chunk kernel on the token-major layout (chunk_mfma.hip):
// bf16, N <= 16, D a multiple of 8, xin and y 16-byte aligned; and whether
// it is the faster token-major path for the shape.
bool tokmajor_mfma_supported(const TokmajorArgs& a);
bool tokmajor_mfma_preferred(const TokmajorArgs& a);
hipError_t launch_chunk_mfma_tokmajor(const TokmajorArgs& a);

// One token per row from the modal state (decode.hip).
hipError_t launch_modal_decode(const DecodeArgs& a);
// FIR continuing from a window of the last K-1 inputs: launch_fir for the
// outputs past the window's reach, then the window kernel (decode.hip).
hipError_t launch_fir_window(const FirArgs& a, const float* win_in, float* win_out);

// Token-major modal operator (tokmajor.hip): segment length TS and count P
// for the shape, the workspace it needs (0 when P = 1), and the launcher.
void tokmajor_segments(int64_t B, int64_t D, int64_t L, bool bf16, int* TS, int* P);
size_t tokmajor_workspace(int64_t B, int64_t D, int64_t L, int64_t N, bool bf16);
hipError_t launch_tokmajor(const TokmajorArgs& a);
// Token-major explicit FIR (K <= 128), then window_out when requested.
void tokmajor_fir_segments(int64_t B, int64_t D, int64_t L, int K, int* TS, int* P);
hipError_t launch_tokmajor_fir(const TokmajorFirArgs& a);
// The matrix-core FIR on the token-major layout (fir_mfma.hip): bf16,
// K <= 128, D a multiple of 8, xin and y 16-byte aligned; y only (the
// window is written by the caller's window kernel).
bool tokmajor_fir_mfma_supported(const TokmajorFirArgs& a);
hipError_t launch_fir_mfma_tokmajor(const TokmajorFirArgs& a);

// state_out <- state_in (or 0 when state_in is null), count floats.
hipError_t launch_state_copy(const float* state_in, float* state_out, int64_t count,
                             hipStream_t stream);

}  // namespace hyena
