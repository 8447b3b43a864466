// fir.hip -- gated explicit-FIR Hyena operator on the vector ALUs.
//
// z[t] = sum_{k<K} w[c,k] u[t-k], u = x1 * v, y = x2 * z + skip * u: the hcs
// (K = 7) and hcm (K = 128) blocks (Evo2-7B-262K model card, Implementation
// Notes, 'Block dispatch').
//
// One workgroup of 256 threads makes 2048 outputs of one row.  u for the
// tile plus a halo of K-1 earlier samples is staged once in LDS; each thread
// keeps 8 consecutive outputs in registers and walks the taps 8 at a time,
// reading 16 consecutive u values (four 16-byte LDS reads) per 64 FMAs.  The
// taps are read with a uniform address (LDS broadcast).
#include "common.hpp"
#include "launch.hpp"

namespace hyena {

constexpr int FIR_T = 256;
constexpr int FIR_OPT = 8;                    // outputs per thread
constexpr int FIR_TILE = FIR_T * FIR_OPT;     // outputs per workgroup
constexpr int FIR_G = 8;                      // taps per register group

// 8 consecutive elements starting at i (16-byte aligned for bf16, 32 for fp32)
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  static __device__ __forceinline__ void ld(const bf16_t* p, int64_t i, float (&o)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = __uint_as_float(ws[j] << 16);
      o[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void st(bf16_t* p, int64_t i, const float (&o)[8]) {
    uint32_t ws[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ws[j] = static_cast<uint32_t>(f32_to_bf16(o[2 * j])) |
              (static_cast<uint32_t>(f32_to_bf16(o[2 * j + 1])) << 16);
    *reinterpret_cast<uint4*>(p + i) = make_uint4(ws[0], ws[1], ws[2], ws[3]);
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void ld(const float* p, int64_t i, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p + i);
    const float4 b = *reinterpret_cast<const float4*>(p + i + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
  static __device__ __forceinline__ void st(float* p, int64_t i, const float (&o)[8]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(p + i + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
};

template <typename IO, bool VEC>
__global__ __launch_bounds__(FIR_T) void fir_kernel(
    const IO* __restrict__ x1, const IO* __restrict__ x2, const IO* __restrict__ v,
    const float* __restrict__ taps, int K, const float* __restrict__ skip,
    IO* __restrict__ y, int D, int L) {
  extern __shared__ float4 sm4[];
  float* sm = reinterpret_cast<float*>(sm4);
  const int Kp = (K + FIR_G - 1) / FIR_G * FIR_G;   // taps padded with zeros
  const int H = Kp;                                  // halo >= K - 1, multiple of 8
  float* w = sm;
  float* us = sm + Kp;                               // us[j] = u[tile0 - H + j]
  const int tid = threadIdx.x;
  const int tile0 = blockIdx.x * FIR_TILE;
  const int64_t row = blockIdx.y;
  const int c = static_cast<int>(row % D);
  const IO* x1r = x1 + row * L;
  const IO* x2r = x2 + row * L;
  const IO* vr = v + row * L;
  IO* yr = y + row * L;

  for (int j = tid; j < Kp; j += FIR_T) w[j] = (j < K) ? taps[static_cast<int64_t>(c) * K + j] : 0.0f;
  const int span = H + FIR_TILE;
  for (int j8 = tid * 8; j8 < span; j8 += FIR_T * 8) {
    const int g = tile0 - H + j8;
    if (VEC && g >= 0 && g + 8 <= L) {
      float a[8], b[8];
      Vec8<IO>::ld(x1r, g, a);
      Vec8<IO>::ld(vr, g, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) us[j8 + e] = a[e] * b[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int gg = g + e;
        us[j8 + e] = (gg >= 0 && gg < L) ? Io<IO>::ld(x1r, gg) * Io<IO>::ld(vr, gg) : 0.0f;
      }
    }
  }
  __syncthreads();

  float acc[FIR_OPT];
#pragma unroll
  for (int e = 0; e < FIR_OPT; ++e) acc[e] = 0.0f;
  const int o0 = H + tid * FIR_OPT;          // us index of this thread's first output
  for (int k0 = 0; k0 < Kp; k0 += FIR_G) {
    float r[FIR_OPT + FIR_G];                // r[j] = us[o0 - k0 - FIR_G + j]
    const float4* src = reinterpret_cast<const float4*>(us + o0 - k0 - FIR_G);
#pragma unroll
    for (int q = 0; q < (FIR_OPT + FIR_G) / 4; ++q) {
      const float4 f = src[q];
      r[4 * q] = f.x; r[4 * q + 1] = f.y; r[4 * q + 2] = f.z; r[4 * q + 3] = f.w;
    }
#pragma unroll
    for (int g = 0; g < FIR_G; ++g) {
      const float wk = w[k0 + g];
#pragma unroll
      for (int e = 0; e < FIR_OPT; ++e) acc[e] = fmaf(wk, r[e - g + FIR_G], acc[e]);
    }
  }

  const float sk = skip ? skip[c] : 0.0f;
  const int o = tile0 + tid * FIR_OPT;
  if (o >= L) return;
  if (VEC && o + FIR_OPT <= L) {
    float g[8], out[8];
    Vec8<IO>::ld(x2r, o, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = fmaf(g[e], acc[e], sk * us[o0 + e]);
    Vec8<IO>::st(yr, o, out);
  } else {
#pragma unroll
    for (int e = 0; e < FIR_OPT; ++e) {
      if (o + e < L) Io<IO>::st(yr, o + e, fmaf(Io<IO>::ld(x2r, o + e), acc[e], sk * us[o0 + e]));
    }
  }
}

template <typename IO>
static hipError_t launch_fir_io(const FirArgs& a, bool vec) {
  const int Kp = (a.K + FIR_G - 1) / FIR_G * FIR_G;
  const size_t shmem = static_cast<size_t>(2 * Kp + FIR_TILE) * sizeof(float);
  dim3 grid((a.L + FIR_TILE - 1) / FIR_TILE, static_cast<unsigned>(a.B * a.D));
  const IO* x1 = static_cast<const IO*>(a.x1);
  const IO* x2 = static_cast<const IO*>(a.x2);
  const IO* v = static_cast<const IO*>(a.v);
  IO* y = static_cast<IO*>(a.y);
  if (vec)
    fir_kernel<IO, true><<<grid, FIR_T, shmem, a.stream>>>(x1, x2, v, a.taps, a.K, a.skip, y, a.D, a.L);
  else
    fir_kernel<IO, false><<<grid, FIR_T, shmem, a.stream>>>(x1, x2, v, a.taps, a.K, a.skip, y, a.D, a.L);
  return hipGetLastError();
}

hipError_t launch_fir(const FirArgs& a) {
  // bf16 activations and up to 128 taps go to the matrix-core kernel
  if (a.bf16 && a.K <= 128) return launch_fir_mfma(a);
  const bool vec = (a.L % 8 == 0) && aligned_all(16, a.x1, a.x2, a.v, a.y);
  return a.bf16 ? launch_fir_io<bf16_t>(a, vec) : launch_fir_io<float>(a, vec);
}

}  // namespace hyena
