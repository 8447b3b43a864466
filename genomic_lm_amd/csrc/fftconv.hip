// fftconv.hip -- single-pass modal Hyena operator, one workgroup per (b, c) row.
//
// y = x2 * (h causal-conv u) + skip * u, u = x1 * v, h[t] = sum_n R_n exp(lam_n t),
// the convolution taken as a zero-padded FFT product of length Nfft = 4S >= 2L
// ('modal-form IIR via FFT': Evo2-7B-262K model card, Implementation Notes,
// 'Block dispatch'; 'FFT-based long convolution': Evo1-1.5-7B-8K model card,
// Implementation Notes, 'Hyena engine').
//
// Layout of the transform (all fp32, all on chip):
//  * the real length-Nfft signals u and h are packed as complex c[m] =
//    x[2m] + i x[2m+1], m < M = 2S; since x is zero from L <= 2S on, c is zero
//    on its upper half;
//  * the first decimation-in-frequency stage of the size-M DFT therefore
//    splits into two size-S DFTs with no butterflies: C[2k+q] is the DFT of
//    c[m] * exp(-2*pi*i*q*m/M), q = 0, 1 (the "parity halves");
//  * the real spectrum U[K], K = 2k+q, comes from C[K] and C[M-K], and M-K
//    has the same parity, so each parity half is processed on its own;
//  * Z = U * H, repacked for the inverse real transform, inverse size-S DFT
//    per parity, and the two halves are recombined with one twiddle:
//    c_z[m] = (B_0[m] + exp(2*pi*i*m/M) B_1[m]) / M.
// Only one size-S transform lives in LDS at a time.  Up to S = 2048 one
// workgroup takes both halves.  From S = 4096 (L > 4096) the two halves are
// two launches with one workgroup per (row, half): the even half writes its
// inverse transform B_0 (S complex, fp32) to a caller workspace and the odd
// half reads it back for the recombination -- 4 bytes per token each way,
// against the 48 of the four-step path that rows longer than 32768 take.  h is
// generated per thread with short exp ladders (<= 16 multiplications from an
// exact anchor) and never touches memory.
#include "common.hpp"
#include "fft.hpp"
#include "launch.hpp"

namespace hyena {

// a[i] = (h[2m], h[2m+1]) for m = t + T*i, zero at and beyond L.
template <int P, int T>
__device__ __forceinline__ void modal_pairs(float2 (&a)[P], const float* lam, const float* res,
                                            int N, int t, int L) {
#pragma unroll
  for (int i = 0; i < P; ++i) a[i] = make_float2(0.0f, 0.0f);
  for (int n = 0; n < N; ++n) {
    const float l = lam[n];
    const float p = expf(l);
    const float step = expf(l * static_cast<float>(2 * T));
    float e = res[n] * expf(l * static_cast<float>(2 * t));
#pragma unroll
    for (int i = 0; i < P; ++i) {
      a[i].x += e;
      a[i].y = fmaf(e, p, a[i].y);
      e *= step;
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int m2 = 2 * (t + T * i);
    if (m2 >= L) a[i].x = 0.0f;
    if (m2 + 1 >= L) a[i].y = 0.0f;
  }
}

// The same pairs for complex modes (lam, res as (re, im) pairs):
// (Re sum_n R_n p_n^(2m), Re sum_n R_n p_n^(2m+1)), a ladder of P steps of
// p^(2T) from an exact anchor per mode.
template <int P, int T>
__device__ __forceinline__ void modal_pairs_cpx(float2 (&a)[P], const float* lam, const float* res,
                                                int N, int t, int L) {
#pragma unroll
  for (int i = 0; i < P; ++i) a[i] = make_float2(0.0f, 0.0f);
  for (int n = 0; n < N; ++n) {
    const CpxMode md = cpx_mode(lam[2 * n], lam[2 * n + 1]);
    const float2 p = cexp_at(md, 1.0f);
    const float2 step = cexp_at(md, static_cast<float>(2 * T));
    float2 e = cmul(make_float2(res[2 * n], res[2 * n + 1]), cexp_at(md, static_cast<float>(2 * t)));
#pragma unroll
    for (int i = 0; i < P; ++i) {
      a[i].x += e.x;
      a[i].y += fmaf(e.x, p.x, -e.y * p.y);      // Re(e p)
      e = cmul(e, step);
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int m2 = 2 * (t + T * i);
    if (m2 >= L) a[i].x = 0.0f;
    if (m2 + 1 >= L) a[i].y = 0.0f;
  }
}

// PART 0: both parity halves in one workgroup.  PART 1: the even half, its
// inverse transform stored to ws (S complex per row of the launch, in the
// order m = t + T*i).  PART 2: the odd half, recombined with ws, gated and
// stored.  A launch covers rows row0 .. row0 + gridDim.x - 1.
template <int S, int T, typename IO, bool VEC, bool CPX, int PART>
__global__ __launch_bounds__(T) void fftconv_kernel(
    const IO* x1, const IO* x2, const IO* v,
    const float* __restrict__ lam, const float* __restrict__ res, int N,
    const float* __restrict__ skip, IO* __restrict__ y, int D, int L,
    float2* __restrict__ ws, int64_t row0) {
  constexpr int P = S / T;
  constexpr int M = 2 * S;
  constexpr int LG_M = ilog2(M);
  constexpr int LG_N = LG_M + 1;
  constexpr int Q0 = PART == 2 ? 1 : 0;
  constexpr int Q1 = PART == 1 ? 0 : 1;
  __shared__ float2 lds[lds_padded_size(S)];
  // From S = 1024 on, the even half's inverse transform waits for the odd
  // half in LDS rather than in 2P registers: there the register budget, not
  // LDS, limits the workgroups per CU (measured at D = 4096: L = 8192 612 ->
  // 377 us, L = 4096 201 -> 175 us; at S = 8192 it also ends a spill).
  constexpr bool B0_LDS = PART == 0 && S >= 1024;
  __shared__ float2 b0s[B0_LDS ? S : 1];

  const int t = threadIdx.x;
  const int64_t row = row0 + blockIdx.x;
  float2* wsr = ws + static_cast<int64_t>(blockIdx.x) * S;
  const int c = static_cast<int>(row % D);
  const IO* x1r = x1 + row * L;
  const IO* x2r = x2 + row * L;
  const IO* vr = v + row * L;
  IO* yr = y + row * L;
  constexpr int W = CPX ? 2 : 1;               // floats per mode parameter
  const float* lamc = lam + static_cast<int64_t>(c) * N * W;
  const float* resc = res + static_cast<int64_t>(c) * N * W;

  float2 b0[PART == 0 && !B0_LDS ? P : 1];   // inverse transform of the even half, kept for the recombination
  float zm_nyq = 0.0f;    // Z[M] (real), only used by thread 0

  // Both parity halves are unrolled: as a loop, the address and twiddle
  // arithmetic common to the two iterations was hoisted out of it and held
  // in registers across both transforms.
#pragma unroll
  for (int q = Q0; q <= Q1; ++q) {
    float2 a[P];
    // ---- u = x1 * v, packed in pairs, parity pre-twiddle
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int m = t + T * i;
      float2 p1, p2;
      if constexpr (VEC) {
        // L even: clamped pair index, zero beyond L without a branch
        const int64_t e = min(2 * m, L - 2);
        Raw2<IO> r1, r2;
        r1.load(x1r + e);
        r2.load(vr + e);
        const bool in = 2 * m < L;
        p1 = in ? r1.get() : make_float2(0.0f, 0.0f);
        p2 = in ? r2.get() : make_float2(0.0f, 0.0f);
      } else {
        p1 = ld_pair<IO, VEC>(x1r, 2 * m, L);
        p2 = ld_pair<IO, VEC>(vr, 2 * m, L);
      }
      a[i] = make_float2(p1.x * p2.x, p1.y * p2.y);
      if (q) a[i] = cmul(a[i], twiddle(m, LG_M));
    }
    fft_forward<S, T>(a, lds, t);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = a[i];
    __syncthreads();
    float2 z[P];
    float um_nyq = 0.0f;
    int ts = t;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (i % SEQ == 0) ts = seq_idx(t);
      const int k = ts + T * i;
      const int kk = q ? (S - 1 - k) : ((S - k) & (S - 1));
      z[i] = real_spectrum(a[i], lds[lds_pad(kk)], twiddle(2 * k + q, LG_N));
      seq_keep(z[i]);
    }
    if (q == 0 && t == 0) um_nyq = a[0].x - a[0].y;

    // ---- h, generated on chip, same packing
    if constexpr (CPX)
      modal_pairs_cpx<P, T>(a, lamc, resc, N, t, L);
    else
      modal_pairs<P, T>(a, lamc, resc, N, t, L);
    if (q) {
#pragma unroll
      for (int i = 0; i < P; ++i) a[i] = cmul(a[i], twiddle(t + T * i, LG_M));
    }
    fft_forward<S, T>(a, lds, t);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = a[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (i % SEQ == 0) ts = seq_idx(t);
      const int k = ts + T * i;
      const int kk = q ? (S - 1 - k) : ((S - k) & (S - 1));
      z[i] = cmul(z[i], real_spectrum(a[i], lds[lds_pad(kk)], twiddle(2 * k + q, LG_N)));
      seq_keep(z[i]);
    }
    if (q == 0 && t == 0) zm_nyq = um_nyq * (a[0].x - a[0].y);

    // ---- repack Z for the inverse real transform
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = z[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (i % SEQ == 0) ts = seq_idx(t);
      const int k = ts + T * i;
      const int kk = q ? (S - 1 - k) : ((S - k) & (S - 1));
      float2 zmir = lds[lds_pad(kk)];
      if (q == 0 && k == 0) zmir = make_float2(zm_nyq, 0.0f);
      a[i] = inverse_pack(z[i], zmir, twiddle(2 * k + q, LG_N));
      seq_keep(a[i]);
    }
    fft_inverse<S, T>(a, lds, t);

    if (q == 0) {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        if constexpr (PART == 1) (wsr + T * i)[t] = a[i];   // uniform base per i, one offset
        else if constexpr (B0_LDS) b0s[t + T * i] = a[i];
        else b0[i] = a[i];
      }
    } else {
      // ---- recombine, gate, store
      const float sk = skip ? skip[c] : 0.0f;
      const float inv_m = 1.0f / static_cast<float>(M);
      if constexpr (VEC) {
        // L is even: pair m is whole for 2m < L and absent beyond.  The
        // operands of a group of 8 elements (B_0, x1, v, x2) are loaded
        // together from pair indices clamped into the row, so no branch
        // separates the loads and none waits for an earlier element's store;
        // pairs beyond L are not stored.
        constexpr int GG = P < 8 ? P : 8;
#pragma unroll
        for (int g0 = 0; g0 < P; g0 += GG) {
          ts = seq_idx(t);
          Raw2<IO> r1[GG], r2[GG], rg[GG];
          float2 e0[GG];
#pragma unroll
          for (int j = 0; j < GG; ++j) {
            const int i = g0 + j;
            const int64_t e = min(2 * (ts + T * i), L - 2);
            if constexpr (PART == 2) e0[j] = (wsr + T * i)[ts];
            else if constexpr (B0_LDS) e0[j] = b0s[ts + T * i];
            else e0[j] = b0[i];
            r1[j].load(x1r + e);
            r2[j].load(vr + e);
            rg[j].load(x2r + e);
          }
#pragma unroll
          for (int j = 0; j < GG; ++j) {
            const int m = ts + T * (g0 + j);
            const float2 zz = cscale(cadd(e0[j], cmul(cconj(twiddle(m, LG_M)), a[g0 + j])), inv_m);
            const float2 p1 = r1[j].get(), p2 = r2[j].get(), g = rg[j].get();
            const float2 out = make_float2(fmaf(g.x, zz.x, sk * (p1.x * p2.x)),
                                           fmaf(g.y, zz.y, sk * (p1.y * p2.y)));
            if (2 * m < L) Io<IO>::st2(yr, 2 * m, out);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < P; ++i) {
          if (i % SEQ == 0) ts = seq_idx(t);
          const int m = ts + T * i;
          if (2 * m >= L) continue;
          float2 e0;
          if constexpr (PART == 2) e0 = (wsr + T * i)[ts];
          else if constexpr (B0_LDS) e0 = b0s[ts + T * i];
          else e0 = b0[i];
          const float2 zz = cscale(cadd(e0, cmul(cconj(twiddle(m, LG_M)), a[i])), inv_m);
          const float2 p1 = ld_pair<IO, VEC>(x1r, 2 * m, L);
          const float2 p2 = ld_pair<IO, VEC>(vr, 2 * m, L);
          const float2 g = ld_pair<IO, VEC>(x2r, 2 * m, L);
          const float2 out = make_float2(fmaf(g.x, zz.x, sk * (p1.x * p2.x)),
                                         fmaf(g.y, zz.y, sk * (p1.y * p2.y)));
          st_pair<IO, VEC>(yr, 2 * m, L, out);
        }
      }
    }
  }
}

template <int S, int T, typename IO, bool VEC, bool CPX, int PART>
static void launch_part(const FftconvArgs& a, int64_t row0, int64_t rows) {
  fftconv_kernel<S, T, IO, VEC, CPX, PART><<<dim3(static_cast<unsigned>(rows)), dim3(T), 0, a.stream>>>(
      static_cast<const IO*>(a.x1), static_cast<const IO*>(a.x2), static_cast<const IO*>(a.v),
      a.lam, a.res, a.N, a.skip, static_cast<IO*>(a.y), a.D, a.L,
      static_cast<float2*>(a.workspace), row0);
}

// Rows of the split form per pass through the workspace (8 S bytes each, at
// most 1 GiB).
static int64_t split_batch_rows(int64_t rows, int S) {
  const int64_t cap = (int64_t(1) << 30) / (8 * static_cast<int64_t>(S));
  return rows < cap ? rows : cap;
}

template <int S, int T, typename IO, bool VEC, bool CPX>
static void launch_k(const FftconvArgs& a) {
  const int64_t rows = static_cast<int64_t>(a.B) * a.D;
  if constexpr (S <= 2048) {
    launch_part<S, T, IO, VEC, CPX, 0>(a, 0, rows);
  } else {
    const int64_t nb = split_batch_rows(rows, S);
    for (int64_t r0 = 0; r0 < rows; r0 += nb) {
      const int64_t n = rows - r0 < nb ? rows - r0 : nb;
      launch_part<S, T, IO, VEC, CPX, 1>(a, r0, n);
      launch_part<S, T, IO, VEC, CPX, 2>(a, r0, n);
    }
  }
}

template <int S, int T, typename IO>
static hipError_t launch_s(const FftconvArgs& a, bool vec) {
  if (a.cpx)
    vec ? launch_k<S, T, IO, true, true>(a) : launch_k<S, T, IO, false, true>(a);
  else
    vec ? launch_k<S, T, IO, true, false>(a) : launch_k<S, T, IO, false, false>(a);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_io(const FftconvArgs& a, int S, bool vec) {
  switch (S) {
    // One workgroup for both halves up to S = 2048, 8 points per thread
    // wherever the workgroup size allows (at 16 points the two-half kernel
    // needs more than 256 registers per thread).  From S = 4096 on, one
    // workgroup per half, 16 points per thread: at S = 8192 that is two
    // 512-thread workgroups per CU instead of one of 1024 threads (L = 16384
    // 1.14 -> 0.89 ms at D = 4096), at S = 4096 four of 256 instead of two of
    // 512 (L = 8192 0.33 -> 0.29 ms, once the loads were branch-free); at
    // S = 2048 it made no difference.  S = 16384 needs 132 KB of LDS, one
    // workgroup per CU either way, and ran about as fast as the four-step
    // path (2.29 ms at L = 32768) with a quarter of its workspace.
    case 256: return launch_s<256, 64, IO>(a, vec);
    case 512: return launch_s<512, 64, IO>(a, vec);
    case 1024: return launch_s<1024, 128, IO>(a, vec);
    case 2048: return launch_s<2048, 256, IO>(a, vec);
    case 4096: return launch_s<4096, 256, IO>(a, vec);
    case 8192: return launch_s<8192, 512, IO>(a, vec);
    case 16384: return launch_s<16384, 1024, IO>(a, vec);
    default: return hipErrorInvalidValue;
  }
}

int fftconv_onchip_S(int64_t L) {
  int64_t half = (L + 1) / 2;
  int64_t S = 256;
  while (S < half) S <<= 1;
  return S <= 16384 ? static_cast<int>(S) : 0;
}

size_t fftconv_onchip_workspace(int64_t B, int64_t D, int64_t L) {
  const int S = fftconv_onchip_S(L);
  if (S <= 2048 || B <= 0 || D <= 0) return 0;
  return static_cast<size_t>(split_batch_rows(B * D, S) * 8 * S);
}

hipError_t launch_fftconv_onchip(const FftconvArgs& a) {
  const int S = fftconv_onchip_S(a.L);
  if (S == 0) return hipErrorInvalidValue;
  const size_t esz = a.bf16 ? 2 : 4;
  const bool vec = (a.L % 2 == 0) && aligned_all(2 * esz, a.x1, a.x2, a.v, a.y);
  return a.bf16 ? launch_io<bf16_t>(a, S, vec) : launch_io<float>(a, S, vec);
}

}  // namespace hyena
