// fftconv_large.hip -- single-pass modal Hyena operator for L > 32768.
//
// Same operation as fftconv.hip (y = x2 * (h causal-conv u) + skip * u, the
// convolution as one zero-padded FFT product of length Nfft = 4S >= 2L:
// 'modal-form IIR via FFT', Evo2-7B-262K model card, Implementation Notes,
// 'Block dispatch'), for rows too long for one CU: beyond L = 32768 one
// parity half (S >= 32768 complex, 256 KB) no longer fits in a CU's LDS.
// The packing is the
// one of fftconv.hip: real signals as complex c[m] = x[2m] + i x[2m+1], and the
// size-M complex DFT (M = 2S) split into its two parity halves, each a size-S
// DFT of c[m] exp(-2 pi i q m / M), m < S.
//
// Each size-S DFT is taken as a four-step transform with S = S1 * S2,
// S2 = 256, m = m1 + S1 m2 and k = S2 k1 + k2:
//   1. cols_fwd: for every column m1, the size-S2 DFT over m2, then the
//      twiddle exp(-2 pi i m1 k2 / S); stored as Y[k2][m1];
//   2. rows: for every row k2, the size-S1 DFT over m1 gives the spectrum at
//      k = S2 k1 + k2.  The partner index of the real-spectrum formulas (M-K
//      in the full transform) lies, within one parity half, in one other row
//      (the "mirror row"), so one workgroup takes a row and its mirror, for u
//      and for h, forms Z = U H and the packed inverse input, runs the inverse
//      row DFTs and applies exp(+2 pi i m1 k2 / S); stored over Y_u;
//   3. cols_inv: for every column, the inverse size-S2 DFT of both parity
//      halves, their recombination c_z[m] = (B_0[m] + exp(2 pi i m / M) B_1[m]) / M,
//      and the gate, written to y.
// h is generated on chip in step 1 and never stored as a signal.  Rows are
// processed in batches through the caller's workspace: per row, the four
// size-S half spectra (u and h, two parities) as fp32 complex, 32 S bytes.
#include "common.hpp"
#include "fft.hpp"
#include "launch.hpp"

namespace hyena {

namespace {

constexpr int LG_S2 = 8;
constexpr int S2 = 1 << LG_S2;                 // column transform size
constexpr int CT = 32;                         // threads per column transform
constexpr int CP = S2 / CT;                    // points per thread (8: at 16 the
                                               // transforms need too many registers)
constexpr int GC = 16;                         // columns per workgroup
constexpr int NTC = CT * GC;                   // threads of the column kernels
constexpr int CSTRIDE = lds_padded_size(S2) + 1;   // odd stride: columns on distinct banks
constexpr int MIN_S1 = 128, MAX_S1 = 1024;
constexpr size_t BATCH_BYTES = size_t(1) << 30;    // workspace of one row batch: larger
                                                   // launches fill the chip better

// Number of mirror-row units of one row: parity 0 has rows 0 and 128 paired
// with themselves and 127 pairs (k2, 256 - k2); parity 1 has 128 pairs
// (k2, 255 - k2).
constexpr int ROW_UNITS = 129 + 128;

}  // namespace

// Column pass, forward.  Thread (t, col): t-major so that one wave touches 16
// consecutive columns of four rows (128-byte segments).
template <typename IO, bool VEC, bool CPX>
__global__ __launch_bounds__(NTC) void fftconv_cols_fwd(
    const IO* x1, const IO* v, const float* __restrict__ lam, const float* __restrict__ res,
    int N, float2* __restrict__ ws, int row0, int D, int L, int lgS1) {
  __shared__ float2 lds[GC * CSTRIDE];
  const int S1 = 1 << lgS1;
  const int lgS = lgS1 + LG_S2, lgM = lgS + 1;
  const int64_t S = int64_t(1) << lgS;
  const int tid = threadIdx.x;
  const int col = tid % GC, t = tid / GC;
  const int m1 = blockIdx.x * GC + col;
  const int sig = blockIdx.y;                  // 0: u = x1 v, 1: h
  const int rb = blockIdx.z;
  const int64_t row = row0 + rb;

  float2 d[CP];
  if (sig == 0) {
    const IO* x1r = x1 + row * L;
    const IO* vr = v + row * L;
#pragma unroll
    for (int i = 0; i < CP; ++i) {
      const int64_t m = m1 + int64_t(S1) * (t + CT * i);
      float2 p1, p2;
      if constexpr (VEC) {
        // L even: clamped pair index, zero beyond L, no branch between loads
        const int64_t e = min(2 * m, int64_t(L) - 2);
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
      d[i] = make_float2(p1.x * p2.x, p1.y * p2.y);
    }
  } else {
    // (h[2m], h[2m+1]), h[t] = (Re) sum_n R_n exp(lam_n t); a ladder of CP
    // steps of exp(2 lam S1 CT) from an exact anchor per mode
    const int c = static_cast<int>(row % D);
    constexpr int W = CPX ? 2 : 1;
    const float* lamc = lam + int64_t(c) * N * W;
    const float* resc = res + int64_t(c) * N * W;
#pragma unroll
    for (int i = 0; i < CP; ++i) d[i] = make_float2(0.0f, 0.0f);
    for (int n = 0; n < N; ++n) {
      if constexpr (CPX) {
        const CpxMode md = cpx_mode(lamc[2 * n], lamc[2 * n + 1]);
        const float2 p = cexp_at(md, 1.0f);
        const float2 step = cexp_at(md, static_cast<float>(2 * S1 * CT));
        float2 e = cmul(make_float2(resc[2 * n], resc[2 * n + 1]),
                        cexp_at(md, static_cast<float>(2 * (m1 + S1 * t))));
#pragma unroll
        for (int i = 0; i < CP; ++i) {
          d[i].x += e.x;
          d[i].y += fmaf(e.x, p.x, -e.y * p.y);   // Re(e p)
          e = cmul(e, step);
        }
      } else {
        const float l = lamc[n];
        const float p = fast_exp(l);
        const float step = fast_exp(l * static_cast<float>(2 * S1 * CT));
        float e = resc[n] * fast_exp(l * static_cast<float>(2 * (m1 + S1 * t)));
#pragma unroll
        for (int i = 0; i < CP; ++i) {
          d[i].x += e;
          d[i].y = fmaf(e, p, d[i].y);
          e *= step;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CP; ++i) {
      const int64_t m2x = 2 * (m1 + int64_t(S1) * (t + CT * i));
      if (m2x >= L) d[i].x = 0.0f;
      if (m2x + 1 >= L) d[i].y = 0.0f;
    }
  }

  float2* out = ws + (int64_t(rb) * 4 + sig * 2) * S;
  float2* lc = lds + col * CSTRIDE;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float2 a[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i)
      a[i] = q ? cmul(d[i], twiddle(m1 + S1 * (t + CT * i), lgM)) : d[i];
    fft_forward<S2, CT>(a, lc, t);
#pragma unroll
    for (int i = 0; i < CP; ++i) {
      const int k2 = t + CT * i;
      out[q * S + int64_t(k2) * S1 + m1] = cmul(a[i], twiddle(m1 * k2, lgS));
    }
  }
}

// Row pass: one workgroup per (mirror-row unit, row).  4 T threads, T = S1/8:
// the forward row transforms of u and h for the row and its mirror run side
// by side (T threads each), the spectrum product and inverse packing use all
// threads, and the two inverse row transforms take 2 T threads each.
template <int S1>
__global__ __launch_bounds__(S1 / 2) void fftconv_rows(float2* __restrict__ ws) {
  constexpr int T = S1 / 8;
  constexpr int SL = lds_padded_size(S1);
  constexpr int lgS = ilog2(S1) + LG_S2;
  constexpr int lgN = lgS + 2;
  constexpr int64_t S = int64_t(S1) * S2;
  __shared__ float2 lds[4 * SL];

  const int unit = blockIdx.x;
  const int q = unit < 129 ? 0 : 1;
  const int rA = q ? unit - 129 : unit;
  const int rB = q ? S2 - 1 - rA : (S2 - rA) & (S2 - 1);
  float2* base = ws + int64_t(blockIdx.y) * 4 * S;
  const int tid = threadIdx.x;

  {
    // slices: 0 u[rA], 1 u[rB], 2 h[rA], 3 h[rB]
    const int g = tid / T, t = tid % T;
    const int k2 = (g & 1) ? rB : rA;
    const float2* src = base + ((g >> 1) * 2 + q) * S + int64_t(k2) * S1;
    float2 a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = src[t + T * i];
    fft_forward<S1, T>(a, lds + g * SL, t);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) lds[g * SL + lds_pad(t + T * i)] = a[i];
  }
  __syncthreads();

  // element k1 = j + 2T i of row R (0: rA, 1: rB); its partner is element c1
  // of the other row
  const int R = tid / (2 * T), j = tid % (2 * T);
  const int k2 = R ? rB : rA;
  const bool row0 = (q == 0 && k2 == 0);      // the row holding K = 0 and its own partners
  const float2* own_u = lds + R * SL;
  const float2* mir_u = lds + (1 - R) * SL;
  const float2* own_h = lds + (2 + R) * SL;
  const float2* mir_h = lds + (3 - R) * SL;
  float2 z[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k1 = j + 2 * T * i;
    const int c1 = row0 ? ((S1 - k1) & (S1 - 1)) : (S1 - 1 - k1);
    const float2 w = twiddle(2 * (S2 * k1 + k2) + q, lgN);
    const float2 U = real_spectrum(own_u[lds_pad(k1)], mir_u[lds_pad(c1)], w);
    const float2 H = real_spectrum(own_h[lds_pad(k1)], mir_h[lds_pad(c1)], w);
    z[i] = cmul(U, H);
  }
  float znyq = 0.0f;                          // Z[M], real
  if (row0 && j == 0) {
    const float2 u0 = own_u[0], h0 = own_h[0];
    znyq = (u0.x - u0.y) * (h0.x - h0.y);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) lds[R * SL + lds_pad(j + 2 * T * i)] = z[i];
  __syncthreads();
  float2 cz[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k1 = j + 2 * T * i;
    const int c1 = row0 ? ((S1 - k1) & (S1 - 1)) : (S1 - 1 - k1);
    float2 zm = lds[(1 - R) * SL + lds_pad(c1)];
    if (row0 && k1 == 0) zm = make_float2(znyq, 0.0f);
    cz[i] = inverse_pack(z[i], zm, twiddle(2 * (S2 * k1 + k2) + q, lgN));
  }
  fft_inverse<S1, 2 * T>(cz, lds + R * SL, j);
  if (R == 1 && rA == rB) return;             // a row paired with itself is written once
  float2* dst = base + q * S + int64_t(k2) * S1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m1 = j + 2 * T * i;
    dst[m1] = cmul(cz[i], cconj(twiddle(m1 * k2, lgS)));
  }
}

// Column pass, inverse, with the parity recombination and the gate.
template <typename IO, bool VEC>
__global__ __launch_bounds__(NTC) void fftconv_cols_inv(
    const IO* x1, const IO* x2, const IO* v, const float* __restrict__ skip,
    IO* y, const float2* __restrict__ ws, int row0, int D, int L, int lgS1) {
  __shared__ float2 lds[GC * CSTRIDE];
  const int S1 = 1 << lgS1;
  const int lgS = lgS1 + LG_S2, lgM = lgS + 1;
  const int64_t S = int64_t(1) << lgS;
  const int tid = threadIdx.x;
  const int col = tid % GC, t = tid / GC;
  const int m1 = blockIdx.x * GC + col;
  const int rb = blockIdx.y;
  const int64_t row = row0 + rb;
  const float2* w = ws + int64_t(rb) * 4 * S;
  float2* lc = lds + col * CSTRIDE;

  float2 b0[CP];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float2 a[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i) a[i] = w[q * S + int64_t(t + CT * i) * S1 + m1];
    fft_inverse<S2, CT>(a, lc, t);
    if (q == 0) {
#pragma unroll
      for (int i = 0; i < CP; ++i) b0[i] = a[i];
    } else {
      const IO* x1r = x1 + row * L;
      const IO* x2r = x2 + row * L;
      const IO* vr = v + row * L;
      IO* yr = y + row * L;
      const float sk = skip ? skip[row % D] : 0.0f;
      const float inv_m = ldexpf(1.0f, -lgM);
      if constexpr (VEC) {
        // gate operands loaded together from clamped pair indices (L even),
        // so no branch separates the loads; pairs beyond L are not stored
        Raw2<IO> r1[CP], r2[CP], rg[CP];
#pragma unroll
        for (int i = 0; i < CP; ++i) {
          const int64_t e = min(2 * int64_t(m1 + S1 * (t + CT * i)), int64_t(L) - 2);
          r1[i].load(x1r + e);
          r2[i].load(vr + e);
          rg[i].load(x2r + e);
        }
#pragma unroll
        for (int i = 0; i < CP; ++i) {
          const int m = m1 + S1 * (t + CT * i);
          const float2 zz = cscale(cadd(b0[i], cmul(cconj(twiddle(m, lgM)), a[i])), inv_m);
          const float2 p1 = r1[i].get(), p2 = r2[i].get(), g = rg[i].get();
          const float2 out = make_float2(fmaf(g.x, zz.x, sk * (p1.x * p2.x)),
                                         fmaf(g.y, zz.y, sk * (p1.y * p2.y)));
          if (2 * int64_t(m) < L) Io<IO>::st2(yr, 2 * int64_t(m), out);
        }
      } else {
#pragma unroll
        for (int i = 0; i < CP; ++i) {
          const int m = m1 + S1 * (t + CT * i);
          if (2 * int64_t(m) >= L) continue;
          const float2 zz = cscale(cadd(b0[i], cmul(cconj(twiddle(m, lgM)), a[i])), inv_m);
          const float2 p1 = ld_pair<IO, VEC>(x1r, 2 * m, L);
          const float2 p2 = ld_pair<IO, VEC>(vr, 2 * m, L);
          const float2 g = ld_pair<IO, VEC>(x2r, 2 * m, L);
          st_pair<IO, VEC>(yr, 2 * m, L,
                           make_float2(fmaf(g.x, zz.x, sk * (p1.x * p2.x)),
                                       fmaf(g.y, zz.y, sk * (p1.y * p2.y))));
        }
      }
    }
  }
}

namespace {

// S (size of one parity half) for L, or 0 when L is outside this path
int64_t large_S(int64_t L) {
  const int64_t half = (L + 1) / 2;
  int64_t S = int64_t(MIN_S1) * S2;
  while (S < half) S <<= 1;
  return (S / S2 <= MAX_S1) ? S : 0;
}

int64_t batch_rows(int64_t rows, int64_t S, size_t bytes = 0) {
  const int64_t per_row = 32 * S;
  int64_t r = static_cast<int64_t>(bytes ? bytes : BATCH_BYTES) / per_row;
  if (r < 1) r = 1;
  return r < rows ? r : rows;
}

template <int S1>
hipError_t launch_rows(float2* ws, int nr, hipStream_t stream) {
  fftconv_rows<S1><<<dim3(ROW_UNITS, nr), S1 / 2, 0, stream>>>(ws);
  return hipGetLastError();
}

template <typename IO, bool VEC, bool CPX>
hipError_t launch_large_io(const FftconvArgs& a, int64_t S) {
  const int S1 = static_cast<int>(S / S2);
  const int lgS1 = ilog2(S1);
  const int64_t rows = int64_t(a.B) * a.D;
  const int64_t nb = batch_rows(rows, S, a.batch_bytes);
  const IO* x1 = static_cast<const IO*>(a.x1);
  const IO* x2 = static_cast<const IO*>(a.x2);
  const IO* v = static_cast<const IO*>(a.v);
  IO* y = static_cast<IO*>(a.y);
  float2* ws = static_cast<float2*>(a.workspace);
  for (int64_t r0 = 0; r0 < rows; r0 += nb) {
    const int nr = static_cast<int>(rows - r0 < nb ? rows - r0 : nb);
    fftconv_cols_fwd<IO, VEC, CPX><<<dim3(S1 / GC, 2, nr), NTC, 0, a.stream>>>(
        x1, v, a.lam, a.res, a.N, ws, static_cast<int>(r0), a.D, a.L, lgS1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (S1) {
      case 128: e = launch_rows<128>(ws, nr, a.stream); break;
      case 256: e = launch_rows<256>(ws, nr, a.stream); break;
      case 512: e = launch_rows<512>(ws, nr, a.stream); break;
      case 1024: e = launch_rows<1024>(ws, nr, a.stream); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    fftconv_cols_inv<IO, VEC><<<dim3(S1 / GC, nr), NTC, 0, a.stream>>>(
        x1, x2, v, a.skip, y, ws, static_cast<int>(r0), a.D, a.L, lgS1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t fftconv_large_workspace(int64_t B, int64_t D, int64_t L, size_t batch_bytes) {
  if (B <= 0 || D <= 0 || L <= 0) return 0;
  const int64_t S = large_S(L);
  if (S == 0 || fftconv_onchip_S(L) != 0) return 0;
  return static_cast<size_t>(batch_rows(B * D, S, batch_bytes) * 32 * S);
}

hipError_t launch_fftconv_large(const FftconvArgs& a) {
  const int64_t S = large_S(a.L);
  if (S == 0) return hipErrorInvalidValue;
  const size_t esz = a.bf16 ? 2 : 4;
  const bool vec = (a.L % 2 == 0) && aligned_all(2 * esz, a.x1, a.x2, a.v, a.y);
  if (a.cpx) {
    if (a.bf16)
      return vec ? launch_large_io<bf16_t, true, true>(a, S) : launch_large_io<bf16_t, false, true>(a, S);
    return vec ? launch_large_io<float, true, true>(a, S) : launch_large_io<float, false, true>(a, S);
  }
  if (a.bf16)
    return vec ? launch_large_io<bf16_t, true, false>(a, S) : launch_large_io<bf16_t, false, false>(a, S);
  return vec ? launch_large_io<float, true, false>(a, S) : launch_large_io<float, false, false>(a, S);
}

}  // namespace hyena
