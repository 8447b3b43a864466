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
// against the 48 of the four-step path that rows longer than 32768 take.  h
// never touches memory: the split halves form it on the matrix cores as a
// rank-N product (modal_pairs_mfma, modal_pairs_mfma_cpx), the other kernels
// per thread with short exp ladders (<= 16 multiplications from an exact
// anchor).
#include "common.hpp"
#include "fft.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace hyena {

// a[i] = (h[2m], h[2m+1]) for m = t + T*i, zero at and beyond L.
template <int P, int T>
__device__ __forceinline__ void modal_pairs(float2 (&a)[P], const float* lam, const float* res,
                                            int N, int t, int L) {
#pragma unroll
  for (int i = 0; i < P; ++i) a[i] = make_float2(0.0f, 0.0f);
  for (int n = 0; n < N; ++n) {
    const float l = lam[n];
    const float p = fast_exp(l);
    const float step = fast_exp(l * static_cast<float>(2 * T));
    float e = res[n] * fast_exp(l * static_cast<float>(2 * t));
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

// Eight values of an MFMA operand (one lane's K slots), each split into
// three bf16 parts x = p0 + p1 + p2 + O(2^-24 x), packed two per word.
struct Split3x8 {
  uint32_t p[3][4];
  __device__ __forceinline__ void set(int j2, float a, float b) {   // slots 2 j2, 2 j2 + 1
    split3_pair(a, b, p[0][j2], p[1][j2], p[2][j2]);
  }
  __device__ __forceinline__ bf16x8 part(int k) const {
    const u32x4 q = {p[k][0], p[k][1], p[k][2], p[k][3]};
    return __builtin_bit_cast(bf16x8, q);
  }
};

// acc + X Y over the part products of order <= 2 (X0Y0, X0Y1, X1Y0, X1Y1,
// X0Y2, X2Y0), the smallest first: about 2^-24 relative per term.
__device__ __forceinline__ f32x16 mfma_split3(const Split3x8& x, const Split3x8& y, f32x16 acc) {
  acc = mfma(x.part(2), y.part(0), acc);
  acc = mfma(x.part(0), y.part(2), acc);
  acc = mfma(x.part(1), y.part(1), acc);
  acc = mfma(x.part(1), y.part(0), acc);
  acc = mfma(x.part(0), y.part(1), acc);
  return mfma(x.part(0), y.part(0), acc);
}

// a[i] = (de[i], dd[i]), zero at and beyond L (pairs m = t + T i).
template <int T>
__device__ __forceinline__ void pairs_from(float2 (&a)[16], const f32x16& de, const f32x16& dd,
                                           int t, int L) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m2 = 2 * (t + T * i);
    a[i] = make_float2(m2 < L ? de[i] : 0.0f, m2 + 1 < L ? dd[i] : 0.0f);
  }
}

// Exponents of a lane's A row and B column in the 32x32x16 products below
// (lane l of wave w, t = 64 w + l): row rho = l % 32 stands for point i =
// 4(rho/8) + rho%4 of half-wave (rho/4)%2, column c = l % 32 for t = 64 w + c.
template <int T>
__device__ __forceinline__ float row_exponent(int t) {
  const int rho = t & 31;
  return static_cast<float>(64 * ((rho >> 2) & 1) + 2 * T * (4 * (rho >> 3) + (rho & 3)));
}
__device__ __forceinline__ float col_exponent(int t) {
  return static_cast<float>(2 * ((t & ~63) + (t & 31)));
}

// The same pairs on the matrix cores, for 16 points per thread (T a multiple
// of 64, every thread of the wave calling).  With t = 64 w + l, lane l of
// wave w needs h at 2m and 2m + 1 for m = t + T i, i < 16, and
//   h[2m] = sum_n R_n p_n^(2(64w + l%32)) * p_n^(64 (l/32) + 2T i),
// a product over the modes of Y[n][c] = p_n^(2(64w + c)) (c < 32, one column
// per lane pair) and X[rho][n] = R_n p_n^(64 hf + 2T i) (32 rows rho, each a
// pair (i, hf)), h[2m + 1] the same with X p_n.  The rows are numbered so
// that register r of a lane in half-wave hf of the 32x32 result (row
// 8(r/4) + 4hf + r%4) is point i = r: rho gives i = 4(rho/8) + rho%4 and hf =
// (rho/4)%2.  X, X p and Y are split into three bf16 parts (mfma_split3), 16
// modes per block of 12 MFMAs.  This replaces 16 x 3 vector operations per
// mode and point of the ladder above.
template <int T>
__device__ __forceinline__ void modal_pairs_mfma(float2 (&a)[16], const float* lam, const float* res,
                                                 int N, int t, int L) {
  static_assert(T % 64 == 0, "whole waves");
  const int hf = (t & 63) >> 5;
  const float xe = row_exponent<T>(t);
  const float ye = col_exponent(t);
  f32x16 de = {}, dd = {};
  for (int n0 = 0; n0 < N; n0 += 16) {
    Split3x8 x, o, y;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      float xv[2], ov[2], yv[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int n = n0 + 8 * hf + j + k;
        const bool live = n < N;
        const int nc = live ? n : 0;
        const float lm = live ? lam[nc] : 0.0f;
        const float r = live ? res[nc] : 0.0f;
        xv[k] = r * fast_exp(lm * xe);
        ov[k] = r * fast_exp(lm * (xe + 1.0f));
        yv[k] = live ? fast_exp(lm * ye) : 0.0f;
      }
      x.set(j / 2, xv[0], xv[1]);
      o.set(j / 2, ov[0], ov[1]);
      y.set(j / 2, yv[0], yv[1]);
    }
    de = mfma_split3(x, y, de);
    dd = mfma_split3(o, y, dd);
  }
  pairs_from<T>(a, de, dd, t, L);
}

// The same for complex modes (lam, res as (re, im) pairs): Re(R p^(a+b)) =
// Re(R p^a) Re(p^b) - Im(R p^a) Im(p^b), so each mode takes two of the
// product's 16 K slots (slot 8 hf + j of a lane: mode 4 hf + j/2, its real
// part for even j), 8 modes per block, with X = (Re, -Im) of R p^(64 hf +
// 2T i) and Y = (Re, Im) of p^(2(64w + c)).
template <int T>
__device__ __forceinline__ void modal_pairs_mfma_cpx(float2 (&a)[16], const float* lam,
                                                     const float* res, int N, int t, int L) {
  static_assert(T % 64 == 0, "whole waves");
  const int hf = (t & 63) >> 5;
  const float xe = row_exponent<T>(t);
  const float ye = col_exponent(t);
  f32x16 de = {}, dd = {};
  for (int n0 = 0; n0 < N; n0 += 8) {
    Split3x8 x, o, y;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * hf + j;
      const bool live = n < N;
      const int nc = live ? n : 0;
      const CpxMode md = cpx_mode(live ? lam[2 * nc] : 0.0f, live ? lam[2 * nc + 1] : 0.0f);
      const float2 r = live ? make_float2(res[2 * nc], res[2 * nc + 1]) : make_float2(0.0f, 0.0f);
      const float2 xv = cmul(r, cexp_at(md, xe));
      const float2 ov = cmul(r, cexp_at(md, xe + 1.0f));
      const float2 yv = live ? cexp_at(md, ye) : make_float2(0.0f, 0.0f);
      x.set(j, xv.x, -xv.y);
      o.set(j, ov.x, -ov.y);
      y.set(j, yv.x, yv.y);
    }
    de = mfma_split3(x, y, de);
    dd = mfma_split3(o, y, dd);
  }
  pairs_from<T>(a, de, dd, t, L);
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
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(PART == 0 ? 1 : 4))) void fftconv_kernel(
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
  // one step serves every ladder below: exp(-2 pi i T / M) = exp(-2 pi i 2T / Nfft)
  const float2 tst = twiddle(T, LG_M);
  float2 tw = make_float2(1.0f, 0.0f);
#pragma unroll
  for (int q = Q0; q <= Q1; ++q) {
    float2 a[P];
    float2 z[P];
    int ts = t;
    // Split halves (one to four workgroups per CU, at most one from
    // S = 16384 on) take h first; bf16 rows then issue the loads of u right
    // after h is generated and transform h while they are in flight: nothing
    // else on the CU would hide their latency.  The pending pairs hold 2P
    // registers, as many as the first spectrum holds through the second
    // transform either way.
    constexpr bool H_FIRST = PART != 0;
    constexpr bool EARLY_U = H_FIRST && VEC && sizeof(IO) == 2;
    Raw2<IO> r1[EARLY_U ? P : 1], r2[EARLY_U ? P : 1];
    float hm_nyq = 0.0f, um_nyq = 0.0f;   // H[M], U[M] (real), only used by thread 0
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      // pass 0 transforms u and pass 1 h, or the other way round (H_FIRST)
      const bool is_h = H_FIRST ? pass == 0 : pass == 1;
      if (is_h) {
        // ---- h, generated on chip, packed in pairs
        if constexpr (CPX && P == 16)
          modal_pairs_mfma_cpx<T>(a, lamc, resc, N, t, L);
        else if constexpr (CPX)
          modal_pairs_cpx<P, T>(a, lamc, resc, N, t, L);
        else if constexpr (P == 16)
          modal_pairs_mfma<T>(a, lamc, resc, N, t, L);
        else
          modal_pairs<P, T>(a, lamc, resc, N, t, L);
        if constexpr (EARLY_U) {
#pragma unroll
          for (int i = 0; i < P; ++i) {
            const int64_t e = min(2 * (t + T * i), L - 2);
            r1[i].load(x1r + e);
            r2[i].load(vr + e);
          }
        }
      } else {
        // ---- u = x1 * v, packed in pairs
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int m = t + T * i;
          float2 p1, p2;
          if constexpr (EARLY_U) {
            const bool in = 2 * m < L;
            p1 = in ? r1[i].get() : make_float2(0.0f, 0.0f);
            p2 = in ? r2[i].get() : make_float2(0.0f, 0.0f);
          } else if constexpr (VEC) {
            // L even: clamped pair index, zero beyond L without a branch
            const int64_t e = min(2 * m, L - 2);
            Raw2<IO> l1, l2;
            l1.load(x1r + e);
            l2.load(vr + e);
            const bool in = 2 * m < L;
            p1 = in ? l1.get() : make_float2(0.0f, 0.0f);
            p2 = in ? l2.get() : make_float2(0.0f, 0.0f);
          } else {
            p1 = ld_pair<IO, VEC>(x1r, 2 * m, L);
            p2 = ld_pair<IO, VEC>(vr, 2 * m, L);
          }
          a[i] = make_float2(p1.x * p2.x, p1.y * p2.y);
        }
      }
      // parity pre-twiddle
      if (q) {
#pragma unroll
        for (int i = 0; i < P; ++i) a[i] = cmul(a[i], tw_next(i, t, T, LG_M, tw, tst));
      }
      fft_forward<S, T>(a, lds, t);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = a[i];
      __syncthreads();
      // real spectrum; the second transform's is multiplied into the first's
      int mb = 0;
#pragma unroll
      for (int i = 0; i < P; ++i) {
        if (i % SEQ == 0) {
          ts = seq_idx(t);
          mb = mirror_base(ts, q);
        }
        const float2 x = real_spectrum(a[i], lds[mirror_slot<S, T>(mb, i, q, ts)],
                                       tw_next(i, 2 * ts + q, 2 * T, LG_N, tw, tst));
        z[i] = pass == 0 ? x : cmul(z[i], x);
        seq_keep(z[i]);
      }
      if (q == 0 && t == 0) (is_h ? hm_nyq : um_nyq) = a[0].x - a[0].y;
    }
    if (q == 0 && t == 0) zm_nyq = um_nyq * hm_nyq;

    // ---- repack Z for the inverse real transform
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = z[i];
    __syncthreads();
    int mb = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (i % SEQ == 0) {
        ts = seq_idx(t);
        mb = mirror_base(ts, q);
      }
      const int k = ts + T * i;
      float2 zmir = lds[mirror_slot<S, T>(mb, i, q, ts)];
      if (q == 0 && k == 0) zmir = make_float2(zm_nyq, 0.0f);
      a[i] = inverse_pack(z[i], zmir, tw_next(i, 2 * ts + q, 2 * T, LG_N, tw, tst));
      seq_keep(a[i]);
    }
    // The gate's operands of a group of GG points (B_0, x1, v, x2), loaded
    // together from pair indices clamped into the row.  The odd half issues
    // the workspace loads of its first group before the inverse transform,
    // whose passes then hide their latency (2 GG registers).
    constexpr int GG = P < 8 ? P : 8;
    constexpr bool PRE_GATE = PART == 2 && VEC;
    Raw2<IO> g1[GG], g2[GG], gg[GG];
    float2 ge[GG];
    auto load_b0 = [&](int g0, int tt) {
#pragma unroll
      for (int j = 0; j < GG; ++j) {
        const int i = g0 + j;
        if constexpr (PART == 2) ge[j] = (wsr + T * i)[tt];
        else if constexpr (B0_LDS) ge[j] = b0s[tt + T * i];
        else ge[j] = b0[i];
      }
    };
    auto load_acts = [&](int g0, int tt) {
#pragma unroll
      for (int j = 0; j < GG; ++j) {
        const int64_t e = min(2 * (tt + T * (g0 + j)), L - 2);
        g1[j].load(x1r + e);
        g2[j].load(vr + e);
        gg[j].load(x2r + e);
      }
    };
    if constexpr (PRE_GATE) load_b0(0, t);
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
        // L is even: pair m is whole for 2m < L and absent beyond.  No
        // branch separates a group's loads and none waits for an earlier
        // element's store; pairs beyond L are not stored.
#pragma unroll
        for (int g0 = 0; g0 < P; g0 += GG) {
          ts = seq_idx(t);
          if (!PRE_GATE || g0 > 0) load_b0(g0, ts);
          load_acts(g0, ts);
#pragma unroll
          for (int j = 0; j < GG; ++j) {
            const int m = ts + T * (g0 + j);
            const float2 zz = cscale(cadd(ge[j], cmul(cconj(tw_next(g0 + j, ts, T, LG_M, tw, tst)),
                                                      a[g0 + j])), inv_m);
            const float2 p1 = g1[j].get(), p2 = g2[j].get(), g = gg[j].get();
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
          const float2 wm = tw_next(i, ts, T, LG_M, tw, tst);     // the ladder advances for every i
          if (2 * m >= L) continue;
          float2 e0;
          if constexpr (PART == 2) e0 = (wsr + T * i)[ts];
          else if constexpr (B0_LDS) e0 = b0s[ts + T * i];
          else e0 = b0[i];
          const float2 zz = cscale(cadd(e0, cmul(cconj(wm), a[i])), inv_m);
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
// most `bytes`, 1 GiB by default).
static int64_t split_batch_rows(int64_t rows, int S, size_t bytes = 0) {
  const size_t b = bytes ? bytes : (size_t(1) << 30);
  int64_t cap = static_cast<int64_t>(b / (8 * static_cast<size_t>(S)));
  if (cap < 1) cap = 1;
  return rows < cap ? rows : cap;
}

template <int S, int T, typename IO, bool VEC, bool CPX>
static void launch_k(const FftconvArgs& a) {
  const int64_t rows = static_cast<int64_t>(a.B) * a.D;
  if constexpr (S <= 2048) {
    launch_part<S, T, IO, VEC, CPX, 0>(a, 0, rows);
  } else {
    const int64_t nb = split_batch_rows(rows, S, a.batch_bytes);
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

size_t fftconv_onchip_workspace(int64_t B, int64_t D, int64_t L, size_t batch_bytes) {
  const int S = fftconv_onchip_S(L);
  if (S <= 2048 || B <= 0 || D <= 0) return 0;
  return static_cast<size_t>(split_batch_rows(B * D, S, batch_bytes) * 8 * S);
}

hipError_t launch_fftconv_onchip(const FftconvArgs& a) {
  const int S = fftconv_onchip_S(a.L);
  if (S == 0) return hipErrorInvalidValue;
  const size_t esz = a.bf16 ? 2 : 4;
  const bool vec = (a.L % 2 == 0) && aligned_all(2 * esz, a.x1, a.x2, a.v, a.y);
  return a.bf16 ? launch_io<bf16_t>(a, S, vec) : launch_io<float>(a, S, vec);
}

}  // namespace hyena
