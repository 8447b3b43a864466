// chunk_fft.hip -- chunked prefill with the modal state carried across chunks,
// the in-chunk convolution done as a zero-padded FFT of length >= 2C.
//
// For the chunk [t0, t0 + C'), C' = min(C, L - t0):
//   z[t] = sum_{k=t0}^{t} h[t-k] u[k] + sum_n R_n p_n^(t-t0+1) s_n
//   s_n <- p_n^C' s_n + sum_{j<C'} p_n^(C'-1-j) u[t0+j]
// which makes the chunked output equal the single-pass output for any C
// (TurboQuant-Bio int4 Evo 2 checkpoints, 'Important: a correctness fix comes
// with this' and 'Chunk size'; the IIR modal state is the layer's inference
// cache: Evo2-7B-262K model card, Implementation Notes, 'Custom cache').  The
// pages' engine runs the in-chunk part through an FFT buffer sized by the
// chunk ('modal-FFT buffer', TurboQuant-Bio, 'Chunk size'); here that buffer
// is LDS.
//
// One workgroup walks all chunks of one (b, c) row in order.  The spectrum of
// h[0:C) is built once per row and kept in registers; per chunk there are two
// forward and two inverse size-S transforms (S = C/2 rounded up to a power of
// two, the parity-half scheme of fftconv.hip), the rank-N carried term, and a
// workgroup reduction for the state update.
#include "common.hpp"
#include "fft.hpp"
#include "launch.hpp"
#include "pow_pair.hpp"

namespace hyena {

constexpr int CHUNK_MAXN = 64;
constexpr int CHUNK_NG = 16;             // modes per reduction group
// The state is decayed by the pole power p^C' as an fp32 pair (pow_pair.hpp)
// at every chunk length: a single fp32 factor's rounding d compounds over the
// chunks a mode remembers, 1 / (|lam| C) of them, a bias of d / (|lam| C)
// of its state -- ~1e-6 for |lam| = 1e-5 even at C = 4096, which two slow
// modes with nearly equal poles and opposite residues raise many times over
// relative to the output.  Real modes take one fp64 exp per mode and chunk;
// complex modes keep the whole-chunk pair in the registers of the thread
// that owns the mode (N <= 64 <= T) and make a pair only for a shorter last
// chunk.

// CPX: complex modes, lam and res as (re, im) pairs, complex state (B, D, N)
// as (re, im) pairs; h = Re sum_n R_n exp(lam_n t) and the carried term is
// Re sum_n R_n p_n^(t-t0+1) s_n.
template <int S, int T, typename IO, bool VEC, bool CPX>
__global__ __launch_bounds__(T) void chunk_fft_kernel(
    const IO* x1, const IO* x2, const IO* v,
    const float* __restrict__ lam, const float* __restrict__ res, int N,
    const float* __restrict__ skip, const float* state_in,
    float* state_out, IO* __restrict__ y, int D, int L, int C) {
  constexpr int P = S / T;
  constexpr int M = 2 * S;
  constexpr int LG_M = ilog2(M);
  constexpr int LG_N = LG_M + 1;
  __shared__ float2 lds[lds_padded_size(S)];
  constexpr int W = CPX ? 2 : 1;                 // floats per mode parameter / state
  static_assert(T >= CHUNK_MAXN, "each thread owns at most one mode (n = t)");
  __shared__ float s_lam[W * CHUNK_MAXN], s_res[W * CHUNK_MAXN], s_st[W * CHUNK_MAXN];
  __shared__ float s_tot[W * CHUNK_MAXN];
  constexpr int NW = T / 64;                     // waves of the workgroup
  __shared__ float red[NW * (CHUNK_NG + 1)];     // per-wave sums of one mode group

  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int c = static_cast<int>(row % D);
  const IO* x1r = x1 + row * L;
  const IO* x2r = x2 + row * L;
  const IO* vr = v + row * L;
  IO* yr = y + row * L;
  const float sk = skip ? skip[c] : 0.0f;

  const int NR = W * N;                          // real slots of the modes
  for (int n = t; n < NR; n += T) {
    s_lam[n] = lam[static_cast<int64_t>(c) * NR + n];
    s_res[n] = res[static_cast<int64_t>(c) * NR + n];
    s_st[n] = state_in ? state_in[row * NR + n] : 0.0f;
  }
  __syncthreads();

  // one step serves every twiddle ladder: exp(-2 pi i T / M) = exp(-2 pi i 2T / Nfft)
  const float2 tst = twiddle(T, LG_M);
  float2 tw = make_float2(1.0f, 0.0f);

  // ---- spectrum of h[0:C) for both parity halves, kept for every chunk
  float2 hs[2][P];
  float h_nyq = 0.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float2 a[P];
#pragma unroll
    for (int i = 0; i < P; ++i) a[i] = make_float2(0.0f, 0.0f);
    for (int n = 0; n < N; ++n) {
      if constexpr (CPX) {
        const CpxMode md = cpx_mode(s_lam[2 * n], s_lam[2 * n + 1]);
        const float2 p = cexp_at(md, 1.0f);
        const float2 step = cexp_at(md, static_cast<float>(2 * T));
        float2 e = cmul(make_float2(s_res[2 * n], s_res[2 * n + 1]),
                        cexp_at(md, static_cast<float>(2 * t)));
#pragma unroll
        for (int i = 0; i < P; ++i) {
          a[i].x += e.x;
          a[i].y += fmaf(e.x, p.x, -e.y * p.y);   // Re(e p)
          e = cmul(e, step);
        }
      } else {
        const float l = s_lam[n];
        const float p = fast_exp(l);
        const float step = fast_exp(l * static_cast<float>(2 * T));
        float e = s_res[n] * fast_exp(l * static_cast<float>(2 * t));
#pragma unroll
        for (int i = 0; i < P; ++i) {
          a[i].x += e;
          a[i].y = fmaf(e, p, a[i].y);
          e *= step;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int m = t + T * i;
      if (2 * m >= C) a[i].x = 0.0f;
      if (2 * m + 1 >= C) a[i].y = 0.0f;
      if (q) a[i] = cmul(a[i], tw_next(i, t, T, LG_M, tw, tst));
    }
    fft_forward<S, T>(a, lds, t);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = a[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int k = t + T * i;
      const int kk = q ? (S - 1 - k) : ((S - k) & (S - 1));
      hs[q][i] = real_spectrum(a[i], lds[lds_pad(kk)], tw_next(i, 2 * t + q, 2 * T, LG_N, tw, tst));
    }
    if (q == 0 && t == 0) h_nyq = a[0].x - a[0].y;
  }

  // ---- chunk-invariant mode factors, once per row: p, p^(2T), and (one
  // wave per row, up to 16 real slots) each thread's anchors of the
  // carried-term ladder p^(2t+1) and of the state-weight ladder
  // p^(2T-2-2t).  Partial chunks recompute the ladders' weights.
  __shared__ float s_p[W * CHUNK_MAXN], s_step[W * CHUNK_MAXN];
  constexpr bool TAB = (T == 64);
  __shared__ float t_ea[TAB ? CHUNK_NG * T : 1], t_wa[TAB ? CHUNK_NG * T : 1];
  const bool use_tab = TAB && NR <= CHUNK_NG;
  for (int n = t; n < N; n += T) {
    if constexpr (CPX) {
      const CpxMode md = cpx_mode(s_lam[2 * n], s_lam[2 * n + 1]);
      const float2 p = cexp_at(md, 1.0f), st = cexp_at(md, static_cast<float>(2 * T));
      s_p[2 * n] = p.x;     s_p[2 * n + 1] = p.y;
      s_step[2 * n] = st.x; s_step[2 * n + 1] = st.y;
    } else {
      const float l = s_lam[n];
      s_p[n] = fast_exp(l);
      s_step[n] = fast_exp(l * static_cast<float>(2 * T));
    }
  }
  // CPX: p^C of the mode this thread owns (n = t), as hi + lo
  float2 pc_hi = make_float2(0.0f, 0.0f), pc_lo = make_float2(0.0f, 0.0f);
  if constexpr (CPX) {
    if (t < N) pc_hi = cpow_pair(s_lam[2 * t], s_lam[2 * t + 1], static_cast<float>(C), pc_lo);
  }
  if (use_tab) {
    for (int n = 0; n < N; ++n) {
      if constexpr (CPX) {
        const CpxMode md = cpx_mode(s_lam[2 * n], s_lam[2 * n + 1]);
        const float2 ea = cexp_at(md, static_cast<float>(2 * t + 1));
        const float2 wa = cexp_at(md, static_cast<float>(2 * T - 2 - 2 * t));
        t_ea[(2 * n) * T + t] = ea.x;
        t_ea[(2 * n + 1) * T + t] = ea.y;
        t_wa[(2 * n) * T + t] = wa.x;
        t_wa[(2 * n + 1) * T + t] = wa.y;
      } else {
        const float l = s_lam[n];
        t_ea[n * T + t] = fast_exp(l * static_cast<float>(2 * t + 1));
        t_wa[n * T + t] = fast_exp(l * static_cast<float>(2 * T - 2 - 2 * t));
      }
    }
  }
  __syncthreads();

  const float inv_m = 1.0f / static_cast<float>(M);
#pragma unroll 1
  for (int t0 = 0; t0 < L; t0 += C) {
    const int Cp = min(C, L - t0);
    const int lim = t0 + Cp;
    float2 u[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int m = t + T * i;
      float2 p1, p2;
      if constexpr (VEC) {
        // L and C even: the chunk holds whole pairs; clamped pair index,
        // zero beyond its end, no branch between the loads
        const int e = min(t0 + 2 * m, lim - 2);
        Raw2<IO> r1, r2;
        r1.load(x1r + e);
        r2.load(vr + e);
        const bool in = t0 + 2 * m < lim;
        p1 = in ? r1.get() : make_float2(0.0f, 0.0f);
        p2 = in ? r2.get() : make_float2(0.0f, 0.0f);
      } else {
        p1 = ld_pair<IO, VEC>(x1r, t0 + 2 * m, lim);
        p2 = ld_pair<IO, VEC>(vr, t0 + 2 * m, lim);
      }
      u[i] = make_float2(p1.x * p2.x, p1.y * p2.y);
    }
    float2 b0[P], a[P];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int i = 0; i < P; ++i) a[i] = q ? cmul(u[i], tw_next(i, t, T, LG_M, tw, tst)) : u[i];
      fft_forward<S, T>(a, lds, t);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = a[i];
      __syncthreads();
      float2 z[P];
      float zm_nyq = 0.0f;
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int k = t + T * i;
        const int kk = q ? (S - 1 - k) : ((S - k) & (S - 1));
        z[i] = cmul(real_spectrum(a[i], lds[lds_pad(kk)], tw_next(i, 2 * t + q, 2 * T, LG_N, tw, tst)),
                    hs[q][i]);
      }
      if (q == 0 && t == 0) zm_nyq = (a[0].x - a[0].y) * h_nyq;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < P; ++i) lds[lds_pad(t + T * i)] = z[i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int k = t + T * i;
        const int kk = q ? (S - 1 - k) : ((S - k) & (S - 1));
        float2 zmir = lds[lds_pad(kk)];
        if (q == 0 && k == 0) zmir = make_float2(zm_nyq, 0.0f);
        a[i] = inverse_pack(z[i], zmir, tw_next(i, 2 * t + q, 2 * T, LG_N, tw, tst));
      }
      fft_inverse<S, T>(a, lds, t);
      if (q == 0) {
#pragma unroll
        for (int i = 0; i < P; ++i) b0[i] = a[i];
      }
    }
    // in-chunk convolution at positions t0 + 2m, t0 + 2m + 1
    float2 zz[P];
#pragma unroll
    for (int i = 0; i < P; ++i)
      zz[i] = cscale(cadd(b0[i], cmul(cconj(tw_next(i, t, T, LG_M, tw, tst)), a[i])), inv_m);

    // carried term sum_n R_n p_n^(tau+1) s_n (old state), and the state
    // partials, reduced over the workgroup 16 modes at a time
    const bool full = (Cp == 2 * S);       // ladder only when the chunk fills the frame
    // groups of CHUNK_NG real slots (a complex mode takes two: re, im)
    for (int n0 = 0; n0 < NR; n0 += CHUNK_NG) {
      const int ng = min(CHUNK_NG, NR - n0);
      if constexpr (CPX) {
        for (int g = 0; g < ng; g += 2) {
          const int n = (n0 + g) >> 1;
          const CpxMode md = cpx_mode(s_lam[2 * n], s_lam[2 * n + 1]);
          const float2 p = make_float2(s_p[2 * n], s_p[2 * n + 1]);
          const float2 step = make_float2(s_step[2 * n], s_step[2 * n + 1]);
          const float2 ea = use_tab ? make_float2(t_ea[(2 * n) * T + t], t_ea[(2 * n + 1) * T + t])
                                    : cexp_at(md, static_cast<float>(2 * t + 1));
          float2 e = cmul(cmul(make_float2(s_res[2 * n], s_res[2 * n + 1]),
                               make_float2(s_st[2 * n], s_st[2 * n + 1])), ea);
#pragma unroll
          for (int i = 0; i < P; ++i) {
            zz[i].x += e.x;
            zz[i].y += fmaf(e.x, p.x, -e.y * p.y);   // Re(e p)
            e = cmul(e, step);
          }
          // weight of position 2m+1 is p^(Cp-2-2m), of 2m it is p^(Cp-1-2m)
          float2 part = make_float2(0.0f, 0.0f);
          if (full) {
            float2 w = use_tab ? make_float2(t_wa[(2 * n) * T + t], t_wa[(2 * n + 1) * T + t])
                               : cexp_at(md, static_cast<float>(Cp - 2 - 2 * (t + T * (P - 1))));
#pragma unroll
            for (int i = P - 1; i >= 0; --i) {
              const float2 wp = cmul(w, p);
              part = make_float2(fmaf(u[i].x, wp.x, fmaf(u[i].y, w.x, part.x)),
                                 fmaf(u[i].x, wp.y, fmaf(u[i].y, w.y, part.y)));
              w = cmul(w, step);
            }
          } else {
#pragma unroll
            for (int i = 0; i < P; ++i) {
              const int m2 = 2 * (t + T * i);
              const float2 w = cexp_at(md, static_cast<float>(max(Cp - 2 - m2, 0)));
              const float2 w0 = (m2 + 1 < Cp) ? cmul(w, p) : w;   // m2 = Cp-1: weight p^0
              part = make_float2(fmaf(u[i].x, w0.x, fmaf(u[i].y, w.x, part.x)),
                                 fmaf(u[i].x, w0.y, fmaf(u[i].y, w.y, part.y)));
            }
          }
          const float sx = wave_sum(part.x), sy = wave_sum(part.y);
          if ((t & 63) == 0) {
            red[(t >> 6) * (CHUNK_NG + 1) + g] = sx;
            red[(t >> 6) * (CHUNK_NG + 1) + g + 1] = sy;
          }
        }
      } else {
        for (int g = 0; g < ng; ++g) {
          const int n = n0 + g;
          const float l = s_lam[n];
          const float p = s_p[n];
          const float step = s_step[n];
          float e = s_res[n] * s_st[n] *
                    (use_tab ? t_ea[n * T + t] : fast_exp(l * static_cast<float>(2 * t + 1)));
#pragma unroll
          for (int i = 0; i < P; ++i) {
            zz[i].x += e;
            zz[i].y = fmaf(e, p, zz[i].y);
            e *= step;
          }
          // weight of position 2m+1 is p^(Cp-2-2m), of 2m it is p^(Cp-1-2m)
          float part = 0.0f;
          if (full) {
            float w = use_tab ? t_wa[n * T + t]
                              : fast_exp(l * static_cast<float>(Cp - 2 - 2 * (t + T * (P - 1))));
#pragma unroll
            for (int i = P - 1; i >= 0; --i) {
              part = fmaf(u[i].x, w * p, part);
              part = fmaf(u[i].y, w, part);
              w *= step;
            }
          } else {
#pragma unroll
            for (int i = 0; i < P; ++i) {
              const int m2 = 2 * (t + T * i);
              const float w = fast_exp(l * static_cast<float>(max(Cp - 2 - m2, 0)));
              part = fmaf(u[i].x, (m2 + 1 < Cp) ? w * p : w, part);   // m2 = Cp-1: weight p^0
              part = fmaf(u[i].y, w, part);                              // zero beyond Cp anyway
            }
          }
          const float sw = wave_sum(part);
          if ((t & 63) == 0) red[(t >> 6) * (CHUNK_NG + 1) + g] = sw;
        }
      }
      // The partials are summed as a tree, a wave's lanes by wave_sum and
      // then the NW waves' sums: a sequential fp32 sum of the T per-thread
      // partials put ~sqrt(T) roundings of the chunk's contribution into the
      // carried state in every chunk (at C = 4096, T = 512, ~1e-6 of a slow
      // mode's state over the chunks it remembers).
      __syncthreads();                     // partials written; old state no longer read
      for (int g = t; g < ng; g += T) {
        float tot = 0.0f;
#pragma unroll
        for (int j = 0; j < NW; ++j) tot += red[j * (CHUNK_NG + 1) + g];
        const int n = n0 + g;
        if constexpr (CPX) {
          s_tot[n] = tot;                  // the complex update needs both slots
        } else {
          // made here: kept per row in LDS the pairs would cost a workgroup per CU
          const float2 pc = pow_pair(s_lam[n], static_cast<float>(Cp));
          s_st[n] = fmaf(pc.x, s_st[n], fmaf(pc.y, s_st[n], tot));
        }
      }
      __syncthreads();                     // red reusable
    }
    if constexpr (CPX) {
      for (int n = t; n < N; n += T) {
        float2 ph = pc_hi, pl = pc_lo;     // n == t: the thread's own mode
        if (Cp != C) ph = cpow_pair(s_lam[2 * n], s_lam[2 * n + 1], static_cast<float>(Cp), pl);
        const float2 so = make_float2(s_st[2 * n], s_st[2 * n + 1]);
        const float2 sn = cadd(cadd(cmul(ph, so), cmul(pl, so)),
                               make_float2(s_tot[2 * n], s_tot[2 * n + 1]));
        s_st[2 * n] = sn.x;
        s_st[2 * n + 1] = sn.y;
      }
      __syncthreads();
    }
    // gate and store
    if constexpr (VEC) {
      // every x2 pair loaded (clamped into the chunk) before the first store
      Raw2<IO> rg[P];
#pragma unroll
      for (int i = 0; i < P; ++i) rg[i].load(x2r + min(t0 + 2 * (t + T * i), lim - 2));
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int pos = t0 + 2 * (t + T * i);
        const float2 g = rg[i].get();
        const float2 out = make_float2(fmaf(g.x, zz[i].x, sk * u[i].x), fmaf(g.y, zz[i].y, sk * u[i].y));
        if (pos < lim) Io<IO>::st2(yr, pos, out);
      }
    } else {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int pos = t0 + 2 * (t + T * i);
        if (pos >= lim) continue;
        const float2 g = ld_pair<IO, VEC>(x2r, pos, lim);
        const float2 out = make_float2(fmaf(g.x, zz[i].x, sk * u[i].x), fmaf(g.y, zz[i].y, sk * u[i].y));
        st_pair<IO, VEC>(yr, pos, lim, out);
      }
    }
  }
  for (int n = t; n < NR; n += T) state_out[row * NR + n] = s_st[n];
}

int chunk_fft_S(int64_t C) {
  int64_t half = (C + 1) / 2;
  int64_t S = 256;
  while (S < half) S <<= 1;
  return S <= 4096 ? static_cast<int>(S) : 0;
}

template <int S, int T, typename IO, bool VEC, bool CPX>
static void launch_chunk_k(const ChunkArgs& a, int C) {
  chunk_fft_kernel<S, T, IO, VEC, CPX><<<dim3(static_cast<unsigned>(a.B * a.D)), dim3(T), 0, a.stream>>>(
      static_cast<const IO*>(a.x1), static_cast<const IO*>(a.x2), static_cast<const IO*>(a.v),
      a.lam, a.res, a.N, a.skip, a.state_in, a.state_out, static_cast<IO*>(a.y), a.D, a.L, C);
}

template <int S, int T, typename IO>
static hipError_t launch_chunk_s(const ChunkArgs& a, int C, bool vec) {
  if (a.cpx)
    vec ? launch_chunk_k<S, T, IO, true, true>(a, C) : launch_chunk_k<S, T, IO, false, true>(a, C);
  else
    vec ? launch_chunk_k<S, T, IO, true, false>(a, C) : launch_chunk_k<S, T, IO, false, false>(a, C);
  return hipGetLastError();
}

// Threads per row: one wave up to S = 512, then 8 points per thread.  At 16
// points per thread (S = 1024 ... 4096 on 64 ... 256 threads) the kernel
// needed all 256 registers and spilled into AGPRs, one wave per SIMD; at 8
// it fits 166-188 and C = 2048 / 4096 / 8192 at D = 4096, L = 32768 took
// 1.72 / 1.95 / 2.34 -> 0.89 / 1.18 / 1.57 ms (4 points per thread were
// slower again, and so was S = 512 on two waves).
template <typename IO>
static hipError_t launch_chunk_io(const ChunkArgs& a, int S, int C, bool vec) {
  switch (S) {
    case 256: return launch_chunk_s<256, 64, IO>(a, C, vec);
    case 512: return launch_chunk_s<512, 64, IO>(a, C, vec);
    case 1024: return launch_chunk_s<1024, 128, IO>(a, C, vec);
    case 2048: return launch_chunk_s<2048, 256, IO>(a, C, vec);
    case 4096: return launch_chunk_s<4096, 512, IO>(a, C, vec);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_fft(const ChunkArgs& a) {
  const int C = a.C < a.L ? a.C : a.L;     // a chunk longer than the sequence is one chunk
  const int S = chunk_fft_S(C);
  if (S == 0 || a.N > CHUNK_MAXN) return hipErrorInvalidValue;
  const size_t esz = a.bf16 ? 2 : 4;
  const bool vec = (a.L % 2 == 0) && (C % 2 == 0) && aligned_all(2 * esz, a.x1, a.x2, a.v, a.y);
  return a.bf16 ? launch_chunk_io<bf16_t>(a, S, C, vec) : launch_chunk_io<float>(a, S, C, vec);
}

}  // namespace hyena
