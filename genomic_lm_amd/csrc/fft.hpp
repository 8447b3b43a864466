// fft.hpp -- Stockham radix-P complex FFT for one workgroup, gfx950.
//
// A size-S transform is held by T threads, P = S / T points each, in
// "strided natural" order: register i of thread t is element t + T*i.  Each
// Stockham pass does P/R radix-R butterflies per thread entirely in
// registers; between passes the data is exchanged through LDS (one write, one
// read, two barriers).  Input and output are both in strided natural order,
// so the caller loads from and stores to global memory coalesced without any
// extra reordering pass.  The butterflies are radix 16 where the size allows
// (the last pass takes the remaining factor), which keeps the number of LDS
// round trips at ceil(log_P S) - 1.
//
// The pass structure is the auto-sorting Stockham formulation: pass with span
// Ns and radix R reads x[j + r*S/R], multiplies by exp(-2*pi*i*r*(j mod Ns)/(Ns*R))
// and writes the length-R DFT to y[(j/Ns)*Ns*R + (j mod Ns) + r*Ns].
//
// LDS rows are padded by one complex every 32 (lds_pad), which keeps the
// 8-byte accesses of every pass within a few percent of conflict-free.
#pragma once

#include "common.hpp"

namespace hyena {

// Raw storage of one element pair [i, i+1] (4 bytes of bf16 or 8 of fp32),
// loaded without conversion so that many can be in flight in few registers;
// p must be aligned to the pair.
template <typename T> struct Raw2;
template <> struct Raw2<bf16_t> {
  uint32_t w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ float2 get() const {
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
  }
};
template <> struct Raw2<float> {
  float2 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ float2 get() const { return w; }
};

__device__ __forceinline__ int lds_pad(int i) { return i + (i >> 5); }
__host__ __device__ constexpr int lds_padded_size(int S) { return S + (S >> 5); }

// ------------------------------------------------------------- small DFTs
// Forward DFT (omega = exp(-2*pi*i/R)), natural order in and out.
template <int R> struct Dft;

template <> struct Dft<2> {
  static __device__ __forceinline__ void run(float2* v) {
    float2 a = v[0], b = v[1];
    v[0] = cadd(a, b);
    v[1] = csub(a, b);
  }
};

template <> struct Dft<4> {
  static __device__ __forceinline__ void run(float2* v) {
    float2 a0 = cadd(v[0], v[2]), a1 = csub(v[0], v[2]);
    float2 a2 = cadd(v[1], v[3]), a3 = cmul_mi(csub(v[1], v[3]));
    v[0] = cadd(a0, a2);
    v[2] = csub(a0, a2);
    v[1] = cadd(a1, a3);
    v[3] = csub(a1, a3);
  }
};

template <> struct Dft<8> {
  static __device__ __forceinline__ void run(float2* v) {
    const float r = 0.70710678118654752f;
    float2 e[4] = {v[0], v[2], v[4], v[6]};
    float2 o[4] = {v[1], v[3], v[5], v[7]};
    Dft<4>::run(e);
    Dft<4>::run(o);
    o[1] = make_float2((o[1].x + o[1].y) * r, (o[1].y - o[1].x) * r);   // * exp(-i pi/4)
    o[2] = cmul_mi(o[2]);                                                // * exp(-i pi/2)
    o[3] = make_float2((o[3].y - o[3].x) * r, -(o[3].x + o[3].y) * r);  // * exp(-3i pi/4)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = cadd(e[k], o[k]);
      v[k + 4] = csub(e[k], o[k]);
    }
  }
};

template <> struct Dft<16> {
  static __device__ __forceinline__ void run(float2* v) {
    const float c1 = 0.92387953251128674f, s1 = 0.38268343236508977f;
    const float r = 0.70710678118654752f;
    float2 e[8], o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      e[k] = v[2 * k];
      o[k] = v[2 * k + 1];
    }
    Dft<8>::run(e);
    Dft<8>::run(o);
    // o[k] *= exp(-i pi k / 8)
    o[1] = cmul(o[1], make_float2(c1, -s1));
    o[2] = make_float2((o[2].x + o[2].y) * r, (o[2].y - o[2].x) * r);
    o[3] = cmul(o[3], make_float2(s1, -c1));
    o[4] = cmul_mi(o[4]);
    o[5] = cmul(o[5], make_float2(-s1, -c1));
    o[6] = make_float2((o[6].y - o[6].x) * r, -(o[6].x + o[6].y) * r);
    o[7] = cmul(o[7], make_float2(-c1, -s1));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = cadd(e[k], o[k]);
      v[k + 8] = csub(e[k], o[k]);
    }
  }
};

__host__ __device__ constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// ------------------------------------------------------------- passes
// Radix of the pass with span NS: all of a thread's points (at most 16) in
// one butterfly, or what is left of S.
template <int S, int T, int NS>
struct PassRadix {
  static constexpr int P = S / T < 16 ? S / T : 16;
  static constexpr int value = (S / NS >= P) ? P : S / NS;
};

template <int S, int T, int R, int NS>
__device__ __forceinline__ void pass_compute(float2 (&reg)[S / T], int t) {
  constexpr int P = S / T;
  constexpr int NB = P / R;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float2 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = reg[b + r * NB];
    if constexpr (NS > 1) {
      const int j = t + T * b;
      const int k = j & (NS - 1);
      const float2 w = twiddle(k, ilog2(NS * R));
      float2 wr = w;
#pragma unroll
      for (int r = 1; r < R; ++r) {
        v[r] = cmul(v[r], wr);
        // the empty asms keep each power of w next to its use: computed all
        // ahead, the powers hold 2(R-1) more registers through the butterfly
        asm volatile("" : "+v"(v[r].x), "+v"(v[r].y));
        if (r + 1 < R) {
          wr = cmul(wr, w);
          asm volatile("" : "+v"(wr.x), "+v"(wr.y));
        }
      }
    }
    Dft<R>::run(v);
#pragma unroll
    for (int r = 0; r < R; ++r) reg[b + r * NB] = v[r];
  }
}

// The LDS addresses of a pass depend only on t and are the same in every
// transform of a kernel; t passes through an empty asm so that the compiler
// recomputes them per pass instead of keeping every pass's addresses live
// across whole kernels, which costs registers.  Within a butterfly the
// padded address is affine in r: for the index sets of these passes (a base
// whose offset within its 32-element row leaves room for r*NS, or a stride
// that is a multiple of 32) lds_pad(base + r*NS) = lds_pad(base) + r*NS +
// (r*NS >> 5); tests/test_fft_layout.py checks it for every thread of every
// instantiated shape.  So
// one padded base is computed per butterfly and the rest are immediate
// offsets.
template <int S, int T, int R, int NS>
__device__ __forceinline__ void pass_store(const float2 (&reg)[S / T], float2* lds, int t) {
  constexpr int P = S / T;
  asm volatile("" : "+v"(t));
  constexpr int NB = P / R;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = t + T * b;
    float2* row = lds + lds_pad((j / NS) * NS * R + (j & (NS - 1)));
#pragma unroll
    for (int r = 0; r < R; ++r) row[r * NS + ((r * NS) >> 5)] = reg[b + r * NB];
  }
}

template <int S, int T, int R>
__device__ __forceinline__ void pass_load(float2 (&reg)[S / T], const float2* lds, int t) {
  constexpr int P = S / T;
  constexpr int Q = S / R;
  asm volatile("" : "+v"(t));
  constexpr int NB = P / R;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float2* row = lds + lds_pad(t + T * b);
#pragma unroll
    for (int r = 0; r < R; ++r) reg[b + r * NB] = row[r * Q + ((r * Q) >> 5)];
  }
}

template <int S, int T, int NS>
__device__ __forceinline__ void fft_from(float2 (&reg)[S / T], float2* lds, int t) {
  constexpr int R = PassRadix<S, T, NS>::value;
  pass_compute<S, T, R, NS>(reg, t);
  if constexpr (NS * R < S) {
    __syncthreads();                    // earlier readers of lds are done
    pass_store<S, T, R, NS>(reg, lds, t);
    __syncthreads();
    constexpr int R2 = PassRadix<S, T, NS * R>::value;
    pass_load<S, T, R2>(reg, lds, t);
    fft_from<S, T, NS * R>(reg, lds, t);
  }
}

// Forward transform X[k] = sum_m x[m] exp(-2*pi*i*m*k/S), in place in
// registers (strided natural order), using lds (lds_padded_size(S) complex) as
// exchange space.  t is the thread's index among the T threads of this
// transform; a workgroup may run several transforms side by side (each group
// of T threads with its own lds), but every thread of the workgroup must call
// it, since the passes are separated by workgroup barriers.  On return lds may
// still be read by other threads: synchronise before writing to it.
template <int S, int T>
__device__ __forceinline__ void fft_forward(float2 (&reg)[S / T], float2* lds, int t) {
  static_assert(S % T == 0 && (S & (S - 1)) == 0, "power-of-two size, T | S");
  static_assert(S / T == 2 || S / T == 4 || S / T == 8 || S / T == 16 || S / T == 32,
                "2 to 32 points per thread");
  fft_from<S, T, 1>(reg, lds, t);
}

// Unnormalised inverse: x[m] = sum_k X[k] exp(+2*pi*i*m*k/S) = conj(F(conj X)).
template <int S, int T>
__device__ __forceinline__ void fft_inverse(float2 (&reg)[S / T], float2* lds, int t) {
#pragma unroll
  for (int i = 0; i < S / T; ++i) reg[i].y = -reg[i].y;
  fft_forward<S, T>(reg, lds, t);
#pragma unroll
  for (int i = 0; i < S / T; ++i) reg[i].y = -reg[i].y;
}

// Sequencing of the per-element loops between transforms (real-spectrum
// formation, repacking, recombination).  Issued freely, the compiler starts
// every element's LDS read and twiddle at once (4P registers on top of the 4P
// of the operands).  Each group of 4 elements
// takes its thread index through an empty asm and keeps its results with
// another; volatile asms stay in order, so group g + 1 cannot start before
// group g is done.
__device__ __forceinline__ int seq_idx(int t) {
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ void seq_keep(float2& x) { asm volatile("" : "+v"(x.x), "+v"(x.y)); }
constexpr int SEQ = 4;

// Twiddles exp(-2 pi i (a + d i) / 2^lg) of a thread's elements i = 0, 1, 2,
// ... taken in order (i a compile-time constant): every SEQ-th from
// twiddle(), whose v_cos / v_sin issue at a quarter of the vector rate, the
// ones between as the previous twiddle times `step` = twiddle(d, lg), one
// complex product (at most SEQ - 1 roundings more than twiddle's).  `w`
// carries the last twiddle from one call to the next.
__device__ __forceinline__ float2 tw_next(int i, int a, int d, int lg, float2& w, float2 step) {
  w = (i % SEQ == 0) ? twiddle(a + d * i, lg) : cmul(w, step);
  return w;
}

// LDS slot of the real-spectrum partner of element i of thread ts (k = ts +
// T i): lds_pad(kk) with kk = (S - k) mod S in the even parity half (q = 0)
// and kk = S - 1 - k in the odd one.  T i is a multiple of 32, and for C a
// multiple of 32 and 0 <= x <= C, lds_pad(C - x) = C + C/32 - x - ceil(x/32);
// so with x = ts + q one per-thread base (mirror_base) and a constant per i
// (mirror_off) give every slot, except k = 0 of the even half, whose partner
// wraps to slot 0.  tests/test_fft_layout.py checks this for every shape.
__device__ __forceinline__ int mirror_base(int ts, int q) {
  const int x = ts + q;
  return -x - ((x + 31) >> 5);
}
__host__ __device__ constexpr int mirror_off(int S, int T, int i) {
  return (S - T * i) + ((S - T * i) >> 5);
}
template <int S, int T>
__device__ __forceinline__ int mirror_slot(int base, int i, int q, int ts) {
  const int slot = base + mirror_off(S, T, i);
  return (i == 0 && q == 0 && ts == 0) ? 0 : slot;
}

// ------------------------------------------------------------- real signals
// A real length-Nfft signal x is transformed as the complex length-M signal
// c[m] = x[2m] + i x[2m+1], M = Nfft / 2.  Its spectrum X[K] (K < M) follows
// from C[K] and C[M-K]:
//   X[K] = (C[K] + conj C[M-K]) / 2 - i w (C[K] - conj C[M-K]) / 2,
//   w = exp(-2 pi i K / Nfft),
// and the inverse real transform takes the length-M complex input
//   C_z[K] = ((Z[K] + conj Z[M-K]) + i conj(w) (Z[K] - conj Z[M-K])) / 2,
// whose unnormalised inverse DFT, divided by M, is z[2m] + i z[2m+1].  At
// K = 0 the partner Z[M] (the real Nyquist bin) replaces Z[M-0].
__device__ __forceinline__ float2 real_spectrum(float2 ck, float2 cm, float2 w) {
  const float2 a = make_float2(ck.x + cm.x, ck.y - cm.y);
  const float2 b = make_float2(ck.x - cm.x, ck.y + cm.y);
  return cscale(cadd(a, cmul_mi(cmul(w, b))), 0.5f);
}

__device__ __forceinline__ float2 inverse_pack(float2 zk, float2 zm, float2 w) {
  const float2 a = make_float2(zk.x + zm.x, zk.y - zm.y);
  const float2 b = make_float2(zk.x - zm.x, zk.y + zm.y);
  return cscale(cadd(a, cmul_pi(cmul(cconj(w), b))), 0.5f);
}

}  // namespace hyena
