// tokmajor.hip -- the modal operator on the token-major layout that in_proj
// produces: (B, L, 3D) with each channel's three streams side by side
// (Hyena channels interleaved per triple: evo2_flash README, Limitations),
// writing y as (B, L, D), the layout out_proj consumes (evo2_flash README,
// layer_names table: 'blocks.N.projections', 'blocks.N.filter').
//
// For G consecutive channels one token's streams are one contiguous span of
// 3G elements, so a workgroup of G lanes (one lane per channel) stages tiles
// of TT token rows through LDS with coalesced 16-byte loads, and each lane
// walks its channel's tokens with the decode step's recurrence
//     s_n <- p_n s_n + u_t,   z_t = sum_n R_n s_n,   y_t = x2_t z_t + skip u_t,
// i.e. the modal state form of the causal convolution (the IIR modal state
// of the inference cache: Evo2-7B-262K model card, Implementation Notes,
// 'Custom cache').  One lane per channel alone gives D / G workgroups, far
// too few for the chip, so the sequence is also cut into P segments of TS
// tokens:
//   1. tm_states:  segment r < P-1 from a zero state; its end state e_r goes
//                  to slot r+1 of the workspace;
//   2. tm_scan:    slot 0 = state_in, slot r = p^TS slot(r-1) + e_(r-1), the
//                  true state entering segment r;
//   3. tm_outputs: every segment from its slot, emitting y; the last one's
//                  end state is state_out.
// Passes 1 and 3 both read the input: 14 bytes per token-channel at bf16
// against the 8 of the channel-major kernels, the price of the parallelism.
//
// Accuracy of the recurrence.  The step uses p_f, the pole rounded to fp32,
// and by itself would weight lag j by p_f^j = p^j (1 + j d), |d| <= 2^-24:
// over the ~1/(1 - p) tokens a slow mode remembers, that drift reaches ~1e-5
// of the output, far above the rest of the error.  So at the start of every
// full tile of K tokens the state is scaled by p^K / p_f^K, as s += g s with
// g = p^K / p_f^K - 1 from fp64 (tiny, so the fma keeps the correction exact
// to ~1e-14): the state then carries the exact decay across tiles and each
// input is off by at most K d.  What remains is the rounding of s itself,
// which decays with p_n (about sqrt(1/(1 - p_n)) ulps of the state).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace hyena {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM_THREADS = 256;                // threads per workgroup
constexpr int TM_G = 256;                      // modal kernels: channels (lanes) per workgroup
constexpr int TM_TILE_BYTES = 12 * 1024;       // modal kernels: input bytes per tile

// Staging of tiles of TT token rows of a span of G channels (3G elements)
// by TM_THREADS threads.
template <typename IO, int G, int TTOK>
struct TmShape {
  static constexpr int TT = TTOK;                       // tokens per tile
  static constexpr int ESZ = sizeof(IO);
  static constexpr int SPAN = 3 * G;                    // elements of one token row's span
  static constexpr int EPC = 16 / ESZ;                  // elements per 16-byte chunk
  static constexpr int CW = SPAN / EPC;                 // chunks per token row
  static constexpr int NCH = TT * CW;                   // chunks per tile
  static constexpr int PER = (NCH + TM_THREADS - 1) / TM_THREADS;        // per thread
  static constexpr int PER_E = (TT * SPAN + TM_THREADS - 1) / TM_THREADS;  // scalar path
  static_assert(SPAN % EPC == 0, "span");
};

// The modal kernels' tile: 12 KB of rows, 8 tokens (bf16) or 4 (f32).
template <typename IO>
using TmModal = TmShape<IO, TM_G, TM_TILE_BYTES / (3 * TM_G * int(sizeof(IO)))>;

// One tile of token rows [t0, t0 + TT) of the span [col0, col0 + cols) of
// the input, rows outside [t_lo, t_end) and columns past cols left as zeros.  VEC: 16-byte
// chunks (needs a 16-byte aligned input and rows of a multiple of 16 bytes);
// otherwise single elements.
template <typename IO, bool VEC, int G, int TT>
struct TmLoader {
  using S = TmShape<IO, G, TT>;
  static constexpr int NREG = VEC ? S::PER : S::PER_E;
  static constexpr int NITEM = VEC ? S::NCH : TT * S::SPAN;   // chunks or elements per tile
  using Reg = typename std::conditional<VEC, u32x4, IO>::type;
  Reg r[NREG];

  __device__ __forceinline__ void load(const IO* __restrict__ xb, int64_t ld, int col0, int cols,
                                       int t0, int t_end, int tid, int t_lo = 0) {
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int k = tid + TM_THREADS * i;
      if constexpr (VEC) {
        const int tt = k / S::CW, pc = k % S::CW;
        if (k < NITEM && t0 + tt >= t_lo && t0 + tt < t_end && pc * S::EPC < cols) {
          const u32x4* src =
              reinterpret_cast<const u32x4*>(xb + int64_t(t0 + tt) * ld + col0) + pc;
          r[i] = __builtin_nontemporal_load(src);
        } else {
          r[i] = u32x4{0u, 0u, 0u, 0u};
        }
      } else {
        const int tt = k / S::SPAN, e = k % S::SPAN;
        r[i] = (k < NITEM && t0 + tt >= t_lo && t0 + tt < t_end && e < cols)
                   ? xb[int64_t(t0 + tt) * ld + col0 + e]
                   : IO(0);
      }
    }
  }

  __device__ __forceinline__ void store(IO* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int k = tid + TM_THREADS * i;
      if (NITEM % TM_THREADS == 0 || k < NITEM) {
        if constexpr (VEC) reinterpret_cast<u32x4*>(tile)[k] = r[i];
        else tile[k] = r[i];
      }
    }
  }
};

// Per-lane poles for n < N: pf[n] = exp(lam_n) rounded to fp32 and the tile
// correction g[n] = p^TT / pf^TT - 1 (0 where pf is so small that the mode
// is gone within a token); zeros in the NM - N padding slots and for lanes
// past the last channel.
template <int NM, int TT>
__device__ __forceinline__ void tm_poles(const float* __restrict__ lam, int N, int c, bool live,
                                         float (&pf)[NM], float (&g)[NM]) {
#pragma unroll
  for (int n = 0; n < NM; ++n) {
    pf[n] = 0.0f;
    g[n] = 0.0f;
    if (live && n < N) {
      const double l = static_cast<double>(lam[int64_t(c) * N + n]);
      pf[n] = static_cast<float>(exp(l));
      double pk = 1.0;
#pragma unroll
      for (int k = 0; k < TT; ++k) pk *= static_cast<double>(pf[n]);
      if (pf[n] > 1e-30f && pk > 0.0) g[n] = static_cast<float>(exp(l * TT) / pk - 1.0);
    }
  }
}

// Pass 1: end state of segment r < P-1 from a zero state, to slot r+1.
// Grid (ceil(D / G), P - 1, B).
template <typename IO, bool VEC, int NM>
__global__ __launch_bounds__(TM_G) void tm_states(
    const IO* __restrict__ xin, int pos1, int posv, const float* __restrict__ lam, int N,
    float* __restrict__ ws, int D, int L, int TS, int P) {
  using S = TmModal<IO>;
  __shared__ IO tile[2][S::TT * S::SPAN];
  const int tid = threadIdx.x;
  const int col0 = 3 * TM_G * blockIdx.x;
  const int c = TM_G * blockIdx.x + tid;
  const bool live = c < D;
  const int r = blockIdx.y;
  const int b = blockIdx.z;
  const int cols = min(S::SPAN, 3 * D - col0);
  const int64_t ld = 3 * int64_t(D);
  const IO* xb = xin + int64_t(b) * L * ld;

  float pf[NM], g[NM], s[NM];
  tm_poles<NM, S::TT>(lam, N, c, live, pf, g);
#pragma unroll
  for (int n = 0; n < NM; ++n) s[n] = 0.0f;

  const int t_begin = r * TS, t_end = t_begin + TS;   // full: r < P-1
  const int o1 = 3 * tid + pos1, ov = 3 * tid + posv;
  TmLoader<IO, VEC, TM_G, S::TT> ldr;
  ldr.load(xb, ld, col0, cols, t_begin, t_end, tid);
  int buf = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += S::TT) {
    ldr.store(tile[buf], tid);
    __syncthreads();
    if (t0 + S::TT < t_end) ldr.load(xb, ld, col0, cols, t0 + S::TT, t_end, tid);
    const IO* tb = tile[buf];
    float u[S::TT];                     // the tile's inputs first: one LDS wait per tile
#pragma unroll
    for (int tt = 0; tt < S::TT; ++tt)
      u[tt] = Io<IO>::ld(tb, tt * S::SPAN + o1) * Io<IO>::ld(tb, tt * S::SPAN + ov);
#pragma unroll
    for (int n = 0; n < NM; ++n) s[n] = fmaf(g[n], s[n], s[n]);   // every tile is full
#pragma unroll
    for (int tt = 0; tt < S::TT; ++tt) {
#pragma unroll
      for (int n = 0; n < NM; ++n) s[n] = fmaf(pf[n], s[n], u[tt]);
    }
    buf ^= 1;
  }
  if (live) {
    float* dst = ws + ((int64_t(b) * P + r + 1) * D + c) * N;
#pragma unroll
    for (int n = 0; n < NM; ++n)
      if (n < N) dst[n] = s[n];
  }
}

// Pass 2: the scan over segments, one thread per (b, c, n).
__global__ __launch_bounds__(256) void tm_scan(const float* __restrict__ lam, int N,
                                               const float* state_in, float* __restrict__ ws,
                                               int D, int TS, int P, int64_t total) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t dn = int64_t(D) * N;
  const int64_t b = i / dn, cn = i % dn;        // cn = c N + n
  const float q = static_cast<float>(exp(static_cast<double>(lam[cn]) * TS));
  float s = state_in ? state_in[i] : 0.0f;
  float* w = ws + b * P * dn + cn;
  w[0] = s;
  // slots in groups of 16 independent loads, so the chain waits on memory
  // once per group instead of once per segment
  constexpr int GRP = 16;
  for (int r0 = 1; r0 < P; r0 += GRP) {
    float e[GRP];
#pragma unroll
    for (int k = 0; k < GRP; ++k) e[k] = (r0 + k < P) ? w[(r0 + k) * dn] : 0.0f;
#pragma unroll
    for (int k = 0; k < GRP; ++k) {
      if (r0 + k < P) {
        s = fmaf(q, s, e[k]);
        w[(r0 + k) * dn] = s;
      }
    }
  }
}

// Pass 3: every segment from its entering state, emitting y.  Grid
// (ceil(D / G), P, B).  With P = 1 the entering state is state_in itself
// (each lane reads its own channel's state before writing it).
template <typename IO, bool VEC, int NM>
__global__ __launch_bounds__(TM_G) void tm_outputs(
    const IO* __restrict__ xin, int pos1, int pos2, int posv, const float* __restrict__ lam,
    const float* __restrict__ res, int N, const float* __restrict__ skip, const float* state_in,
    const float* __restrict__ ws, float* state_out, IO* __restrict__ y, int D, int L, int TS,
    int P) {
  using S = TmModal<IO>;
  __shared__ IO tile[2][S::TT * S::SPAN];
  const int tid = threadIdx.x;
  const int col0 = 3 * TM_G * blockIdx.x;
  const int c = TM_G * blockIdx.x + tid;
  const bool live = c < D;
  const int r = blockIdx.y;
  const int b = blockIdx.z;
  const int cols = min(S::SPAN, 3 * D - col0);
  const int64_t ld = 3 * int64_t(D);
  const IO* xb = xin + int64_t(b) * L * ld;
  IO* yb = y + int64_t(b) * L * D + c;

  float pf[NM], g[NM], R[NM], s[NM];
  tm_poles<NM, S::TT>(lam, N, c, live, pf, g);
#pragma unroll
  for (int n = 0; n < NM; ++n) R[n] = (live && n < N) ? res[int64_t(c) * N + n] : 0.0f;
  const float* s0 = (P > 1) ? ws + ((int64_t(b) * P + r) * D + c) * N
                            : (state_in ? state_in + (int64_t(b) * D + c) * N : nullptr);
#pragma unroll
  for (int n = 0; n < NM; ++n) s[n] = (live && n < N && s0) ? s0[n] : 0.0f;
  const float sk = (live && skip) ? skip[c] : 0.0f;

  const int t_begin = r * TS, t_end = min(L, t_begin + TS);
  const int o1 = 3 * tid + pos1, o2 = 3 * tid + pos2, ov = 3 * tid + posv;
  TmLoader<IO, VEC, TM_G, S::TT> ldr;
  ldr.load(xb, ld, col0, cols, t_begin, t_end, tid);
  int buf = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += S::TT) {
    ldr.store(tile[buf], tid);
    __syncthreads();
    if (t0 + S::TT < t_end) ldr.load(xb, ld, col0, cols, t0 + S::TT, t_end, tid);
    const IO* tb = tile[buf];
    const int nt = min(S::TT, t_end - t0);
    if (nt == S::TT) {
      // a partial last tile goes uncorrected: its drift is at most nt d
#pragma unroll
      for (int n = 0; n < NM; ++n) s[n] = fmaf(g[n], s[n], s[n]);
    }
    float u[S::TT], x2[S::TT];          // the tile's inputs first: one LDS wait per tile
#pragma unroll
    for (int tt = 0; tt < S::TT; ++tt) {
      u[tt] = Io<IO>::ld(tb, tt * S::SPAN + o1) * Io<IO>::ld(tb, tt * S::SPAN + ov);
      x2[tt] = Io<IO>::ld(tb, tt * S::SPAN + o2);
    }
#pragma unroll
    for (int tt = 0; tt < S::TT; ++tt) {
      if (tt < nt) {
        float z0 = 0.0f, z1 = 0.0f;
#pragma unroll
        for (int n = 0; n < NM; n += 2) {
          s[n] = fmaf(pf[n], s[n], u[tt]);
          z0 = fmaf(R[n], s[n], z0);
          s[n + 1] = fmaf(pf[n + 1], s[n + 1], u[tt]);
          z1 = fmaf(R[n + 1], s[n + 1], z1);
        }
        if (live) Io<IO>::st_nt(yb, int64_t(t0 + tt) * D, fmaf(x2[tt], z0 + z1, sk * u[tt]));
      }
    }
    buf ^= 1;
  }
  if (r == P - 1 && live) {
    float* dst = state_out + (int64_t(b) * D + c) * N;
#pragma unroll
    for (int n = 0; n < NM; ++n)
      if (n < N) dst[n] = s[n];
  }
}

// ---------------------------------------------------------------- FIR
// The explicit-FIR operator (hcm / hcs blocks) on the same layout:
//   z[t] = sum_{k<K} w[c, k] u[t-k],  y = x2 z + skip u,
// u[t < 0] from the caller's window of the K-1 inputs before the call (or 0).
// A workgroup of 256 threads covers G = 256 / LPC channels and LPC blocks of
// TPL taps: thread (j, ch) = (tid / G, tid % G) holds taps [j TPL, (j+1) TPL)
// of channel ch, so each wave (64 consecutive channels, one tap block) touches
// LDS only across consecutive channels, free of bank conflicts.  Tiles of
// FT = 8 token rows are staged through LDS; the tile's u goes into a ring of
// RD = LPC TPL + FT token slots x G channels, from which thread (j, ch) reads
// the window u[t0 - (j+1) TPL, t0 - j TPL + FT) and forms its partial sums for
// the tile's 8 outputs; the LPC partials meet in LDS.  No state crosses
// segments: segments of TS tokens run in parallel, each starting with LPC TPL
// tokens of halo that only fill the ring.  fp32 vector work, 2K flops per
// token and channel.

// Grid (ceil(D / G), P, B); segment r covers [r TS, min(L, (r+1) TS)).
// win_out, when not null, is written by the last segment from its ring (the
// caller passes it only when no other segment still reads win_in there).
template <typename IO, bool VEC, int TPL, int LPC, int FT>
__global__ __launch_bounds__(TM_THREADS) void tm_fir(
    const IO* __restrict__ xin, int pos1, int pos2, int posv, const float* __restrict__ taps,
    int K, const float* __restrict__ skip, const float* win_in, float* win_out,
    IO* __restrict__ y, int D, int L, int TS) {
  constexpr int G = TM_THREADS / LPC;
  constexpr int TAPS = LPC * TPL;              // >= K
  constexpr int RD = TAPS + FT;                // ring slots, a multiple of FT
  constexpr int EPT = FT * G / TM_THREADS;     // (token, channel) elements per thread
  static_assert(TPL % FT == 0 && G % 64 == 0 && FT * G % TM_THREADS == 0, "shape");
  using S = TmShape<IO, G, FT>;
  __shared__ IO tile[2][FT * S::SPAN];
  __shared__ float ring[RD][G];
  __shared__ float zpart[LPC > 1 ? LPC * FT * G : 1];    // [j][i][ch]

  const int tid = threadIdx.x;
  const int j = tid / G, ch = tid % G;         // this thread's taps and channel
  const int gbase = G * static_cast<int>(blockIdx.x);
  const int r = blockIdx.y;
  const int b = blockIdx.z;
  const int col0 = 3 * gbase;
  const int cols = min(S::SPAN, 3 * D - col0);
  const int64_t ld = 3 * int64_t(D);
  const IO* xb = xin + int64_t(b) * L * ld;
  const int W = K - 1;

  float w[TPL];
  {
    const int c = gbase + ch;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const int kk = j * TPL + k;
      w[k] = (c < D && kk < K) ? taps[int64_t(c) * K + kk] : 0.0f;
    }
  }
  // elements (token i, channel ce) this thread gates: e = tid + 256 q
  float ske[EPT];
  const float* wrow[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int ce = (tid + TM_THREADS * q) % G, c = gbase + ce;
    ske[q] = (c < D && skip) ? skip[c] : 0.0f;
    wrow[q] = (c < D && win_in) ? win_in + (int64_t(b) * D + c) * W : nullptr;
  }

  const int t_begin = r * TS, t_end = min(L, t_begin + TS);
  const int t_first = t_begin - TAPS;          // halo start, a multiple of FT
  TmLoader<IO, VEC, G, FT> ldr;
  ldr.load(xb, ld, col0, cols, t_first, t_end, tid);
  int buf = 0;
  for (int t0 = t_first; t0 < t_end; t0 += FT) {
    ldr.store(tile[buf], tid);
    __syncthreads();                           // tile visible; the last tile's LDS reads done
    if (t0 + FT < t_end) ldr.load(xb, ld, col0, cols, t0 + FT, t_end, tid);
    const IO* tb = tile[buf];
    const int slot0 = (t0 - t_first) % RD;
    // u of this thread's elements into the ring; x2 kept for the gate
    float ue[EPT], x2e[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = tid + TM_THREADS * q, i = e / G, ce = e % G, t = t0 + i;
      float u = 0.0f;
      if (t >= 0) {
        u = Io<IO>::ld(tb, i * S::SPAN + 3 * ce + pos1) * Io<IO>::ld(tb, i * S::SPAN + 3 * ce + posv);
      } else if (wrow[q] && t >= -W) {
        u = wrow[q][W + t];
      }
      ue[q] = u;
      x2e[q] = Io<IO>::ld(tb, i * S::SPAN + 3 * ce + pos2);
      ring[slot0 + i][ce] = u;
    }
    __syncthreads();                           // the tile's u in the ring
    if (t0 < t_begin) {                        // uniform: halo tiles only fill the ring
      buf ^= 1;
      continue;
    }
    // window: tokens [t0 - (j+1) TPL, t0 - j TPL + FT), slot order kept by
    // whole groups of FT (the ring never splits one)
    float win[TPL + FT];
    const int tw = t0 - (j + 1) * TPL;
#pragma unroll
    for (int gq = 0; gq < TPL / FT + 1; ++gq) {
      const int s0 = (tw + FT * gq - t_first) % RD;
#pragma unroll
      for (int m = 0; m < FT; ++m) win[FT * gq + m] = ring[s0 + m][ch];
    }
    // partial sums: token t0 + i, tap j TPL + k reads u[t0 + i - j TPL - k]
    // = win[TPL + i - k]
    float z[FT];
#pragma unroll
    for (int i = 0; i < FT; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < TPL; ++k) acc = fmaf(w[k], win[TPL + i - k], acc);
      z[i] = acc;
    }
    if constexpr (LPC > 1) {
#pragma unroll
      for (int i = 0; i < FT; ++i) zpart[(j * FT + i) * G + ch] = z[i];
      __syncthreads();                         // every tap block's partials in
    }
    const int nt = min(FT, t_end - t0);
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = tid + TM_THREADS * q, i = e / G, ce = e % G;
      float zz;
      if constexpr (LPC > 1) {
        zz = zpart[i * G + ce];
#pragma unroll
        for (int jj = 1; jj < LPC; ++jj) zz += zpart[(jj * FT + i) * G + ce];
      } else {
        zz = z[q];                             // LPC = 1: element q is token q of this channel
      }
      if (i < nt && gbase + ce < D)
        Io<IO>::st_nt(y, (int64_t(b) * L + t0 + i) * D + gbase + ce, fmaf(x2e[q], zz, ske[q] * ue[q]));
    }
    buf ^= 1;
  }
  // the new window, u of tokens [L - W, L), is in the ring of the last
  // segment (its halo reaches back at least K tokens before L - 1); read
  // across consecutive channels (conflict-free), written once per call
  if (win_out && r == static_cast<int>(gridDim.y) - 1) {
    for (int e = tid; e < G * W; e += TM_THREADS) {
      const int k = e / G, cc = e % G;
      if (gbase + cc < D)
        win_out[(int64_t(b) * D + gbase + cc) * W + k] = ring[(L - W + k - t_first) % RD][cc];
    }
  }
}

// window_out[j] = e[L + j] for e = [window_in, u[0:L)], one thread per row
// (L = 0, or several segments with window_out overlapping window_in); ascending
// j reads index L + j >= j before writing j, so window_out may be window_in.
template <typename IO>
__global__ __launch_bounds__(256) void tm_fir_window(const IO* __restrict__ xin, int pos1,
                                                     int posv, const float* win_in,
                                                     float* win_out, int W, int D, int L,
                                                     int64_t rows) {
  const int64_t row = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (row >= rows) return;
  const int64_t b = row / D;
  const int c = static_cast<int>(row % D);
  const int64_t ld = 3 * int64_t(D);
  const IO* xc = xin + b * L * ld + 3 * c;
  const float* wi = win_in ? win_in + row * W : nullptr;
  float* wo = win_out + row * W;
  for (int k = 0; k < W; ++k) {
    const int64_t src = int64_t(L) + k;
    float val;
    if (src < W) {
      val = wi ? wi[src] : 0.0f;
    } else {
      const int64_t t = src - W;
      val = Io<IO>::ld(xc, t * ld + pos1) * Io<IO>::ld(xc, t * ld + posv);
    }
    wo[k] = val;
  }
}

// The same for L >= W, where every entry comes from this call's input:
// window_out[b, c, k] = u[b, L - W + k, c], one thread per entry, consecutive
// threads on consecutive channels (the reads of one token row coalesce).
// (window_in is not read, so window_out may be window_in.)
template <typename IO>
__global__ __launch_bounds__(256) void tm_fir_window_par(const IO* __restrict__ xin, int pos1,
                                                         int posv, float* __restrict__ win_out,
                                                         int W, int D, int L, int64_t total) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int c = static_cast<int>(i % D);
  const int64_t rk = i / D;
  const int k = static_cast<int>(rk % W);
  const int64_t b = rk / W;
  const int64_t ld = 3 * int64_t(D);
  const IO* xr = xin + (b * L + (L - W + k)) * ld + 3 * c;
  win_out[(b * D + c) * W + k] = Io<IO>::ld(xr, pos1) * Io<IO>::ld(xr, posv);
}

template <typename IO>
hipError_t launch_tm_fir_window(const TokmajorFirArgs& a) {
  const int W = a.K - 1;
  if (a.L >= W) {
    const int64_t total = int64_t(a.B) * W * a.D;
    tm_fir_window_par<IO><<<static_cast<unsigned>((total + 255) / 256), 256, 0, a.stream>>>(
        static_cast<const IO*>(a.xin), a.pos_x1, a.pos_v, a.win_out, W, a.D, a.L, total);
  } else {
    const int64_t rows = int64_t(a.B) * a.D;
    tm_fir_window<IO><<<static_cast<unsigned>((rows + 255) / 256), 256, 0, a.stream>>>(
        static_cast<const IO*>(a.xin), a.pos_x1, a.pos_v, a.win_in, a.win_out, W, a.D, a.L, rows);
  }
  return hipGetLastError();
}

// Tap blocks and tile lengths: K <= 8 -> one block of 8 taps, K <= 32 -> one
// block of 32 (tiles of 8 tokens); K <= 64 -> two blocks, K <= 128 -> four
// (tiles of TM_FIR_FT_WIDE tokens: longer tiles amortise the window reads
// and barriers over more fmas, measured 0.89 against 1.09 ms for K = 128 at
// D = 4096, L = 32768).
constexpr int TM_FIR_FT_WIDE = 16;
struct TmFirShape {
  int TPL, LPC, FT;
};
TmFirShape tm_fir_shape(int K) {
  if (K <= 8) return {8, 1, 8};
  if (K <= 32) return {32, 1, 8};
  if (K <= 64) return {32, 2, TM_FIR_FT_WIDE};
  return {32, 4, TM_FIR_FT_WIDE};
}

template <typename IO, bool VEC, int TPL, int LPC, int FT>
hipError_t launch_tm_fir_k(const TokmajorFirArgs& a, int TS, int P) {
  constexpr int G = TM_THREADS / LPC;
  // the FIR kernel writes the window itself unless another segment may still
  // read a window_in that window_out overlaps
  const bool want_win = a.win_out && a.K > 1;
  const size_t wbytes = size_t(a.B) * a.D * (a.K - 1) * sizeof(float);
  const auto* wi = reinterpret_cast<const char*>(a.win_in);
  const auto* wo = reinterpret_cast<const char*>(a.win_out);
  const bool overlap = wi && wo && wi < wo + wbytes && wo < wi + wbytes;
  const bool in_kernel = want_win && a.L > 0 && (!overlap || P == 1);
  if (a.L > 0) {
    tm_fir<IO, VEC, TPL, LPC, FT><<<dim3((a.D + G - 1) / G, P, a.B), TM_THREADS, 0, a.stream>>>(
        static_cast<const IO*>(a.xin), a.pos_x1, a.pos_x2, a.pos_v, a.taps, a.K, a.skip,
        a.win_in, in_kernel ? a.win_out : nullptr, static_cast<IO*>(a.y), a.D, a.L, TS);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (want_win && !in_kernel) return launch_tm_fir_window<IO>(a);
  return hipGetLastError();
}

template <typename IO, bool VEC>
hipError_t launch_tm_fir_io(const TokmajorFirArgs& a, int TS, int P) {
  if (a.K <= 8) return launch_tm_fir_k<IO, VEC, 8, 1, 8>(a, TS, P);
  if (a.K <= 32) return launch_tm_fir_k<IO, VEC, 32, 1, 8>(a, TS, P);
  if (a.K <= 64) return launch_tm_fir_k<IO, VEC, 32, 2, TM_FIR_FT_WIDE>(a, TS, P);
  return launch_tm_fir_k<IO, VEC, 32, 4, TM_FIR_FT_WIDE>(a, TS, P);
}

int tm_tile_tokens(bool bf16) { return bf16 ? TmModal<bf16_t>::TT : TmModal<float>::TT; }

template <typename IO, bool VEC, int NM>
hipError_t launch_tm(const TokmajorArgs& a, int TS, int P) {
  const IO* xin = static_cast<const IO*>(a.xin);
  const unsigned gx = static_cast<unsigned>((a.D + TM_G - 1) / TM_G);
  float* ws = static_cast<float*>(a.workspace);
  if (P > 1) {
    tm_states<IO, VEC, NM><<<dim3(gx, P - 1, a.B), TM_G, 0, a.stream>>>(
        xin, a.pos_x1, a.pos_v, a.lam, a.N, ws, a.D, a.L, TS, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = int64_t(a.B) * a.D * a.N;
    tm_scan<<<static_cast<unsigned>((total + 255) / 256), 256, 0, a.stream>>>(
        a.lam, a.N, a.state_in, ws, a.D, TS, P, total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  tm_outputs<IO, VEC, NM><<<dim3(gx, P, a.B), TM_G, 0, a.stream>>>(
      xin, a.pos_x1, a.pos_x2, a.pos_v, a.lam, a.res, a.N, a.skip, a.state_in, ws, a.state_out,
      static_cast<IO*>(a.y), a.D, a.L, TS, P);
  return hipGetLastError();
}

template <typename IO, bool VEC>
hipError_t launch_tm_modes(const TokmajorArgs& a, int TS, int P) {
  if (a.N <= 8) return launch_tm<IO, VEC, 8>(a, TS, P);
  if (a.N <= 16) return launch_tm<IO, VEC, 16>(a, TS, P);
  if (a.N <= 32) return launch_tm<IO, VEC, 32>(a, TS, P);
  return launch_tm<IO, VEC, 64>(a, TS, P);
}

}  // namespace

// Segment length: a multiple of the tile, chosen so that about TM_TARGET
// workgroups run per pass (about four per CU) when the shape allows it, and
// at least TM_MIN_SEG tokens, so that the per-segment state traffic (4 N
// floats per channel through the workspace) stays small next to the input.
void tokmajor_segments(int64_t B, int64_t D, int64_t L, bool bf16, int* TS, int* P) {
  constexpr int64_t TM_TARGET = 1024;
  constexpr int64_t TM_MIN_SEG = 64;
  const int64_t tt = tm_tile_tokens(bf16);
  const int64_t groups = B * ((D + TM_G - 1) / TM_G);
  int64_t want = (TM_TARGET + groups - 1) / groups;
  if (want < 1) want = 1;
  int64_t ts = (L + want - 1) / want;
  if (ts < TM_MIN_SEG) ts = TM_MIN_SEG;
  ts = (ts + tt - 1) / tt * tt;
  *TS = static_cast<int>(ts);
  *P = static_cast<int>((L + ts - 1) / ts);
}

size_t tokmajor_workspace(int64_t B, int64_t D, int64_t L, int64_t N, bool bf16) {
  if (B <= 0 || D <= 0 || L <= 0 || N <= 0) return 0;
  int TS = 0, P = 0;
  tokmajor_segments(B, D, L, bf16, &TS, &P);
  return P > 1 ? static_cast<size_t>(B * P * D * N) * sizeof(float) : 0;
}

// FIR: G = 256 / LPC channels per workgroup; segments a multiple of the tile,
// at least 8 times the halo (LPC TPL tokens), cut for about TM_TARGET
// workgroups.
void tokmajor_fir_segments(int64_t B, int64_t D, int64_t L, int K, int* TS, int* P) {
  constexpr int64_t TM_TARGET = 1024;
  const TmFirShape sh = tm_fir_shape(K);
  const int64_t G = TM_THREADS / sh.LPC;
  const int64_t groups = B * ((D + G - 1) / G);
  int64_t want = (TM_TARGET + groups - 1) / groups;
  if (want < 1) want = 1;
  int64_t ts = (L + want - 1) / want;
  const int64_t lo = 8 * sh.LPC * sh.TPL > 64 ? 8 * sh.LPC * sh.TPL : 64;
  if (ts < lo) ts = lo;
  ts = (ts + sh.FT - 1) / sh.FT * sh.FT;
  *TS = static_cast<int>(ts);
  *P = static_cast<int>(L > 0 ? (L + ts - 1) / ts : 0);
}

hipError_t launch_tokmajor_fir(const TokmajorFirArgs& a) {
  // bf16 with more than 32 taps: the matrix-core kernel (fir_mfma.hip), then
  // the window kernel.  The fp32 tap loop below costs 2K flops per token and
  // channel; the matrix-core kernel's cost hardly depends on K.  Measured at
  // B=1 D=4096 L=32768 (ms, tap loop / matrix cores): K=7 0.211/0.446,
  // K=20 0.368/0.453, K=33 0.496/0.457, K=64 0.510/0.480, K=128 0.788/0.517.
  if (a.K > 32 && tokmajor_fir_mfma_supported(a)) {
    hipError_t e = launch_fir_mfma_tokmajor(a);
    if (e != hipSuccess || !a.win_out) return e;
    return launch_tm_fir_window<bf16_t>(a);
  }
  int TS = 0, P = 0;
  tokmajor_fir_segments(a.B, a.D, a.L, a.K, &TS, &P);
  const size_t esz = a.bf16 ? 2 : 4;
  const bool vec = aligned_to(a.xin, 16) && (3 * static_cast<size_t>(a.D) * esz) % 16 == 0;
  if (a.bf16)
    return vec ? launch_tm_fir_io<bf16_t, true>(a, TS, P) : launch_tm_fir_io<bf16_t, false>(a, TS, P);
  return vec ? launch_tm_fir_io<float, true>(a, TS, P) : launch_tm_fir_io<float, false>(a, TS, P);
}

hipError_t launch_tokmajor(const TokmajorArgs& a) {
  int TS = 0, P = 0;
  tokmajor_segments(a.B, a.D, a.L, a.bf16, &TS, &P);
  const size_t esz = a.bf16 ? 2 : 4;
  const bool vec = aligned_to(a.xin, 16) && (3 * static_cast<size_t>(a.D) * esz) % 16 == 0;
  if (a.bf16)
    return vec ? launch_tm_modes<bf16_t, true>(a, TS, P) : launch_tm_modes<bf16_t, false>(a, TS, P);
  return vec ? launch_tm_modes<float, true>(a, TS, P) : launch_tm_modes<float, false>(a, TS, P);
}

}  // namespace hyena
