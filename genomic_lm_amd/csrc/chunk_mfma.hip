// chunk_mfma.hip -- chunked prefill with carried modal state on the matrix cores.
//
// Same function as chunk_fft.hip (see there for the chunk recurrence and its
// sources), computed as a blocked Toeplitz product.  Because the filter is a
// sum of N exponentials, the state s_n at any block boundary carries all of
// the past exactly, so the sequence is cut into 32-token blocks and
//
//   z[blk][i] = sum_{j<=i} h[i-j] u[blk][j]                 (Toeplitz T, 32x32)
//             + sum_n R_n p_n^(i+1) s_n(before blk)           (G, 32xN)
//   e[blk][n] = sum_j p_n^(31-j) u[blk][j]                    (block-local end state)
//   s(after blk) = p^32 s(before blk) + e[blk]                (scan over blocks)
//
// Chunk boundaries at any multiple of C fall on exact states of this
// recurrence, so the output is the same for every C and equal to the single
// pass (TurboQuant-Bio int4 Evo 2 checkpoints, 'Chunk size': fidelity does not
// depend on the chunk size).
//
// Mapping: one 64-lane wave per (b, c) row, 1024-token tiles (32 blocks x 32
// tokens) walked in order.  Per tile: T.U, G.S and the transposed E^T = U^T.P^T
// are v_mfma_f32_32x32x16_bf16 products of fp32 operands split into three
// bf16 parts x = x0 + x1 + x2 (each the rounded remainder of the previous);
// every product keeps the part pairs of order <= 2 (x0y0, x0y1, x1y0, x1y1,
// x0y2, x2y0), which leaves ~2^-24 relative error per term, fp32-like.
// u = x1*v of two bf16 values is exactly u0 + u1; fp32 inputs take three
// parts.  22 MFMAs per 1024-token tile for bf16 I/O.
// The contraction index of T.U is permuted so that each lane's B-operand
// tokens are exactly the tokens of its output rows: u, x2 and y move in 8-byte
// runs of 4 tokens and never cross lanes.  The scan runs one mode (hi or lo
// part) per lane: 4 runs of 4 blocks in registers, 8 run carries exchanged
// with the partner half-wave.  The state before each block goes through 4 KB
// of LDS to become the B operand of G.S.
//
// Complex modes (CPX; the complex-pole form of Evo 1's poles / residues,
// Evo1-1.5-7B-8K model card, Architecture): N <= 8 complex modes occupy the
// 16 slots as (Re, Im) pairs, slot 2m + k -- the order of the (D, N, 2)
// parameter and (B, D, N, 2) state arrays.  Every product stays real:
// Re(R p^(i+1) s) = Re(R p^(i+1)) Re s - Im(R p^(i+1)) Im s gives G's two
// columns of a mode, the end-state weights are Re and Im of p^(31-j), and h is
// real.  Only the scan mixes a slot pair (multiplying by p^32 is a complex
// product): each step takes the partner slot's value from lane l ^ 1.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace hyena {

// The three bf16 parts (split3) of the 16 operand slots (s, j) of one lane,
// val(s, j) -> parts[k][s][j], formed two slots at a time (one packed
// conversion per pair; the same bits as split3 value by value).
template <typename F>
__device__ __forceinline__ void split3_slots(F&& val, bf16x8 (&parts)[3][2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    u32x4 w0, w1, w2;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t a, b, c;
      split3_pair(val(s, 2 * jj), val(s, 2 * jj + 1), a, b, c);
      w0[jj] = a;
      w1[jj] = b;
      w2[jj] = c;
    }
    parts[0][s] = __builtin_bit_cast(bf16x8, w0);
    parts[1][s] = __builtin_bit_cast(bf16x8, w1);
    parts[2][s] = __builtin_bit_cast(bf16x8, w2);
  }
}

// B operands of E^T = U^T . P^T for one lane: column nn (mode nn & 15, part
// nn >> 4), slots (s, j) -> token blk_tok(8s + j, hf), from the weights
// w(tok) = p^(ref - tok) for tok <= ref, else 0, split as w0 + w1 + w2.
// Summing columns n and n + 16 of  U0.A + U1.A + U0.B (+ U2.C)  gives every
// product of order <= 2:  A = [w0 | w1], B = [w2 | 0], C = [w0 | 0].
template <typename F>
__device__ __forceinline__ void state_weight_operands(F&& w, int part, int hf, int ref,
                                                      bf16x8 (&pa)[2], bf16x8 (&pb)[2],
                                                      bf16x8 (&pc)[2]) {
  bf16x8 parts[3][2];
  split3_slots(
      [&](int s, int j) {
        const int tok = blk_tok(8 * s + j, hf);
        return (tok <= ref) ? w(ref - tok) : 0.0f;
      },
      parts);
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const u32x4 q0 = __builtin_bit_cast(u32x4, parts[0][s]);
    const u32x4 q1 = __builtin_bit_cast(u32x4, parts[1][s]);
    const u32x4 q2 = __builtin_bit_cast(u32x4, parts[2][s]);
    pa[s] = __builtin_bit_cast(bf16x8, part ? q1 : q0);
    pb[s] = __builtin_bit_cast(bf16x8, part ? zero : q2);
    pc[s] = __builtin_bit_cast(bf16x8, part ? zero : q0);
  }
}

__device__ __forceinline__ void build_state_weights(float lam_n, int part, int hf, int ref,
                                                    bf16x8 (&pa)[2], bf16x8 (&pb)[2],
                                                    bf16x8 (&pc)[2]) {
  state_weight_operands([&](int d) { return expf(lam_n * static_cast<float>(d)); }, part, hf,
                        ref, pa, pb, pc);
}

// The same weights for complex mode `md`: slot component k takes Re (k = 0)
// or Im (k = 1) of p^(ref - tok).
__device__ __forceinline__ void build_state_weights_cpx(const CpxMode& md, int k, int part,
                                                        int hf, int ref, bf16x8 (&pa)[2],
                                                        bf16x8 (&pb)[2], bf16x8 (&pc)[2]) {
  state_weight_operands(
      [&](int d) {
        const float2 e = cexp_at(md, static_cast<float>(d));
        return k ? e.y : e.x;
      },
      part, hf, ref, pa, pb, pc);
}

// VEC: rows of whole 16-byte chunks, 16-byte aligned (full tiles take the
// unchecked path).  PIPE (bf16, VEC, L >= 2048): at least two full tiles, so
// the first two DMAs are issued without a branch.  CPX: N complex modes as
// 2N slots (above).
template <typename IO, bool VEC, bool PIPE, bool CPX>
__global__ __launch_bounds__(64) void chunk_mfma_kernel(
    const IO* __restrict__ x1, const IO* __restrict__ x2, const IO* __restrict__ v,
    const float* __restrict__ lam, const float* __restrict__ res, int N,
    const float* __restrict__ skip, const float* state_in,
    float* state_out, IO* __restrict__ y, int D, int L) {
  // parts of u: x1*v of two bf16 values is exactly two bf16 parts
  constexpr int NU = (sizeof(IO) == 2) ? 2 : 3;
  __shared__ float hbuf[32];
  // state before block b, per part and mode (row 32: unused); two copies
  // used by alternate tiles, so a tile's writes never meet the previous
  // tile's reads
  __shared__ float sbufs[1][2][33][17];
  // staged x1, v, x2 tiles (bf16, swizzled chunks), two tiles in turn, and
  // the staged y tile
  __shared__ uint4 tin_a[3][128], tin_b[3][128];
  __shared__ uint4 tout[128];

  const int l = threadIdx.x;
  const int hf = l >> 5;                      // half-wave
  const int i32 = l & 31;                     // row of A / column of B and C
  const int64_t row = blockIdx.x;
  const int c = static_cast<int>(row % D);
  const int NS = CPX ? 2 * N : N;             // slots: floats per channel of lam, res, state
  const float* lamc = lam + static_cast<int64_t>(c) * NS;
  const float* resc = res + static_cast<int64_t>(c) * NS;
  const IO* x1r = x1 + row * L;
  const IO* x2r = x2 + row * L;
  const IO* vr = v + row * L;
  IO* yr = y + row * L;
  const float sk = skip ? skip[c] : 0.0f;
  const int lane_off = 32 * i32 + 4 * hf;     // token offset of run 0 within a tile
  const int nfull = VEC ? (L >> 10) : 0;      // full 1024-token tiles
  // bf16 tiles: coalesced 16-byte chunks DMA'd into LDS, read from there in
  // the MFMA run layout
  // The wave's issue priority is raised while it issues a tile's six DMAs, so
  // that they leave before the other wave on the SIMD resumes its MFMA / scan
  // work: 205.0-206.0 -> 202.7-203.1 us per 32k-token step at D = 4096 (four
  // alternating measurements, rotating input sets).
  auto prefetch = [&](int64_t t0, uint4 (*tin)[128]) {
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = unswz(64 * h + l);
      dma16(x1r + t0 + 8 * ch, &tin[0][64 * h]);
      dma16(vr + t0 + 8 * ch, &tin[1][64 * h]);
      dma16(x2r + t0 + 8 * ch, &tin[2][64 * h]);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // The same for the partial last tile of a VEC row (L a multiple of 8, so
  // its 8-token chunks are whole or absent): chunks at or past L re-read the
  // tile's first chunk, an in-bounds address, and their runs are zeroed after
  // they are read out.
  auto prefetch_part = [&](int64_t t0, uint4 (*tin)[128]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = unswz(64 * h + l);
      const int64_t src = (t0 + 8 * ch < L) ? t0 + 8 * ch : t0;
      dma16(x1r + src, &tin[0][64 * h]);
      dma16(vr + src, &tin[1][64 * h]);
      dma16(x2r + src, &tin[2][64 * h]);
    }
  };

  // ---- per-lane parameters, then the first two tiles in flight while the
  // per-row constants are set up
  const int part = i32 >> 4;                  // scan lane: mode n_sc, part 0 or 1
  const int n_sc = i32 & 15;
  // Every load is issued unconditionally from an in-bounds address (index
  // clamped, the value dropped afterwards), so that they are all in flight
  // together.
  // the scan lane's pole: real lam, or (Re, Im) of its complex mode
  const int m_sc = CPX ? (n_sc >> 1) : n_sc;
  const int lam_i = CPX ? 2 * min(m_sc, N - 1) : min(n_sc, N - 1);
  const float lam_ld = lamc[lam_i];
  const float lam_ld_im = CPX ? lamc[lam_i + 1] : 0.0f;
  float g_lam[8], g_res[8];                   // slots 8 hf + j of G
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = min(8 * hf + j, NS - 1);
    g_lam[j] = lamc[n];
    g_res[j] = resc[n];
  }
  const float* sp = state_in ? state_in + row * NS + min(n_sc, NS - 1) : lamc;
  const float st_ld = *sp;
  // Wait for the parameters before the first DMAs: with only these loads
  // outstanding the wait costs their latency alone, whereas a wait placed
  // after the DMAs is compiled as a wait for everything.
  asm volatile("" ::"v"(lam_ld), "v"(lam_ld_im), "v"(st_ld), "v"(g_lam[0]), "v"(g_lam[1]), "v"(g_lam[2]),
               "v"(g_lam[3]), "v"(g_lam[4]), "v"(g_lam[5]), "v"(g_lam[6]), "v"(g_lam[7]),
               "v"(g_res[0]), "v"(g_res[1]), "v"(g_res[2]), "v"(g_res[3]), "v"(g_res[4]),
               "v"(g_res[5]), "v"(g_res[6]), "v"(g_res[7]) : "memory");
  if constexpr (sizeof(IO) == 2) {
    if (PIPE || nfull > 0) prefetch(0, tin_a);
    if (PIPE || nfull > 1) prefetch(1024, tin_b);
    if constexpr (VEC && !PIPE) {
      if (nfull == 0) prefetch_part(0, tin_a);   // a row shorter than one tile
    }
  }

  const float lam_n = (n_sc < NS) ? lam_ld : 0.0f;
  // CPX: the slot's mode (padding slots: p = 1) and its component
  const CpxMode md = cpx_mode(n_sc < NS ? lam_ld : 0.0f, n_sc < NS ? lam_ld_im : 0.0f);
  const int kc = n_sc & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (8 * hf + j >= NS) g_res[j] = 0.0f;
  }
  float carry = (part == 0 && n_sc < NS && state_in) ? st_ld : 0.0f;

  // ---- per-row constants
  // h[d], d < 32.  The mode loop has its fixed maximum trip count so that
  // all parameter loads are issued together (a loop over the runtime N
  // waited on one load per mode, the bulk of a one-tile call's set-up).
  {
    float hd = 0.0f;
    if constexpr (CPX) {
#pragma unroll
      for (int n = 0; n < MFMA_MAXN / 2; ++n) {
        if (n < N) {
          const float2 e = cexp_at(cpx_mode(lamc[2 * n], lamc[2 * n + 1]), static_cast<float>(i32));
          hd = fmaf(resc[2 * n], e.x, fmaf(-resc[2 * n + 1], e.y, hd));
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < MFMA_MAXN; ++n) {
        if (n < N) hd = fmaf(resc[n], expf(lamc[n] * static_cast<float>(i32)), hd);
      }
    }
    if (hf == 0) hbuf[i32] = hd;
  }
  lds_sync();
  // A = T (row i32, slot (s,j) -> token blk_tok): T[i][tok] = h[i - tok] for tok <= i
  bf16x8 tm[3][2];
  split3_slots(
      [&](int s, int j) {
        const int d = i32 - blk_tok(8 * s + j, hf);
        return (d >= 0) ? hbuf[d] : 0.0f;
      },
      tm);
  // A = G (row i32, slot j -> mode 8*hf + j): G[i][n] = R_n p_n^(i+1);
  // CPX: slot 2m holds Re(R_m p_m^(i+1)), slot 2m + 1 holds -Im(R_m p_m^(i+1))
  auto gval = [&](int j) {
    if constexpr (CPX) {
      const int j0 = j & ~1;
      const float2 e = cexp_at(cpx_mode(g_lam[j0], g_lam[j0 + 1]), static_cast<float>(i32 + 1));
      const float2 rp = cmul(make_float2(g_res[j0], g_res[j0 + 1]), e);
      return (j & 1) ? -rp.y : rp.x;          // padding slots: g_res = 0
    } else {
      return g_res[j] * expf(g_lam[j] * static_cast<float>(i32 + 1));
    }
  };
  bf16x8 gm[3];
  {
    u32x4 w0, w1, w2;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t a, b, c;
      split3_pair(gval(2 * jj), gval(2 * jj + 1), a, b, c);
      w0[jj] = a;
      w1[jj] = b;
      w2[jj] = c;
    }
    gm[0] = __builtin_bit_cast(bf16x8, w0);
    gm[1] = __builtin_bit_cast(bf16x8, w1);
    gm[2] = __builtin_bit_cast(bf16x8, w2);
  }
  // scan lane: mode n_sc (part 0 or 1 of the column pair) for all 32
  // blocks; padded modes have p = 1 and R = 0
  bf16x8 pa[2], pb[2], pc[2];
  if constexpr (CPX) {
    build_state_weights_cpx(md, kc, part, hf, 31, pa, pb, pc);
  } else {
    build_state_weights(lam_n, part, hf, 31, pa, pb, pc);
  }
  // p^32, p^64, p^96, p^128: real part (CPX: and the imaginary part times
  // the sign of the partner term, -1 for a Re slot, +1 for an Im slot)
  float a1, a2, a3, a4, b1 = 0.0f, b2 = 0.0f, b3 = 0.0f, b4 = 0.0f;
  if constexpr (CPX) {
    const float sg = kc ? 1.0f : -1.0f;
    const float2 e1 = cexp_at(md, 32.0f), e2 = cexp_at(md, 64.0f);
    const float2 e3 = cexp_at(md, 96.0f), e4 = cexp_at(md, 128.0f);
    a1 = e1.x; a2 = e2.x; a3 = e3.x; a4 = e4.x;
    b1 = sg * e1.y; b2 = sg * e2.y; b3 = sg * e3.y; b4 = sg * e4.y;
  } else {
    a1 = expf(lam_n * 32.0f); a2 = expf(lam_n * 64.0f);
    a3 = expf(lam_n * 96.0f); a4 = expf(lam_n * 128.0f);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    pin(pa[s]);
    pin(pb[s]);
    if constexpr (NU == 3) pin(pc[s]);
#pragma unroll
    for (int k = 0; k < 3; ++k) pin(tm[k][s]);
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) pin(gm[k]);
  pin(a1);
  pin(a2);
  pin(a3);
  pin(a4);
  if constexpr (CPX) {
    pin(b1);
    pin(b2);
    pin(b3);
    pin(b4);
  }
  // consume the state load here: a load still pending at the loop would make
  // the compiler wait for all vector memory (the DMAs in flight included) at
  // its first use in every iteration
  asm volatile("" : "+v"(carry));

  // One 1024-token tile: inputs in `in` (u = x1 * v, gate x2), output to y.
  // Returns nothing; updates `carry` (state after the tile, in part-0 lanes)
  // and leaves sbuf holding the state before each block of the tile.
  // Runs of the tile: from `in` (registers) or, for bf16 tiles staged in
  // LDS, from the staged chunks.  All inputs are read first; `released` is
  // called once they are in registers, so the caller may refill `tin`.
  auto tile = [&](const TileIn<IO>& in, int64_t t0, bool full, bf16x8 (&um)[NU][2],
                  uint4 (*tin)[128], bool staged, auto&& released) {
    float (*sbuf)[33][17] = sbufs[0];
    Raw4<IO> rx[4], rv[4], rg[4];              // x1, v, gate x2
    if constexpr (sizeof(IO) == 2) {
      if (staged) {
        read_staged_runs(tin, i32, hf, rx, rv, rg);
        if (!full) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (t0 + lane_off + 8 * q >= L) {   // a run is whole or past L
              rx[q].w = make_uint2(0u, 0u);
              rv[q].w = make_uint2(0u, 0u);
              rg[q].w = make_uint2(0u, 0u);
            }
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rx[q] = in.a[q];
          rv[q] = in.b[q];
          rg[q] = in.g[q];
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rx[q] = in.a[q];
        rv[q] = in.b[q];
        rg[q] = in.g[q];
      }
    }
    float su[16];                              // skip * u, for the output
    u32x4 uw[NU][2];                           // parts of u as packed bf16 pairs
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const Raw4<IO> ra = rx[q], rb = rv[q];
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int r = 4 * q + e;
        const float u0 = ra.get(e) * rb.get(e);
        const float u1 = ra.get(e + 1) * rb.get(e + 1);
        su[r] = sk * u0;
        su[r + 1] = sk * u1;
        uint32_t p0, p1, p2;
        if constexpr (NU == 2) {
          // exact: the remainder of a product of two bf16 fits one bf16
          p0 = cvt2(u0, u1);
          p1 = cvt2(u0 - lo_f(p0), u1 - hi_f(p0));
          p2 = 0;
        } else {
          split3_pair(u0, u1, p0, p1, p2);
        }
        uw[0][r >> 3][(r & 7) >> 1] = p0;
        uw[1][r >> 3][(r & 7) >> 1] = p1;
        if constexpr (NU == 3) uw[NU - 1][r >> 3][(r & 7) >> 1] = p2;
      }
    }
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      um[k][0] = __builtin_bit_cast(bf16x8, uw[k][0]);
      um[k][1] = __builtin_bit_cast(bf16x8, uw[k][1]);
    }
    released();
    // block-local end states, transposed: lane = mode column, 16 blocks per lane
    f32x16 ce = {};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      ce = mfma(um[0][s], pa[s], ce);
      ce = mfma(um[1][s], pa[s], ce);
      ce = mfma(um[0][s], pb[s], ce);
      if constexpr (NU == 3) ce = mfma(um[NU - 1][s], pc[s], ce);
    }
    // in-block Toeplitz part of z; independent of the scan, so the matrix
    // cores work on it while the scan runs on the vector ALUs
    f32x16 cz = {};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      cz = mfma(tm[0][s], um[0][s], cz);
      cz = mfma(tm[0][s], um[1][s], cz);
      cz = mfma(tm[1][s], um[0][s], cz);
      cz = mfma(tm[1][s], um[1][s], cz);
      cz = mfma(tm[2][s], um[0][s], cz);
      if constexpr (NU == 3) cz = mfma(tm[0][s], um[NU - 1][s], cz);
    }
    // scan over the 32 blocks; register r holds block 8(r>>2) + 4hf + (r&3)
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = ce[r];
    // x <- a x (+ b x_partner for CPX: a complex product with p^32k)
    auto step = [&](float a, float b, float xin, float xadd) {
      if constexpr (CPX) return fmaf(a, xin, fmaf(b, xor1(xin), xadd));
      return fmaf(a, xin, xadd);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 1; e < 4; ++e) x[4 * q + e] = step(a1, b1, x[4 * q + e - 1], x[4 * q + e]);
    }
    float own[4], oth[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      own[q] = x[4 * q + 3];
      oth[q] = xor32(own[q], hf);
    }
    // run rho = 2q + half covers blocks 4*rho .. 4*rho+3; cin[rho] = state before it
    float cin[9];
    cin[0] = carry;
#pragma unroll
    for (int rho = 0; rho < 8; ++rho) {
      const float end = ((rho & 1) == hf) ? own[rho >> 1] : oth[rho >> 1];
      cin[rho + 1] = step(a4, b4, cin[rho], end);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float ci = hf ? cin[2 * q + 1] : cin[2 * q];
      x[4 * q + 0] = step(a1, b1, ci, x[4 * q + 0]);
      x[4 * q + 1] = step(a2, b2, ci, x[4 * q + 1]);
      x[4 * q + 2] = step(a3, b3, ci, x[4 * q + 2]);
      x[4 * q + 3] = step(a4, b4, ci, x[4 * q + 3]);
    }
    // state before block b+1 = x for block b (b = 31 lands in the unused row
    // 32); before block 0 = cin[0], identical in both half-waves
#pragma unroll
    for (int r = 0; r < 16; ++r) sbuf[part][blk_tok(r, hf) + 1][n_sc] = x[r];
    sbuf[part][0][n_sc] = cin[0];
    {
      const float fin = cin[8];
      const float tot = fin + xor16(fin, l);
      carry = (part == 0) ? tot : 0.0f;
    }
    lds_sync();
    // B = state before block i32, modes 8hf + j (column pair summed)
    u32x4 sw[3];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int n = 8 * hf + j;
      uint32_t p0, p1, p2;
      split3_pair(sbuf[0][i32][n] + sbuf[1][i32][n], sbuf[0][i32][n + 1] + sbuf[1][i32][n + 1],
                  p0, p1, p2);
      sw[0][j >> 1] = p0;
      sw[1][j >> 1] = p1;
      sw[2][j >> 1] = p2;
    }
    const bf16x8 sm[3] = {__builtin_bit_cast(bf16x8, sw[0]), __builtin_bit_cast(bf16x8, sw[1]),
                          __builtin_bit_cast(bf16x8, sw[2])};
    // z = T.U + G.S, products of order <= 2 (G.S added after the scan)
    cz = mfma(gm[0], sm[0], cz);
    cz = mfma(gm[0], sm[1], cz);
    cz = mfma(gm[1], sm[0], cz);
    cz = mfma(gm[1], sm[1], cz);
    cz = mfma(gm[0], sm[2], cz);
    cz = mfma(gm[2], sm[0], cz);
    // y = x2 * z + skip * u
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q + e;
        o[e] = fmaf(rg[q].get(e), cz[r], su[r]);
      }
      const int64_t pos = t0 + lane_off + 8 * q;
      if (full || staged) {
        if constexpr (sizeof(IO) == 2) {
          reinterpret_cast<uint2*>(&tout[swz(4 * i32 + q)])[hf] = make_uint2(cvt2(o[0], o[1]), cvt2(o[2], o[3]));
        } else {
          *reinterpret_cast<float4*>(yr + pos) = make_float4(o[0], o[1], o[2], o[3]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (pos + e < L) Io<IO>::st(yr, pos + e, o[e]);
      }
    }
    if constexpr (sizeof(IO) == 2) {
      if (full) {
        lds_sync();
#pragma unroll
        for (int h = 0; h < 2; ++h)
          store16_nt(yr + t0 + 8 * (l + 64 * h), tout[swz(l + 64 * h)]);
      } else if (staged) {
        lds_sync();
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (t0 + 8 * (l + 64 * h) < L)
            store16_nt(yr + t0 + 8 * (l + 64 * h), tout[swz(l + 64 * h)]);
      }
    }
  };

  // ---- full tiles, the next one in flight while the current one computes
  // (two buffers used alternately, so nothing is copied between iterations;
  // past the last tile the prefetch re-reads the last tile instead of
  // branching)
  if constexpr (sizeof(IO) == 2) {
    const TileIn<IO> none{};
    // Two tiles in flight: tile k is read out of its buffer at the top of
    // its computation, and the buffer is refilled at once with tile k + 2.
    // vmcnt retires in issue order, so waiting for tile k means allowing
    // the operations issued after its DMA to stay in flight: the y stores of
    // tiles k-2 and k-1 (2 each) and the DMA of tile k+1 (6), where they
    // exist.  Tiles 0 and 1 were issued before the constant setup.
    int k = 0;
#pragma unroll 1
    for (; k + 1 < nfull; k += 2) {
      const int64_t t0 = static_cast<int64_t>(k) << 10;
      if (k == 0) {
        wait_vmem<6>();                   // nfull > 1 here: DMA(1) may fly
      } else if (k + 1 < nfull) {
        wait_vmem<10>();
      } else {
        wait_vmem<4>();
      }
      lds_sync();                         // tile k in tin_a
      {
        bf16x8 um[NU][2];
        tile(none, t0, true, um, tin_a, true, [&] {
          lds_sync();                     // tin_a read out
          if (k + 2 < nfull) prefetch(t0 + 2048, tin_a);
        });
      }
      if (k + 2 < nfull) {
        if (k == 0) wait_vmem<8>(); else wait_vmem<10>();
      } else {
        if (k == 0) wait_vmem<2>(); else wait_vmem<4>();
      }
      lds_sync();                         // tile k+1 in tin_b
      {
        bf16x8 um[NU][2];
        tile(none, t0 + 1024, true, um, tin_b, true, [&] {
          lds_sync();                     // tin_b read out
          if (k + 3 < nfull) prefetch(t0 + 3072, tin_b);
        });
      }
    }
    if (k < nfull) {
      if (k == 0) wait_vmem<0>(); else wait_vmem<4>();
      lds_sync();
      bf16x8 um[NU][2];
      tile(none, static_cast<int64_t>(k) << 10, true, um, tin_a, true, [] {});
    }
  } else {
    TileIn<IO> ta, tb;
    if (nfull > 0) ta.load(x1r, vr, x2r, lane_off);
    int k = 0;
#pragma unroll 1
    for (; k + 1 < nfull; k += 2) {
      const int64_t t0 = static_cast<int64_t>(k) << 10;
      tb.load(x1r, vr, x2r, t0 + 1024 + lane_off);
      {
        bf16x8 um[NU][2];
        tile(ta, t0, true, um, tin_a, false, [] {});
      }
      const int64_t nxt = (static_cast<int64_t>(min(k + 2, nfull - 1)) << 10) + lane_off;
      ta.load(x1r, vr, x2r, nxt);
      {
        bf16x8 um[NU][2];
        tile(tb, t0 + 1024, true, um, tin_a, false, [] {});
      }
    }
    if (k < nfull) {
      bf16x8 um[NU][2];
      tile(ta, static_cast<int64_t>(k) << 10, true, um, tin_a, false, [] {});
    }
  }
  lds_sync();
  if (nfull > 0 && (static_cast<int64_t>(nfull) << 10) == L) {
    if (part == 0 && hf == 0 && n_sc < NS) state_out[row * NS + n_sc] = carry;
    return;
  }

  // ---- remaining tokens: tiles with bounds checks (at most one when VEC)
#pragma unroll 1
  for (int64_t t0 = static_cast<int64_t>(nfull) << 10; t0 < L; t0 += 1024) {
    TileIn<IO> in;
    bool staged = false;
    if constexpr (sizeof(IO) == 2 && VEC) {
      if (t0 > 0) {                       // (a row shorter than one tile issued it on entry)
        wait_vmem<0>();                   // no DMA of the full tiles left in flight
        prefetch_part(t0, tin_a);
      }
      wait_vmem<0>();
      lds_sync();
      staged = true;
    } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float fa[4], fb[4], fg[4];
      const int64_t pos = t0 + lane_off + 8 * q;
      ld4<IO, false>(x1r, pos, L, fa);
      ld4<IO, false>(vr, pos, L, fb);
      ld4<IO, false>(x2r, pos, L, fg);
      if constexpr (sizeof(IO) == 2) {
        auto pk = [](const float (&f)[4]) {
          uint2 w;
          w.x = (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
          w.y = (__float_as_uint(f[2]) >> 16) | (__float_as_uint(f[3]) & 0xFFFF0000u);
          return w;
        };
        in.a[q].w = pk(fa);
        in.b[q].w = pk(fb);
        in.g[q].w = pk(fg);
      } else {
        in.a[q].w = make_float4(fa[0], fa[1], fa[2], fa[3]);
        in.b[q].w = make_float4(fb[0], fb[1], fb[2], fb[3]);
        in.g[q].w = make_float4(fg[0], fg[1], fg[2], fg[3]);
      }
    }
    }
    bf16x8 um[NU][2];
    tile(in, t0, false, um, tin_a, staged, [] {});
    float (*sbuf)[33][17] = sbufs[0];
    const int64_t rem = L - t0;
    if (rem == 1024) {
      if (part == 0 && hf == 0 && n_sc < NS) state_out[row * NS + n_sc] = carry;
    } else if (rem < 1024) {
      // the sequence ends inside this tile: state after token L-1
      const int bstar = static_cast<int>(rem - 1) >> 5;
      const int estar = static_cast<int>(rem - 1) & 31;
      bf16x8 qa[2], qb[2], qc[2];
      if constexpr (CPX) {
        build_state_weights_cpx(md, kc, part, hf, estar, qa, qb, qc);
      } else {
        build_state_weights(lam_n, part, hf, estar, qa, qb, qc);
      }
      f32x16 cf = {};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        cf = mfma(um[0][s], qa[s], cf);
        cf = mfma(um[1][s], qa[s], cf);
        cf = mfma(um[0][s], qb[s], cf);
        if constexpr (NU == 3) cf = mfma(um[NU - 1][s], qc[s], cf);
      }
      const bool mine = (((bstar >> 2) & 1) == hf);
      const int rs = 4 * (bstar >> 3) + (bstar & 3);
      float ev = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ev = (r == rs) ? cf[r] : ev;
      float fin = 0.0f;
      if (mine) {
        if constexpr (CPX) {
          // p^(estar+1) s, component kc: Re = pr sr - pi si, Im = pr si + pi sr
          const float2 pe = cexp_at(md, static_cast<float>(estar + 1));
          const float sg = kc ? 1.0f : -1.0f;
          fin = fmaf(pe.x, sbuf[part][bstar][n_sc], fmaf(sg * pe.y, sbuf[part][bstar][n_sc ^ 1], ev));
        } else {
          fin = fmaf(expf(lam_n * static_cast<float>(estar + 1)), sbuf[part][bstar][n_sc], ev);
        }
      }
      const float tot = fin + __shfl_xor(fin, 16);
      if (mine && part == 0 && n_sc < NS) state_out[row * NS + n_sc] = tot;
    }
    lds_sync();                           // sbuf reads done before the next tile writes
  }
}

template <typename IO, bool VEC, bool PIPE, bool CPX>
static hipError_t launch_mfma_k(const ChunkArgs& a) {
  dim3 grid(static_cast<unsigned>(a.B * a.D)), block(64);
  chunk_mfma_kernel<IO, VEC, PIPE, CPX><<<grid, block, 0, a.stream>>>(
      static_cast<const IO*>(a.x1), static_cast<const IO*>(a.x2), static_cast<const IO*>(a.v),
      a.lam, a.res, a.N, a.skip, a.state_in, a.state_out, static_cast<IO*>(a.y), a.D, a.L);
  return hipGetLastError();
}

template <bool CPX>
static hipError_t launch_mfma_modes(const ChunkArgs& a) {
  const int esz = a.bf16 ? 2 : 4;
  const bool vec = (a.L % (16 / esz) == 0) && aligned_all(16, a.x1, a.x2, a.v, a.y);
  if (!a.bf16)
    return vec ? launch_mfma_k<float, true, false, CPX>(a) : launch_mfma_k<float, false, false, CPX>(a);
  if (!vec) return launch_mfma_k<bf16_t, false, false, CPX>(a);
  return a.L >= 2048 ? launch_mfma_k<bf16_t, true, true, CPX>(a)
                     : launch_mfma_k<bf16_t, true, false, CPX>(a);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
  if ((a.cpx ? 2 * a.N : a.N) > MFMA_MAXN) return hipErrorInvalidValue;
  return a.cpx ? launch_mfma_modes<true>(a) : launch_mfma_modes<false>(a);
}

}  // namespace hyena
