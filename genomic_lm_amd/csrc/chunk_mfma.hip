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
#include "pow_pair.hpp"

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

// The three parts w0, w1, w2 of the same weights as B operands, for the
// kernel with one mode per lane (32 slots), whose end-state product sums
// U0.W0 + U1.W0 + U0.W1 + U1.W1 + U0.W2 (+ U2.W0) in one column per mode.
template <typename F>
__device__ __forceinline__ void state_weight_parts(F&& w, int hf, int ref, bf16x8 (&parts)[3][2]) {
  split3_slots(
      [&](int s, int j) {
        const int tok = blk_tok(8 * s + j, hf);
        return (tok <= ref) ? w(ref - tok) : 0.0f;
      },
      parts);
}

__device__ __forceinline__ void build_state_weights(float lam_n, int part, int hf, int ref,
                                                    bf16x8 (&pa)[2], bf16x8 (&pb)[2],
                                                    bf16x8 (&pc)[2]) {
  state_weight_operands([&](int d) { return fast_exp(lam_n * static_cast<float>(d)); }, part, hf,
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

// Double-float values hi + lo (an unevaluated sum of two floats) for the
// scan's carried state.  The carry is multiplied by p^1024 once per tile
// along the whole row; rounded to fp32 at every tile (or every 128 tokens,
// as the scan over blocks first did) it would collect one rounding per step
// over the ~1 / (1024 |lam|) steps a slow mode remembers, and a single fp32
// factor's rounding would compound into a bias (~1e-4 of the state for
// |lam| = 1e-5 at one step per 128 tokens).  Two slow modes with nearly
// equal poles and opposite residues make that many times the output's rms.
// Carried as a pair, each step is exact to ~2^-44.  No FP contraction in
// these helpers: fusing a product into the sum after it would change the
// value whose rounding error the next line computes.
struct DF {
  float hi, lo;
};

__device__ __forceinline__ DF df_two_sum(float a, float b) {
#pragma clang fp contract(off)
  const float s = a + b;
  const float bb = s - a;
  return {s, (a - (s - bb)) + (b - bb)};
}

// (ah + al) (c.hi + c.lo) + e
__device__ __forceinline__ DF df_step(float ah, float al, DF c, float e) {
#pragma clang fp contract(off)
  const float p = ah * c.hi;
  const float pe = fmaf(ah, c.hi, -p);          // exact: ah c.hi = p + pe
  const DF sm = df_two_sum(p, e);
  const float lo = (sm.lo + pe) + fmaf(ah, c.lo, al * c.hi);
  return df_two_sum(sm.hi, lo);
}

// (ah + al) (c.hi + c.lo) + (bh + bl) (cp.hi + cp.lo) + e: one component of
// a complex product with the state, cp the partner component
__device__ __forceinline__ DF df_step_cpx(float ah, float al, DF c, float bh, float bl, DF cp,
                                          float e) {
#pragma clang fp contract(off)
  const float p1 = ah * c.hi;
  const float e1 = fmaf(ah, c.hi, -p1);
  const float p2 = bh * cp.hi;
  const float e2 = fmaf(bh, cp.hi, -p2);
  const DF s1 = df_two_sum(p1, p2);
  const DF s2 = df_two_sum(s1.hi, e);
  const float lo = ((s2.lo + s1.lo) + (e1 + e2)) +
                   fmaf(ah, c.lo, fmaf(al, c.hi, fmaf(bh, cp.lo, bl * cp.hi)));
  return df_two_sum(s2.hi, lo);
}

// TM (below): the per-wave block states go through LDS in asm blocks.  With
// 8 waves a workgroup indexes its state buffers by the wave, which the
// compiler cannot tell apart from the tile buffers that DMA loads are
// filling, so it would make every plain access wait for all of them.
// States after the lane's 16 blocks, sbuf[part][blk + 1][n_sc], and the state
// before block 0, sbuf[part][0][n_sc] (rows of 17 floats, 68 bytes): `wr` is
// &sbuf[part][4 hf + 1][n_sc], `w0` &sbuf[part][0][n_sc].
__device__ __forceinline__ void sbuf_store_asm(uint32_t wr, uint32_t w0, const float (&x)[16],
                                               float carry) {
  asm volatile(
      "ds_write_b32 %0, %2\n\t"
      "ds_write_b32 %0, %3 offset:68\n\t"
      "ds_write_b32 %0, %4 offset:136\n\t"
      "ds_write_b32 %0, %5 offset:204\n\t"
      "ds_write_b32 %0, %6 offset:544\n\t"
      "ds_write_b32 %0, %7 offset:612\n\t"
      "ds_write_b32 %0, %8 offset:680\n\t"
      "ds_write_b32 %0, %9 offset:748\n\t"
      "ds_write_b32 %0, %10 offset:1088\n\t"
      "ds_write_b32 %0, %11 offset:1156\n\t"
      "ds_write_b32 %0, %12 offset:1224\n\t"
      "ds_write_b32 %0, %13 offset:1292\n\t"
      "ds_write_b32 %0, %14 offset:1632\n\t"
      "ds_write_b32 %0, %15 offset:1700\n\t"
      "ds_write_b32 %0, %16 offset:1768\n\t"
      "ds_write_b32 %0, %17 offset:1836\n\t"
      "ds_write_b32 %1, %18"
      :
      : "v"(wr), "v"(w0), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]),
        "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]),
        "v"(x[13]), "v"(x[14]), "v"(x[15]), "v"(carry)
      : "memory");
}

// sbuf[0][i32][8 hf + j] + sbuf[1][i32][8 hf + j], j < 8 (the parts are 33
// rows = 2244 bytes apart); `rd` is &sbuf[0][i32][8 hf].  Waits for its reads.
__device__ __forceinline__ void sbuf_load_asm(uint32_t rd, float (&sv)[8]) {
  float a[16];
  asm volatile(
      "ds_read_b32 %0, %16\n\t"
      "ds_read_b32 %1, %16 offset:4\n\t"
      "ds_read_b32 %2, %16 offset:8\n\t"
      "ds_read_b32 %3, %16 offset:12\n\t"
      "ds_read_b32 %4, %16 offset:16\n\t"
      "ds_read_b32 %5, %16 offset:20\n\t"
      "ds_read_b32 %6, %16 offset:24\n\t"
      "ds_read_b32 %7, %16 offset:28\n\t"
      "ds_read_b32 %8, %16 offset:2244\n\t"
      "ds_read_b32 %9, %16 offset:2248\n\t"
      "ds_read_b32 %10, %16 offset:2252\n\t"
      "ds_read_b32 %11, %16 offset:2256\n\t"
      "ds_read_b32 %12, %16 offset:2260\n\t"
      "ds_read_b32 %13, %16 offset:2264\n\t"
      "ds_read_b32 %14, %16 offset:2268\n\t"
      "ds_read_b32 %15, %16 offset:2272\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7]), "=&v"(a[8]), "=&v"(a[9]), "=&v"(a[10]), "=&v"(a[11]),
        "=&v"(a[12]), "=&v"(a[13]), "=&v"(a[14]), "=&v"(a[15])
      : "v"(rd)
      : "memory");
#pragma unroll
  for (int j = 0; j < 8; ++j) sv[j] = a[j] + a[8 + j];
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)(p)));
}

// VEC: rows of whole 16-byte chunks, 16-byte aligned (full tiles take the
// unchecked path).  PIPE (bf16, VEC, L >= 2048): at least two full tiles, so
// the first two DMAs are issued without a branch.  CPX: N complex modes as
// 2N slots (above).
//
// TM: the token-major layout of in_proj's output, xin (B, L, 3D) with each
// channel's x1, x2, v side by side at elements 3c + pos1 / pos2 / posv
// (Hyena channels interleaved per triple: evo2_flash README, Limitations),
// y (B, L, D) for out_proj.  A workgroup of 8 waves takes 8 consecutive
// channels, one wave per channel running the per-wave computation above
// unchanged; only the staging differs.  A tile's 1024 token rows of the
// block's 48-byte span (3 x 16-byte chunks per row, 6 DMA loads per thread as
// in the channel-major case) go to LDS row by row, slot 3 tm_swz(t) + j for
// chunk j of token t, and each wave gathers its channel's runs from
// there (the three chunks of a row side by side, so that one DMA instruction
// reads whole 48-byte pieces of ~21 rows: one piece per lane measured 0.47
// against 0.26 ms with the same bytes read contiguously); y goes back through
// a token-major tile (16 bytes = the block's 8 channels per token) and leaves
// as one 16-byte piece per token row.  The
// rows are read and written 48 / 16 bytes at a time, so each group of 8
// neighbouring channel blocks (whole 128-byte lines) is put on one XCD
// (workgroups are dispatched round-robin over the 8 XCDs), where they share
// the L2 lines, and the groups an XCD holds at once lie 64 blocks apart along
// the row, spread over its L2 channels.  Measured at B=1 D=4096 L=32768:
// 0.41 ms, against 0.86 ms with the blocks in launch order and 0.44 ms with
// the groups of one XCD side by side.
// Every input byte is read once and y written once: 8 bytes per token and
// channel at bf16.  Waves of a workgroup meet at s_barrier where a tile
// buffer or the y tile changes hands (wg_sync below).
// NSL: mode slots per wave.  16: each scan lane carries one part (the
// column pair of the end-state product) of mode i32 & 15.  32 (17 to 32 real
// or 9 to 16 complex modes): one mode per lane and one column per mode, G.S
// in two K-steps of 16 modes; 32 MFMAs per bf16 tile instead of 22.
template <typename IO, bool VEC, bool PIPE, bool CPX, bool TM = false, int NSL = 16>
__global__ __launch_bounds__(TM ? 512 : 64) void chunk_mfma_kernel(
    const IO* __restrict__ x1, const IO* __restrict__ x2, const IO* __restrict__ v,
    const float* __restrict__ lam, const float* __restrict__ res, int N,
    const float* __restrict__ skip, const float* state_in,
    float* state_out, IO* __restrict__ y, int D, int L, int pos1, int pos2, int posv) {
  static_assert(!TM || (sizeof(IO) == 2 && VEC && !CPX), "TM: bf16 rows of 16-byte chunks, real modes");
  static_assert(NSL == 16 || NSL == 32, "16 or 32 mode slots");
  static_assert(!TM || NSL == 16, "TM: 16 slots (its state buffers are read and written in asm)");
  constexpr int NPT = (NSL == 16) ? 2 : 1;    // end-state column parts per mode
  constexpr int NK = NSL / 16;                // K-steps of G.S
  // parts of u: x1*v of two bf16 values is exactly two bf16 parts
  constexpr int NU = (sizeof(IO) == 2) ? 2 : 3;
  constexpr int NWV = TM ? 8 : 1;             // waves (channels) per workgroup
  __shared__ float hbufs[NWV][32];
  // state before block b, per part and mode (row 32: unused)
  __shared__ float sbufs[NWV][NPT][33][NSL + 1];
  // staged x1, v, x2 tiles (bf16, swizzled chunks; TM: 3 chunks of each of
  // 1024 token rows), two tiles in turn, and the staged y tile
  __shared__ uint4 tin_a_s[TM ? 3 * 1024 : 3 * 128], tin_b_s[TM ? 3 * 1024 : 3 * 128];
  __shared__ uint4 tout[TM ? 1024 : 128];
  uint4 (*const tin_a)[128] = reinterpret_cast<uint4 (*)[128]>(tin_a_s);
  uint4 (*const tin_b)[128] = reinterpret_cast<uint4 (*)[128]>(tin_b_s);

  const int l = static_cast<int>(threadIdx.x & 63);
  // (a scalar, so that the channel's parameters are scalar loads)
  const int wv = TM ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) : 0;
  float* const hbuf = hbufs[wv];
  const int hf = l >> 5;                      // half-wave
  const int i32 = l & 31;                     // row of A / column of B and C
  int64_t row;
  int c;
  int64_t bat = 0;                            // TM: batch item and channel block
  int cblk = 0;
  if constexpr (TM) {
    const int64_t nwg = gridDim.x, g = blockIdx.x;
    const int64_t lg = (nwg % 64 == 0) ? 64 * (g / 64) + 8 * (g % 8) + (g / 8) % 8 : g;
    const int nblk = D >> 3;
    bat = lg / nblk;
    cblk = static_cast<int>(lg % nblk);
    c = 8 * cblk + wv;
    row = bat * D + c;
  } else {
    row = blockIdx.x;
    c = static_cast<int>(row % D);
  }
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
  // TM: token rows of the channel block; instruction k of wave wv fills
  // slots [64 (6 wv + k), +64): chunk j = slot % 3 of token tm_swz(slot / 3)
  const int64_t ld3 = 3 * static_cast<int64_t>(D);
  const IO* const xb = x1 + bat * L * ld3 + 24 * cblk;
  IO* const yb = y + bat * L * static_cast<int64_t>(D) + 8 * cblk;
  // (byte offsets within a tile fit 32 bits: 1024 rows of 6 D bytes)
  auto prefetch_tm = [&](int64_t t0, uint4 (*tin)[128], bool clamp) {
    uint4* const tf = &tin[0][0];
    const char* const xt = reinterpret_cast<const char*>(xb + t0 * ld3);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int g = 6 * wv + k;
      const int s = 64 * g + l;
      const int tt = tm_swz(s / 3);
      const int te = (clamp && t0 + tt >= L) ? 0 : tt;
      dma16_shared(xt + (static_cast<uint32_t>(te) * static_cast<uint32_t>(2 * ld3) + 16u * (s % 3)),
                   tf + 64 * g);
    }
  };
  auto prefetch = [&](int64_t t0, uint4 (*tin)[128]) {
    __builtin_amdgcn_s_setprio(2);
    if constexpr (TM) {
      prefetch_tm(t0, tin, false);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = unswz(64 * h + l);
        dma16(x1r + t0 + 8 * ch, &tin[0][64 * h]);
        dma16(vr + t0 + 8 * ch, &tin[1][64 * h]);
        dma16(x2r + t0 + 8 * ch, &tin[2][64 * h]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // The same for the partial last tile of a VEC row (L a multiple of 8, so
  // its 8-token chunks are whole or absent): chunks at or past L re-read the
  // tile's first chunk, an in-bounds address, and their runs are zeroed after
  // they are read out.
  auto prefetch_part = [&](int64_t t0, uint4 (*tin)[128]) {
    if constexpr (TM) {
      prefetch_tm(t0, tin, true);
      return;
    }
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
  const int part = (NSL == 16) ? (i32 >> 4) : 0;   // scan lane: mode n_sc, part 0 or 1
  const int n_sc = (NSL == 16) ? (i32 & 15) : i32;
  // Every load is issued unconditionally from an in-bounds address (index
  // clamped, the value dropped afterwards), so that they are all in flight
  // together.
  // the scan lane's pole: real lam, or (Re, Im) of its complex mode
  const int m_sc = CPX ? (n_sc >> 1) : n_sc;
  const int lam_i = CPX ? 2 * min(m_sc, N - 1) : min(n_sc, N - 1);
  const float lam_ld = lamc[lam_i];
  const float lam_ld_im = CPX ? lamc[lam_i + 1] : 0.0f;
  float g_lam[8 * NK], g_res[8 * NK];         // slots 16 k + 8 hf + j of G, [8 k + j]
#pragma unroll
  for (int k = 0; k < NK; ++k) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = min(16 * k + 8 * hf + j, NS - 1);
      g_lam[8 * k + j] = lamc[n];
      g_res[8 * k + j] = resc[n];
    }
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
  if constexpr (NK == 2) {
#pragma unroll
    for (int j = 8; j < 16; ++j) asm volatile("" ::"v"(g_lam[j]), "v"(g_res[j]) : "memory");
  }
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
  for (int k = 0; k < NK; ++k) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (16 * k + 8 * hf + j >= NS) g_res[8 * k + j] = 0.0f;
    }
  }
  DF carry = {(part == 0 && n_sc < NS && state_in) ? st_ld : 0.0f, 0.0f};

  // ---- per-row constants
  // h[d], d < 32.  The mode loop has its fixed maximum trip count so that
  // all parameter loads are issued together (a loop over the runtime N
  // waited on one load per mode, the bulk of a one-tile call's set-up).
  float hsh = 0.0f;
  {
    float hd = 0.0f;
    if constexpr (CPX) {
#pragma unroll
      for (int n = 0; n < NSL / 2; ++n) {
        if (n < N) {
          const float2 e = cexp_at(cpx_mode(lamc[2 * n], lamc[2 * n + 1]), static_cast<float>(i32));
          hd = fmaf(resc[2 * n], e.x, fmaf(-resc[2 * n + 1], e.y, hd));
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < NSL; ++n) {
        if (n < N) hd = fmaf(resc[n], fast_exp(lamc[n] * static_cast<float>(i32)), hd);
      }
    }
    if constexpr (TM) {
      hsh = hd;                               // both half-waves hold h[i32]
    } else {
      if (hf == 0) hbuf[i32] = hd;
    }
  }
  lds_sync();
  // A = T (row i32, slot (s,j) -> token blk_tok): T[i][tok] = h[i - tok] for tok <= i
  // (TM: h[d] from lane d by a shuffle, which touches no LDS memory)
  bf16x8 tm[3][2];
  split3_slots(
      [&](int s, int j) {
        const int d = i32 - blk_tok(8 * s + j, hf);
        if constexpr (TM) {
          const float hv = __shfl(hsh, d & 31);
          return (d >= 0) ? hv : 0.0f;
        } else {
          return (d >= 0) ? hbuf[d] : 0.0f;
        }
      },
      tm);
  // A = G (row i32, K-step k, slot j -> mode 16k + 8*hf + j): G[i][n] = R_n p_n^(i+1);
  // CPX: slot 2m holds Re(R_m p_m^(i+1)), slot 2m + 1 holds -Im(R_m p_m^(i+1))
  // Padding slots (16k + 8hf + slot >= NS) are zero without evaluating
  // anything: their loads hold the last slot's values, for complex modes an
  // imaginary part, which as the real part of a pole could overflow
  // p^(i+1) and make 0 * inf.
  auto gval = [&](int j) {                    // j = 8 k + slot
    if (16 * (j >> 3) + 8 * hf + (j & 7) >= NS) return 0.0f;
    if constexpr (CPX) {
      const int j0 = j & ~1;
      const float2 e = cexp_at(cpx_mode(g_lam[j0], g_lam[j0 + 1]), static_cast<float>(i32 + 1));
      const float2 rp = cmul(make_float2(g_res[j0], g_res[j0 + 1]), e);
      return (j & 1) ? -rp.y : rp.x;
    } else {
      return g_res[j] * fast_exp(g_lam[j] * static_cast<float>(i32 + 1));
    }
  };
  bf16x8 gm[NK][3];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    u32x4 w0, w1, w2;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t a, b, c;
      split3_pair(gval(8 * k + 2 * jj), gval(8 * k + 2 * jj + 1), a, b, c);
      w0[jj] = a;
      w1[jj] = b;
      w2[jj] = c;
    }
    gm[k][0] = __builtin_bit_cast(bf16x8, w0);
    gm[k][1] = __builtin_bit_cast(bf16x8, w1);
    gm[k][2] = __builtin_bit_cast(bf16x8, w2);
  }
  // scan lane: mode n_sc (part 0 or 1 of the column pair) for all 32
  // blocks; padded modes have p = 1 and R = 0
  // (NSL = 32: the three parts wp[k] of the lane's own mode column instead)
  bf16x8 pa[2], pb[2], pc[2];
  bf16x8 wp[NSL == 32 ? 3 : 1][2];
  if constexpr (NSL == 32) {
    if constexpr (CPX) {
      state_weight_parts([&](int d) {
        const float2 e = cexp_at(md, static_cast<float>(d));
        return kc ? e.y : e.x;
      }, hf, 31, wp);
    } else {
      state_weight_parts([&](int d) { return fast_exp(lam_n * static_cast<float>(d)); }, hf, 31, wp);
    }
  } else if constexpr (CPX) {
    build_state_weights_cpx(md, kc, part, hf, 31, pa, pb, pc);
  } else {
    build_state_weights(lam_n, part, hf, 31, pa, pb, pc);
  }
  // p^32, p^64, p^96, p^128: real part (CPX: and the imaginary part times
  // the sign of the partner term, -1 for a Re slot, +1 for an Im slot), in
  // fp32: within a tile each is applied once to a value.
  float a1, a2, a3, a4, b1 = 0.0f, b2 = 0.0f, b3 = 0.0f, b4 = 0.0f;
  if constexpr (CPX) {
    const float sg = kc ? 1.0f : -1.0f;
    const float2 e1 = cexp_at(md, 32.0f), e2 = cexp_at(md, 64.0f);
    const float2 e3 = cexp_at(md, 96.0f), e4 = cexp_at(md, 128.0f);
    a1 = e1.x; a2 = e2.x; a3 = e3.x; a4 = e4.x;
    b1 = sg * e1.y; b2 = sg * e2.y; b3 = sg * e3.y; b4 = sg * e4.y;
  } else {
    a1 = fast_exp(lam_n * 32.0f); a2 = fast_exp(lam_n * 64.0f);
    a3 = fast_exp(lam_n * 96.0f); a4 = fast_exp(lam_n * 128.0f);
  }
  // The state carried from tile to tile is multiplied by p^1024 once per
  // tile along the whole row.  Every factor that reaches it is an fp32 pair
  // hi + lo from an fp64 exp (pow_pair.hpp) and the carry itself a
  // double-float (DF above): p^128 for the chain over a tile's 8 runs,
  // p^(128 rho) for the carry-in of run rho = 2q + hf, p^1024 for the carry
  // out.  (CPX: Re and sign * Im parts as for a1..a4.)
  float c4h, c4l, c4bh = 0.0f, c4bl = 0.0f;            // p^128
  float fh[5], fl[5], fbh[5], fbl[5];                  // p^(128 (2q + hf)), q < 4; [4]: p^1024
  {
    // one fp64 exp for p^128, the other powers by fp64 products (each
    // exact to ~2^-53, far below the pairs' 2^-48)
    const double la = n_sc < NS ? lam_ld : 0.0;
    const double lb = CPX ? (n_sc < NS ? lam_ld_im : 0.0) : 0.0;
    const float sg = kc ? 1.0f : -1.0f;
    const double m = exp(la * 128.0);
    const double e_re = CPX ? m * cos(lb * 128.0) : m, e_im = CPX ? m * sin(lb * 128.0) : 0.0;
    auto put = [&](double re, double im, float& h, float& lo, float& bh, float& bl) {
      const float2 r = split_pair(re);
      h = r.x;
      lo = r.y;
      if constexpr (CPX) {
        const float2 i = split_pair(im);
        bh = sg * i.x;
        bl = sg * i.y;
      }
    };
    put(e_re, e_im, c4h, c4l, c4bh, c4bl);
    const double s_re = e_re * e_re - e_im * e_im, s_im = 2.0 * e_re * e_im;   // p^256
    double f_re = hf ? e_re : 1.0, f_im = hf ? e_im : 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      put(f_re, f_im, fh[q], fl[q], fbh[q], fbl[q]);
      const double t = f_re * s_re - f_im * s_im;
      f_im = f_re * s_im + f_im * s_re;
      f_re = t;
    }
    const double q_re = s_re * s_re - s_im * s_im, q_im = 2.0 * s_re * s_im;   // p^512
    put(q_re * q_re - q_im * q_im, 2.0 * q_re * q_im, fh[4], fl[4], fbh[4], fbl[4]);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if constexpr (NSL == 32) {
#pragma unroll
      for (int k = 0; k < 3; ++k) pin(wp[k][s]);
    } else {
      pin(pa[s]);
      pin(pb[s]);
      if constexpr (NU == 3) pin(pc[s]);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) pin(tm[k][s]);
  }
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
    for (int k = 0; k < 3; ++k) pin(gm[kk][k]);
  }
  pin(a1);
  pin(a2);
  pin(a3);
  pin(a4);
  pin(c4h);
  pin(c4l);
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    pin(fh[q]);
    pin(fl[q]);
  }
  if constexpr (CPX) {
    pin(b1);
    pin(b2);
    pin(b3);
    pin(b4);
    pin(c4bh);
    pin(c4bl);
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      pin(fbh[q]);
      pin(fbl[q]);
    }
  }
  // consume the state load here: a load still pending at the loop would make
  // the compiler wait for all vector memory (the DMAs in flight included) at
  // its first use in every iteration
  asm volatile("" : "+v"(carry.hi));

  // One 1024-token tile: inputs in `in` (u = x1 * v, gate x2), output to y.
  // Returns nothing; updates `carry` (state after the tile, in part-0 lanes,
  // as a double-float)
  // and leaves sbuf holding the state before each block of the tile.
  // Runs of the tile: from `in` (registers) or, for bf16 tiles staged in
  // LDS, from the staged chunks.  All inputs are read first; `released` is
  // called once they are in registers, so the caller may refill `tin`.
  auto tile = [&](const TileIn<IO>& in, int64_t t0, bool full, bf16x8 (&um)[NU][2],
                  uint4 (*tin)[128], bool staged, auto&& released) {
    float (*sbuf)[33][NSL + 1] = sbufs[wv];
    Raw4<IO> rx[4], rv[4], rg[4];              // x1, v, gate x2
    if constexpr (sizeof(IO) == 2) {
      if (staged) {
        if constexpr (TM) {
          read_tm_runs(&tin[0][0], i32, hf, 3 * wv + pos1, 3 * wv + posv, 3 * wv + pos2, rx, rv, rg);
        } else {
          read_staged_runs(tin, i32, hf, rx, rv, rg);
        }
        if (!full) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t tq = t0 + lane_off + 8 * q;
            if constexpr (TM) {
              // token by token: any L
              const uint32_t m0 = (tq < L ? 0xFFFFu : 0u) | (tq + 1 < L ? 0xFFFF0000u : 0u);
              const uint32_t m1 = (tq + 2 < L ? 0xFFFFu : 0u) | (tq + 3 < L ? 0xFFFF0000u : 0u);
              rx[q].w.x &= m0; rx[q].w.y &= m1;
              rv[q].w.x &= m0; rv[q].w.y &= m1;
              rg[q].w.x &= m0; rg[q].w.y &= m1;
            } else if (tq >= L) {   // a run is whole or past L
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
      if constexpr (NSL == 32) {
        ce = mfma(um[0][s], wp[0][s], ce);
        ce = mfma(um[1][s], wp[0][s], ce);
        ce = mfma(um[0][s], wp[1][s], ce);
        ce = mfma(um[1][s], wp[1][s], ce);
        ce = mfma(um[0][s], wp[2][s], ce);
        if constexpr (NU == 3) ce = mfma(um[NU - 1][s], wp[0][s], ce);
      } else {
        ce = mfma(um[0][s], pa[s], ce);
        ce = mfma(um[1][s], pa[s], ce);
        ce = mfma(um[0][s], pb[s], ce);
        if constexpr (NU == 3) ce = mfma(um[NU - 1][s], pc[s], ce);
      }
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
    // run rho = 2q + half covers blocks 4*rho .. 4*rho+3.  loc[rho]: the
    // state before run rho from a zero state at the tile's start (the chain
    // over the runs, fp32 with p^128 as a pair: its rounding stays within the
    // tile); the true state adds p^(128 rho) times the carry.
    float loc[9];
    loc[0] = 0.0f;
#pragma unroll
    for (int rho = 0; rho < 8; ++rho) {
      const float end = ((rho & 1) == hf) ? own[rho >> 1] : oth[rho >> 1];
      if constexpr (CPX) {
        const float xp = xor1(loc[rho]);
        loc[rho + 1] = fmaf(c4h, loc[rho], fmaf(c4bh, xp, fmaf(c4l, loc[rho], fmaf(c4bl, xp, end))));
      } else {
        loc[rho + 1] = fmaf(c4h, loc[rho], fmaf(c4l, loc[rho], end));
      }
    }
    const DF cpy = CPX ? DF{xor1(carry.hi), xor1(carry.lo)} : DF{0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rho = 2 * q + hf;
      // carry-in of the run, rounded once: p^(128 rho) carry + loc[rho]
      float ci;
      if constexpr (CPX) {
        ci = fmaf(fh[q], carry.hi, fmaf(fbh[q], cpy.hi, fmaf(fh[q], carry.lo, fmaf(fbh[q], cpy.lo,
             fmaf(fl[q], carry.hi, fmaf(fbl[q], cpy.hi, loc[rho]))))));
      } else {
        ci = fmaf(fh[q], carry.hi, fmaf(fh[q], carry.lo, fmaf(fl[q], carry.hi, loc[rho])));
      }
      x[4 * q + 0] = step(a1, b1, ci, x[4 * q + 0]);
      x[4 * q + 1] = step(a2, b2, ci, x[4 * q + 1]);
      x[4 * q + 2] = step(a3, b3, ci, x[4 * q + 2]);
      x[4 * q + 3] = step(a4, b4, ci, x[4 * q + 3]);
    }
    // state before block b+1 = x for block b (b = 31 lands in the unused row
    // 32); before block 0 = the carry, identical in both half-waves
    if constexpr (TM) {
      sbuf_store_asm(lds_addr(&sbuf[part][4 * hf + 1][n_sc]), lds_addr(&sbuf[part][0][n_sc]), x,
                     carry.hi + carry.lo);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) sbuf[part][blk_tok(r, hf) + 1][n_sc] = x[r];
      sbuf[part][0][n_sc] = carry.hi + carry.lo;
    }
    {
      // carry out: p^1024 carry + loc[8], then the two parts' states summed
      // into the part-0 lane's carry
      DF fin;
      if constexpr (CPX) {
        fin = df_step_cpx(fh[4], fl[4], carry, fbh[4], fbl[4], cpy, loc[8]);
      } else {
        fin = df_step(fh[4], fl[4], carry, loc[8]);
      }
      if constexpr (NSL == 32) {
        carry = fin;                          // one column per mode: nothing to combine
      } else {
        const DF oth2 = {xor16(fin.hi, l), xor16(fin.lo, l)};
        const DF sm = df_two_sum(fin.hi, oth2.hi);
        const DF tot = df_two_sum(sm.hi, sm.lo + (fin.lo + oth2.lo));
        carry = (part == 0) ? tot : DF{0.0f, 0.0f};
      }
    }
    lds_sync();
    // B = state before block i32, K-step k: modes 16k + 8hf + j (NSL = 16:
    // the column pair summed)
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      u32x4 sw[3];
      float sv[8];
      if constexpr (TM) {
        sbuf_load_asm(lds_addr(&sbuf[0][i32][8 * hf]), sv);
      } else if constexpr (NSL == 32) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = sbuf[0][i32][16 * k + 8 * hf + j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = sbuf[0][i32][8 * hf + j] + sbuf[1][i32][8 * hf + j];
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        uint32_t p0, p1, p2;
        split3_pair(sv[j], sv[j + 1], p0, p1, p2);
        sw[0][j >> 1] = p0;
        sw[1][j >> 1] = p1;
        sw[2][j >> 1] = p2;
      }
      const bf16x8 sm[3] = {__builtin_bit_cast(bf16x8, sw[0]), __builtin_bit_cast(bf16x8, sw[1]),
                            __builtin_bit_cast(bf16x8, sw[2])};
      // z = T.U + G.S, products of order <= 2 (G.S added after the scan)
      cz = mfma(gm[k][0], sm[0], cz);
      cz = mfma(gm[k][0], sm[1], cz);
      cz = mfma(gm[k][1], sm[0], cz);
      cz = mfma(gm[k][1], sm[1], cz);
      cz = mfma(gm[k][0], sm[2], cz);
      cz = mfma(gm[k][2], sm[0], cz);
    }
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
        if constexpr (TM) {
          // token t = 32 i32 + 8q + 4hf + e of the tile -> element wv of slot
          // tm_swz(t): index 256 i32 + wv + ((64 q + 8 e) ^ 8 ((i32 & 15) ^ 4 hf))
          uint32_t yl = 256u * static_cast<uint32_t>(i32) + static_cast<uint32_t>(wv);
          uint32_t m8 = 8u * static_cast<uint32_t>((i32 & 15) ^ (4 * hf));
          asm volatile("" : "+v"(yl), "+v"(m8));   // formed here, not kept across tiles
          uint16_t* const yt = reinterpret_cast<uint16_t*>(tout);
          const uint32_t p01 = cvt2(o[0], o[1]), p23 = cvt2(o[2], o[3]);
          yt[yl + ((64u * q + 0u) ^ m8)] = static_cast<uint16_t>(p01);
          yt[yl + ((64u * q + 8u) ^ m8)] = static_cast<uint16_t>(p01 >> 16);
          yt[yl + ((64u * q + 16u) ^ m8)] = static_cast<uint16_t>(p23);
          yt[yl + ((64u * q + 24u) ^ m8)] = static_cast<uint16_t>(p23 >> 16);
        } else if constexpr (sizeof(IO) == 2) {
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
    // bf16 full tiles leave y staged in tout; flush_y stores it once the
    // next tile's DMA has been waited for (below)
    if constexpr (TM) {
      if (!full) {
        wg_sync();                        // every wave's y of the tile in tout
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int sl = static_cast<int>(threadIdx.x) + 512 * h;
          const int64_t t = t0 + tm_swz(sl);
          if (t < L) *reinterpret_cast<uint4*>(yb + t * D) = tout[sl];
        }
      }
    } else if constexpr (sizeof(IO) == 2) {
      if (!full && staged) {
        lds_sync();
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (t0 + 8 * (l + 64 * h) < L)
            store16_nt(yr + t0 + 8 * (l + 64 * h), tout[swz(l + 64 * h)]);
      }
    }
  };

  // y of the full bf16 tile starting at t0, staged in tout by tile(): 16-byte
  // coalesced non-temporal stores
  // TM: all waves' y, after a workgroup barrier, one token row's 16 bytes
  // per store (plain stores: neighbouring channel blocks fill the rest of
  // each line, which the L2 merges before writing it back).
  auto flush_y = [&](int64_t t0) {
    if constexpr (TM) {
      wg_sync();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sl = static_cast<int>(threadIdx.x) + 512 * h;
        *reinterpret_cast<uint4*>(yb + (t0 + tm_swz(sl)) * D) = tout[sl];
      }
    } else {
      lds_sync();
#pragma unroll
      for (int h = 0; h < 2; ++h) store16_nt(yr + t0 + 8 * (l + 64 * h), tout[swz(l + 64 * h)]);
    }
  };
  // A staged tile is complete for the workgroup / a buffer read out by it:
  // TM needs every wave, the single-wave workgroup only its own LDS work.
  auto sync_tile = [&] {
    if constexpr (TM) wg_sync(); else lds_sync();
  };

  // ---- full tiles, the next one in flight while the current one computes
  // (two buffers used alternately, so nothing is copied between iterations;
  // past the last tile the prefetch re-reads the last tile instead of
  // branching)
  if constexpr (sizeof(IO) == 2) {
    const TileIn<IO> none{};
    // Two tiles in flight: tile k is read out of its buffer at the top of
    // its computation, and the buffer is refilled at once with tile k + 2.
    // The waits assume only that one wave's LDS-DMA loads complete in the
    // order they were issued (the property AMD's ck_tile async pipelines
    // rely on when they wait with vmcnt(n) for all but the n DMA loads
    // issued last), and nothing about stores against loads: each counts the
    // DMA loads issued after tile k's (those of tile k + 1, 6 per lane,
    // when it exists).  Any store issued before them must then have
    // completed too, so y of tile k - 1 is stored only after tile k's wait
    // (flush_y), a whole tile after it was issued rather than just before.
    // Tiles 0 and 1 were issued before the constant setup.
    int k = 0;
#pragma unroll 1
    for (; k + 1 < nfull; k += 2) {
      const int64_t t0 = static_cast<int64_t>(k) << 10;
      wait_vmem<6>();                     // tile k + 1 < nfull may still fly
      sync_tile();                        // tile k in tin_a
      if (k > 0) flush_y(t0 - 1024);
      {
        bf16x8 um[NU][2];
        tile(none, t0, true, um, tin_a, true, [&] {
          sync_tile();                    // tin_a read out (TM: and tout)
          if (k + 2 < nfull) prefetch(t0 + 2048, tin_a);
        });
      }
      if (k + 2 < nfull) wait_vmem<6>(); else wait_vmem<0>();
      sync_tile();                        // tile k+1 in tin_b
      flush_y(t0);
      {
        bf16x8 um[NU][2];
        tile(none, t0 + 1024, true, um, tin_b, true, [&] {
          sync_tile();                    // tin_b read out (TM: and tout)
          if (k + 3 < nfull) prefetch(t0 + 3072, tin_b);
        });
      }
    }
    if (k < nfull) {
      wait_vmem<0>();
      sync_tile();
      if (k > 0) flush_y((static_cast<int64_t>(k) << 10) - 1024);
      bf16x8 um[NU][2];
      tile(none, static_cast<int64_t>(k) << 10, true, um, tin_a, true, [&] {
        if constexpr (TM) wg_sync();      // tout read out by every thread
      });
    }
    if (nfull > 0) flush_y(static_cast<int64_t>(nfull - 1) << 10);
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
    if (part == 0 && hf == 0 && n_sc < NS) state_out[row * NS + n_sc] = carry.hi + carry.lo;
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
      sync_tile();
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
    tile(in, t0, false, um, tin_a, staged, [&] {
      if constexpr (TM) wg_sync();        // tout read out by every thread
    });
    float (*sbuf)[33][NSL + 1] = sbufs[wv];
    const int64_t rem = L - t0;
    if (rem == 1024) {
      if (part == 0 && hf == 0 && n_sc < NS) state_out[row * NS + n_sc] = carry.hi + carry.lo;
    } else if (rem < 1024) {
      // the sequence ends inside this tile: state after token L-1
      const int bstar = static_cast<int>(rem - 1) >> 5;
      const int estar = static_cast<int>(rem - 1) & 31;
      f32x16 cf = {};
      if constexpr (NSL == 32) {
        bf16x8 qp[3][2];
        if constexpr (CPX) {
          state_weight_parts([&](int d) {
            const float2 e = cexp_at(md, static_cast<float>(d));
            return kc ? e.y : e.x;
          }, hf, estar, qp);
        } else {
          state_weight_parts([&](int d) { return fast_exp(lam_n * static_cast<float>(d)); }, hf,
                             estar, qp);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          cf = mfma(um[0][s], qp[0][s], cf);
          cf = mfma(um[1][s], qp[0][s], cf);
          cf = mfma(um[0][s], qp[1][s], cf);
          cf = mfma(um[1][s], qp[1][s], cf);
          cf = mfma(um[0][s], qp[2][s], cf);
          if constexpr (NU == 3) cf = mfma(um[NU - 1][s], qp[0][s], cf);
        }
      } else {
        bf16x8 qa[2], qb[2], qc[2];
        if constexpr (CPX) {
          build_state_weights_cpx(md, kc, part, hf, estar, qa, qb, qc);
        } else {
          build_state_weights(lam_n, part, hf, estar, qa, qb, qc);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          cf = mfma(um[0][s], qa[s], cf);
          cf = mfma(um[1][s], qa[s], cf);
          cf = mfma(um[0][s], qb[s], cf);
          if constexpr (NU == 3) cf = mfma(um[NU - 1][s], qc[s], cf);
        }
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
          fin = fmaf(fast_exp(lam_n * static_cast<float>(estar + 1)), sbuf[part][bstar][n_sc], ev);
        }
      }
      const float tot = (NSL == 16) ? fin + __shfl_xor(fin, 16) : fin;
      if (mine && part == 0 && n_sc < NS) state_out[row * NS + n_sc] = tot;
    }
    lds_sync();                           // sbuf reads done before the next tile writes
  }
}

// One-tile rows: bf16, whole 16-byte chunks, 1 <= L <= 1024 -- one chunk per
// call in chunk-by-chunk prefill (TurboQuant-Bio int4 Evo 2 checkpoints,
// 'Chunk size': 1024-token chunks).  The products are those of
// chunk_mfma_kernel's single tile, but a call of one tile is dominated by
// setting up the per-row operands, so they are formed more cheaply and only
// right before the products that use them, within 128 VGPRs: 4 waves per
// SIMD keep 4096 rows resident at once (the general kernel, 2 waves per
// SIMD, takes two rounds).
//  - h and G share their exponentials: lane (i, hf) forms R_n p_n^(i+1) for
//    the 8 modes of its G slots and the two half-waves' sums give h[i+1].
//  - The end-state weights of a run of 4 consecutive tokens come from one
//    exp and 3 products.
//  - The carry factors are plain fp32 exps: the state enters and leaves the
//    call as fp32, so the pair factors that keep a long scan of many tiles
//    exact have nothing to preserve here.
// LDS: the staged inputs (6 KB) are read into registers before the block
// states and the staged y are written over them; with h, 6.5 KB.
__global__ __launch_bounds__(64, 4) void chunk_one_kernel(
    const bf16_t* __restrict__ x1, const bf16_t* __restrict__ x2, const bf16_t* __restrict__ v,
    const float* __restrict__ lam, const float* __restrict__ res, int N,
    const float* __restrict__ skip, const float* state_in, float* state_out,
    bf16_t* __restrict__ y, int D, int L) {
  constexpr int kTinBytes = 3 * 128 * 16;
  constexpr int kSbufBytes = (2 * 33 * 17 * 4 + 15) / 16 * 16;
  constexpr int kLdsBytes = (kSbufBytes + 128 * 16 > kTinBytes) ? kSbufBytes + 128 * 16 : kTinBytes;
  __shared__ __align__(16) unsigned char lds_raw[kLdsBytes];
  // h's three bf16 parts by reversed lag: htab[0][k][x] = part k of
  // h[31 - x], zero for x > 31 (lags below zero); htab[1] the same one entry
  // later.  A lane's pair of T slots (lags d and d - 1) is then one aligned
  // 32-bit word of one of the two copies.
  __shared__ __align__(4) uint16_t htab[2][3][66];
  const uint4 (*const tin)[128] = reinterpret_cast<const uint4 (*)[128]>(lds_raw);
  uint4 (*const tin_w)[128] = reinterpret_cast<uint4 (*)[128]>(lds_raw);
  float (*const sbuf)[33][17] = reinterpret_cast<float (*)[33][17]>(lds_raw);
  uint4* const tout = reinterpret_cast<uint4*>(lds_raw + kSbufBytes);

  const int l = threadIdx.x;
  const int hf = l >> 5;
  const int i32 = l & 31;
  const int part = i32 >> 4;
  const int n_sc = i32 & 15;
  const int c = static_cast<int>(blockIdx.x);                // grid (D, B): no division
  const int64_t row = static_cast<int64_t>(blockIdx.y) * D + c;
  const float* lamc = lam + static_cast<int64_t>(c) * N;
  const float* resc = res + static_cast<int64_t>(c) * N;
  const bf16_t* x1r = x1 + row * L;
  const bf16_t* x2r = x2 + row * L;
  const bf16_t* vr = v + row * L;
  bf16_t* yr = y + row * L;
  const bool whole = (L == 1024);

  // The parameters first, then the inputs: chunks at or past L re-read the
  // row's first chunk, an in-bounds address, and their runs are zeroed after
  // they are read out.  Everything before the inputs' 6 DMA loads is waited
  // for with vmcnt(6), so the setup below runs while the inputs are in flight.
  // With fewer than 16 modes the padded slots read mode 0 and are given
  // pole and residue 0 once loaded, so that they contribute R p^k = 0.
  float lam_ld, st_ld = 0.0f;                            // the scan lane's pole and state
  float g_lam[8], g_res[8];                              // G's slots: modes 8 hf + j
  if (N >= 16) {
    lam_ld = lamc[n_sc];
    if (state_in) st_ld = state_in[row * N + n_sc];
    const float* const gl = lamc + 8 * hf;
    const float* const gr = resc + 8 * hf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      g_lam[j] = gl[j];
      g_res[j] = gr[j];
    }
  } else {
    const bool live_sc = n_sc < N;
    lam_ld = lamc[live_sc ? n_sc : 0];
    if (state_in) st_ld = state_in[row * N + (live_sc ? n_sc : 0)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = (8 * hf + j < N) ? 8 * hf + j : 0;
      g_lam[j] = lamc[n];
      g_res[j] = resc[n];
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ch = unswz(64 * h + l);
    const int src = (8 * ch < L) ? 8 * ch : 0;
    dma16(x1r + src, &tin_w[0][64 * h]);
    dma16(vr + src, &tin_w[1][64 * h]);
    dma16(x2r + src, &tin_w[2][64 * h]);
  }

  // ---- h and G while the inputs are in flight.  The loaded values pass
  // through an empty asm after the wait, so that no use of them is scheduled
  // above it (the compiler would guard such a use with a wait for every
  // load, the DMAs included).
  wait_vmem<6>();
  float lam_sc = lam_ld, st_sc = st_ld;
  pin(lam_sc);
  pin(st_sc);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pin(g_lam[j]);
    pin(g_res[j]);
  }
  if (N < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool live = 8 * hf + j < N;
      g_lam[j] = live ? g_lam[j] : 0.0f;
      g_res[j] = live ? g_res[j] : 0.0f;
    }
  }
  float gv[8];                                 // G[i32][8 hf + j] = R_n p_n^(i32+1)
  float hpart = 0.0f, h0part = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    gv[j] = g_res[j] * fast_exp(g_lam[j] * static_cast<float>(i32 + 1));
    hpart += gv[j];
    h0part += g_res[j];
  }
  const float hnext = hpart + xor32(hpart, hf);            // h[i32 + 1]
  const float h0 = h0part + xor32(h0part, hf);             // h[0]
  {
    // lane (i32, 0): h[i32 + 1] at x = 30 - i32, lane 0 also h[0] at x = 31;
    // lane (i32, 1): the zero at x = 32 + i32
    uint32_t hp[3];
    split3_pair(hf ? 0.0f : hnext, h0, hp[0], hp[1], hp[2]);
    const int x = hf ? 32 + i32 : 30 - i32;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint16_t lo = static_cast<uint16_t>(hp[k]), hi = static_cast<uint16_t>(hp[k] >> 16);
      if (x >= 0) {
        htab[0][k][x] = lo;
        htab[1][k][x + 1] = lo;
      }
      if (hf == 0 && i32 == 0) {
        htab[0][k][31] = hi;
        htab[1][k][32] = hi;
      }
    }
  }
  bf16x8 gm[3];
  {
    u32x4 w0, w1, w2;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t a, b, cc;
      split3_pair(gv[2 * jj], gv[2 * jj + 1], a, b, cc);
      w0[jj] = a;
      w1[jj] = b;
      w2[jj] = cc;
    }
    gm[0] = __builtin_bit_cast(bf16x8, w0);
    gm[1] = __builtin_bit_cast(bf16x8, w1);
    gm[2] = __builtin_bit_cast(bf16x8, w2);
  }
  // split here, in the inputs' latency, not next to G S after the wait
  pin(gm[0]);
  pin(gm[1]);
  pin(gm[2]);
  lds_sync();
  // T[i32][tok] = h[i32 - tok] (zero for tok > i32): slot pair (s, 2jj) at
  // x = 31 - i32 + tok, tok = 4hf + t(s, jj), t in {0, 2, 8, 10, 16, 18, 24, 26};
  // x has the parity of 31 - i32, so odd rows read copy 0 at x and even rows
  // copy 1 at x + 1, both word-aligned.  One asm block that waits for its
  // reads (the inputs' DMAs are in flight; see read_staged_runs).
  bf16x8 tm[3][2];
  {
    const uint16_t* hb = (i32 & 1) ? &htab[0][0][31 - i32 + 4 * hf] : &htab[1][0][32 - i32 + 4 * hf];
    const uint32_t ha = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)(hb)));
    uint32_t r[24];
    asm volatile(
        "ds_read_b32 %0, %24\n\t"
        "ds_read_b32 %1, %24 offset:4\n\t"
        "ds_read_b32 %2, %24 offset:16\n\t"
        "ds_read_b32 %3, %24 offset:20\n\t"
        "ds_read_b32 %4, %24 offset:32\n\t"
        "ds_read_b32 %5, %24 offset:36\n\t"
        "ds_read_b32 %6, %24 offset:48\n\t"
        "ds_read_b32 %7, %24 offset:52\n\t"
        "ds_read_b32 %8, %24 offset:132\n\t"
        "ds_read_b32 %9, %24 offset:136\n\t"
        "ds_read_b32 %10, %24 offset:148\n\t"
        "ds_read_b32 %11, %24 offset:152\n\t"
        "ds_read_b32 %12, %24 offset:164\n\t"
        "ds_read_b32 %13, %24 offset:168\n\t"
        "ds_read_b32 %14, %24 offset:180\n\t"
        "ds_read_b32 %15, %24 offset:184\n\t"
        "ds_read_b32 %16, %24 offset:264\n\t"
        "ds_read_b32 %17, %24 offset:268\n\t"
        "ds_read_b32 %18, %24 offset:280\n\t"
        "ds_read_b32 %19, %24 offset:284\n\t"
        "ds_read_b32 %20, %24 offset:296\n\t"
        "ds_read_b32 %21, %24 offset:300\n\t"
        "ds_read_b32 %22, %24 offset:312\n\t"
        "ds_read_b32 %23, %24 offset:316\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
          "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15]), "=&v"(r[16]), "=&v"(r[17]),
          "=&v"(r[18]), "=&v"(r[19]), "=&v"(r[20]), "=&v"(r[21]), "=&v"(r[22]), "=&v"(r[23])
        : "v"(ha)
        : "memory");
#pragma unroll
    for (int k = 0; k < 3; ++k) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const u32x4 w = {r[8 * k + 4 * sl], r[8 * k + 4 * sl + 1], r[8 * k + 4 * sl + 2],
                         r[8 * k + 4 * sl + 3]};
        tm[k][sl] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  // ---- the scan lane's operands, also before the inputs arrive: the
  // end-state weights and the scan's decay factors.  Scan lane: mode n_sc,
  // part `part`; padded modes have p = 1 (their states never reach y: R = 0).
  const float lam_n = (n_sc < N) ? lam_sc : 0.0f;
  const float p1 = fast_exp(lam_n);
  // weights p^(31 - tok): run m of the lane holds tokens 8m + 4hf + e, whose
  // weight is p^(28 - 8m - 4hf) p^(3 - e)
  auto run_weights = [&](float lam_v, int top, float (&w)[16]) {
    const float p2 = p1 * p1, p3 = p2 * p1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d3 = top - 8 * m - 4 * hf - 3;
      const float b = fast_exp(lam_v * static_cast<float>(d3));
      w[4 * m + 3] = b;
      w[4 * m + 2] = b * p1;
      w[4 * m + 1] = b * p2;
      w[4 * m + 0] = b * p3;
    }
  };
  // slot (s, j) of the B operand holds run m = 2s + (j >> 2), element j & 3
  auto weight_operands = [&](const float (&w)[16], bf16x8 (&pa)[2], bf16x8 (&pb)[2]) {
    bf16x8 parts[3][2];
    split3_slots([&](int s, int j) { return w[8 * s + j]; }, parts);
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 q0 = __builtin_bit_cast(u32x4, parts[0][s]);
      const u32x4 q1 = __builtin_bit_cast(u32x4, parts[1][s]);
      const u32x4 q2 = __builtin_bit_cast(u32x4, parts[2][s]);
      pa[s] = __builtin_bit_cast(bf16x8, part ? q1 : q0);
      pb[s] = __builtin_bit_cast(bf16x8, part ? zero : q2);
    }
  };
  bf16x8 pa[2], pb[2];
  {
    float w[16];
    run_weights(lam_n, 31, w);
    weight_operands(w, pa, pb);
  }
  float a1 = fast_exp(lam_n * 32.0f), a2 = fast_exp(lam_n * 64.0f);
  float a3 = fast_exp(lam_n * 96.0f), a4 = fast_exp(lam_n * 128.0f);   // a4 = p^128
  float fr[4];                                 // p^(128 rho), rho = 2q + hf
#pragma unroll
  for (int q = 0; q < 4; ++q) fr[q] = fast_exp(lam_n * (128.0f * static_cast<float>(2 * q + hf)));
  const float p1024 = fast_exp(lam_n * 1024.0f);
  // formed here, not next to their uses after the wait below
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    pin(pa[s]);
    pin(pb[s]);
  }
  pin(a1);
  pin(a2);
  pin(a3);
  pin(a4);

  // ---- the inputs: u = x1 v (two exact bf16 parts), skip * u, the gate
  wait_vmem<0>();
  Raw4<bf16_t> rx[4], rv[4], rg[4];
  read_staged_runs(tin, i32, hf, rx, rv, rg);
  if (!whole) {
    asm volatile("");                        // a branch: whole tiles skip the selects
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (32 * i32 + 4 * hf + 8 * q >= L) {
        rx[q].w = make_uint2(0u, 0u);
        rv[q].w = make_uint2(0u, 0u);
        rg[q].w = make_uint2(0u, 0u);
      }
    }
  }
  const float sk = skip ? skip[c] : 0.0f;
  float su[16];
  bf16x8 um[2][2];
  {
    u32x4 uw[2][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int r = 4 * q + e;
        const float u0 = rx[q].get(e) * rv[q].get(e);
        const float u1 = rx[q].get(e + 1) * rv[q].get(e + 1);
        su[r] = sk * u0;
        su[r + 1] = sk * u1;
        const uint32_t p0 = cvt2(u0, u1);
        uw[0][r >> 3][(r & 7) >> 1] = p0;
        uw[1][r >> 3][(r & 7) >> 1] = cvt2(u0 - lo_f(p0), u1 - hi_f(p0));
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      um[k][0] = __builtin_bit_cast(bf16x8, uw[k][0]);
      um[k][1] = __builtin_bit_cast(bf16x8, uw[k][1]);
    }
  }
  // in-block Toeplitz part of z
  f32x16 cz = {};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    cz = mfma(tm[0][s], um[0][s], cz);
    cz = mfma(tm[0][s], um[1][s], cz);
    cz = mfma(tm[1][s], um[0][s], cz);
    cz = mfma(tm[1][s], um[1][s], cz);
    cz = mfma(tm[2][s], um[0][s], cz);
  }

  // ---- block-local end states, E^T = U^T P^T
  f32x16 ce = {};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    ce = mfma(um[0][s], pa[s], ce);
    ce = mfma(um[1][s], pa[s], ce);
    ce = mfma(um[0][s], pb[s], ce);
  }

  // ---- scan over the 32 blocks; register r holds block 8(r>>2) + 4hf + (r&3)
  const float carry = (part == 0 && n_sc < N) ? st_sc : 0.0f;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = ce[r];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int e = 1; e < 4; ++e) x[4 * q + e] = fmaf(a1, x[4 * q + e - 1], x[4 * q + e]);
  }
  // loc[rho]: state before run rho = 2q + half from a zero state at the
  // tile's start; the true state adds p^(128 rho) carry
  float loc[9];
  loc[0] = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float own = x[4 * q + 3], oth = xor32(own, hf);
    loc[2 * q + 1] = fmaf(a4, loc[2 * q], hf ? oth : own);
    loc[2 * q + 2] = fmaf(a4, loc[2 * q + 1], hf ? own : oth);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float ci = fmaf(fr[q], carry, hf ? loc[2 * q + 1] : loc[2 * q]);
    x[4 * q + 0] = fmaf(a1, ci, x[4 * q + 0]);
    x[4 * q + 1] = fmaf(a2, ci, x[4 * q + 1]);
    x[4 * q + 2] = fmaf(a3, ci, x[4 * q + 2]);
    x[4 * q + 3] = fmaf(a4, ci, x[4 * q + 3]);
  }
  // the inputs are in registers (read_staged_runs waited for its reads), so
  // the states may go over them
#pragma unroll
  for (int r = 0; r < 16; ++r) sbuf[part][blk_tok(r, hf) + 1][n_sc] = x[r];
  sbuf[part][0][n_sc] = carry;
  lds_sync();
  // ---- z += G S, S = state before block i32 (the two parts summed)
  {
    u32x4 sw[3];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int n = 8 * hf + j;
      uint32_t s0, s1, s2;
      split3_pair(sbuf[0][i32][n] + sbuf[1][i32][n], sbuf[0][i32][n + 1] + sbuf[1][i32][n + 1],
                  s0, s1, s2);
      sw[0][j >> 1] = s0;
      sw[1][j >> 1] = s1;
      sw[2][j >> 1] = s2;
    }
    const bf16x8 sm0 = __builtin_bit_cast(bf16x8, sw[0]);
    const bf16x8 sm1 = __builtin_bit_cast(bf16x8, sw[1]);
    const bf16x8 sm2 = __builtin_bit_cast(bf16x8, sw[2]);
    cz = mfma(gm[0], sm0, cz);
    cz = mfma(gm[0], sm1, cz);
    cz = mfma(gm[1], sm0, cz);
    cz = mfma(gm[1], sm1, cz);
    cz = mfma(gm[0], sm2, cz);
    cz = mfma(gm[2], sm0, cz);
  }
  // ---- y = x2 z + skip u, staged and stored in coalesced 16-byte chunks
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = fmaf(rg[q].get(e), cz[4 * q + e], su[4 * q + e]);
    reinterpret_cast<uint2*>(&tout[swz(4 * i32 + q)])[hf] =
        make_uint2(cvt2(o[0], o[1]), cvt2(o[2], o[3]));
  }
  lds_sync();
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (whole || 8 * (l + 64 * h) < L) store16_nt(yr + 8 * (l + 64 * h), tout[swz(l + 64 * h)]);

  // ---- state after token L - 1
  if (whole) {
    // p^1024 carry + loc[8], the two parts summed
    const float fin = fmaf(p1024, carry, loc[8]);
    const float tot = fin + xor16(fin, l);
    if (part == 0 && hf == 0 && n_sc < N) state_out[row * N + n_sc] = tot;
  } else {
    // the sequence ends in block bstar after token estar: p^(estar+1) times
    // the state before the block plus the block's own end state at estar
    const int bstar = (L - 1) >> 5;
    const int estar = (L - 1) & 31;
    float w[16];
    run_weights(lam_n, estar, w);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int tok = blk_tok(8 * (k >> 3) + (k & 7), hf);
      if (tok > estar) w[k] = 0.0f;
    }
    bf16x8 qa[2], qb[2];
    weight_operands(w, qa, qb);
    f32x16 cf = {};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      cf = mfma(um[0][s], qa[s], cf);
      cf = mfma(um[1][s], qa[s], cf);
      cf = mfma(um[0][s], qb[s], cf);
    }
    const bool mine = (((bstar >> 2) & 1) == hf);
    const int rs = 4 * (bstar >> 3) + (bstar & 3);
    float ev = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ev = (r == rs) ? cf[r] : ev;
    const float fin =
        mine ? fmaf(fast_exp(lam_n * static_cast<float>(estar + 1)), sbuf[part][bstar][n_sc], ev)
             : 0.0f;
    const float tot = fin + xor16(fin, l);
    if (mine && part == 0 && n_sc < N) state_out[row * N + n_sc] = tot;
  }
}

template <typename IO, bool VEC, bool PIPE, bool CPX, int NSL>
static hipError_t launch_mfma_k(const ChunkArgs& a) {
  dim3 grid(static_cast<unsigned>(a.B * a.D)), block(64);
  chunk_mfma_kernel<IO, VEC, PIPE, CPX, false, NSL><<<grid, block, 0, a.stream>>>(
      static_cast<const IO*>(a.x1), static_cast<const IO*>(a.x2), static_cast<const IO*>(a.v),
      a.lam, a.res, a.N, a.skip, a.state_in, a.state_out, static_cast<IO*>(a.y), a.D, a.L, 0, 0, 0);
  return hipGetLastError();
}

template <bool CPX, int NSL>
static hipError_t launch_mfma_modes(const ChunkArgs& a) {
  const int esz = a.bf16 ? 2 : 4;
  const bool vec = (a.L % (16 / esz) == 0) && aligned_all(16, a.x1, a.x2, a.v, a.y);
  if (!a.bf16)
    return vec ? launch_mfma_k<float, true, false, CPX, NSL>(a)
               : launch_mfma_k<float, false, false, CPX, NSL>(a);
  if (!vec) return launch_mfma_k<bf16_t, false, false, CPX, NSL>(a);
  if constexpr (!CPX && NSL == 16) {
    if (a.L <= 1024 && a.B <= 65535) {
      dim3 grid(static_cast<unsigned>(a.D), static_cast<unsigned>(a.B)), block(64);
      chunk_one_kernel<<<grid, block, 0, a.stream>>>(
          static_cast<const bf16_t*>(a.x1), static_cast<const bf16_t*>(a.x2),
          static_cast<const bf16_t*>(a.v), a.lam, a.res, a.N, a.skip, a.state_in, a.state_out,
          static_cast<bf16_t*>(a.y), a.D, a.L);
      return hipGetLastError();
    }
  }
  return a.L >= 2048 ? launch_mfma_k<bf16_t, true, true, CPX, NSL>(a)
                     : launch_mfma_k<bf16_t, true, false, CPX, NSL>(a);
}

// Token-major input and output (TM above): bf16, real modes, N <= 16, D a
// multiple of 8 (below 349526) and xin, y 16-byte aligned.
bool tokmajor_mfma_supported(const TokmajorArgs& a) {
  return a.bf16 && a.N <= MFMA_MAXN && a.D % 8 == 0 && a.L > 0 && a.B > 0 &&
         int64_t(a.D) * 6 * 1024 <= INT32_MAX && aligned_all(16, a.xin, a.y);
}

// Where the one-pass kernel is the faster token-major path: its workgroups
// (one per 8 channels, one per CU) fill the 256 CUs, and the prefill is at
// most 32 tile steps (1024 tokens each) per CU.  Measured against the
// per-token segments (B, D, L: ms one-pass / per-token): 1,4096,8192
// 0.110/0.148; 2,2048,16384 0.201/0.226; 1,4096,32768 0.409/0.391;
// 4,4096,8192 0.411/0.381; 1,8192,32768 0.874/0.711; 1,1024,32768
// 0.178/0.155 (128 workgroups).  Longer prefills lose to the per-token
// segments, whose requests to the L2 are whole lines.
bool tokmajor_mfma_preferred(const TokmajorArgs& a) {
  const int64_t wgs = int64_t(a.B) * (a.D / 8);
  return wgs >= 256 && wgs * ((int64_t(a.L) + 1023) / 1024) <= 256 * 32;
}

hipError_t launch_chunk_mfma_tokmajor(const TokmajorArgs& a) {
  if (!tokmajor_mfma_supported(a)) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(a.B * (a.D / 8))), block(512);
  const bf16_t* xin = static_cast<const bf16_t*>(a.xin);
  bf16_t* y = static_cast<bf16_t*>(a.y);
  if (a.L >= 2048) {
    chunk_mfma_kernel<bf16_t, true, true, false, true><<<grid, block, 0, a.stream>>>(
        xin, nullptr, nullptr, a.lam, a.res, a.N, a.skip, a.state_in, a.state_out, y, a.D, a.L,
        a.pos_x1, a.pos_x2, a.pos_v);
  } else {
    chunk_mfma_kernel<bf16_t, true, false, false, true><<<grid, block, 0, a.stream>>>(
        xin, nullptr, nullptr, a.lam, a.res, a.N, a.skip, a.state_in, a.state_out, y, a.D, a.L,
        a.pos_x1, a.pos_x2, a.pos_v);
  }
  return hipGetLastError();
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
  const int slots = a.cpx ? 2 * a.N : a.N;
  if (slots > MFMA_MAXN_WIDE) return hipErrorInvalidValue;
  if (slots > MFMA_MAXN)
    return a.cpx ? launch_mfma_modes<true, 32>(a) : launch_mfma_modes<false, 32>(a);
  return a.cpx ? launch_mfma_modes<true, 16>(a) : launch_mfma_modes<false, 16>(a);
}

}  // namespace hyena
