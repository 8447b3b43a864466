// fir_mfma.hip -- gated explicit-FIR Hyena operator on the matrix cores
// (bf16 I/O, K <= 128: the hcs K = 7 and hcm K = 128 blocks of the
// Evo2-7B-262K model card, Implementation Notes, 'Block dispatch').
//
// z[t] = sum_{k<K} w[k] u[t-k] is a banded Toeplitz product.  Cut into
// 32-token blocks, output block m is
//     z_m = sum_{d<ND} T_d . u_{m-d},    T_d[i][j] = w[32d + i - j]  (0 <= . < K)
// with ND = ceil((K-1)/32) + 1 block diagonals.  One wave owns a row and walks
// 1024-token tiles (32 blocks = one 32x32 MFMA output); u's bf16 parts for the
// tile plus ND-1 halo blocks of the previous tile sit in LDS, and the B operand
// of each diagonal is read from there at a block offset.  Taps are split into
// two bf16 parts (exact when the taps are bf16 values, as in bf16 models; the
// second part's products are then skipped); u = x1*v of two bf16 values is
// exactly two bf16 parts.  Tiles move HBM<->LDS as in chunk_mfma.hip.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace hyena {

template <int ND>
__global__ __launch_bounds__(64) void fir_mfma_kernel(
    const bf16_t* x1, const bf16_t* x2, const bf16_t* v, const float* __restrict__ taps, int K,
    const float* __restrict__ skip, bf16_t* y, int D, int L, bool vec) {
  constexpr int NB = 32 + ND - 1;             // blocks held in ub: halo + tile
  __shared__ float wbuf[32 * ND];
  __shared__ uint4 tin_a[3][128], tin_b[3][128];
  __shared__ uint4 ub[2][NB * 4];             // u parts, 16-byte chunks, swizzled

  const int l = threadIdx.x;
  const int hf = l >> 5;
  const int i32 = l & 31;
  const int64_t row = blockIdx.x;
  const int c = static_cast<int>(row % D);
  const bf16_t* x1r = x1 + row * L;
  const bf16_t* x2r = x2 + row * L;
  const bf16_t* vr = v + row * L;
  bf16_t* yr = y + row * L;
  const float sk = skip ? skip[c] : 0.0f;

  for (int j = l; j < 32 * ND; j += 64) wbuf[j] = (j < K) ? taps[static_cast<int64_t>(c) * K + j] : 0.0f;
  for (int j = l; j < 2 * NB * 4; j += 64) ub[j / (NB * 4)][j % (NB * 4)] = make_uint4(0, 0, 0, 0);
  lds_sync();

  // A operands: T_d parts, row i32, slot (s, j) -> token blk_tok(8s + j, hf)
  bf16x8 ta[ND][2][2];
  uint32_t lo_bits = 0;
#pragma unroll
  for (int d = 0; d < ND; ++d) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = 32 * d + i32 - blk_tok(8 * s + j, hf);
        const float w = (idx >= 0 && idx < 32 * ND) ? wbuf[idx] : 0.0f;
        const __bf16 w0 = static_cast<__bf16>(w);
        const __bf16 w1 = static_cast<__bf16>(w - static_cast<float>(w0));
        ta[d][0][s][j] = w0;
        ta[d][1][s][j] = w1;
        lo_bits |= __builtin_bit_cast(uint16_t, w1);
      }
      pin(ta[d][0][s]);
      pin(ta[d][1][s]);
    }
  }
  // taps that are bf16 values have no second part anywhere in the wave
  const bool exact_taps = !__any(lo_bits != 0);

  // One 1024-token tile whose x1, v, x2 chunks are in `tin`.
  auto tile = [&](uint4 (*tin)[128], int64_t t0, bool full) {
    float su[16];
    uint2 up[2][4];                           // u parts of this lane's runs
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = swz(4 * i32 + q);
      const uint2 ra = reinterpret_cast<const uint2*>(&tin[0][slot])[hf];
      const uint2 rb = reinterpret_cast<const uint2*>(&tin[1][slot])[hf];
      const float u0 = lo_f(ra.x) * lo_f(rb.x), u1 = hi_f(ra.x) * hi_f(rb.x);
      const float u2 = lo_f(ra.y) * lo_f(rb.y), u3 = hi_f(ra.y) * hi_f(rb.y);
      su[4 * q + 0] = sk * u0;
      su[4 * q + 1] = sk * u1;
      su[4 * q + 2] = sk * u2;
      su[4 * q + 3] = sk * u3;
      const uint32_t a0 = cvt2(u0, u1), a1 = cvt2(u2, u3);
      up[0][q] = make_uint2(a0, a1);
      up[1][q] = make_uint2(cvt2(u0 - lo_f(a0), u1 - hi_f(a0)), cvt2(u2 - lo_f(a1), u3 - hi_f(a1)));
      const int us = swz(4 * (i32 + ND - 1) + q);
      reinterpret_cast<uint2*>(&ub[0][us])[hf] = up[0][q];
      reinterpret_cast<uint2*>(&ub[1][us])[hf] = up[1][q];
    }
    lds_sync();
    f32x16 cz = {};
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int blk = i32 + ND - 1 - d;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 b[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint2 r0 = reinterpret_cast<const uint2*>(&ub[p][swz(4 * blk + 2 * s)])[hf];
          const uint2 r1 = reinterpret_cast<const uint2*>(&ub[p][swz(4 * blk + 2 * s + 1)])[hf];
          const u32x4 w4 = {r0.x, r0.y, r1.x, r1.y};
          b[p] = __builtin_bit_cast(bf16x8, w4);
        }
        cz = mfma(ta[d][0][s], b[0], cz);
        cz = mfma(ta[d][0][s], b[1], cz);
        if (!exact_taps) {
          cz = mfma(ta[d][1][s], b[0], cz);
          cz = mfma(ta[d][1][s], b[1], cz);
        }
      }
    }
    // y = x2 * z + skip * u, staged over the x1 slice of tin
    uint4* tout = tin[0];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = swz(4 * i32 + q);
      const uint2 rg = reinterpret_cast<const uint2*>(&tin[2][slot])[hf];
      const float o0 = fmaf(lo_f(rg.x), cz[4 * q + 0], su[4 * q + 0]);
      const float o1 = fmaf(hi_f(rg.x), cz[4 * q + 1], su[4 * q + 1]);
      const float o2 = fmaf(lo_f(rg.y), cz[4 * q + 2], su[4 * q + 2]);
      const float o3 = fmaf(hi_f(rg.y), cz[4 * q + 3], su[4 * q + 3]);
      reinterpret_cast<uint2*>(&tout[slot])[hf] = make_uint2(cvt2(o0, o1), cvt2(o2, o3));
    }
    lds_sync();
    // full tiles leave y staged over tin[0]; flush_y stores it after the
    // next tile's DMA wait
#pragma unroll
    for (int h = 0; h < 2 && !full; ++h) {
      const int ch = l + 64 * h;
      const uint4 w4 = tout[swz(ch)];
      const int64_t pos = t0 + 8 * ch;
      if (vec && pos < L) {                 // vec: L is a multiple of 8, chunks are whole
        store16_nt(yr + pos, w4);
      } else if (!vec) {
        const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (pos + e < L) yr[pos + e] = static_cast<bf16_t>((e & 1) ? (ws[e >> 1] >> 16) : (ws[e >> 1] & 0xFFFFu));
      }
    }
    // the last ND-1 blocks become the next tile's halo
    if (ND > 1 && i32 >= 33 - ND) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int hs = swz(4 * (i32 - (33 - ND)) + q);
        reinterpret_cast<uint2*>(&ub[0][hs])[hf] = up[0][q];
        reinterpret_cast<uint2*>(&ub[1][hs])[hf] = up[1][q];
      }
    }
    lds_sync();
  };

  // Issued at raised wave priority, as in the chunk kernel: FIR-128 at
  // D = 4096, L = 32768 went from 203.8-205.2 to 196.6-197.2 us (three
  // alternating measurements, rotating inputs), FIR-7 stayed at ~204 us.
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

  // y of the full tile at t0, staged over tin[0] of its buffer
  auto flush_y = [&](uint4 (*tin)[128], int64_t t0) {
    lds_sync();
#pragma unroll
    for (int h = 0; h < 2; ++h) store16_nt(yr + t0 + 8 * (l + 64 * h), tin[0][swz(l + 64 * h)]);
    lds_sync();                               // read out before the buffer is refilled
  };

  // One tile in flight: tile k + 1 is issued once tile k has arrived and
  // tile k - 1's y has left its buffer.  When tile k is waited for, no DMA
  // was issued after it, so the wait is vmcnt(0), and y of tile k - 1 is
  // stored only after that wait: the stores it covers were issued a tile
  // earlier.  No ordering between loads and stores is assumed.
  const int nfull = vec ? (L >> 10) : 0;
  if (nfull > 0) prefetch(0, tin_a);
  int k = 0;
#pragma unroll 1
  for (; k + 1 < nfull; k += 2) {
    const int64_t t0 = static_cast<int64_t>(k) << 10;
    wait_vmem<0>();
    lds_sync();
    if (k > 0) flush_y(tin_b, t0 - 1024);
    prefetch(t0 + 1024, tin_b);
    tile(tin_a, t0, true);
    wait_vmem<0>();
    lds_sync();
    flush_y(tin_a, t0);
    if (k + 2 < nfull) prefetch(t0 + 2048, tin_a);
    tile(tin_b, t0 + 1024, true);
  }
  if (k < nfull) {
    wait_vmem<0>();
    lds_sync();
    if (k > 0) flush_y(tin_b, (static_cast<int64_t>(k) << 10) - 1024);
    tile(tin_a, static_cast<int64_t>(k) << 10, true);
  }
  if (nfull > 0) flush_y((nfull & 1) ? tin_a : tin_b, static_cast<int64_t>(nfull - 1) << 10);
  // remaining tokens: with vec at most one partial tile, staged like a full
  // one -- L is a multiple of 8, so its 8-token chunks are whole or absent;
  // chunks at or past L re-read the tile's first chunk (an in-bounds
  // address) and are then zeroed in LDS, as the bounded loads below would
  // leave them.  Rows that are not 16-byte aligned take bounded element loads.
  if (vec && (static_cast<int64_t>(nfull) << 10) < L) {
    const int64_t t0 = static_cast<int64_t>(nfull) << 10;
    wait_vmem<0>();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = unswz(64 * h + l);
      const int64_t src = (t0 + 8 * ch < L) ? t0 + 8 * ch : t0;
      dma16(x1r + src, &tin_a[0][64 * h]);
      dma16(vr + src, &tin_a[1][64 * h]);
      dma16(x2r + src, &tin_a[2][64 * h]);
    }
    wait_vmem<0>();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (t0 + 8 * unswz(64 * h + l) >= L) {
#pragma unroll
        for (int a = 0; a < 3; ++a) tin_a[a][64 * h + l] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    lds_sync();
    tile(tin_a, t0, false);
    return;
  }
#pragma unroll 1
  for (int64_t t0 = static_cast<int64_t>(nfull) << 10; t0 < L; t0 += 1024) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = l + 64 * h;
      const int64_t pos = t0 + 8 * ch;
      const bf16_t* src[3] = {x1r, vr, x2r};
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        uint32_t ws[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (pos + e < L) ws[e >> 1] |= static_cast<uint32_t>(src[a][pos + e]) << (16 * (e & 1));
        tin_a[a][swz(ch)] = make_uint4(ws[0], ws[1], ws[2], ws[3]);
      }
    }
    lds_sync();
    tile(tin_a, t0, false);
  }
}

int fir_mfma_diagonals(int K) { return (K - 1 + 31) / 32 + 1; }

// Token-major form (in_proj's (B, L, 3D) with each channel's x1, x2, v at
// elements 3c + pos1 / pos2 / posv, y (B, L, D), u for t < 0 from the
// caller's window): a workgroup of 8 waves takes 8 consecutive channels, one
// wave per channel running the tile computation above.  A tile's 1024 token
// rows of the block's 48-byte span are loaded into registers one tile ahead
// (6 x 16 bytes per thread, three consecutive threads per row) and stored to
// LDS row by row, slot 3 tm_swz(t) + j for chunk j of token t, once every
// wave has read the previous tile; each wave gathers its channel's runs from
// there.  Staging through registers leaves no LDS-DMA in flight, so the
// per-wave u buffers are ordinary LDS accesses.  y goes back through a
// token-major LDS tile as one 16-byte piece per token row; workgroups are
// grouped on the XCDs as in chunk_mfma.hip's token-major form.
template <int ND>
__global__ __launch_bounds__(512) void fir_mfma_tm_kernel(
    const bf16_t* __restrict__ xin, int pos1, int pos2, int posv, const float* __restrict__ taps,
    int K, const float* __restrict__ skip, const float* __restrict__ win_in,
    bf16_t* __restrict__ y, int D, int L) {
  constexpr int NB = 32 + ND - 1;
  constexpr int NWV = 8;
  __shared__ float wbufs[NWV][32 * ND];
  __shared__ uint4 tin[3 * 1024];
  __shared__ uint4 ubs[NWV][2][NB * 4];
  __shared__ uint4 tout[1024];

  const int tid = static_cast<int>(threadIdx.x);
  const int l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = l >> 5;
  const int i32 = l & 31;
  const int64_t nwg = gridDim.x, g = blockIdx.x;
  const int64_t lg = (nwg % 64 == 0) ? 64 * (g / 64) + 8 * (g % 8) + (g / 8) % 8 : g;
  const int nblk = D >> 3;
  const int64_t bat = lg / nblk;
  const int cblk = static_cast<int>(lg % nblk);
  const int c = 8 * cblk + wv;
  const int64_t row = bat * D + c;
  const int64_t ld3 = 3 * static_cast<int64_t>(D);
  const bf16_t* const xb = xin + bat * L * ld3 + 24 * cblk;
  bf16_t* const yb = y + bat * L * static_cast<int64_t>(D) + 8 * cblk;
  const float sk = skip ? skip[c] : 0.0f;
  float* const wbuf = wbufs[wv];
  uint4 (*const ub)[NB * 4] = ubs[wv];

  // taps, and the halo before the first tile: u[t] for -32 (ND-1) <= t < 0
  // from the window (its last K-1 entries), else zero, as two bf16 parts
  for (int j = l; j < 32 * ND; j += 64) wbuf[j] = (j < K) ? taps[static_cast<int64_t>(c) * K + j] : 0.0f;
  for (int j = l; j < 2 * NB * 4; j += 64) ub[j / (NB * 4)][j % (NB * 4)] = make_uint4(0, 0, 0, 0);
  lds_sync();
  if (win_in) {
    uint16_t* const u16 = reinterpret_cast<uint16_t*>(&ub[0][0]);
    for (int k = l; k < 32 * (ND - 1); k += 64) {
      const int t = k - 32 * (ND - 1);
      const float w = (t >= -(K - 1)) ? win_in[row * (K - 1) + (K - 1) + t] : 0.0f;
      const uint32_t pw = cvt2(w, 0.0f);
      const float w0 = lo_f(pw);
      const uint32_t pr = cvt2(w - w0, 0.0f);
      const int e = 8 * swz(4 * (k >> 5) + ((k & 31) >> 3)) + (k & 7);
      u16[e] = static_cast<uint16_t>(pw);
      u16[8 * NB * 4 + e] = static_cast<uint16_t>(pr);
    }
    lds_sync();
  }

  // A operands: T_d parts, as in fir_mfma_kernel
  bf16x8 ta[ND][2][2];
  uint32_t lo_bits = 0;
#pragma unroll
  for (int d = 0; d < ND; ++d) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = 32 * d + i32 - blk_tok(8 * s + j, hf);
        const float w = (idx >= 0 && idx < 32 * ND) ? wbuf[idx] : 0.0f;
        const __bf16 w0 = static_cast<__bf16>(w);
        const __bf16 w1 = static_cast<__bf16>(w - static_cast<float>(w0));
        ta[d][0][s][j] = w0;
        ta[d][1][s][j] = w1;
        lo_bits |= __builtin_bit_cast(uint16_t, w1);
      }
      pin(ta[d][0][s]);
      pin(ta[d][1][s]);
    }
  }
  const bool exact_taps = !__any(lo_bits != 0);

  // tile loads: thread tid takes slots tid + 512 k, k < 6 (chunk s % 3 of
  // token tm_swz(s / 3)); rows at or past L load as zeros
  uint4 pre[6];
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int s = tid + 512 * k;
      const int64_t t = t0 + tm_swz(s / 3);
      pre[k] = (t < L) ? *reinterpret_cast<const uint4*>(xb + t * ld3 + 8 * (s % 3))
                       : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  const int nt = (L + 1023) >> 10;
  if (nt > 0) load_tile(0);
  const int e1 = 3 * wv + pos1, ev = 3 * wv + posv, e2 = 3 * wv + pos2;
#pragma unroll 1
  for (int kt = 0; kt < nt; ++kt) {
    const int64_t t0 = static_cast<int64_t>(kt) << 10;
    wg_sync();                                // every wave has read the previous tile and y
#pragma unroll
    for (int k = 0; k < 6; ++k) tin[tid + 512 * k] = pre[k];
    if (kt + 1 < nt) load_tile(t0 + 1024);
    wg_sync();                                // the tile is in LDS
    // this lane's runs: token 32 i32 + 8q + 4hf + e at row tm_swz(t) = 32 i32 + ((8q + e) ^ m)
    uint32_t rb = 768u * static_cast<uint32_t>(i32);     // 24 elements per row
    uint32_t m = static_cast<uint32_t>((i32 & 15) ^ (4 * hf));
    asm volatile("" : "+v"(rb), "+v"(m));     // formed here, not kept across tiles
    const uint16_t* const tu = reinterpret_cast<const uint16_t*>(tin);
    float su[16];
    uint2 up[2][4];
    uint2 gq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float u[4];
      uint32_t gw[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t r = rb + 24u * ((8u * q + e) ^ m);
        const float xa = __uint_as_float(static_cast<uint32_t>(tu[r + e1]) << 16);
        const float xv = __uint_as_float(static_cast<uint32_t>(tu[r + ev]) << 16);
        gw[e >> 1] |= static_cast<uint32_t>(tu[r + e2]) << (16 * (e & 1));
        u[e] = xa * xv;
        su[4 * q + e] = sk * u[e];
      }
      gq[q] = make_uint2(gw[0], gw[1]);
      const uint32_t a0 = cvt2(u[0], u[1]), a1 = cvt2(u[2], u[3]);
      up[0][q] = make_uint2(a0, a1);
      up[1][q] = make_uint2(cvt2(u[0] - lo_f(a0), u[1] - hi_f(a0)), cvt2(u[2] - lo_f(a1), u[3] - hi_f(a1)));
      const int us = swz(4 * (i32 + ND - 1) + q);
      reinterpret_cast<uint2*>(&ub[0][us])[hf] = up[0][q];
      reinterpret_cast<uint2*>(&ub[1][us])[hf] = up[1][q];
    }
    lds_sync();
    f32x16 cz = {};
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int blk = i32 + ND - 1 - d;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 b[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint2 r0 = reinterpret_cast<const uint2*>(&ub[p][swz(4 * blk + 2 * s)])[hf];
          const uint2 r1 = reinterpret_cast<const uint2*>(&ub[p][swz(4 * blk + 2 * s + 1)])[hf];
          const u32x4 w4 = {r0.x, r0.y, r1.x, r1.y};
          b[p] = __builtin_bit_cast(bf16x8, w4);
        }
        cz = mfma(ta[d][0][s], b[0], cz);
        cz = mfma(ta[d][0][s], b[1], cz);
        if (!exact_taps) {
          cz = mfma(ta[d][1][s], b[0], cz);
          cz = mfma(ta[d][1][s], b[1], cz);
        }
      }
    }
    lds_sync();                               // ub read out before the halo moves
    // the last ND-1 blocks become the next tile's halo
    if (ND > 1 && i32 >= 33 - ND) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int hs = swz(4 * (i32 - (33 - ND)) + q);
        reinterpret_cast<uint2*>(&ub[0][hs])[hf] = up[0][q];
        reinterpret_cast<uint2*>(&ub[1][hs])[hf] = up[1][q];
      }
    }
    // y = x2 z + skip u into the token-major y tile: token t -> element wv
    // of slot tm_swz(t)
    {
      uint32_t yl = 256u * static_cast<uint32_t>(i32) + static_cast<uint32_t>(wv);
      uint32_t m8 = 8u * static_cast<uint32_t>((i32 & 15) ^ (4 * hf));
      asm volatile("" : "+v"(yl), "+v"(m8));
      uint16_t* const yt = reinterpret_cast<uint16_t*>(tout);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float o0 = fmaf(lo_f(gq[q].x), cz[4 * q + 0], su[4 * q + 0]);
        const float o1 = fmaf(hi_f(gq[q].x), cz[4 * q + 1], su[4 * q + 1]);
        const float o2 = fmaf(lo_f(gq[q].y), cz[4 * q + 2], su[4 * q + 2]);
        const float o3 = fmaf(hi_f(gq[q].y), cz[4 * q + 3], su[4 * q + 3]);
        const uint32_t p01 = cvt2(o0, o1), p23 = cvt2(o2, o3);
        yt[yl + ((64u * q + 0u) ^ m8)] = static_cast<uint16_t>(p01);
        yt[yl + ((64u * q + 8u) ^ m8)] = static_cast<uint16_t>(p01 >> 16);
        yt[yl + ((64u * q + 16u) ^ m8)] = static_cast<uint16_t>(p23);
        yt[yl + ((64u * q + 24u) ^ m8)] = static_cast<uint16_t>(p23 >> 16);
      }
    }
    wg_sync();                                // every wave's y in tout
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sl = tid + 512 * h;
      const int64_t t = t0 + tm_swz(sl);
      if (t < L) *reinterpret_cast<uint4*>(yb + t * D) = tout[sl];
    }
  }
}

// Token-major FIR on blocks of 32 channels.  Each token row of the block is
// one 192-byte span of xin and one 64-byte span of y, so a workgroup reads and
// writes whole cache lines or halves of them instead of 48- and 16-byte
// pieces: at B = 1, D = 4096, L = 32768 the 8-channel form above spends about
// a third of its time on the request rate of those pieces.  With 32 channels
// the tile is 256 tokens (48 KB of inputs), cut into 16-token blocks for the
// 16x16x32 matrix instruction:
//     z_n = sum_{d<ND} A_d . U_{n,d},   A_d[i][k] = w[i + 32d + 16 - k],
// U_{n,d} the 32 tokens from 16(n - 2d - 1) on, so that output block n of
// the tile (one column) needs the tile and the 32 ND - 16 tokens before it.
// Wave w takes channels 4w .. 4w+3 of the block, one after the other, with
// their A operands in registers (the first bf16 part of the taps; taps that
// are not bf16 values form their second part from the tap array on every
// tile, a slow path that bf16 models do not take).  The
// sequence is cut into segments so that the grid fills the chip; a segment
// after the first starts with one tile that only fills the u buffers.
// LDS: the tile in rows of 256 bytes (192 used) with the 16-byte chunks of a
// row permuted by bits of the row index, so that the 64 rows a wave gathers
// from at once spread over the banks (also the tap table at setup); per wave
// and channel both u parts of the tile and its halo; the y tile.  The four
// channels of a wave are 24 adjacent bytes of a row, read as three 8-byte
// words; u = x1 v takes the two elements of each triple that are not the
// gate, so only the gate's position PG is needed, as a template parameter.
template <int ND, int PG>
__global__ __launch_bounds__(512) void fir_mfma_tm32_kernel(
    const bf16_t* __restrict__ xin, int pos1, int pos2, int posv, const float* __restrict__ taps,
    int K, const float* __restrict__ skip, const float* __restrict__ win_in,
    bf16_t* __restrict__ y, int D, int L, int nseg, int seg_len) {
  constexpr int HT = 32 * ND - 16;            // tokens before the tile that the products read
  constexpr int UBC = (HT + 256) / 8;         // 16-byte chunks of one u part of one channel
  constexpr int KP = 32 * ND + 16;            // tap table row: lag + 16
  __shared__ uint4 tin[256 * 16];
  __shared__ uint4 ubs[8][4][2][UBC];
  __shared__ uint32_t tout[256 * 16];

  const int tid = static_cast<int>(threadIdx.x);
  const int l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = l & 15, g = l >> 4;
  // neighbouring blocks (which share a 128-byte line of each row) on one XCD
  const int ncb = D >> 5;
  const int64_t nwg = gridDim.x, gid = blockIdx.x;
  const int64_t lg = (nwg % 16 == 0) ? 16 * (gid / 16) + 2 * (gid % 8) + (gid / 8) % 2 : gid;
  const int cb = static_cast<int>(lg % ncb);
  const int64_t rest = lg / ncb;
  const int seg = static_cast<int>(rest % nseg);
  const int64_t bat = rest / nseg;
  const int64_t ld3 = 3 * static_cast<int64_t>(D);
  const bf16_t* const xb = xin + bat * L * ld3 + 96 * cb;
  bf16_t* const yb = y + bat * L * static_cast<int64_t>(D) + 32 * cb;
  const int64_t t_begin = static_cast<int64_t>(seg) * seg_len;
  const int64_t t_end = min(static_cast<int64_t>(L), t_begin + seg_len);

  // taps of the block's channels by lag + 16 (zero outside [0, K)), and
  // cleared u buffers
  float* const wtab = reinterpret_cast<float*>(tin);
  for (int x = tid; x < 32 * KP; x += 512) {
    const int cl = x / KP, k = x % KP - 16;
    wtab[x] = (k >= 0 && k < K) ? taps[static_cast<int64_t>(32 * cb + cl) * K + k] : 0.0f;
  }
  for (int x = tid; x < 8 * 4 * 2 * UBC; x += 512) (&ubs[0][0][0][0])[x] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  // A operands: lane (row n, k-group g) holds A_d[n][8g + e] = w[n + 32d + 16 - 8g - e]
  bf16x8 ta[4][ND];
  uint32_t lo_bits = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float* const wr = wtab + (4 * wv + j) * KP;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = wr[n + 32 * d + 32 - 8 * g - e];
        const __bf16 w0 = static_cast<__bf16>(w);
        ta[j][d][e] = w0;
        lo_bits |= __builtin_bit_cast(uint16_t, static_cast<__bf16>(w - static_cast<float>(w0)));
      }
      pin(ta[j][d]);
    }
  }
  // taps that are bf16 values have no second part anywhere in the wave
  const bool exact_taps = !__any(lo_bits != 0);
  // the first segment's halo from the window: u[t], -HT <= t < 0, as two bf16 parts
  if (seg == 0 && win_in && K > 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = bat * D + 32 * cb + 4 * wv + j;
      uint16_t* const u0 = reinterpret_cast<uint16_t*>(&ubs[wv][j][0][0]);
      uint16_t* const u1 = reinterpret_cast<uint16_t*>(&ubs[wv][j][1][0]);
      for (int p = l; p < HT; p += 64) {
        const int t = p - HT;
        const float w = (t >= -(K - 1)) ? win_in[row * (K - 1) + (K - 1) + t] : 0.0f;
        const uint32_t pw = cvt2(w, 0.0f);
        u0[p] = static_cast<uint16_t>(pw);
        u1[p] = static_cast<uint16_t>(cvt2(w - lo_f(pw), 0.0f));
      }
    }
  }
  __syncthreads();                            // tap table read out before the tile goes over it

  float sk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sk[j] = skip ? skip[32 * cb + 4 * wv + j] : 0.0f;
  // tile loads: thread tid takes slots tid + 512 k (k < 6), chunk s % 12 of
  // row s / 12, at a 32-bit byte offset from the tile's first row; only a
  // tile that reaches past L tests its rows
  uint4 pre[6];
  const uint32_t rowb = static_cast<uint32_t>(2 * ld3);
  auto load_tile = [&](int64_t t0, const int (&rw)[6], const int (&ck)[6]) {
    const char* const base = reinterpret_cast<const char*>(xb + t0 * ld3);
    if (t0 + 256 <= L) {
#pragma unroll
      for (int k = 0; k < 6; ++k)
        pre[k] = *reinterpret_cast<const uint4*>(base + (static_cast<uint32_t>(rw[k]) * rowb + 16u * ck[k]));
    } else {
#pragma unroll
      for (int k = 0; k < 6; ++k)
        pre[k] = (t0 + rw[k] < L)
                     ? *reinterpret_cast<const uint4*>(base + (static_cast<uint32_t>(rw[k]) * rowb + 16u * ck[k]))
                     : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto slots = [&](int (&rw)[6], int (&ck)[6]) {
    int tt = tid;
    asm volatile("" : "+v"(tt));              // formed per tile, not kept across the loop
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      rw[k] = (tt + 512 * k) / 12;
      ck[k] = (tt + 512 * k) - 12 * rw[k];
    }
  };
  int64_t t0 = (seg > 0) ? t_begin - 256 : t_begin;
  {
    int rw[6], ck[6];
    slots(rw, ck);
    load_tile(t0, rw, ck);
  }
  // the lane's tokens are rows 16n + 4g + e (e < 4) of the tile; their chunk
  // permutation h = (row >> 2) & 15 is the same for all four
  const uint32_t h = static_cast<uint32_t>((4 * n + g) & 15);
#pragma unroll 1
  for (; t0 < t_end; t0 += 256) {
    wg_sync();                                // every wave has read the previous tile and y
    {
      int rw[6], ck[6];
      slots(rw, ck);
#pragma unroll
      for (int k = 0; k < 6; ++k) tin[16 * rw[k] + (ck[k] ^ ((rw[k] >> 2) & 15))] = pre[k];
      if (t0 + 256 < t_end) load_tile(t0 + 256, rw, ck);
    }
    wg_sync();                                // the tile is in LDS
    const bool emit = t0 >= t_begin;          // not the filling tile of a later segment
    uint32_t rbase = 128u * static_cast<uint32_t>(16 * n + 4 * g);
    uint32_t hl = h;
    asm volatile("" : "+v"(rbase), "+v"(hl)); // formed here, not kept across tiles
    // the four channels in phases, so that each phase's LDS latency is met
    // once: their inputs, then their u parts into the buffers, then the
    // products and y, then the halos.  Row 16n + 4g + e holds the wave's
    // triples at bytes 24 wv .. 24 wv + 23: three 8-byte words, each inside
    // one 16-byte chunk.
    uint32_t wd[4][6];
    {
      const uint2* const t2 = reinterpret_cast<const uint2*>(tin);
      uint32_t q8[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const uint32_t off = static_cast<uint32_t>(24 * wv + 8 * i);           // bytes in the row
        q8[i] = (rbase >> 2) + 2u * ((off >> 4) ^ hl) + ((off >> 3) & 1u);    // in 8-byte units
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const uint2 w2 = t2[q8[i] + 32u * e];
          wd[e][2 * i] = w2.x;
          wd[e][2 * i + 1] = w2.y;
        }
      }
    }
    constexpr int PA = (PG == 0) ? 1 : 0, PB = (PG == 2) ? 1 : 2;     // the two factors of u
    auto el = [&](int e, int k) {             // element k (< 12) of row e as the high half of a float
      const uint32_t w = wd[e][k >> 1];
      return (k & 1) ? (w & 0xFFFF0000u) : (w << 16);
    };
    float su[4][4];
    uint32_t gw[4][2];
    uint2 uh[4], ul[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[e] = __uint_as_float(el(e, 3 * j + PA)) * __uint_as_float(el(e, 3 * j + PB));
        su[j][e] = sk[j] * u[e];
      }
      gw[j][0] = (el(0, 3 * j + PG) >> 16) | el(1, 3 * j + PG);
      gw[j][1] = (el(2, 3 * j + PG) >> 16) | el(3, 3 * j + PG);
      // u = x1 v is exactly two bf16 parts
      const uint32_t p0 = cvt2(u[0], u[1]), p1 = cvt2(u[2], u[3]);
      uh[j] = make_uint2(p0, p1);
      ul[j] = make_uint2(cvt2(u[0] - lo_f(p0), u[1] - hi_f(p0)), cvt2(u[2] - lo_f(p1), u[3] - hi_f(p1)));
    }
    const int up = (HT + 16 * n + 4 * g) >> 2;            // in 8-byte units
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      reinterpret_cast<uint2*>(&ubs[wv][j][0][0])[up] = uh[j];
      reinterpret_cast<uint2*>(&ubs[wv][j][1][0])[up] = ul[j];
    }
    lds_sync();
    if (emit) {
      float yv[4][4];                         // [channel][token]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cl = 4 * wv + j;
        f32x4 cz = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int ci = HT / 8 + 2 * n - 4 * d - 2 + g;
          const bf16x8 b0 = __builtin_bit_cast(bf16x8, ubs[wv][j][0][ci]);
          const bf16x8 b1 = __builtin_bit_cast(bf16x8, ubs[wv][j][1][ci]);
          cz = mfma16(ta[j][d], b0, cz);
          cz = mfma16(ta[j][d], b1, cz);
          if (!exact_taps) {
            // the taps' second bf16 part, from the tap array
            const float* const wc = taps + static_cast<int64_t>(32 * cb + cl) * K;
            int kb = n + 32 * d + 16 - 8 * g;
            asm volatile("" : "+v"(kb));      // per tile: not hoisted out of the loop
            bf16x8 t1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int k = kb - e;
              const float w = (k >= 0 && k < K) ? wc[k] : 0.0f;
              t1[e] = static_cast<__bf16>(w - static_cast<float>(static_cast<__bf16>(w)));
            }
            cz = mfma16(t1, b0, cz);
            cz = mfma16(t1, b1, cz);
          }
        }
        // y = x2 z + skip u
        yv[j][0] = fmaf(lo_f(gw[j][0]), cz[0], su[j][0]);
        yv[j][1] = fmaf(hi_f(gw[j][0]), cz[1], su[j][1]);
        yv[j][2] = fmaf(lo_f(gw[j][1]), cz[2], su[j][2]);
        yv[j][3] = fmaf(hi_f(gw[j][1]), cz[3], su[j][3]);
      }
      // the y tile: row 16n + 4g + e, the wave's four channels as one 8-byte
      // word, word wv of the row's eight permuted by h & 7
      uint2* const y2 = reinterpret_cast<uint2*>(tout);
      const uint32_t ya = 8u * static_cast<uint32_t>(16 * n + 4 * g) + (static_cast<uint32_t>(wv) ^ (hl & 7u));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y2[ya + 8u * e] = make_uint2(cvt2(yv[0][e], yv[1][e]), cvt2(yv[2][e], yv[3][e]));
    }
    // the last HT tokens become the next tile's halo (the reads above are
    // issued first, and one wave's LDS accesses complete in order)
    if (l < 2 * (HT / 8)) {
      const int pp = l / (HT / 8), q = l % (HT / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) ubs[wv][j][pp][q] = ubs[wv][j][pp][32 + q];
    }
    wg_sync();                                // every wave's y in the tile
    if (emit) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int sl = tid + 512 * hh;
        const int row = sl >> 2, q = sl & 3;
        const int64_t t = t0 + row;
        const uint32_t hr = static_cast<uint32_t>((row >> 2) & 7);
        const uint2* const yr = reinterpret_cast<const uint2*>(tout) + 8 * row;
        const uint2 wa = yr[(2u * q) ^ hr], wb = yr[(2u * q + 1u) ^ hr];
        const uint4 w4 = make_uint4(wa.x, wa.y, wb.x, wb.y);
        if (t < t_end) *reinterpret_cast<uint4*>(yb + t * D + 8 * q) = w4;
      }
    }
  }
}

// bf16, K <= 128, D a multiple of 8 below 349526, xin and y 16-byte aligned.
bool tokmajor_fir_mfma_supported(const TokmajorFirArgs& a) {
  return a.bf16 && a.K <= 128 && a.D % 8 == 0 && a.L > 0 && a.B > 0 &&
         int64_t(a.D) * 6 * 1024 <= INT32_MAX && aligned_all(16, a.xin, a.y);
}

// The 32-channel form: D a multiple of 32.
static bool tokmajor_fir_mfma32_supported(const TokmajorFirArgs& a) {
  return tokmajor_fir_mfma_supported(a) && a.D % 32 == 0;
}

// 16-token blocks: output block n reads 32-token spans 16(n - 2d - 1) for
// d < ND, which reach lag K - 1 at the block's first row.
static int fir_mfma16_diagonals(int K) { return (K - 1 <= 16) ? 1 : (K - 17 + 31) / 32 + 1; }

static hipError_t launch_fir_mfma_tokmajor32(const TokmajorFirArgs& a) {
  const int64_t ncb = a.D / 32;
  // segments of whole 256-token tiles, until the grid covers the CUs or a
  // segment would drop below 2048 tokens
  int64_t nseg = 1;
  while (a.B * ncb * nseg < 256 && (a.L + 2 * nseg - 1) / (2 * nseg) >= 2048) nseg *= 2;
  const int64_t seg_len = ((a.L + nseg - 1) / nseg + 255) / 256 * 256;
  nseg = (a.L + seg_len - 1) / seg_len;
  const int64_t nwg = a.B * ncb * nseg;
  if (nwg > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(nwg)), block(512);
  const bf16_t* x = static_cast<const bf16_t*>(a.xin);
  bf16_t* y = static_cast<bf16_t*>(a.y);
  if (a.pos_x2 < 0 || a.pos_x2 > 2) return hipErrorInvalidValue;
#define HYENA_FIR_TM32(NDV, PGV)                                                                \
  fir_mfma_tm32_kernel<NDV, PGV><<<grid, block, 0, a.stream>>>(                                 \
      x, a.pos_x1, a.pos_x2, a.pos_v, a.taps, a.K, a.skip, a.win_in, y, a.D, a.L,               \
      static_cast<int>(nseg), static_cast<int>(seg_len))
#define HYENA_FIR_TM32_PG(NDV)                          \
  switch (a.pos_x2) {                                   \
    case 0: HYENA_FIR_TM32(NDV, 0); break;              \
    case 1: HYENA_FIR_TM32(NDV, 1); break;              \
    default: HYENA_FIR_TM32(NDV, 2); break;             \
  }
  switch (fir_mfma16_diagonals(a.K)) {
    case 1: HYENA_FIR_TM32_PG(1); break;
    case 2: HYENA_FIR_TM32_PG(2); break;
    case 3: HYENA_FIR_TM32_PG(3); break;
    case 4: HYENA_FIR_TM32_PG(4); break;
    case 5: HYENA_FIR_TM32_PG(5); break;
    default: return hipErrorInvalidValue;
  }
#undef HYENA_FIR_TM32_PG
#undef HYENA_FIR_TM32
  return hipGetLastError();
}

hipError_t launch_fir_mfma_tokmajor(const TokmajorFirArgs& a) {
  if (!tokmajor_fir_mfma_supported(a)) return hipErrorInvalidValue;
  if (tokmajor_fir_mfma32_supported(a)) return launch_fir_mfma_tokmajor32(a);
  const int nd = fir_mfma_diagonals(a.K);
  dim3 grid(static_cast<unsigned>(a.B * (a.D / 8))), block(512);
  const bf16_t* x = static_cast<const bf16_t*>(a.xin);
  bf16_t* y = static_cast<bf16_t*>(a.y);
#define HYENA_FIR_TM(NDV)                                                                      \
  fir_mfma_tm_kernel<NDV><<<grid, block, 0, a.stream>>>(x, a.pos_x1, a.pos_x2, a.pos_v, a.taps, \
                                                         a.K, a.skip, a.win_in, y, a.D, a.L)
  switch (nd) {
    case 1: HYENA_FIR_TM(1); break;
    case 2: HYENA_FIR_TM(2); break;
    case 3: HYENA_FIR_TM(3); break;
    case 4: HYENA_FIR_TM(4); break;
    case 5: HYENA_FIR_TM(5); break;
    default: return hipErrorInvalidValue;
  }
#undef HYENA_FIR_TM
  return hipGetLastError();
}



hipError_t launch_fir_mfma(const FirArgs& a) {
  const int nd = fir_mfma_diagonals(a.K);
  const bool vec = (a.L % 8 == 0) && aligned_all(16, a.x1, a.x2, a.v, a.y);
  dim3 grid(static_cast<unsigned>(a.B * a.D)), block(64);
  const bf16_t* x1 = static_cast<const bf16_t*>(a.x1);
  const bf16_t* x2 = static_cast<const bf16_t*>(a.x2);
  const bf16_t* v = static_cast<const bf16_t*>(a.v);
  bf16_t* y = static_cast<bf16_t*>(a.y);
  switch (nd) {
    case 1: fir_mfma_kernel<1><<<grid, block, 0, a.stream>>>(x1, x2, v, a.taps, a.K, a.skip, y, a.D, a.L, vec); break;
    case 2: fir_mfma_kernel<2><<<grid, block, 0, a.stream>>>(x1, x2, v, a.taps, a.K, a.skip, y, a.D, a.L, vec); break;
    case 3: fir_mfma_kernel<3><<<grid, block, 0, a.stream>>>(x1, x2, v, a.taps, a.K, a.skip, y, a.D, a.L, vec); break;
    case 4: fir_mfma_kernel<4><<<grid, block, 0, a.stream>>>(x1, x2, v, a.taps, a.K, a.skip, y, a.D, a.L, vec); break;
    case 5: fir_mfma_kernel<5><<<grid, block, 0, a.stream>>>(x1, x2, v, a.taps, a.K, a.skip, y, a.D, a.L, vec); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hyena
