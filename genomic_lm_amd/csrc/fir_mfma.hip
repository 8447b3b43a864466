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
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = l + 64 * h;
      const uint4 w4 = tout[swz(ch)];
      const int64_t pos = t0 + 8 * ch;
      if (full || (vec && pos < L)) {       // vec: L is a multiple of 8, chunks are whole
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

  const int nfull = vec ? (L >> 10) : 0;
  if (nfull > 0) prefetch(0, tin_a);
  int k = 0;
#pragma unroll 1
  for (; k + 1 < nfull; k += 2) {
    const int64_t t0 = static_cast<int64_t>(k) << 10;
    if (k == 0) wait_vmem<0>(); else wait_vmem<2>();
    lds_sync();
    prefetch(t0 + 1024, tin_b);
    tile(tin_a, t0, true);
    wait_vmem<2>();
    lds_sync();
    if (k + 2 < nfull) prefetch(t0 + 2048, tin_a);
    tile(tin_b, t0 + 1024, true);
  }
  if (k < nfull) {
    if (k == 0) wait_vmem<0>(); else wait_vmem<2>();
    lds_sync();
    tile(tin_a, static_cast<int64_t>(k) << 10, true);
  }
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
