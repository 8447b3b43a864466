// mfma_common.hpp -- pieces shared by the matrix-core kernels (chunk_mfma.hip,
// fir_mfma.hip): bf16 operand vectors and splits, the 32x32x16 and 16x16x32
// MFMAs, the per-lane token layout, and the LDS staging of 1024-token tiles.
#pragma once

#include "common.hpp"

namespace hyena {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int MFMA_MAXN = 16;        // mode slots of the 16-slot kernels (one-tile, token-major)
constexpr int MFMA_MAXN_WIDE = 32;   // slots of the chunk kernel's 32-slot form

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Per-row operands are computed once and must stay in registers: the empty
// asm hides how they were made, so the compiler cannot recompute them (with
// their exp calls) inside the tile loop to save registers.
__device__ __forceinline__ void pin(bf16x8& x) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
  asm volatile("" : "+v"(w));
  x = __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32: lane l holds row l % 16 of A and column l % 16 of B, each with
// K elements 8 (l / 16) .. + 7, and rows 4 (l / 16) .. + 3 of column l % 16
// of the result (checked against a host product on gfx950).
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x = p0 + p1 + p2 + r with p_k = rne_bf16 of the remainder so far; |r| <= 2^-24 |x|
__device__ __forceinline__ void split3(float x, __bf16& p0, __bf16& p1, __bf16& p2) {
  p0 = static_cast<__bf16>(x);
  const float r1 = x - static_cast<float>(p0);
  p1 = static_cast<__bf16>(r1);
  p2 = static_cast<__bf16>(r1 - static_cast<float>(p1));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair (one v_cvt_pk_bf16_f32), and back.
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// split3 on a pair, each part a packed bf16 pair
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
  p0 = cvt2(a, b);
  float ra = a - lo_f(p0), rb = b - hi_f(p0);
  p1 = cvt2(ra, rb);
  ra -= lo_f(p1);
  rb -= hi_f(p1);
  p2 = cvt2(ra, rb);
}

// token (within a 32-token block) of output register r / operand slot
// (s, j) = r = 8s + j of a lane in half-wave hf
__device__ __forceinline__ int blk_tok(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// 4 consecutive elements at [i, i+4) of a row, zero at and beyond L
template <typename IO, bool VEC>
__device__ __forceinline__ void ld4(const IO* row, int64_t i, int64_t L, float (&o)[4]) {
  if constexpr (VEC) {
    if (i + 4 <= L) {
      if constexpr (sizeof(IO) == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(row + i);
        o[0] = __uint_as_float(w.x << 16);
        o[1] = __uint_as_float(w.x & 0xFFFF0000u);
        o[2] = __uint_as_float(w.y << 16);
        o[3] = __uint_as_float(w.y & 0xFFFF0000u);
      } else {
        const float4 f = *reinterpret_cast<const float4*>(row + i);
        o[0] = f.x; o[1] = f.y; o[2] = f.z; o[3] = f.w;
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (i + e < L) ? Io<IO>::ld(row, i + e) : 0.0f;
}

// Raw storage of 4 consecutive activations (one run of a lane): 8 bytes of
// bf16 or 16 bytes of fp32, loaded without conversion so that the next tile
// can be in flight while the current one is computed.
template <typename IO> struct Raw4;
template <> struct Raw4<bf16_t> {
  uint2 w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t x = (e < 2) ? w.x : w.y;
    return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
};
template <> struct Raw4<float> {
  float4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float get(int e) const {
    return e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
  }
};

// The three input runs of one lane for one tile.
template <typename IO> struct TileIn {
  Raw4<IO> a[4], b[4], g[4];     // x1, v, x2 at tokens base + 8q .. +3
  __device__ __forceinline__ void load(const IO* x1r, const IO* vr, const IO* x2r, int64_t base) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q].load(x1r + base + 8 * q);
      b[q].load(vr + base + 8 * q);
      g[q].load(x2r + base + 8 * q);
    }
  }
};

// bf16 tiles move between HBM and LDS in 16-byte chunks (8 tokens), one
// chunk per lane per instruction, which keeps every load and store fully
// coalesced.  Chunk c = 4m + q holds tokens 32m + 8q .. +7 of block m and
// lives in LDS slot swz(c) = 4m + ((q + m/4) & 3): the coalesced writes stay
// conflict-free and so do the reads of a lane's run (block m, half hf),
// which for a fixed q touch 16 distinct slots per 256 bytes.
__device__ __forceinline__ int swz(int c) { return (c & ~3) | (((c & 3) + (c >> 4)) & 3); }

__device__ __forceinline__ int unswz(int s) { return (s & ~3) | (((s & 3) - (s >> 4)) & 3); }

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte chunk per lane from global memory straight into LDS (no
// registers): the wave writes 1 KB at `dst`, lane l at dst + 16 l.  The
// activations are read exactly once, so the load is marked non-temporal
// (cache-policy bit nt).  Measured on MI355X with new inputs every launch the
// bit gains 1-2 % on the chunk kernel; it gains far more when a launch
// re-reads the previous one's inputs, which the last-level cache then holds.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  constexpr int kNonTemporal = 2;
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst), 16, 0, kNonTemporal);
}

// The same with the default cache policy, for data whose cache lines other
// loads of the workgroup or of its neighbours read too (token-major rows,
// where one 128-byte line holds several channel blocks' pieces): non-temporal
// loads of such pieces measured ~4x the algorithmic bytes fetched from HBM.
__device__ __forceinline__ void dma16_shared(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst), 16, 0, 0);
}

// One 16-byte output chunk per lane, stored non-temporal (the output is not
// read back by this launch).  Measured on MI355X with new inputs every launch:
// the chunk kernel goes from ~219 to ~204 us per step at 32k tokens x 4096
// channels, because the written lines no longer displace into, and later drain
// from, the memory-side last-level cache between the inputs' reads.  When a
// launch re-reads what the previous one read, plain stores are faster (the
// cache then also serves inputs), which is not the case this is tuned for.
__device__ __forceinline__ void store16_nt(void* dst, const uint4 q) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  v4u w;
  w.x = q.x; w.y = q.y; w.z = q.z; w.w = q.w;
  __builtin_nontemporal_store(w, static_cast<v4u*>(dst));
}

// The workgroup is a single wave: its LDS operations execute in order, so
// making LDS writes visible to the other lanes needs only that they have
// completed and that the compiler keeps program order -- no s_barrier and, in
// particular, no wait for outstanding global loads (the DMA of the next
// tile), which a __syncthreads() fence would add.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The three staged runs (x1, v, x2) of one lane for one tile, from a buffer
// of three 2 KB slices filled by dma16.  The twelve reads form one asm block
// that waits for them itself (outputs early-clobber, all used).  The compiler
// therefore sees no LDS read that may alias a DMA it considers in flight; it
// would guard such a read by waiting for every vector memory operation, the
// DMAs of later tiles included.  Ordering against the DMA that filled this
// buffer is the caller's explicit wait_vmem.
__device__ __forceinline__ void read_staged_runs(const uint4 (*tin)[128], int i32, int hf,
                                                 Raw4<bf16_t> (&a)[4], Raw4<bf16_t> (&b)[4],
                                                 Raw4<bf16_t> (&g)[4]) {
  const uint32_t base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const lds_void*)(&tin[0][0])));
  uint32_t ad[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ad[q] = base + 16u * swz(4 * i32 + q) + 8u * hf;
  uint64_t r[12];
  asm volatile(
      "ds_read_b64 %0, %12\n\t"
      "ds_read_b64 %1, %12 offset:2048\n\t"
      "ds_read_b64 %2, %12 offset:4096\n\t"
      "ds_read_b64 %3, %13\n\t"
      "ds_read_b64 %4, %13 offset:2048\n\t"
      "ds_read_b64 %5, %13 offset:4096\n\t"
      "ds_read_b64 %6, %14\n\t"
      "ds_read_b64 %7, %14 offset:2048\n\t"
      "ds_read_b64 %8, %14 offset:4096\n\t"
      "ds_read_b64 %9, %15\n\t"
      "ds_read_b64 %10, %15 offset:2048\n\t"
      "ds_read_b64 %11, %15 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a[q].w = make_uint2(static_cast<uint32_t>(r[3 * q]), static_cast<uint32_t>(r[3 * q] >> 32));
    b[q].w = make_uint2(static_cast<uint32_t>(r[3 * q + 1]), static_cast<uint32_t>(r[3 * q + 1] >> 32));
    g[q].w = make_uint2(static_cast<uint32_t>(r[3 * q + 2]), static_cast<uint32_t>(r[3 * q + 2] >> 32));
  }
}

// Token-major staging of a block of 8 channels (24 elements, 48 bytes per
// token row): LDS slot 3 tm_swz(t) + j holds chunk j (elements 8j .. 8j+7)
// of token row t of the tile, so that the three chunks of a row are adjacent
// and one DMA instruction (64 consecutive slots) fetches whole 48-byte pieces
// of ~21 rows.  tm_swz is an involution on [0, 1024) that spreads the rows a
// wave reads together (t = 32 i + const, i < 32) over the 16 groups of 4 LDS
// banks a 16-byte slot spans (3 tm_swz(t) mod 16 takes 16 values).
__device__ __forceinline__ int tm_swz(int t) { return t ^ ((t >> 5) & 15); }

// The runs of one channel of a token-major tile, as read_staged_runs gives
// them for the channel-major layout: x1, v, x2 at tokens 32 i32 + 8q + 4hf + e
// (e < 4), elements e1, ev, e2 of the span.  Per run, 12 two-byte reads in
// one asm block that waits for them itself, for the reason given at
// read_staged_runs; outputs early-clobber, all used.
__device__ __forceinline__ void read_tm_runs(const uint4* tin, int i32, int hf, int e1, int ev,
                                             int e2, Raw4<bf16_t> (&a)[4], Raw4<bf16_t> (&b)[4],
                                             Raw4<bf16_t> (&g)[4]) {
  // token t = 32 i32 + c (c = 8q + 4hf + e < 32) is row tm_swz(t) = 32 i32 + ((8q + e) ^ m),
  // m = (i32 & 15) ^ 4 hf, at byte 48 tm_swz(t) of the tile.  The lane's
  // bases pass through an empty asm, so the addresses are formed here on
  // every call instead of being kept in registers across the tile loop.
  uint32_t lb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)(tin))) +
                1536u * static_cast<uint32_t>(i32);
  uint32_t m = static_cast<uint32_t>((i32 & 15) ^ (4 * hf));
  asm volatile("" : "+v"(lb), "+v"(m));
  auto off = [](int e) { return static_cast<uint32_t>((e >> 3) * 16 + (e & 7) * 2); };
  const uint32_t bs[3] = {lb + off(e1), lb + off(ev), lb + off(e2)};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t ad[12];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = 48u * ((8u * q + e) ^ m);
#pragma unroll
      for (int st = 0; st < 3; ++st) ad[3 * e + st] = bs[st] + x;
    }
    uint32_t r[12];
    asm volatile(
        "ds_read_u16 %0, %12\n\t"
        "ds_read_u16 %1, %13\n\t"
        "ds_read_u16 %2, %14\n\t"
        "ds_read_u16 %3, %15\n\t"
        "ds_read_u16 %4, %16\n\t"
        "ds_read_u16 %5, %17\n\t"
        "ds_read_u16 %6, %18\n\t"
        "ds_read_u16 %7, %19\n\t"
        "ds_read_u16 %8, %20\n\t"
        "ds_read_u16 %9, %21\n\t"
        "ds_read_u16 %10, %22\n\t"
        "ds_read_u16 %11, %23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7]), "v"(ad[8]), "v"(ad[9]), "v"(ad[10]), "v"(ad[11])
        : "memory");
    // r[3e + st]: stream st (x1, v, x2) at token e of the run
    a[q].w = make_uint2(r[0] | (r[3] << 16), r[6] | (r[9] << 16));
    b[q].w = make_uint2(r[1] | (r[4] << 16), r[7] | (r[10] << 16));
    g[q].w = make_uint2(r[2] | (r[5] << 16), r[8] | (r[11] << 16));
  }
}

// Both half-waves of every wave of the workgroup meet here, with their LDS
// operations complete.  No wait for vector memory: DMA loads issued for later
// tiles stay in flight (a __syncthreads() fence would wait for them).
__device__ __forceinline__ void wg_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector memory operations of this wave are
// outstanding.  The callers pass N = the number of LDS-DMA loads issued after
// the one they wait for and rely only on DMA loads of one wave completing in
// issue order; stores may be outstanding or not, either way the wait holds.
// (The compiler's own wait insertion for gfx950 counts plain loads and
// stores as one in-order stream but falls back to vmcnt(0) while an LDS DMA
// is pending, so no ordering between DMAs and stores is assumed here.)
// (s_waitcnt simm16 on gfx9: vmcnt[3:0] in bits
// 3:0, expcnt in bits 6:4, lgkmcnt in bits 11:8, vmcnt[5:4] in bits 15:14;
// expcnt and lgkmcnt are left free.)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}

}  // namespace hyena
