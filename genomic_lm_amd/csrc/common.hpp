// common.hpp -- element formats, complex arithmetic and twiddles shared by the
// gfx950 kernels of libhyena.  Device code only; no host state.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hyena {

typedef uint16_t bf16_t;   // bfloat16 bit pattern as stored in memory

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (gfx950 v_cvt_pk_bf16_f32); NaN stays NaN, overflow
// goes to +-inf as IEEE rounding says.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// ------------------------------------------------------------------ I/O
// Element access for the two activation formats.  Loads return fp32, stores
// round once.
template <typename T> struct Io;

template <> struct Io<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
  // non-temporal: for outputs that this launch never reads back
  static __device__ __forceinline__ void st_nt(float* p, int64_t i, float x) {
    __builtin_nontemporal_store(x, p + i);
  }
  // two consecutive elements [i, i+1]; requires 8-byte alignment of p + i
  static __device__ __forceinline__ float2 ld2(const float* p, int64_t i) {
    return *reinterpret_cast<const float2*>(p + i);
  }
  static __device__ __forceinline__ void st2(float* p, int64_t i, float2 x) {
    *reinterpret_cast<float2*>(p + i) = x;
  }
};

template <> struct Io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
  static __device__ __forceinline__ void st_nt(bf16_t* p, int64_t i, float x) {
    __builtin_nontemporal_store(f32_to_bf16(x), p + i);
  }
  // requires 4-byte alignment of p + i
  static __device__ __forceinline__ float2 ld2(const bf16_t* p, int64_t i) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(p + i);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
  }
  static __device__ __forceinline__ void st2(bf16_t* p, int64_t i, float2 x) {
    uint32_t w = static_cast<uint32_t>(f32_to_bf16(x.x)) |
                 (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
    *reinterpret_cast<uint32_t*>(p + i) = w;
  }
};

// Elements [i, i+1] of a row of length L, zero beyond the end.  VEC selects
// the paired access, valid when the row start is aligned to two elements.
template <typename T, bool VEC>
__device__ __forceinline__ float2 ld_pair(const T* row, int64_t i, int64_t L) {
  if (VEC && i + 1 < L) return Io<T>::ld2(row, i);
  float a = (i < L) ? Io<T>::ld(row, i) : 0.0f;
  float b = (i + 1 < L) ? Io<T>::ld(row, i + 1) : 0.0f;
  return make_float2(a, b);
}

template <typename T, bool VEC>
__device__ __forceinline__ void st_pair(T* row, int64_t i, int64_t L, float2 x) {
  if (VEC && i + 1 < L) { Io<T>::st2(row, i, x); return; }
  if (i < L) Io<T>::st(row, i, x.x);
  if (i + 1 < L) Io<T>::st(row, i + 1, x.y);
}

// ------------------------------------------------------------------ complex
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
// multiply by -i and +i
__device__ __forceinline__ float2 cmul_mi(float2 a) { return make_float2(a.y, -a.x); }
__device__ __forceinline__ float2 cmul_pi(float2 a) { return make_float2(-a.y, a.x); }

// exp(x), x <= 0, as v_exp_f32 of x * log2(e): two instructions against the
// fourteen of expf's exactly rounded range reduction.  The product's rounding
// moves the exponent by up to |x| 2^-24, so the relative error is about
// (|x| + 1) 2^-24 and the absolute error at most about 2^-24 / e: the size of
// the rounding of the terms these weights multiply.  Used for the filter's
// and the weights' exponentials; the factors that compound along a row (the
// carried state's decays) come from fp64 (pow_pair.hpp), not from here.
__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// exp(-2*pi*i * num / 2^lg), 0 <= num < 2^lg.  v_sin_f32 / v_cos_f32 take
// the angle in revolutions; -num / 2^lg is exact in fp32, and on gfx950 the
// result is within 1.3e-7 of the true value for such arguments (checked
// against fp64 over 2^20 points).
//
// The argument passes through an empty asm so that the compiler recomputes a
// twiddle where it is used (two transcendental ops) instead of keeping
// earlier copies live across whole transforms, which costs registers.
__device__ __forceinline__ float2 twiddle(int num, int lg) {
  asm volatile("" : "+v"(num));
  const float x = -ldexpf(static_cast<float>(num), -lg);
  return make_float2(__builtin_amdgcn_cosf(x), __builtin_amdgcn_sinf(x));
}

// ------------------------------------------------------------------ lane exchanges
// x of lane l ^ 32 (the other half-wave).  v_permlane32_swap exchanges the
// upper half-wave of its first operand with the lower half-wave of its
// second; with x in both, the first result holds lanes 0..31 of x in both
// halves and the second lanes 32..63.  A VALU op, unlike ds_bpermute.
__device__ __forceinline__ float xor32(float x, int hf) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(hf ? r[0] : r[1]);
}

// x of lane l ^ 16.  v_permlane16_swap exchanges the odd 16-lane rows of its
// first operand with the even rows of its second.
__device__ __forceinline__ float xor16(float x, int l) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((l & 16) ? r[0] : r[1]);
}

// x of lane l ^ 1 (DPP quad permutation 1, 0, 3, 2; a VALU op).
__device__ __forceinline__ float xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}

// Sum of x over the 64 lanes of the wave, returned in every lane: a tree of
// six additions, each lane adding a partner's partial -- quad permutations
// (lanes ^ 1, ^ 2), the half-row and row mirrors (the other quad of 8 lanes,
// the other half of 16), then the row and half-wave swaps.  All VALU (DPP and
// permlane), no LDS; ~sqrt(6) roundings of the sum instead of one per term
// of a sequential sum.
__device__ __forceinline__ float wave_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // half mirror
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row mirror
  const int l = static_cast<int>(threadIdx.x);
  x += xor16(x, l);
  x += xor32(x, (l >> 5) & 1);
  return x;
}

// ------------------------------------------------------------------ complex modes
// A complex mode exp(lam x), lam = a + i b, evaluated for real x >= 0 (up to
// 2^20).  The phase b x is reduced in revolutions at double-float precision:
// b / (2 pi) = fhi + flo, fhi x is split exactly by an fma, and only the
// fractional part reaches v_cos / v_sin (which take revolutions); a plain
// fp32 b * x would lose ~1e-3 revolutions at x = 2^15.
struct CpxMode {
  float a, fhi, flo;
};

__device__ __forceinline__ CpxMode cpx_mode(float a, float b) {
  constexpr float c_hi = 0.15915494f;   // 1 / (2 pi), high part
  constexpr float c_lo = static_cast<float>(0.15915494309189535 - static_cast<double>(c_hi));
  CpxMode m;
  m.a = a;
  m.fhi = b * c_hi;
  m.flo = fmaf(b, c_hi, -m.fhi) + b * c_lo;
  return m;
}

__device__ __forceinline__ float2 cexp_at(const CpxMode& m, float x) {
  // no contraction here: fused into p - rint(p), the product fhi x would be
  // taken exactly there and its rounding error e then added a second time
#pragma clang fp contract(off)
  const float p = m.fhi * x;
  const float e = fmaf(m.fhi, x, -p);              // exact: fhi x = p + e
  const float r = (p - rintf(p)) + fmaf(m.flo, x, e);
  const float mag = fast_exp(m.a * x);
  return make_float2(mag * __builtin_amdgcn_cosf(r), mag * __builtin_amdgcn_sinf(r));
}

}  // namespace hyena
