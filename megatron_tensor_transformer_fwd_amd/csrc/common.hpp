// Shared device helpers for the gfx950 kernels: vector types, buffer
// resources (out-of-range loads return zero and never fault), bf16 packing,
// and the activation functions with their derivatives.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace tpk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes).  Loads beyond the range
// return zero; stores beyond it are dropped.  The range is clamped to 4 GiB;
// callers keep per-block bases close to the data they touch.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// Retire loads issued before a loop whose waits are inline asm (the flash
// kernels' "s_waitcnt ... s_barrier"): the compiler's wait-count tracking
// cannot see an asm s_waitcnt, so it would keep such loads pending through
// the loop, and its waits for them (vmcnt counts in issue order) would also
// wait for the loop's own DMAs in flight.  An asm use makes the compiler
// wait for them here, once.
template <class T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

// Round-to-nearest-even fp32 -> bf16, two at a time (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

// Eight consecutive elements to and from fp32 with 16-byte accesses.  NT
// selects streaming (nontemporal) accesses for data touched once: they do
// not displace reusable lines in L2 and the Infinity Cache, and a stream of
// them runs at about twice the HBM bandwidth of ordinary accesses when the
// caches hold other kernels' dirty lines.
template <bool NT, class V>
__device__ __forceinline__ V ld16(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, class V>
__device__ __forceinline__ void st16(V* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

constexpr bool kNtIn = true;    // streamed inputs of the HBM-bound kernels
constexpr bool kNtOut = true;   // their large outputs

template <class T> struct Vec8;
template <> struct Vec8<bf16> {
  template <bool NT = false>
  static __device__ __forceinline__ void load(const bf16* p, float* o) {
    const u32x4 w = ld16<NT>(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(w[i]); o[2 * i + 1] = bf16_hi(w[i]); }
  }
  template <bool NT = false>
  static __device__ __forceinline__ void store(bf16* p, const float* v) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    st16<NT>(reinterpret_cast<u32x4*>(p), w);
  }
};
template <> struct Vec8<float> {
  template <bool NT = false>
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const f32x4 a = ld16<NT>(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = ld16<NT>(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
  }
  template <bool NT = false>
  static __device__ __forceinline__ void store(float* p, const float* v) {
    st16<NT>(reinterpret_cast<f32x4*>(p), f32x4{v[0], v[1], v[2], v[3]});
    st16<NT>(reinterpret_cast<f32x4*>(p) + 1, f32x4{v[4], v[5], v[6], v[7]});
  }
};

// ---------------------------------------------------------------------------
// Activations.  GeLU is the exact erf form, GeLU(x) = x Phi(x), with
// GeLU'(x) = Phi(x) + x phi(x).  Swish(x) = x sigmoid(x),
// Swish'(x) = sigmoid(x) (1 + x (1 - sigmoid(x))).
//
// Phi comes from erfc in the Chebyshev-fitted form
//   erfc(z) = t exp(-z^2 + P(t)),  t = 1 / (1 + z/2),  z >= 0,
// P a degree-9 polynomial, fractional error about 1e-7 at every z (Press et
// al., Numerical Recipes, 2nd ed., section 6.2).  Evaluated in fp32 it stays
// within about 1e-6 (relative) for z <= 5 and keeps that relative accuracy in
// the lower tail, where Phi(x) for x < 0 is 0.5 erfc(|x| / sqrt 2) and no
// cancellation occurs.  One reciprocal, one exp and ten FMAs: the fp32
// epilogues evaluate it for every output of the products they finish.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float erfc_nonneg(float z) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  return t * __expf(fmaf(-z, z, p));
}

// Standard normal CDF, Phi(x) = erfc(-x / sqrt 2) / 2.
__device__ __forceinline__ float norm_cdf(float x) {
  const float h = 0.5f * erfc_nonneg(fabsf(x) * 0.70710678118654752f);
  return x >= 0.f ? 1.0f - h : h;
}

__device__ __forceinline__ float gelu_f(float x) { return x * norm_cdf(x); }

__device__ __forceinline__ float gelu_prime_f(float x) {
  const float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
  return fmaf(x, pdf, norm_cdf(x));
}

// The bf16 epilogues store 8 significant bits, so they take Phi from a
// cheaper fit of the same form,
//   erfc(z) = t e^{-z^2} S(t),  t = 1 / (1 + p z),  p = 0.395,
// S a degree-6 polynomial with relative error below 3.5e-6 over z >= 0
// (fit_erfc.py beside this file: least maximum relative error).  Factoring
// e^{-z^2} out of the exp lets GeLU' reuse it as the normal density's
// e^{-x^2/2}: one reciprocal and one exp2 for either function, and seven
// fewer FMAs than the form above.  In fp32 the result stays within about
// 4e-6 (relative) for |x| <= 4 and 1.4e-5 in the far lower tail, where the
// rounding of x^2 in the exponent dominates, as it does for the form above.
struct PhiTail {
  float h;   // Phi(-|x|) = erfc(|x| / sqrt 2) / 2
  float e;   // e^{-x^2 / 2}
};
__device__ __forceinline__ PhiTail phi_tail_bf16(float x) {
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(x), 0.395f * 0.70710678118654752f, 1.0f));
  const float y = x * 0.84932180028801904f;   // sqrt(log2(e) / 2): 2^{-y^2} = e^{-x^2/2}
  const float e = __builtin_amdgcn_exp2f(-y * y);
  float s = -0.0508769453f;                   // S / 2, highest order first
  s = fmaf(s, t, 0.108530633f);
  s = fmaf(s, t, 0.0224856846f);
  s = fmaf(s, t, 0.0954376161f);
  s = fmaf(s, t, 0.101512372f);
  s = fmaf(s, t, 0.111481868f);
  s = fmaf(s, t, 0.111427054f);
  return PhiTail{t * e * s, e};
}

__device__ __forceinline__ float norm_cdf_bf16(float h, float x) { return x >= 0.f ? 1.0f - h : h; }

__device__ __forceinline__ float gelu_bf16(float x) { return x * norm_cdf_bf16(phi_tail_bf16(x).h, x); }

__device__ __forceinline__ float gelu_prime_bf16(float x) {
  const PhiTail q = phi_tail_bf16(x);
  return fmaf(x * 0.39894228040143268f, q.e, norm_cdf_bf16(q.h, x));
}

// 1 / (1 + e^-x) with the hardware reciprocal (1 ulp); saturates to 0 and 1.
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace tpk
