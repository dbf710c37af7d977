// GEMM epilogues.  An epilogue describes the fused elementwise step of the
// TP shard that follows a product and where its outputs go:
//   NOUT                       number of output tensors
//   OutT<O>                    storage type of output O (bf16 or float)
//   has_out<O>()               whether output O is wanted (runtime, uniform)
//   out_ptr<O>(m, n, split, z) address of element (m, n) of output O; eight
//                              consecutive n starting at a multiple of 8 are
//                              contiguous
//   value<O>(m, n, v)          output O's values for the fp32 product quad v
//                              at (m, n..n+3) (value2<O>(m, n, g, u) for
//                              dual-B products)
// Quads never straddle a row (n is a multiple of 4, widths multiples of 8).
// The GEMM kernels stage each output through LDS and write whole rows with
// 16-byte stores; the fp32 SIMT kernel stores quads directly.
#pragma once
#include "common.hpp"

namespace tpk {

template <class T> struct Quad;
template <> struct Quad<bf16> {
  using Raw = u32x2;
  static __device__ __forceinline__ void store(bf16* p, f32x4 v) {
    u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(p) = w;
  }
  static __device__ __forceinline__ Raw load_raw(const bf16* p) { return *reinterpret_cast<const u32x2*>(p); }
  static __device__ __forceinline__ f32x4 unpack(Raw w) {
    return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  }
  static __device__ __forceinline__ f32x4 load(const bf16* p) { return unpack(load_raw(p)); }
};
template <> struct Quad<float> {
  using Raw = f32x4;
  static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ f32x4 unpack(Raw w) { return w; }
  static __device__ __forceinline__ f32x4 load(const float* p) { return load_raw(p); }
};

// C = AB stored in T.  With split-K, split s writes its partial sum to
// C + s * split_stride (fp32 workspace), summed afterwards in split order.
template <class T>
struct EpiStore {
  static constexpr int NOUT = 1;
  template <int O> using OutT = T;
  T* C;
  int64_t ldc;
  int64_t split_stride;
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ T* out_ptr(int64_t m, int64_t n, int split, int) const {
    return C + split * split_stride + m * ldc + n;
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const { return v; }
};

// Column-parallel product with GeLU ([JY] FFN, [HC] Figure 3.4): output 0 is
// the pre-activation A (optional), output 1 is H = GeLU(A) from the fp32 sum.
// KEEP: A and H are stored without the streaming hint (keep<O>()), for the
// products that read them next (H at once, A in the backward's GeLU' dgrad).
template <class T, bool KEEP = false>
struct EpiGelu {
  static constexpr int NOUT = 2;
  template <int O> using OutT = T;
  T* A;   // may be null
  T* H;
  int64_t ld;
  template <int O> static constexpr bool keep() { return KEEP; }
  template <int O> __device__ __forceinline__ bool has_out() const { return O == 1 || A != nullptr; }
  template <int O> __device__ __forceinline__ T* out_ptr(int64_t m, int64_t n, int, int) const {
    return (O == 0 ? A : H) + m * ld + n;
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const {
    if constexpr (O == 0) return v;
    f32x4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = std::is_same_v<T, bf16> ? gelu_bf16(v[q]) : gelu_f(v[q]);
    return h;
  }
};

// Backward dgrad of the row-parallel product with GeLU' fused:
// dA = (dY W2^T) * GeLU'(A), A read back from the forward's saved copy.
// KEEP: dA is stored without the streaming hint, as A and H above.
template <class T, bool KEEP = false>
struct EpiDGelu {
  static constexpr int NOUT = 1;
  template <int O> using OutT = T;
  const T* A;
  T* dA;
  int64_t ld;
  template <int O> static constexpr bool keep() { return KEEP; }
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ T* out_ptr(int64_t m, int64_t n, int, int) const {
    return dA + m * ld + n;
  }
  struct Aux { typename Quad<T>::Raw a; };
  template <int O> __device__ __forceinline__ Aux aux_load(int64_t m, int64_t n) const {
    return Aux{Quad<T>::load_raw(A + m * ld + n)};
  }
  template <int O> __device__ __forceinline__ f32x4 value_aux(int64_t, int64_t, f32x4 v, const Aux& x) const {
    const f32x4 a = Quad<T>::unpack(x.a);
    f32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = v[q] * (std::is_same_v<T, bf16> ? gelu_prime_bf16(a[q]) : gelu_prime_f(a[q]));
    return r;
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t m, int64_t n, f32x4 v) const {
    return value_aux<O>(m, n, v, aux_load<O>(m, n));
  }
};

// Dual product X [W1 | W3] with SwiGLU: outputs G = X W1 (optional),
// U = X W3 (optional) and H = Swish(G) * U.
template <class T>
struct EpiSwiGLU {
  static constexpr int NOUT = 3;
  template <int O> using OutT = T;
  T* G;   // may be null
  T* U;   // may be null
  T* H;
  int64_t ld;
  template <int O> __device__ __forceinline__ bool has_out() const {
    return O == 2 || (O == 0 ? G != nullptr : U != nullptr);
  }
  template <int O> __device__ __forceinline__ T* out_ptr(int64_t m, int64_t n, int, int) const {
    return (O == 0 ? G : O == 1 ? U : H) + m * ld + n;
  }
  template <int O> __device__ __forceinline__ f32x4 value2(int64_t, int64_t, f32x4 g, f32x4 u) const {
    if constexpr (O == 0) return g;
    if constexpr (O == 1) return u;
    f32x4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = g[q] * sigmoid_f(g[q]) * u[q];
    return h;
  }
};

// SwiGLU backward dgrad: given dH = dY W2^T, outputs dG = dH * U * Swish'(G)
// (output 0) and dU = dH * Swish(G) (output 1) into the two halves of one
// [M x 2f] buffer (dG in columns [0, f), dU in [f, 2f)).  Stored without the
// streaming hint (bf16): the dX product reads them at once, and at C3 it took
// 301-302 instead of 313-315 us with them still in the caches.
template <class T>
struct EpiDSwiGLU {
  static constexpr int NOUT = 2;
  template <int O> using OutT = T;
  const T* G;
  const T* U;
  T* dGU;
  int64_t ld;    // f
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ T* out_ptr(int64_t m, int64_t n, int, int) const {
    return dGU + m * (2 * ld) + (O == 0 ? 0 : ld) + n;
  }
  template <int O> static constexpr bool keep() { return std::is_same_v<T, bf16>; }
  // output 0 reads G and U, output 1 only G
  struct Aux { typename Quad<T>::Raw g, u; };
  template <int O> __device__ __forceinline__ Aux aux_load(int64_t m, int64_t n) const {
    Aux x;
    x.g = Quad<T>::load_raw(G + m * ld + n);
    if constexpr (O == 0) x.u = Quad<T>::load_raw(U + m * ld + n);
    return x;
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t m, int64_t n, f32x4 v) const {
    return value_aux<O>(m, n, v, aux_load<O>(m, n));
  }
  template <int O> __device__ __forceinline__ f32x4 value_aux(int64_t, int64_t, f32x4 v, const Aux& x) const {
    const f32x4 g = Quad<T>::unpack(x.g);
    f32x4 r;
    if constexpr (O == 0) {
      const f32x4 u = Quad<T>::unpack(x.u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s = sigmoid_f(g[q]);
        r[q] = v[q] * u[q] * s * (1.0f + g[q] * (1.0f - s));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = v[q] * g[q] * sigmoid_f(g[q]);
    }
    return r;
  }
};

// fp32 output whose columns [0, split_col) go to C1 and the rest to C2 (each
// with row pitch split_col), e.g. X^T [dG | dU] -> dW1 and dW3.
struct EpiF32Halves {
  static constexpr int NOUT = 1;
  template <int O> using OutT = float;
  float* C1;
  float* C2;
  int64_t split_col;
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ float* out_ptr(int64_t m, int64_t n, int, int) const {
    return n < split_col ? C1 + m * split_col + n : C2 + m * split_col + (n - split_col);
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const { return v; }
};

// Column-parallel Q/K/V projection ([BM] Megatron_MHA; [JY] Attention): batch
// z of the launch is Q (0), K (1) or V (2); output (m, n) with m = bi*s + t
// and n = j*d_head + c goes to the head-major [b, h_local, s, d_head] tensor.
template <class T>
struct EpiHeadScatter {
  static constexpr int NOUT = 1;
  template <int O> using OutT = T;
  T* out[3];
  int s, h_local, d_head;
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ T* out_ptr(int64_t m, int64_t n, int, int z) const {
    const int64_t bi = m / s, t = m % s;
    const int64_t j = n / d_head, c = n % d_head;
    return out[z] + ((bi * h_local + j) * s + t) * d_head + c;
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const { return v; }
};

// Direct quad stores of every output (the fp32 SIMT kernel's epilogue).
template <class Epi>
__device__ __forceinline__ void epi_store_direct(const Epi& e, int64_t m, int64_t n, f32x4 v, int split,
                                                 int z) {
  [&]<int... O>(std::integer_sequence<int, O...>) {
    ((e.template has_out<O>() ? Quad<typename Epi::template OutT<O>>::store(
                                    e.template out_ptr<O>(m, n, split, z), e.template value<O>(m, n, v))
                              : void()),
     ...);
  }(std::make_integer_sequence<int, Epi::NOUT>{});
}

template <class Epi>
__device__ __forceinline__ void epi_store_direct2(const Epi& e, int64_t m, int64_t n, f32x4 g, f32x4 u) {
  [&]<int... O>(std::integer_sequence<int, O...>) {
    ((e.template has_out<O>() ? Quad<typename Epi::template OutT<O>>::store(
                                    e.template out_ptr<O>(m, n, 0, 0), e.template value2<O>(m, n, g, u))
                              : void()),
     ...);
  }(std::make_integer_sequence<int, Epi::NOUT>{});
}

}  // namespace tpk
