// GEMM epilogues.  Each receives the fp32 results of one output quad
// (m, n..n+3) (n is a multiple of 4 and every output width is a multiple of
// 8, so a quad never straddles a row) and performs the fused elementwise
// step of the TP shard before a single store.  T is the storage type of the
// activations (bf16 or float).
#pragma once
#include "common.hpp"

namespace tpk {

template <class T> struct Quad;
template <> struct Quad<bf16> {
  static __device__ __forceinline__ void store(bf16* p, f32x4 v) {
    u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(p) = w;
  }
  static __device__ __forceinline__ f32x4 load(const bf16* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  }
};
template <> struct Quad<float> {
  static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
  static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
};

// C = AB, stored in T.  With split-K, split s writes its partial sum to
// C + s * split_stride (fp32 workspace), summed afterwards in split order.
template <class T>
struct EpiStore {
  T* C;
  int64_t ldc;
  int64_t split_stride;
  __device__ __forceinline__ void apply(int64_t m, int64_t n, f32x4 v, int split, int) const {
    Quad<T>::store(C + split * split_stride + m * ldc + n, v);
  }
};

// Column-parallel product with GeLU ([JY] FFN, [HC] Figure 3.4): keeps the
// pre-activation A (optional) and writes H = GeLU(A) from the fp32 sum.
template <class T>
struct EpiGelu {
  T* A;   // may be null
  T* H;
  int64_t ld;
  __device__ __forceinline__ void apply(int64_t m, int64_t n, f32x4 v, int, int) const {
    if (A) Quad<T>::store(A + m * ld + n, v);
    f32x4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = gelu_f(v[q]);
    Quad<T>::store(H + m * ld + n, h);
  }
};

// Backward dgrad of the row-parallel product with GeLU' fused:
// dA = (dY W2^T) * GeLU'(A), A read back from the forward's saved copy.
template <class T>
struct EpiDGelu {
  const T* A;
  T* dA;
  int64_t ld;
  __device__ __forceinline__ void apply(int64_t m, int64_t n, f32x4 v, int, int) const {
    const f32x4 a = Quad<T>::load(A + m * ld + n);
    f32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = v[q] * gelu_prime_f(a[q]);
    Quad<T>::store(dA + m * ld + n, r);
  }
};

// Dual product X [W1 | W3] with SwiGLU: G = X W1, U = X W3, H = Swish(G) * U.
template <class T>
struct EpiSwiGLU {
  T* G;   // may be null
  T* U;   // may be null
  T* H;
  int64_t ld;
  __device__ __forceinline__ void apply2(int64_t m, int64_t n, f32x4 g, f32x4 u) const {
    if (G) Quad<T>::store(G + m * ld + n, g);
    if (U) Quad<T>::store(U + m * ld + n, u);
    f32x4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = g[q] * sigmoid_f(g[q]) * u[q];
    Quad<T>::store(H + m * ld + n, h);
  }
};

// SwiGLU backward dgrad: given dH = dY W2^T, writes
// dG = dH * U * Swish'(G) and dU = dH * Swish(G) into the two halves of one
// [M x 2f] buffer (dG in columns [0, f), dU in [f, 2f)).
template <class T>
struct EpiDSwiGLU {
  const T* G;
  const T* U;
  T* dGU;
  int64_t ld;    // f
  __device__ __forceinline__ void apply(int64_t m, int64_t n, f32x4 v, int, int) const {
    const f32x4 g = Quad<T>::load(G + m * ld + n);
    const f32x4 u = Quad<T>::load(U + m * ld + n);
    f32x4 dg, du;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float s = sigmoid_f(g[q]);
      du[q] = v[q] * g[q] * s;
      dg[q] = v[q] * u[q] * s * (1.0f + g[q] * (1.0f - s));
    }
    T* row = dGU + m * (2 * ld);
    Quad<T>::store(row + n, dg);
    Quad<T>::store(row + ld + n, du);
  }
};

// fp32 output whose columns [0, split_col) go to C1 and the rest to C2 (each
// with row pitch split_col), e.g. X^T [dG | dU] -> dW1 and dW3.  Split-K
// partials go to the workspace as one [M x N] matrix per split.
struct EpiF32Halves {
  float* C1;
  float* C2;
  int64_t split_col;
  float* ws;              // non-null: split-K partials [split][M][N]
  int64_t N;
  int64_t split_stride;
  __device__ __forceinline__ void apply(int64_t m, int64_t n, f32x4 v, int split, int) const {
    if (ws) {
      Quad<float>::store(ws + split * split_stride + m * N + n, v);
    } else if (n < split_col) {
      Quad<float>::store(C1 + m * split_col + n, v);
    } else {
      Quad<float>::store(C2 + m * split_col + (n - split_col), v);
    }
  }
};

// Column-parallel Q/K/V projection ([BM] Megatron_MHA; [JY] Attention): batch
// z of the launch is Q (0), K (1) or V (2); output (m, n) with m = bi*s + t
// and n = j*d_head + c goes to the head-major [b, h_local, s, d_head] tensor.
template <class T>
struct EpiHeadScatter {
  T* out[3];
  int s, h_local, d_head;
  __device__ __forceinline__ void apply(int64_t m, int64_t n, f32x4 v, int, int z) const {
    const int64_t bi = m / s, t = m % s;
    const int64_t j = n / d_head, c = n % d_head;
    Quad<T>::store(out[z] + ((bi * h_local + j) * s + t) * d_head + c, v);
  }
};

}  // namespace tpk
