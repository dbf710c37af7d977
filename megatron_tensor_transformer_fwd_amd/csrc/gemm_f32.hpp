// fp32 GEMM for the all-fp32 path (small shards, where launch latency and
// not the matrix cores bound the time): 64 x 64 output tile, 16 x 16 threads
// with 4 x 4 outputs each, k staged through LDS in slices of 16.  Same
// operand layouts, K segments, dual-B products and epilogues as the bf16
// MFMA kernel, so both paths compute the same quantities.
#pragma once
#include "common.hpp"
#include "epilogues.hpp"

namespace tpk {

struct GemmSegF32 {
  const float* A;
  const float* B;
  const float* B2;
  int64_t lda, ldb;
  int64_t K;
  int64_t a_rows;   // extent of A in its m/n dimension (= M for the A operand)
  int64_t b_cols;   // extent of B in its n dimension (= N)
};

struct GemmParamsF32 {
  int M, N, nseg;
  GemmSegF32 seg[2];
  int split_k;
};

template <bool A_KM, bool B_KM, bool DUAL, class Epi>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const GemmParamsF32 p, const Epi epi) {
  constexpr int BT = 64, BK = 16, PAD = 4;
  __shared__ float As[BK][BT + PAD];
  __shared__ float Bs[BK][BT + PAD];
  __shared__ float B2s[DUAL ? BK : 1][BT + PAD];

  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.x * BT, n0 = (int64_t)blockIdx.z * BT;
  float acc[4][4] = {}, acc2[4][4] = {};

  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegF32& g = p.seg[s];
    const int64_t kt_n = (g.K + BK - 1) / BK;
    const int64_t kb = kt_n * blockIdx.y / p.split_k, ke = kt_n * (blockIdx.y + 1) / p.split_k;
    for (int64_t kt = kb; kt < ke; ++kt) {
      const int64_t k0 = kt * BK;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = tid + e * 256;           // 1024 elements per 64 x 16 tile
        const int r = idx % BT, kk = idx / BT;   // r along m/n, kk along k
        const int64_t m = m0 + r, n = n0 + r, k = k0 + kk;
        float a = 0.f, b = 0.f, b2 = 0.f;
        if (m < g.a_rows && k < g.K) a = A_KM ? g.A[m * g.lda + k] : g.A[k * g.lda + m];
        if (n < g.b_cols && k < g.K) {
          b = B_KM ? g.B[n * g.ldb + k] : g.B[k * g.ldb + n];
          if constexpr (DUAL) b2 = B_KM ? g.B2[n * g.ldb + k] : g.B2[k * g.ldb + n];
        }
        As[kk][r] = a;
        Bs[kk][r] = b;
        if constexpr (DUAL) B2s[kk][r] = b2;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4], b2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b[j] = Bs[kk][tx * 4 + j];
          if constexpr (DUAL) b2[j] = B2s[kk][tx * 4 + j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            if constexpr (DUAL) acc2[i][j] = fmaf(a[i], b2[j], acc2[i][j]);
          }
      }
      __syncthreads();
    }
  }

  const int64_t n = n0 + tx * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m < p.M && n < p.N) {
      const f32x4 v = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      if constexpr (DUAL) {
        const f32x4 v2 = {acc2[i][0], acc2[i][1], acc2[i][2], acc2[i][3]};
        epi_store_direct2(epi, m, n, v, v2);
      } else {
        epi_store_direct(epi, m, n, v, (int)blockIdx.y, 0);
      }
    }
  }
}

}  // namespace tpk
