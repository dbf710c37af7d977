// fp32 GEMM for the all-fp32 path (small shards, where launch latency and
// not the matrix cores bound the time): 64 x 64 output tile, 16 x 16 threads
// with 4 x 4 outputs each, k staged through LDS in slices of 32.  Same
// operand layouts, K segments, dual-B products and epilogues as the bf16
// MFMA kernel, so both paths compute the same quantities.
//
// At these sizes a k-slice's global loads are a round trip of one to two
// microseconds, against a fraction of that for its arithmetic.  So each
// thread loads 16-byte vectors along the operand's contiguous dimension into
// a register ring of DEPTH slices, issued DEPTH slices ahead of their
// products: a K of up to DEPTH x 32 (the fp32 shards' 32 to 128) costs one
// round trip, and longer ones overlap each trip with DEPTH slices of work.
// (Wider slices were slower: a short K then pads them with zeros.)  The
// barriers order the LDS only, so the ring's loads stay in flight across them.
//
// Batched launches (grid z = batch x column tiles) run one product per shard:
// operand pointers advance by a_zs / b_zs elements per batch and the epilogue
// sees output row m + batch * z_rows, so row-stacked outputs need no copies.
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
  int tiles_n;        // column tiles per batch (grid z = nbatch * tiles_n)
  int64_t a_zs, b_zs; // per-batch operand offsets, elements
  int z_rows;         // per-batch output row offset
  int vec;            // every operand 16-byte aligned with a leading dimension divisible by 4
};

namespace f32g {

constexpr int BT = 64, BK = 32, PAD = 4, DEPTH = 4;
constexpr int NV = BT * BK / 4 / 256;   // 16-byte vectors per thread per operand slice
constexpr int KV = BK / 4;              // vectors along k in a k-major row

// One operand's share of a 64 x BK slice: NV 16-byte vectors per thread.
// A k-major operand (element (r, k) at base[r * ld + k]) is read as 64 rows
// of KV vectors along k; an m/n-major one (element (r, k) at base[k * ld + r])
// as BK rows of 16 vectors along r.  Out-of-range elements read as 0.
template <bool KM>
__device__ __forceinline__ void load_slice(const float* __restrict__ base, int64_t ld, int64_t ext, int64_t K,
                                           int64_t r0, int64_t k0, int tid, bool vec, f32x4 (&v)[NV]) {
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int idx = tid + e * 256;
    const int64_t r = KM ? r0 + idx / KV : r0 + (idx % 16) * 4;
    const int64_t k = KM ? k0 + (idx % KV) * 4 : k0 + idx / 16;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (KM) {
      if (r < ext) {
        const float* p = base + r * ld + k;
        if (vec && k + 3 < K) {
          x = *reinterpret_cast<const f32x4*>(p);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (k + j < K) x[j] = p[j];
        }
      }
    } else {
      if (k < K) {
        const float* p = base + k * ld + r;
        if (vec && r + 3 < ext) {
          x = *reinterpret_cast<const f32x4*>(p);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (r + j < ext) x[j] = p[j];
        }
      }
    }
    v[e] = x;
  }
}

// The slice into LDS as [k][r].
template <bool KM>
__device__ __forceinline__ void store_slice(float (*S)[BT + PAD], int tid, const f32x4 (&v)[NV]) {
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int idx = tid + e * 256;
    if (KM) {
      const int r = idx / KV, kk = (idx % KV) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) S[kk + j][r] = v[e][j];
    } else {
      const int r = (idx % 16) * 4, kk = idx / 16;
      *reinterpret_cast<f32x4*>(&S[kk][r]) = v[e];
    }
  }
}

// Workgroup barrier that orders only the LDS: __syncthreads() would also wait
// for every global load in flight, which drains the register ring at each
// slice.  The ring's registers get their own waits where they are used.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace f32g

template <bool A_KM, bool B_KM, bool DUAL, class Epi>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const GemmParamsF32 p, const Epi epi) {
  using namespace f32g;
  __shared__ __attribute__((aligned(16))) float As[BK][BT + PAD];
  __shared__ __attribute__((aligned(16))) float Bs[BK][BT + PAD];
  __shared__ __attribute__((aligned(16))) float B2s[DUAL ? BK : 1][BT + PAD];

  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int zb = (int)blockIdx.z / p.tiles_n;
  const int64_t m0 = (int64_t)blockIdx.x * BT, n0 = (int64_t)(blockIdx.z % p.tiles_n) * BT;
  const bool vec = p.vec != 0;
  float acc[4][4] = {}, acc2[4][4] = {};

  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegF32& g = p.seg[s];
    const float* A = g.A + zb * p.a_zs;
    const float* B = g.B + zb * p.b_zs;
    const float* B2 = DUAL ? g.B2 + zb * p.b_zs : nullptr;
    const int64_t kt_n = (g.K + BK - 1) / BK;
    const int64_t kb = kt_n * blockIdx.y / p.split_k, ke = kt_n * (blockIdx.y + 1) / p.split_k;
    if (kb >= ke) continue;
    f32x4 ra[DEPTH][NV], rb[DEPTH][NV], rb2[DUAL ? DEPTH : 1][NV];
    auto fetch = [&](int slot, int64_t kt) {
      load_slice<A_KM>(A, g.lda, g.a_rows, g.K, m0, kt * BK, tid, vec, ra[slot]);
      load_slice<B_KM>(B, g.ldb, g.b_cols, g.K, n0, kt * BK, tid, vec, rb[slot]);
      if constexpr (DUAL) load_slice<B_KM>(B2, g.ldb, g.b_cols, g.K, n0, kt * BK, tid, vec, rb2[slot]);
    };
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
      if (kb + i < ke) fetch(i, kb + i);
    for (int64_t kt0 = kb; kt0 < ke; kt0 += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {   // slot i holds slice kt0 + i
        const int64_t kt = kt0 + i;
        if (kt >= ke) break;
        store_slice<A_KM>(As, tid, ra[i]);
        store_slice<B_KM>(Bs, tid, rb[i]);
        if constexpr (DUAL) store_slice<B_KM>(B2s, tid, rb2[i]);
        lds_barrier();
        if (kt + DEPTH < ke) fetch(i, kt + DEPTH);   // in flight during the next DEPTH slices' products
        // KG k-rows of fragments read together, then their products: one LDS
        // round trip per group rather than per k
        constexpr int KG = DUAL ? 4 : 6;
#pragma unroll
        for (int kk0 = 0; kk0 < BK; kk0 += KG) {
          f32x4 a[KG], b[KG], b2[KG];
#pragma unroll
          for (int q = 0; q < KG; ++q) {
            if (kk0 + q >= BK) break;
            a[q] = *reinterpret_cast<const f32x4*>(&As[kk0 + q][ty * 4]);
            b[q] = *reinterpret_cast<const f32x4*>(&Bs[kk0 + q][tx * 4]);
            if constexpr (DUAL) b2[q] = *reinterpret_cast<const f32x4*>(&B2s[kk0 + q][tx * 4]);
          }
#pragma unroll
          for (int q = 0; q < KG; ++q) {
            if (kk0 + q >= BK) break;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                acc[r][c] = fmaf(a[q][r], b[q][c], acc[r][c]);
                if constexpr (DUAL) acc2[r][c] = fmaf(a[q][r], b2[q][c], acc2[r][c]);
              }
          }
        }
        lds_barrier();
      }
    }
  }

  const int64_t n = n0 + tx * 4;
  const int64_t zrow = (int64_t)zb * p.z_rows;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m < p.M && n < p.N) {
      const f32x4 v = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      if constexpr (DUAL) {
        const f32x4 v2 = {acc2[i][0], acc2[i][1], acc2[i][2], acc2[i][3]};
        epi_store_direct2(epi, m + zrow, n, v, v2);
      } else {
        epi_store_direct(epi, m + zrow, n, v, (int)blockIdx.y, zb);
      }
    }
  }
}

}  // namespace tpk
