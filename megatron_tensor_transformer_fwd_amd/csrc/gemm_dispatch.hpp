// Host-side tile-shape choice and launch of the GEMM kernels.
#pragma once
#include <algorithm>
#include <cmath>
#include "gemm.hpp"
#include "gemm_f32.hpp"
#include "launch.hpp"
#include "profile.hpp"

#define TPK_TRY(expr)                         \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return e_;          \
  } while (0)

namespace tpk {

// Tile shapes.  L: 256x256, 8 waves of 128x64 (two per SIMD), the shape for
// large shards; M: 256x128, 4 waves of 128x64; S: 128x128, 4 waves of 64x64
// for narrow outputs such as a TP-8 slice of a 4096-wide feed-forward layer.
// Wave layout, k-tile depth, A/B ring slots, per-ring DMA spread (k-steps)
// and k-order rotation of each shape are compile-time tuning knobs.
#ifndef TPK_L_CFG
#define TPK_L_CFG 256, 256, 2, 4, 64, 2, 2, 1, 1, 1
#endif
#ifndef TPK_M_CFG
#define TPK_M_CFG 256, 128, 2, 2, 64, 2, 2, 1, 1, 0
#endif
#ifndef TPK_S_CFG
#define TPK_S_CFG 128, 128, 2, 2, 64, 2, 2, 1, 1, 0
#endif
using CfgL = TileCfg<TPK_L_CFG>;
using CfgM = TileCfg<TPK_M_CFG>;
using CfgS = TileCfg<TPK_S_CFG>;

enum { CFG_L = 0, CFG_M = 1, CFG_S = 2 };

struct GemmPlan {
  int cfg;
  int split;
  int tail = 0;      // > 1: the last partial round of 256x256 tiles is split along K this many ways
  double est = 0.0;  // the planner's estimated duration in seconds
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t tiles_for(int cfg, int64_t M, int64_t N, bool dual) {
  const int bm = cfg == CFG_S ? 128 : 256;
  int bn = cfg == CFG_L ? 256 : 128;
  if (dual) bn /= 2;
  return cdiv(M, bm) * cdiv(N, bn);
}

// Relative MFMA rate of a CU running the M and S shapes, against the L shape
// (tuning constants, measured on the workloads' products).
#ifndef TPK_RATE_M
#define TPK_RATE_M 0.75
#endif
#ifndef TPK_RATE_S
#define TPK_RATE_S 0.60
#endif
// Batched split-K weight gradients (all shards of a layer in one launch):
// the S shape's 64 KiB of LDS lets two of its workgroups share a CU, and on
// eight 512 x 1024 shard gradients over 8192 tokens two 128 x 128 tiles per
// CU over K 4096 take as long as one 256 x 256 tile over K 2048, with half
// the fp32 partials to reduce.  On unbatched products the pairing did not
// hold (forward products, dgrads and the other workloads' gradients were
// 3-6% slower), so the paired rate is used for this case only.
#ifndef TPK_RATE_S2
#define TPK_RATE_S2 0.95
#endif

// Tile shape and K split of a product: the choice with the smallest
// estimated duration, where a launch takes ceil(tiles / 256) rounds of tiles
// (one per CU at a time; a partly filled last round costs a whole one) times
// a tile's work over its shape's rate, and a K split adds the deterministic
// fp32 reduce of its partials (split + 1 passes over the output at about
// 4 TB/s).  Splitting is allowed only where the caller has an fp32 workspace
// (weight gradients).  Near-ties go to the larger tile and the smaller split.
// Dual-B products always take the L shape (two 128-column sub-tiles).
//
// With allow_tail (the caller has a workspace for it), the 256x256 shape may
// also run its whole rounds as usual and split the tiles of a last round
// that fills at most half the CUs along K (tail = 2..8 ways, at least 8
// k-tiles each): the round then costs a tile's work / tail, plus a pass that
// writes and reads the fp32 partial tiles and applies the epilogue.
constexpr int kTailMaxSplit = 8;
constexpr double kGemmLaunchS = 4e-6;   // per extra launch

// nbatch: the launch runs that many products of this shape side by side
// (grid z), so their tiles share the rounds.
inline GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool dual, bool allow_split, bool allow_tail = false,
                          int64_t nbatch = 1) {
  constexpr double CUS = 256.0, CU_FLOPS = 4.4e12, REDUCE_BPS = 4.0e12, LAUNCH_S = kGemmLaunchS;
  const double rate[3] = {1.0, TPK_RATE_M, TPK_RATE_S};
  GemmPlan best{CFG_L, 1};
  double best_t = 1e30;
  for (int cfg = CFG_L; cfg <= CFG_S; ++cfg) {
    if (dual && cfg != CFG_L) break;
    const int64_t bm = cfg == CFG_S ? 128 : 256;
    const int64_t bn = cfg == CFG_L ? 256 : 128;   // output columns per tile (dual: two halves)
    const int64_t tiles = cdiv(M, bm) * cdiv(N, dual ? bn / 2 : bn) * nbatch;
    for (int s = 1; s <= (allow_split ? 16 : 1); s *= 2) {
      const int64_t kc = cdiv(K, s);
      if (s > 1 && kc < 512) break;
      const double tile_flop = 2.0 * (double)(bm * bn * kc);
      double t = std::ceil((double)(tiles * s) / CUS) * tile_flop / (rate[cfg] * CU_FLOPS);
      if (cfg == CFG_S && allow_split && nbatch > 1 && tiles * s > 256)   // two S tiles per CU
        t = std::ceil((double)(tiles * s) / (2.0 * CUS)) * 2.0 * tile_flop / (TPK_RATE_S2 * CU_FLOPS);
      // An unbatched product without a K split whose 256x256 tiles would leave
      // one partly filled round (a narrow output: C4's V projection and dO,
      // E1's dZ E) fills all of it with 128x128 tiles, two per CU, at the
      // paired rate: 78.8 -> 70.1 and 94.8 -> 77.2 us at C4 against 256x128
      // tiles one per CU.
      if (cfg == CFG_S && !allow_split && nbatch == 1 && s == 1 && tiles > 256 && tiles <= 512 &&
          cdiv(M, 256) * cdiv(N, 256) < 256)
        t = 2.0 * tile_flop / (TPK_RATE_S2 * CU_FLOPS);
      if (s > 1) t += (double)(s + 1) * (double)M * (double)N * (double)nbatch * 4.0 / REDUCE_BPS + LAUNCH_S;
      if (t < best_t * 0.97) {
        best_t = t;
        best = GemmPlan{cfg, s};
      }
    }
    if (cfg == CFG_L && allow_tail && !dual && nbatch == 1) {
      const int64_t full = tiles / 256 * 256, rem = tiles - full;
      const int64_t kt = cdiv(K, 64);
      int ways = rem > 0 ? (int)std::min<int64_t>(kTailMaxSplit, 256 / rem) : 0;
      while (ways > 1 && kt / ways < 8) --ways;
      if (ways > 1) {
        const double tile_t = 2.0 * (double)(bm * bn * K) / CU_FLOPS;
        const double fix_bytes = (double)rem * ways * bm * bn * 4.0 * 2.0 + (double)rem * bm * bn * 4.0;
        const double t = (double)(full / 256) * tile_t + tile_t / ways + fix_bytes / REDUCE_BPS + 2 * LAUNCH_S;
        if (t < best_t * 0.97) {
          best_t = t;
          best = GemmPlan{CFG_L, 1, ways};
        }
      }
    }
  }
  best.est = best_t;
  return best;
}

// fp32 workspace the tail split of `plan` needs (0 without one).
inline size_t gemm_tail_ws_bytes(const GemmPlan& plan, int64_t M, int64_t N) {
  if (plan.tail <= 1) return 0;
  const int64_t tiles = cdiv(M, 256) * cdiv(N, 256);
  return (size_t)(tiles % 256) * plan.tail * 256 * 256 * 4;
}

// Partial sums of the split tail tiles: the tile at grouped position base + j,
// split s, is stored densely (BM x BN floats, row-major) at ws + (s * count + j) * BM * BN.
template <int BM, int BN>
struct EpiTilePartial {
  static constexpr int NOUT = 1;
  template <int O> using OutT = float;
  float* ws;
  int count, base, tiles_m, tiles_n;
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ float* out_ptr(int64_t m, int64_t n, int split, int) const {
    const int j = position_of((int)(m / BM), (int)(n / BN), tiles_m, tiles_n) - base;
    return ws + ((int64_t)split * count + j) * (BM * BN) + (m % BM) * BN + (n % BN);
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const { return v; }
};

// Sum of the tail tiles' partials in split order, then the product's own
// epilogue; one thread per four consecutive outputs.
template <int BM, int BN, class Epi>
__global__ void __launch_bounds__(256)
gemm_tail_fixup_kernel(const float* __restrict__ ws, int splits, int count, int base, int tiles_m, int tiles_n,
                       int M, int N, Epi epi) {
  constexpr int QPT = BM * BN / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)count * QPT) return;
  const int j = (int)(i / QPT), q = (int)(i % QPT);
  int tm, tn;
  tile_of(base + j, tiles_m, tiles_n, tm, tn);
  const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
  const int64_t m = (int64_t)tm * BM + r, n = (int64_t)tn * BN + c;
  if (m >= M || n >= N) return;
  const float* p = ws + (int64_t)j * (BM * BN) + r * BN + c;
  f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  for (int s = 1; s < splits; ++s)
    v += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + (int64_t)s * count * (BM * BN)));
  epi_store_direct(epi, m, n, v, 0, 0);
}

template <class Cfg, bool A_KM, bool B_KM, bool DUAL, class Epi>
hipError_t launch_gemm_cfg(hipStream_t st, const char* label, GemmParams p, const Epi& epi, int nz) {
  constexpr int BNL = DUAL ? Cfg::BN / 2 : Cfg::BN;
  p.tiles_m = (int)cdiv(p.M, Cfg::BM);
  p.tiles_n = (int)cdiv(p.N, BNL);
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n), (unsigned)p.split_k, (unsigned)nz);
  return launch(label, gemm_bf16_kernel<Cfg, A_KM, B_KM, DUAL, Epi>, grid, dim3(Cfg::NT), st, p, epi);
}

// The whole rounds of 256x256 tiles as usual, then the remaining tiles split
// `plan.tail` ways along K into the fp32 workspace, then the fixup pass.
template <bool A_KM, bool B_KM, class Epi>
hipError_t launch_gemm_tail(hipStream_t st, const char* label, GemmParams p, const Epi& epi, GemmPlan plan,
                            float* tail_ws) {
  p.tiles_m = (int)cdiv(p.M, CfgL::BM);
  p.tiles_n = (int)cdiv(p.N, CfgL::BN);
  const int tiles = p.tiles_m * p.tiles_n;
  const int full = tiles / 256 * 256, rem = tiles - full;
  if (full > 0) {
    GemmParams p1 = p;
    p1.split_k = 1;
    p1.tile_base = 0;
    TPK_TRY(launch(label, gemm_bf16_kernel<CfgL, A_KM, B_KM, false, Epi>, dim3((unsigned)full), dim3(CfgL::NT), st,
                   p1, epi));
  }
  GemmParams p2 = p;
  p2.split_k = plan.tail;
  p2.tile_base = full;
  EpiTilePartial<CfgL::BM, CfgL::BN> e2{tail_ws, rem, full, p.tiles_m, p.tiles_n};
  TPK_TRY(launch("gemm.tail_split", gemm_bf16_kernel<CfgL, A_KM, B_KM, false, EpiTilePartial<CfgL::BM, CfgL::BN>>,
                 dim3((unsigned)rem, (unsigned)plan.tail), dim3(CfgL::NT), st, p2, e2));
  const int64_t quads = (int64_t)rem * (CfgL::BM * CfgL::BN / 4);
  return launch("gemm.tail_fixup", gemm_tail_fixup_kernel<CfgL::BM, CfgL::BN, Epi>,
                dim3((unsigned)cdiv(quads, 256)), dim3(256), st, (const float*)tail_ws, plan.tail, rem, full,
                p.tiles_m, p.tiles_n, p.M, p.N, epi);
}

template <bool A_KM, bool B_KM, bool DUAL, class Epi>
hipError_t launch_gemm(hipStream_t st, const char* label, GemmParams p, const Epi& epi, GemmPlan plan,
                       int nz = 1, float* tail_ws = nullptr) {
  if constexpr (!DUAL && !epi_row_reduce<Epi>::value) {
    if (plan.tail > 1) {
      if (nz != 1 || plan.cfg != CFG_L || plan.split != 1 || !tail_ws) return hipErrorInvalidValue;
      return launch_gemm_tail<A_KM, B_KM>(st, label, p, epi, plan, tail_ws);
    }
  }
  if (plan.tail > 1) return hipErrorInvalidValue;
  p.split_k = plan.split;
  switch (plan.cfg) {
    case CFG_L: return launch_gemm_cfg<CfgL, A_KM, B_KM, DUAL, Epi>(st, label, p, epi, nz);
    case CFG_M:
      if constexpr (DUAL) return hipErrorInvalidValue;
      else return launch_gemm_cfg<CfgM, A_KM, B_KM, DUAL, Epi>(st, label, p, epi, nz);
    default:
      if constexpr (DUAL) return hipErrorInvalidValue;
      else return launch_gemm_cfg<CfgS, A_KM, B_KM, DUAL, Epi>(st, label, p, epi, nz);
  }
}

// Two independent products of the 256x256 shape without K splits in one
// launch (gemm_pair_kernel), the first product's tiles dispatched first.
// Estimated duration: with tile times t1, t2 (the plans' estimates over their
// rounds), about (n1 t1 + n2 t2) / 256 plus half the shorter tile for the
// uneven end, against ceil(n1 / 256) t1 + ceil(n2 / 256) t2 for two launches:
// it pays where one of them leaves a partial last round.  A huge value where
// the plans do not fit the pair kernel.
inline double gemm_pair_est(const GemmPlan& a, int64_t n1, const GemmPlan& b, int64_t n2) {
  if (a.cfg != CFG_L || b.cfg != CFG_L || a.split != 1 || b.split != 1 || a.tail > 1 || b.tail > 1 || n1 <= 0 ||
      n2 <= 0)
    return 1e30;
  const double t1 = a.est / std::ceil(n1 / 256.0), t2 = b.est / std::ceil(n2 / 256.0);
  return ((double)n1 * t1 + (double)n2 * t2) / 256.0 + 0.5 * std::min(t1, t2);
}

template <bool A1, bool B1, class E1, bool A2, bool B2, class E2>
hipError_t launch_gemm_pair(hipStream_t st, const char* label, GemmParams p1, const E1& e1, GemmParams p2,
                            const E2& e2) {
  for (GemmParams* p : {&p1, &p2}) {
    p->tiles_m = (int)cdiv(p->M, CfgL::BM);
    p->tiles_n = (int)cdiv(p->N, CfgL::BN);
    p->split_k = 1;
    p->tile_base = 0;
  }
  const int n1 = p1.tiles_m * p1.tiles_n, n2 = p2.tiles_m * p2.tiles_n;
  return launch(label, gemm_pair_kernel<CfgL, A1, B1, E1, A2, B2, E2>, dim3((unsigned)(n1 + n2)), dim3(CfgL::NT),
                st, p1, e1, p2, e2, n1);
}

// One K segment of a bf16 product.  a_rows_or_k / b: the extent of each
// operand's slow dimension, used for the readable range.
inline GemmSeg make_seg(const void* A, int64_t lda, int64_t a_elems,
                        const void* B, int64_t ldb, int64_t b_elems, int64_t K,
                        const void* B2 = nullptr) {
  GemmSeg s;
  s.A = static_cast<const bf16*>(A);
  s.B = static_cast<const bf16*>(B);
  s.B2 = static_cast<const bf16*>(B2);
  s.lda = lda;
  s.ldb = ldb;
  s.a_elems = a_elems;
  s.b_elems = b_elems;
  s.K = (int)K;
  return s;
}

inline GemmParams make_params(int64_t M, int64_t N, GemmSeg s0) {
  GemmParams p{};
  p.M = (int)M;
  p.N = (int)N;
  p.nseg = 1;
  p.seg[0] = s0;
  p.Bz[0] = p.Bz[1] = p.Bz[2] = nullptr;
  p.split_k = 1;
  return p;
}

// fp32 path
// nbatch > 1: one product per batch (grid z = batch x column tiles), operands
// advanced by p.a_zs / p.b_zs elements per batch, outputs row-stacked by p.z_rows.
template <bool A_KM, bool B_KM, bool DUAL, class Epi>
hipError_t launch_gemm_f32(hipStream_t st, const char* label, GemmParamsF32 p, const Epi& epi, int nbatch = 1) {
  p.tiles_n = (int)cdiv(p.N, 64);
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  bool vec = (p.a_zs % 4 == 0) && (p.b_zs % 4 == 0);
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegF32& g = p.seg[s];
    vec = vec && al16(g.A) && al16(g.B) && (!DUAL || al16(g.B2)) && g.lda % 4 == 0 && g.ldb % 4 == 0;
  }
  p.vec = vec ? 1 : 0;
  const dim3 grid((unsigned)cdiv(p.M, 64), (unsigned)p.split_k, (unsigned)(p.tiles_n * nbatch));
  return launch(label, gemm_f32_kernel<A_KM, B_KM, DUAL, Epi>, grid, dim3(256), st, p, epi);
}

inline GemmSegF32 make_seg_f32(const void* A, int64_t lda, int64_t a_rows,
                               const void* B, int64_t ldb, int64_t b_cols, int64_t K,
                               const void* B2 = nullptr) {
  GemmSegF32 s;
  s.A = static_cast<const float*>(A);
  s.B = static_cast<const float*>(B);
  s.B2 = static_cast<const float*>(B2);
  s.lda = lda;
  s.ldb = ldb;
  s.K = K;
  s.a_rows = a_rows;
  s.b_cols = b_cols;
  return s;
}

inline GemmParamsF32 make_params_f32(int64_t M, int64_t N, GemmSegF32 s0) {
  GemmParamsF32 p{};
  p.M = (int)M;
  p.N = (int)N;
  p.nseg = 1;
  p.seg[0] = s0;
  p.split_k = 1;
  return p;
}

// fp32 weight gradient C[Mo x No] = A^T B over K tokens, through the split-K
// workspace when the plan splits.  With nbatch > 1 the launch computes
// nbatch such products (grid z, outputs row-stacked: [nbatch x Mo x No]); the
// split partials are laid out [split][nbatch][Mo x No] and summed in split
// order by one reduce over all batches.
template <class Launch>
inline hipError_t wgrad_f32_out(hipStream_t st, GemmPlan plan, int64_t Mo, int64_t No,
                                float* out, float* split_ws, Launch&& run, int64_t nbatch = 1) {
  if (plan.split > 1) {
    EpiStore<float> e{split_ws, No, nbatch * Mo * No};
    TPK_TRY(run(e, plan));
    return launch_shard_reduce(st, DT_F32, DT_F32, plan.split, nbatch * Mo * No, split_ws, nbatch * Mo * No,
                               nullptr, 0, out);
  }
  EpiStore<float> e{out, No, 0};
  return run(e, plan);
}


}  // namespace tpk
