// SwiGLU MLP shard, forward and backward ([JY] FFN, SwiGLU part: W1 and W3
// split by columns, W2 by rows; W1 is the Swish'd gate; [HC] Figure 3.6).
//
// Forward:  one dual-B product reads each X tile once for both slices:
//           G = X W1, U = X W3, H = Swish(G) * U (epilogue); Z = H W2.
// Backward: dH = dY W2^T with the SwiGLU derivative fused:
//             dG = dH * U * Swish'(G), dU = dH * Swish(G), into [dG | dU];
//           dW2 = H^T dY;  dX = [dG | dU] [W1 | W3]^T (two K segments, one
//           accumulator);  [dW1 | dW3] = X^T [dG | dU] (one product, N = 2f).
#include "epilogues.hpp"
#include "gemm_dispatch.hpp"

namespace tpk {

static inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

static hipError_t swiglu_fwd_bf16(hipStream_t st, int64_t M, int64_t d, int64_t f,
                                  const void* X, const void* W1, const void* W3, const void* W2,
                                  void* G, void* U, void* H, void* Z) {
  {
    GemmParams p = make_params(M, f, make_seg(X, d, M * d, W1, f, d * f, d, W3));
    EpiSwiGLU<bf16> e{static_cast<bf16*>(G), static_cast<bf16*>(U), static_cast<bf16*>(H), f};
    TPK_TRY((launch_gemm<true, false, true>(st, "swiglu_fwd.x_w1w3_swiglu", p, e, plan_gemm(M, f, d, true, false))));
  }
  {
    GemmParams p = make_params(M, d, make_seg(H, f, M * f, W2, d, f * d, f));
    EpiStore<bf16> e{static_cast<bf16*>(Z), d, 0};
    TPK_TRY((launch_gemm<true, false, false>(st, "swiglu_fwd.hw2", p, e, plan_gemm(M, d, f, false, false))));
  }
  return hipSuccess;
}

struct SwigluBwdPlan {
  GemmPlan dH, dW2, dW13;
  size_t dGU_bytes, split_bytes, tail_bytes;
};

// Workspace: [dG | dU], then the split-K partials of dW2, then the fp32
// partial tiles of a split last round (shared by the dH and [dW1 | dW3]
// products, which run one after the other).
static SwigluBwdPlan swiglu_bwd_plan(int dt, int64_t M, int64_t d, int64_t f) {
  SwigluBwdPlan pl;
  const size_t es = dt == DT_BF16 ? 2 : 4;
  pl.dGU_bytes = align256((size_t)M * 2 * f * es);
  const bool bf = dt == DT_BF16;
  pl.dH = bf ? plan_gemm(M, f, d, false, false, true) : GemmPlan{CFG_S, 1};
  pl.dW2 = bf ? plan_gemm(f, d, M, false, true) : GemmPlan{CFG_S, 1};
  pl.dW13 = bf ? plan_gemm(d, 2 * f, M, false, false, true) : GemmPlan{CFG_S, 1};
  pl.split_bytes = pl.dW2.split > 1 ? align256((size_t)pl.dW2.split * f * d * 4) : 0;
  pl.tail_bytes = align256(std::max(gemm_tail_ws_bytes(pl.dH, M, f), gemm_tail_ws_bytes(pl.dW13, d, 2 * f)));
  return pl;
}

size_t swiglu_bwd_ws_bytes(int dt, int64_t M, int64_t d, int64_t f) {
  const SwigluBwdPlan pl = swiglu_bwd_plan(dt, M, d, f);
  return pl.dGU_bytes + pl.split_bytes + pl.tail_bytes;
}

static hipError_t swiglu_bwd_bf16(hipStream_t st, int64_t M, int64_t d, int64_t f,
                                  const void* X, const void* W1, const void* W3, const void* W2,
                                  const void* G, const void* U, const void* H, const void* dY,
                                  void* dX, float* dW1, float* dW3, float* dW2, void* ws) {
  const SwigluBwdPlan pl = swiglu_bwd_plan(DT_BF16, M, d, f);
  bf16* dGU = static_cast<bf16*>(ws);
  float* split_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.dGU_bytes);
  float* tail_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.dGU_bytes + pl.split_bytes);
  // dH = dY W2^T -> dG, dU and dW2 = H^T dY are independent, as are dX and
  // [dW1 | dW3] below: each pair runs as one launch where that beats two
  // (partial last rounds; gemm_pair_est), the weight gradient (K = M, the
  // longer) first.
  GemmParams ph = make_params(M, f, make_seg(dY, d, M * d, W2, d, f * d, d));
  EpiDSwiGLU<bf16> eh{static_cast<const bf16*>(G), static_cast<const bf16*>(U), dGU, f};
  GemmParams p2 = make_params(f, d, make_seg(H, f, M * f, dY, d, M * d, M));
  EpiStore<float> e2{dW2, d, 0};
  const GemmPlan ph_plain = plan_gemm(M, f, d, false, false);
  if (pl.dW2.split == 1 &&
      gemm_pair_est(pl.dW2, tiles_for(CFG_L, f, d, false), ph_plain, tiles_for(CFG_L, M, f, false)) <
          0.97 * (pl.dW2.est + pl.dH.est)) {
    TPK_TRY((launch_gemm_pair<false, false, EpiStore<float>, true, true, EpiDSwiGLU<bf16>>(
        st, "swiglu_bwd.htdy_dswiglu_pair", p2, e2, ph, eh)));
  } else {
    TPK_TRY((launch_gemm<true, true, false>(st, "swiglu_bwd.dyw2t_dswiglu", ph, eh, pl.dH, 1, tail_ws)));
    GemmParams p = p2;
    if (pl.dW2.split > 1) {
      EpiStore<float> e{split_ws, d, f * d};
      TPK_TRY((launch_gemm<false, false, false>(st, "swiglu_bwd.htdy", p, e, pl.dW2)));
      TPK_TRY(launch_shard_reduce(st, DT_F32, DT_F32, pl.dW2.split, f * d, split_ws, f * d, nullptr, 0, dW2));
    } else {
      EpiStore<float> e{dW2, d, 0};
      TPK_TRY((launch_gemm<false, false, false>(st, "swiglu_bwd.htdy", p, e, pl.dW2)));
    }
  }
  // dX = dG W1^T + dU W3^T and [dW1 | dW3] = X^T [dG | dU]
  GemmParams px = make_params(M, d, make_seg(dGU, 2 * f, M * 2 * f, W1, f, d * f, f));
  px.nseg = 2;
  px.seg[1] = make_seg(dGU + f, 2 * f, M * 2 * f - f, W3, f, d * f, f);
  EpiStore<bf16> ex{static_cast<bf16*>(dX), d, 0};
  const GemmPlan plx = plan_gemm(M, d, 2 * f, false, false);
  GemmParams pw = make_params(d, 2 * f, make_seg(X, d, M * d, dGU, 2 * f, M * 2 * f, M));
  EpiF32Halves ew{dW1, dW3, f};
  const GemmPlan pw_plain = plan_gemm(d, 2 * f, M, false, false);
  if (gemm_pair_est(pw_plain, tiles_for(CFG_L, d, 2 * f, false), plx, tiles_for(CFG_L, M, d, false)) <
      0.97 * (pl.dW13.est + plx.est))
    return launch_gemm_pair<false, false, EpiF32Halves, true, true, EpiStore<bf16>>(st, "swiglu_bwd.xtdgu_dx_pair",
                                                                                    pw, ew, px, ex);
  TPK_TRY((launch_gemm<true, true, false>(st, "swiglu_bwd.dgu_w13t", px, ex, plx)));
  TPK_TRY((launch_gemm<false, false, false>(st, "swiglu_bwd.xtdgu", pw, ew, pl.dW13, 1, tail_ws)));
  return hipSuccess;
}

// ------------------------------------------------------------------ fp32
static hipError_t swiglu_fwd_f32(hipStream_t st, int64_t M, int64_t d, int64_t f,
                                 const void* X, const void* W1, const void* W3, const void* W2,
                                 void* G, void* U, void* H, void* Z) {
  {
    GemmParamsF32 p = make_params_f32(M, f, make_seg_f32(X, d, M, W1, f, f, d, W3));
    EpiSwiGLU<float> e{static_cast<float*>(G), static_cast<float*>(U), static_cast<float*>(H), f};
    TPK_TRY((launch_gemm_f32<true, false, true>(st, "swiglu_f32.nn_dual", p, e)));
  }
  {
    GemmParamsF32 p = make_params_f32(M, d, make_seg_f32(H, f, M, W2, d, d, f));
    EpiStore<float> e{static_cast<float*>(Z), d, 0};
    TPK_TRY((launch_gemm_f32<true, false, false>(st, "swiglu_f32.nn", p, e)));
  }
  return hipSuccess;
}

static hipError_t swiglu_bwd_f32(hipStream_t st, int64_t M, int64_t d, int64_t f,
                                 const void* X, const void* W1, const void* W3, const void* W2,
                                 const void* G, const void* U, const void* H, const void* dY,
                                 void* dX, float* dW1, float* dW3, float* dW2, void* ws) {
  float* dGU = static_cast<float*>(ws);
  {
    GemmParamsF32 p = make_params_f32(M, f, make_seg_f32(dY, d, M, W2, d, f, d));
    EpiDSwiGLU<float> e{static_cast<const float*>(G), static_cast<const float*>(U), dGU, f};
    TPK_TRY((launch_gemm_f32<true, true, false>(st, "swiglu_f32.nt", p, e)));
  }
  {
    GemmParamsF32 p = make_params_f32(f, d, make_seg_f32(H, f, f, dY, d, d, M));
    EpiStore<float> e{dW2, d, 0};
    TPK_TRY((launch_gemm_f32<false, false, false>(st, "swiglu_f32.tn", p, e)));
  }
  {
    GemmParamsF32 p = make_params_f32(M, d, make_seg_f32(dGU, 2 * f, M, W1, f, d, f));
    p.nseg = 2;
    p.seg[1] = make_seg_f32(dGU + f, 2 * f, M, W3, f, d, f);
    EpiStore<float> e{static_cast<float*>(dX), d, 0};
    TPK_TRY((launch_gemm_f32<true, true, false>(st, "swiglu_f32.nt", p, e)));
  }
  {
    GemmParamsF32 p = make_params_f32(d, 2 * f, make_seg_f32(X, d, d, dGU, 2 * f, 2 * f, M));
    EpiF32Halves e{dW1, dW3, f};
    TPK_TRY((launch_gemm_f32<false, false, false>(st, "swiglu_f32.tn", p, e)));
  }
  return hipSuccess;
}

hipError_t launch_swiglu_fwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                             const void* X, const void* W1, const void* W3, const void* W2,
                             void* G, void* U, void* H, void* Z) {
  return dt == DT_BF16 ? swiglu_fwd_bf16(st, M, d, f, X, W1, W3, W2, G, U, H, Z)
                       : swiglu_fwd_f32(st, M, d, f, X, W1, W3, W2, G, U, H, Z);
}

hipError_t launch_swiglu_bwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                             const void* X, const void* W1, const void* W3, const void* W2,
                             const void* G, const void* U, const void* H, const void* dY,
                             void* dX, float* dW1, float* dW3, float* dW2, void* ws) {
  return dt == DT_BF16
             ? swiglu_bwd_bf16(st, M, d, f, X, W1, W3, W2, G, U, H, dY, dX, dW1, dW3, dW2, ws)
             : swiglu_bwd_f32(st, M, d, f, X, W1, W3, W2, G, U, H, dY, dX, dW1, dW3, dW2, ws);
}

}  // namespace tpk
