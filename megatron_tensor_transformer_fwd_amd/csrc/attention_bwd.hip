// Backward of the head-group attention shard ([BM] Megatron_MHA; [HC] 3.4):
// the products around the flash kernels of attention_bwd_core.hip, and the
// workspace they share.
//
//   dO = dY W_O^T;  dW_O = O^T dY;  D = rowsum(dO * O);  flash dQ, dK, dV;
//   dX = [dQ | dK | dV] [W_Q | W_K | W_V]^T;  [dW_Q | dW_K | dW_V] = X^T [dQ | dK | dV]
#include "epilogues.hpp"
#include "gemm_dispatch.hpp"
#include "launch.hpp"

namespace tpk {

// fp32 output of a product whose columns [off[k], off[k] + w[k]) go to C[k]
// (row pitch w[k]), e.g. X^T [dQ | dK | dV] -> dW_Q, dW_K, dW_V.
struct EpiF32Parts {
  static constexpr int NOUT = 1;
  template <int O> using OutT = float;
  float* C[3];
  int64_t w0, w1;   // widths: w0, w1, w1 (offsets 0, w0, w0 + w1)
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ float* out_ptr(int64_t m, int64_t n, int, int) const {
    if (n < w0) return C[0] + m * w0 + n;
    if (n < w0 + w1) return C[1] + m * w1 + (n - w0);
    return C[2] + m * w1 + (n - w0 - w1);
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const { return v; }
};

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: dO [M x N] bf16, [dQ | dK | dV] [M x (N + 2 Nkv)] bf16,
// [W_Q | W_K | W_V] [d x (N + 2 Nkv)] bf16, D and L2 [b h s] fp32, with
// grouped K/V heads the per-query-head fp32 dK and dV contributions [M x N]
// each, then the split-K partials of dW_O, then the fp32 partial tiles of the
// weight-gradient product's split last round.
struct AttnBwdLayout {
  size_t dO, dQKV, Wcat, Dv, L2, part, split, tail, total;
  GemmPlan wqkv;     // [dW_Q | dW_K | dW_V] = X^T [dQ | dK | dV]
};

static AttnBwdLayout attn_bwd_layout(int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t h_kv,
                                     int64_t d_head) {
  const int64_t M = b * s, N = h_local * d_head, Nt = N + 2 * h_kv * d_head;
  const GemmPlan pwo = plan_gemm(N, d, M, false, true);
  AttnBwdLayout l;
  l.dO = 0;
  l.dQKV = l.dO + up256((size_t)M * N * 2);
  l.Wcat = l.dQKV + up256((size_t)M * Nt * 2);
  l.Dv = l.Wcat + up256((size_t)d * Nt * 2);
  l.L2 = l.Dv + up256((size_t)b * h_local * s * 4);
  l.part = l.L2 + up256((size_t)b * h_local * s * 4);
  l.split = l.part + (h_kv != h_local ? 2 * up256((size_t)M * N * 4) : 0);
  l.tail = l.split + (pwo.split > 1 ? up256((size_t)pwo.split * N * d * 4) : 0);
  l.wqkv = plan_gemm(d, Nt, M, false, false, true);
  l.total = l.tail + up256(gemm_tail_ws_bytes(l.wqkv, d, Nt));
  return l;
}

size_t attn_bwd_ws_bytes(int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t h_kv, int64_t d_head) {
  return attn_bwd_layout(b, s, d, h_local, h_kv, d_head).total;
}

hipError_t launch_attn_bwd(hipStream_t st, int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t h_kv,
                           int64_t d_head, int causal, float scale,
                           const void* X, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                           const void* Q, const void* K, const void* V, const void* O, const float* L,
                           const void* dY, void* dX, float* dWq, float* dWk, float* dWv, float* dWo,
                           void* ws) {
  if (d_head != 128 || h_kv <= 0 || h_local % h_kv) return hipErrorInvalidValue;   // the flash kernels' width
  const int64_t M = b * s, N = h_local * d_head, Nkv = h_kv * d_head, Nt = N + 2 * Nkv;
  const int group = (int)(h_local / h_kv);
  const AttnBwdLayout lay = attn_bwd_layout(b, s, d, h_local, h_kv, d_head);
  char* w = static_cast<char*>(ws);
  bf16* dO = reinterpret_cast<bf16*>(w + lay.dO);
  bf16* dQKV = reinterpret_cast<bf16*>(w + lay.dQKV);  // [M x Nt]: dQ | dK | dV
  bf16* Wcat = reinterpret_cast<bf16*>(w + lay.Wcat);  // [d x Nt]: W_Q | W_K | W_V
  float* Dv = reinterpret_cast<float*>(w + lay.Dv);
  float* L2 = reinterpret_cast<float*>(w + lay.L2);
  float* part = reinterpret_cast<float*>(w + lay.part);
  float* split_ws = reinterpret_cast<float*>(w + lay.split);
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d_head);

  {  // dO = dY W_O^T
    GemmParams p = make_params(M, N, make_seg(dY, d, M * d, Wo, d, N * d, d));
    EpiStore<bf16> e{dO, N, 0};
    TPK_TRY((launch_gemm<true, true, false>(st, "attn_bwd.dy_wot", p, e, plan_gemm(M, N, d, false, false))));
  }
  {  // dW_O = O^T dY (fp32; split along K = M when the output is narrow):
     // A(m, k) = O[k][m], B(k, n) = dY[k][n]
    GemmParams p = make_params(N, d, make_seg(O, N, M * N, dY, d, M * d, M));
    TPK_TRY(wgrad_f32_out(st, plan_gemm(N, d, M, false, true), N, d, dWo, split_ws,
                          [&](const EpiStore<float>& e, GemmPlan g) {
                            return launch_gemm<false, false, false>(st, "attn_bwd.ot_dy", p, e, g);
                          }));
  }
  // D = rowsum(dO * O) and L in base 2, then the flash kernels
  TPK_TRY(launch_attn_bwd_rowdot(st, dO, O, L, Dv, L2, M, (int)h_local, (int)s, N));
  {
    float* pk = part;
    float* pv = reinterpret_cast<float*>(reinterpret_cast<char*>(part) + up256((size_t)M * N * 4));
    TPK_TRY(launch_attn_bwd_flash(st, (int)b, (int)h_local, group, (int)s, causal, sc, Q, K, V, dO, L2, Dv, N,
                                  dQKV, Nt, N, Nkv, pk, pv));
  }
  TPK_TRY(launch_attn_concat3(st, Wq, Wk, Wv, Wcat, d, N, Nkv));   // [W_Q | W_K | W_V]
  // dX = [dQ | dK | dV] [W_Q | W_K | W_V]^T and [dW_Q | dW_K | dW_V] = X^T [dQ | dK | dV]
  GemmParams px = make_params(M, d, make_seg(dQKV, Nt, M * Nt, Wcat, Nt, d * Nt, Nt));
  EpiStore<bf16> ex{static_cast<bf16*>(dX), d, 0};
  const GemmPlan plx = plan_gemm(M, d, Nt, false, false);
  GemmParams pw = make_params(d, Nt, make_seg(X, d, M * d, dQKV, Nt, M * Nt, M));
  EpiF32Parts ew{{dWq, dWk, dWv}, N, Nkv};
  // The two are independent: one launch where the weight gradient's tiles
  // (K = M, the longer) would leave a partial round (C4: 192 tiles), the
  // dX tiles filling it.
  const GemmPlan plw = plan_gemm(d, Nt, M, false, false);
  if (gemm_pair_est(plw, tiles_for(CFG_L, d, Nt, false), plx, tiles_for(CFG_L, M, d, false)) <
      0.97 * (lay.wqkv.est + plx.est))
    return launch_gemm_pair<false, false, EpiF32Parts, true, true, EpiStore<bf16>>(st, "attn_bwd.wgrad_dx_pair",
                                                                                    pw, ew, px, ex);
  TPK_TRY((launch_gemm<true, true, false>(st, "attn_bwd.dqkv_wt", px, ex, plx)));
  TPK_TRY((launch_gemm<false, false, false>(st, "attn_bwd.xt_dqkv", pw, ew, lay.wqkv, 1,
                                            reinterpret_cast<float*>(w + lay.tail))));
  return hipSuccess;
}

}  // namespace tpk
