// GeLU MLP shard, forward and backward ([JY] FFN; [HC] 3.4, Figure 3.4).
//
// Forward:  A = X W1 (column-parallel, GeLU fused: H = GeLU(A)),
//           Z = H W2 (row-parallel partial).
// Backward: dA = (dY W2^T) * GeLU'(A)      NT product, GeLU' fused
//           dW2 = H^T dY                   TN product (fp32, split-K if narrow)
//           dX = dA W1^T                   NT product (this shard's summand)
//           dW1 = X^T dA                   TN product (fp32, split-K if narrow)
#include <mutex>
#include <type_traits>

#include "epilogues.hpp"
#include "gemm_dispatch.hpp"
#include "tp_shard.h"

namespace tpk {

// Workspace of the allocation-free MLP backward: a device array in this code
// object, so every GPU the library runs on holds its own copy from the
// library's first use there until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: kernels and copies
// take the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[TP_MLP_BWD_NOALLOC_MAX_WORKSPACE];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t mlp_bwd_scratch(void** ptr) {
  int dev = -1;
  TPK_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    TPK_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));   // with device `dev` current
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

static inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// ------------------------------------------------------------------ bf16
// H and dA are the left operand of the next products, over K = f.  With a
// short K those products' tiles are mostly operand fetch and epilogue, and
// H and dA stored without the streaming hint are still in the caches when
// they start: at C2 (f 512, all shards) the Z and dX products took 79-81
// instead of 87-88 us (A, kept as well, saves the GeLU' dgrad another 1 us).
// At f 4096 (C5) the same made the GeLU product 1.5% slower and its readers
// no faster, so only narrow shards keep them.
constexpr int64_t kKeepOperandMaxK = 1024;

template <class F>
static hipError_t with_keep(int64_t f, F&& run) {
  return f <= kKeepOperandMaxK ? run(std::true_type{}) : run(std::false_type{});
}

static hipError_t mlp_fwd_bf16(hipStream_t st, int64_t M, int64_t d, int64_t f,
                               const void* X, const void* W1, const void* W2,
                               void* A, void* H, void* Z) {
  {  // A = X W1, H = GeLU(A)
    GemmParams p = make_params(M, f, make_seg(X, d, M * d, W1, f, d * f, d));
    TPK_TRY(with_keep(f, [&](auto keep) {
      EpiGelu<bf16, decltype(keep)::value> e{static_cast<bf16*>(A), static_cast<bf16*>(H), f};
      return launch_gemm<true, false, false>(st, "mlp_fwd.xw1_gelu", p, e, plan_gemm(M, f, d, false, false));
    }));
  }
  {  // Z = H W2
    GemmParams p = make_params(M, d, make_seg(H, f, M * f, W2, d, f * d, f));
    EpiStore<bf16> e{static_cast<bf16*>(Z), d, 0};
    TPK_TRY((launch_gemm<true, false, false>(st, "mlp_fwd.hw2", p, e, plan_gemm(M, d, f, false, false))));
  }
  return hipSuccess;
}

struct MlpBwdPlan {
  GemmPlan dW2, dW1;
  size_t dA_bytes, split_bytes;
};

static MlpBwdPlan mlp_bwd_plan(int dt, int64_t M, int64_t d, int64_t f) {
  MlpBwdPlan pl;
  const size_t es = dt == DT_BF16 ? 2 : 4;
  pl.dA_bytes = align256((size_t)M * f * es);
  if (dt == DT_BF16) {
    pl.dW2 = plan_gemm(f, d, M, false, true);
    pl.dW1 = plan_gemm(d, f, M, false, true);
  } else {
    pl.dW2 = pl.dW1 = GemmPlan{CFG_S, 1};
  }
  const int smax = std::max(pl.dW2.split, pl.dW1.split);
  pl.split_bytes = smax > 1 ? align256((size_t)smax * d * f * 4) : 0;
  return pl;
}

size_t mlp_bwd_ws_bytes(int dt, int64_t M, int64_t d, int64_t f) {
  const MlpBwdPlan pl = mlp_bwd_plan(dt, M, d, f);
  return pl.dA_bytes + pl.split_bytes;
}

static hipError_t mlp_bwd_bf16(hipStream_t st, int64_t M, int64_t d, int64_t f,
                               const void* X, const void* W1, const void* W2,
                               const void* A, const void* H, const void* dY,
                               void* dX, float* dW1, float* dW2, void* ws) {
  const MlpBwdPlan pl = mlp_bwd_plan(DT_BF16, M, d, f);
  bf16* dA = static_cast<bf16*>(ws);
  float* split_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.dA_bytes);
  // dW2 first: it reads dY, which the dgrad then finds in the Infinity Cache,
  // and the dgrad's output dA is then fresh for the two products that read it.
  {  // dW2 = H^T dY:  A(m, k) = H[k][m], B(k, n) = dY[k][n]
    GemmParams p = make_params(f, d, make_seg(H, f, M * f, dY, d, M * d, M));
    TPK_TRY(wgrad_f32_out(st, pl.dW2, f, d, dW2, split_ws, [&](const EpiStore<float>& e, GemmPlan g) {
      return launch_gemm<false, false, false>(st, "mlp_bwd.htdy", p, e, g);
    }));
  }
  {  // dA = (dY W2^T) * GeLU'(A);  B(k, n) = W2[n][k]
    GemmParams p = make_params(M, f, make_seg(dY, d, M * d, W2, d, f * d, d));
    TPK_TRY(with_keep(f, [&](auto keep) {
      EpiDGelu<bf16, decltype(keep)::value> e{static_cast<const bf16*>(A), dA, f};
      return launch_gemm<true, true, false>(st, "mlp_bwd.dyw2t_dgelu", p, e, plan_gemm(M, f, d, false, false));
    }));
  }
  {  // dX = dA W1^T;  B(k, n) = W1[n][k]
    GemmParams p = make_params(M, d, make_seg(dA, f, M * f, W1, f, d * f, f));
    EpiStore<bf16> e{static_cast<bf16*>(dX), d, 0};
    TPK_TRY((launch_gemm<true, true, false>(st, "mlp_bwd.daw1t", p, e, plan_gemm(M, d, f, false, false))));
  }
  {  // dW1 = X^T dA:  A(m, k) = X[k][m], B(k, n) = dA[k][n]
    GemmParams p = make_params(d, f, make_seg(X, d, M * d, dA, f, M * f, M));
    TPK_TRY(wgrad_f32_out(st, pl.dW1, d, f, dW1, split_ws, [&](const EpiStore<float>& e, GemmPlan g) {
      return launch_gemm<false, false, false>(st, "mlp_bwd.xtda", p, e, g);
    }));
  }
  return hipSuccess;
}

// ------------------------------------------------------------------ fp32
// n shards per launch (n = 1: one shard), shard-stacked as in the bf16 path;
// dA ([n x M x f]) lives in the workspace.
static hipError_t mlp_fwd_f32(hipStream_t st, int64_t n, int64_t M, int64_t d, int64_t f,
                              const void* X, const void* W1s, const void* W2s,
                              void* A, void* H, void* Z) {
  {  // A_i = X W1_i, H_i = GeLU(A_i)
    GemmParamsF32 p = make_params_f32(M, f, make_seg_f32(X, d, M, W1s, f, f, d));
    p.b_zs = d * f;
    p.z_rows = (int)M;
    EpiGelu<float> e{static_cast<float*>(A), static_cast<float*>(H), f};
    TPK_TRY((launch_gemm_f32<true, false, false>(st, "mlp_f32.nn", p, e, (int)n)));
  }
  {  // Z_i = H_i W2_i
    GemmParamsF32 p = make_params_f32(M, d, make_seg_f32(H, f, M, W2s, d, d, f));
    p.a_zs = M * f;
    p.b_zs = f * d;
    p.z_rows = (int)M;
    EpiStore<float> e{static_cast<float*>(Z), d, 0};
    TPK_TRY((launch_gemm_f32<true, false, false>(st, "mlp_f32.nn", p, e, (int)n)));
  }
  return hipSuccess;
}

static hipError_t mlp_bwd_f32(hipStream_t st, int64_t n, int64_t M, int64_t d, int64_t f,
                              const void* X, const void* W1s, const void* W2s,
                              const void* A, const void* H, const void* dY,
                              void* dX, float* dW1s, float* dW2s, void* ws) {
  float* dA = static_cast<float*>(ws);
  {  // dA_i = (dY W2_i^T) * GeLU'(A_i)
    GemmParamsF32 p = make_params_f32(M, f, make_seg_f32(dY, d, M, W2s, d, f, d));
    p.b_zs = f * d;
    p.z_rows = (int)M;
    EpiDGelu<float> e{static_cast<const float*>(A), dA, f};
    TPK_TRY((launch_gemm_f32<true, true, false>(st, "mlp_f32.nt", p, e, (int)n)));
  }
  {  // dW2_i = H_i^T dY
    GemmParamsF32 p = make_params_f32(f, d, make_seg_f32(H, f, f, dY, d, d, M));
    p.a_zs = M * f;
    p.z_rows = (int)f;
    EpiStore<float> e{dW2s, d, 0};
    TPK_TRY((launch_gemm_f32<false, false, false>(st, "mlp_f32.tn", p, e, (int)n)));
  }
  {  // dX_i = dA_i W1_i^T
    GemmParamsF32 p = make_params_f32(M, d, make_seg_f32(dA, f, M, W1s, f, d, f));
    p.a_zs = M * f;
    p.b_zs = d * f;
    p.z_rows = (int)M;
    EpiStore<float> e{static_cast<float*>(dX), d, 0};
    TPK_TRY((launch_gemm_f32<true, true, false>(st, "mlp_f32.nt", p, e, (int)n)));
  }
  {  // dW1_i = X^T dA_i
    GemmParamsF32 p = make_params_f32(d, f, make_seg_f32(X, d, d, dA, f, f, M));
    p.b_zs = M * f;
    p.z_rows = (int)d;
    EpiStore<float> e{dW1s, f, 0};
    TPK_TRY((launch_gemm_f32<false, false, false>(st, "mlp_f32.tn", p, e, (int)n)));
  }
  return hipSuccess;
}

// Shards per fp32 launch: all of them while the grid's z extent (shards x
// column tiles of the widest product) stays within the launch limit.
static int64_t f32_shards_per_launch(int64_t n, int64_t d, int64_t f) {
  const int64_t tiles = cdiv(std::max(d, f), 64);
  return std::max<int64_t>(1, std::min<int64_t>(n, 65535 / tiles));
}

// ------------------------------------------- all shards of the layer at once
// Every shard's products are independent given X (forward) or dY (backward)
// ([HC] 3.4), so with all n shards held on one GPU each product runs as one
// launch over the n shards (grid z = shard): the n narrow products fill the
// chip together where one alone would leave most compute units idle.
// Weights are shard-stacked ([n x d x f] and [n x f x d]), as are the
// per-shard activations, partials and weight gradients.

struct MlpShardsPlan {
  GemmPlan xw1, hw2, htdy, dyw2t, daw1t, xtda;
  size_t dA_bytes, split_bytes;
};

static MlpShardsPlan mlp_shards_plan(int64_t n, int64_t M, int64_t d, int64_t f) {
  MlpShardsPlan pl;
  pl.xw1 = plan_gemm(M, f, d, false, false, false, n);
  pl.hw2 = plan_gemm(M, d, f, false, false, false, n);
  pl.htdy = plan_gemm(f, d, M, false, true, false, n);
  pl.dyw2t = plan_gemm(M, f, d, false, false, false, n);
  pl.daw1t = plan_gemm(M, d, f, false, false, false, n);
  pl.xtda = plan_gemm(d, f, M, false, true, false, n);
  pl.dA_bytes = align256((size_t)n * M * f * 2);
  const int smax = std::max(pl.htdy.split, pl.xtda.split);
  pl.split_bytes = smax > 1 ? align256((size_t)smax * n * d * f * 4) : 0;
  return pl;
}

size_t mlp_shards_bwd_ws_bytes(int dt, int64_t n, int64_t M, int64_t d, int64_t f) {
  if (dt != DT_BF16)   // fp32: dA of the shards one launch covers
    return align256((size_t)f32_shards_per_launch(n, d, f) * M * f * 4);
  const MlpShardsPlan pl = mlp_shards_plan(n, M, d, f);
  return pl.dA_bytes + pl.split_bytes;
}

hipError_t launch_mlp_fwd_shards(hipStream_t st, int dt, int64_t n, int64_t M, int64_t d, int64_t f,
                                 const void* X, const void* W1s, const void* W2s, void* A, void* H, void* Z) {
  if (dt != DT_BF16) {
    const int64_t per = f32_shards_per_launch(n, d, f);
    for (int64_t i = 0; i < n; i += per) {
      const int64_t k = std::min(per, n - i);
      auto at = [&](const void* b, int64_t elems) { return static_cast<const float*>(b) + i * elems; };
      auto mt = [&](void* b, int64_t elems) { return b ? static_cast<float*>(b) + i * elems : nullptr; };
      TPK_TRY(mlp_fwd_f32(st, k, M, d, f, X, at(W1s, d * f), at(W2s, f * d), mt(A, M * f), mt(H, M * f),
                          mt(Z, M * d)));
    }
    return hipSuccess;
  }
  const MlpShardsPlan pl = mlp_shards_plan(n, M, d, f);
  {  // A_i = X W1_i, H_i = GeLU(A_i): X shared, W1_i and the outputs per shard
    GemmParams p = make_params(M, f, make_seg(X, d, M * d, W1s, f, d * f, d));
    p.b_zs = d * f;
    p.z_rows = (int)M;
    TPK_TRY(with_keep(f, [&](auto keep) {
      EpiGelu<bf16, decltype(keep)::value> e{static_cast<bf16*>(A), static_cast<bf16*>(H), f};
      return launch_gemm<true, false, false>(st, "mlp_fwd.xw1_gelu", p, e, pl.xw1, (int)n);
    }));
  }
  {  // Z_i = H_i W2_i
    GemmParams p = make_params(M, d, make_seg(H, f, M * f, W2s, d, f * d, f));
    p.a_zs = M * f;
    p.b_zs = f * d;
    p.z_rows = (int)M;
    EpiStore<bf16> e{static_cast<bf16*>(Z), d, 0};
    TPK_TRY((launch_gemm<true, false, false>(st, "mlp_fwd.hw2", p, e, pl.hw2, (int)n)));
  }
  return hipSuccess;
}

hipError_t launch_mlp_bwd_shards(hipStream_t st, int dt, int64_t n, int64_t M, int64_t d, int64_t f,
                                 const void* X, const void* W1s, const void* W2s, const void* A, const void* H,
                                 const void* dY, void* dX, float* dW1s, float* dW2s, void* ws) {
  if (dt != DT_BF16) {
    const int64_t per = f32_shards_per_launch(n, d, f);
    for (int64_t i = 0; i < n; i += per) {
      const int64_t k = std::min(per, n - i);
      auto at = [&](const void* b, int64_t elems) { return static_cast<const float*>(b) + i * elems; };
      TPK_TRY(mlp_bwd_f32(st, k, M, d, f, X, at(W1s, d * f), at(W2s, f * d), at(A, M * f), at(H, M * f), dY,
                          static_cast<float*>(dX) + i * M * d, dW1s + i * d * f, dW2s + i * f * d, ws));
    }
    return hipSuccess;
  }
  const MlpShardsPlan pl = mlp_shards_plan(n, M, d, f);
  bf16* dA = static_cast<bf16*>(ws);
  float* split_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.dA_bytes);
  {  // dW2_i = H_i^T dY
    GemmParams p = make_params(f, d, make_seg(H, f, M * f, dY, d, M * d, M));
    p.a_zs = M * f;
    p.z_rows = (int)f;
    TPK_TRY(wgrad_f32_out(
        st, pl.htdy, f, d, dW2s, split_ws,
        [&](const EpiStore<float>& e, GemmPlan g) { return launch_gemm<false, false, false>(st, "mlp_bwd.htdy", p, e, g, (int)n); },
        n));
  }
  {  // dA_i = (dY W2_i^T) * GeLU'(A_i)
    GemmParams p = make_params(M, f, make_seg(dY, d, M * d, W2s, d, f * d, d));
    p.b_zs = f * d;
    p.z_rows = (int)M;
    TPK_TRY(with_keep(f, [&](auto keep) {
      EpiDGelu<bf16, decltype(keep)::value> e{static_cast<const bf16*>(A), dA, f};
      return launch_gemm<true, true, false>(st, "mlp_bwd.dyw2t_dgelu", p, e, pl.dyw2t, (int)n);
    }));
  }
  {  // dX_i = dA_i W1_i^T
    GemmParams p = make_params(M, d, make_seg(dA, f, M * f, W1s, f, d * f, f));
    p.a_zs = M * f;
    p.b_zs = d * f;
    p.z_rows = (int)M;
    EpiStore<bf16> e{static_cast<bf16*>(dX), d, 0};
    TPK_TRY((launch_gemm<true, true, false>(st, "mlp_bwd.daw1t", p, e, pl.daw1t, (int)n)));
  }
  {  // dW1_i = X^T dA_i
    GemmParams p = make_params(d, f, make_seg(X, d, M * d, dA, f, M * f, M));
    p.b_zs = M * f;
    p.z_rows = (int)d;
    TPK_TRY(wgrad_f32_out(
        st, pl.xtda, d, f, dW1s, split_ws,
        [&](const EpiStore<float>& e, GemmPlan g) { return launch_gemm<false, false, false>(st, "mlp_bwd.xtda", p, e, g, (int)n); },
        n));
  }
  return hipSuccess;
}

hipError_t launch_mlp_fwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                          const void* X, const void* W1, const void* W2,
                          void* A, void* H, void* Z) {
  return dt == DT_BF16 ? mlp_fwd_bf16(st, M, d, f, X, W1, W2, A, H, Z)
                       : mlp_fwd_f32(st, 1, M, d, f, X, W1, W2, A, H, Z);
}

hipError_t launch_mlp_bwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                          const void* X, const void* W1, const void* W2,
                          const void* A, const void* H, const void* dY,
                          void* dX, float* dW1, float* dW2, void* ws) {
  return dt == DT_BF16 ? mlp_bwd_bf16(st, M, d, f, X, W1, W2, A, H, dY, dX, dW1, dW2, ws)
                       : mlp_bwd_f32(st, 1, M, d, f, X, W1, W2, A, H, dY, dX, dW1, dW2, ws);
}

}  // namespace tpk
