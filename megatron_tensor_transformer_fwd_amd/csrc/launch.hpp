// Internal launchers behind the C ABI (host side).  Arguments are already
// validated by tp_shard.cpp; these only choose tile shapes and enqueue.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpk {

enum { DT_F32 = 0, DT_BF16 = 1 };

// Most stripes one all-gather launch copies (their pointers travel in the
// kernel arguments).
constexpr int kSpMaxShards = 64;

hipError_t launch_shard_reduce(hipStream_t st, int dt_in, int dt_out, int n, int64_t numel,
                               const void* P, int64_t stride, const void* bias, int64_t bias_len,
                               void* out);

hipError_t launch_mlp_fwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                          const void* X, const void* W1, const void* W2,
                          void* A, void* H, void* Z);
size_t mlp_bwd_ws_bytes(int dt, int64_t M, int64_t d, int64_t f);
// All n shards of the GeLU MLP (shard-stacked weights, activations and outputs).
hipError_t launch_mlp_fwd_shards(hipStream_t st, int dt, int64_t n, int64_t M, int64_t d, int64_t f,
                                 const void* X, const void* W1s, const void* W2s, void* A, void* H, void* Z);
hipError_t launch_mlp_bwd_shards(hipStream_t st, int dt, int64_t n, int64_t M, int64_t d, int64_t f,
                                 const void* X, const void* W1s, const void* W2s, const void* A, const void* H,
                                 const void* dY, void* dX, float* dW1s, float* dW2s, void* ws);
size_t mlp_shards_bwd_ws_bytes(int dt, int64_t n, int64_t M, int64_t d, int64_t f);
// The current device's address of the allocation-free MLP backward's scratch
// array (looked up once per device).
hipError_t mlp_bwd_scratch(void** ptr);
hipError_t launch_mlp_bwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                          const void* X, const void* W1, const void* W2,
                          const void* A, const void* H, const void* dY,
                          void* dX, float* dW1, float* dW2, void* ws);

hipError_t launch_swiglu_fwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                             const void* X, const void* W1, const void* W3, const void* W2,
                             void* G, void* U, void* H, void* Z);
size_t swiglu_bwd_ws_bytes(int dt, int64_t M, int64_t d, int64_t f);
hipError_t launch_swiglu_bwd(hipStream_t st, int dt, int64_t M, int64_t d, int64_t f,
                             const void* X, const void* W1, const void* W3, const void* W2,
                             const void* G, const void* U, const void* H, const void* dY,
                             void* dX, float* dW1, float* dW3, float* dW2, void* ws);

hipError_t launch_attn_fwd(hipStream_t st, int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t h_kv,
                           int64_t d_head, int causal, float scale,
                           const void* X, const void* Wq, const void* Wk, const void* Wv,
                           const void* Wo, void* Q, void* K, void* V, void* O, void* Z, float* L);
// Flash-attention backward kernels (attention_bwd_core.hip); bf16 tensors.
hipError_t launch_attn_bwd_rowdot(hipStream_t st, const void* dO, const void* O, const float* L, float* Dv,
                                  float* L2, int64_t rows, int hl, int s, int64_t ld);
hipError_t launch_attn_bwd_flash(hipStream_t st, int b, int hl, int group, int s, int causal, float scale,
                                 const void* Q, const void* K, const void* V, const void* dO, const float* L2,
                                 const float* Dv, int64_t ld_o, void* dQKV, int64_t ld_g, int64_t n_q,
                                 int64_t n_kv, float* part_k, float* part_v);
hipError_t launch_attn_concat3(hipStream_t st, const void* A, const void* B, const void* C, void* out, int64_t rows,
                               int64_t n0, int64_t n1);
size_t attn_bwd_ws_bytes(int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t h_kv, int64_t d_head);
hipError_t launch_attn_bwd(hipStream_t st, int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t h_kv,
                           int64_t d_head, int causal, float scale,
                           const void* X, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                           const void* Q, const void* K, const void* V, const void* O, const float* L,
                           const void* dY, void* dX, float* dWq, float* dWk, float* dWv, float* dWo,
                           void* ws);

hipError_t launch_sp_reduce_scatter_ln(hipStream_t st, int dt, int n, int64_t rows, int64_t cols,
                                       int64_t index, const void* P, int64_t stride, const void* bias,
                                       const void* residual, const uint8_t* keep, float p_drop,
                                       const void* gamma, const void* beta, float eps, void* h_out,
                                       void* x_out);
size_t sp_ln_bwd_ws_bytes(int64_t rows, int64_t cols, int n);
hipError_t launch_sp_ln_bwd(hipStream_t st, int dt, int n, int64_t rows, int64_t cols, int64_t index,
                            const void* P, int64_t stride, const void* h, const void* gamma, float eps,
                            const uint8_t* keep, float p_drop, const void* dres, void* dh_out, void* dy_out,
                            float* dgamma, float* dbeta, float* dbias, void* ws);
hipError_t launch_sp_all_gather(hipStream_t st, int dt, int n, int64_t stripe_rows, int64_t cols,
                                const void* const* stripes, void* full);

hipError_t launch_vocab_embed_fwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                                  int64_t vstart, const int64_t* ids, const void* E, void* Y);
hipError_t launch_vocab_embed_bwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                                  int64_t vstart, const int64_t* ids, const void* dY, float* dE);
size_t vocab_ce_fwd_ws_bytes(int dt, int64_t n_tokens, int64_t vlocal);
hipError_t launch_vocab_ce_fwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                               int64_t vstart, const void* X, const void* E, const int64_t* targets,
                               void* logits, float* stats, void* ws);
hipError_t launch_vocab_ce_combine(hipStream_t st, int n, int64_t n_tokens, const float* stats,
                                   int64_t shard_stride, float* loss, float* lse);
size_t vocab_ce_bwd_ws_bytes(int dt, int64_t n_tokens, int64_t d, int64_t vlocal);
hipError_t launch_vocab_ce_bwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                               int64_t vstart, const void* X, const void* E, const int64_t* targets,
                               const void* logits, const float* lse, const float* dloss, void* dX, float* dE,
                               void* ws);

}  // namespace tpk
