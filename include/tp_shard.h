/*
 * tp_shard.h — C ABI of libtpshard: one GPU's shard of a Megatron-LM
 * tensor-parallel transformer layer, hand-written for AMD gfx950 (MI355X).
 *
 * The operations follow these pages (cited by title and section):
 *  [JY] "Parallelism on Jiang Yi's Homepage", note "megatron-lm", sections
 *       FFN (Y = GeLU(X W1) W2; W1 split by columns, W2 by rows; the f/g
 *       table; the SwiGLU split) and Attention (heads split across GPUs,
 *       O = [o_1 .. o_h] W_O).
 *  [HC] "Splitting the model: five parallelisms and the traffic they make",
 *       section 3.4 "Tensor parallelism", Figures 3.4-3.6 (Z = sum_k Z_k;
 *       g all-reduces the partial outputs forward, f all-reduces dX backward).
 *  [BM] "tensor-parallelism" (brunomaga.github.io), section "Megatron-LM tensor
 *       parallelism" (Megatron_f/Megatron_g, the feed-forward block with the
 *       bias added after the reduction, Megatron_MHA with its causal mask and
 *       1/sqrt(head_dim) scale).
 *  [DW] "Chapter 8: Distributed Training", section 8.4.2 NCCL (all_reduce SUM).
 *
 * Conventions shared by every entry point
 *  - Matrices are dense, row-major, contiguous: an [R x C] matrix has element
 *    (r, c) at offset r*C + c.  Weights are [in x out] and products are X W,
 *    as in [JY] FFN (W1 in R^{d x d_ff}, W2 in R^{d_ff x d}).
 *  - M = b*s tokens (rows of X).  f is this shard's slice of d_ff.
 *  - dtype TP_DT_BF16: bf16 operands, activations and partial outputs; every
 *    product accumulates in fp32; weight gradients are fp32.  TP_DT_F32: all
 *    fp32.  bf16 results are rounded to nearest, ties to even.
 *  - Every pointer except `stream` is a device pointer (tp_sp_all_gather's
 *    stripe array and tp_shard_range's results are host memory), 16-byte
 *    aligned unless an entry point says otherwise.  The
 *    caller owns all memory; the library allocates nothing, never
 *    synchronises and never changes the current device.  The only state it
 *    keeps between calls is thread-local (the last error text and the
 *    optional kernel-timing hook, tp_profile_begin), plus the per-device
 *    scratch array of tp_mlp_bwd_noalloc and its address on each device.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; faults raised while a kernel runs surface at
 *    the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call.  Every entry
 *    point returns TP_OK (0) or a negative status; tp_last_error_detail()
 *    then holds a thread-local description.  No exception crosses the ABI.
 *  - Size limits (TP_E_DIM beyond them): every size <= 2^30; row pitches
 *    d, f and h_local*d_head <= 2^21 elements (the kernels address a tile of
 *    up to 256 rows with 32-bit offsets); attention s <= 2^22.
 *  - Outputs must not overlap any input or each other (except where noted).
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TP_ABI_VERSION 11

/* dtype codes; tp_dtype_t is a plain 32-bit int so that any value a caller
 * passes is well defined on both sides of the ABI, and values other than
 * these are refused with TP_E_DTYPE */
typedef int32_t tp_dtype_t;
enum { TP_DT_F32 = 0, TP_DT_BF16 = 1 };

/* status codes */
#define TP_OK           0
#define TP_E_NULL      -1   /* a required pointer is NULL                     */
#define TP_E_DIM       -2   /* a size is <= 0, too large, or not supported    */
#define TP_E_DIVIS     -3   /* a size is not a multiple of what it must be    */
#define TP_E_DTYPE     -4   /* unsupported dtype for this entry point         */
#define TP_E_ALIGN     -5   /* a pointer is not aligned as required           */
#define TP_E_ALIAS     -6   /* an output overlaps an input or another output  */
#define TP_E_WORKSPACE -7   /* workspace NULL or smaller than required        */
#define TP_E_HIP       -8   /* a HIP launch failed (text in the detail)       */

/* ---------------------------------------------------------------------------
 * tp_shard_range — the contiguous equal split of `total` features, heads or
 * rows over `n_shards` shards: shard `index` owns [index*k, (index+1)*k) with
 * k = total / n_shards.  Returns TP_E_DIVIS when total % n_shards != 0 (the
 * pages' listings assert divisibility: [JY] Implementation; [BM]
 * Megatron_MHA raises ValueError), TP_E_DIM for non-positive sizes or an
 * index outside [0, n_shards), TP_E_NULL for NULL outputs.  Host only.
 * ------------------------------------------------------------------------- */
int tp_shard_range(int64_t total, int64_t n_shards, int64_t index,
                   int64_t* start, int64_t* len);

/* ---------------------------------------------------------------------------
 * tp_mlp_fwd — GeLU MLP shard forward ([JY] FFN; [HC] Figure 3.4):
 *   A = X W1        (column-parallel product; W1 is this shard's column slice)
 *   H = GeLU(A)     (exact erf form, applied in the product's epilogue)
 *   Z = H W2        (row-parallel product; this shard's summand of Y)
 * X [M x d], W1 [d x f], W2 [f x d], A and H [M x f], Z [M x d].
 * A may be NULL (pre-activation not kept); H and Z are required.
 * d and f must be multiples of 8.
 * ------------------------------------------------------------------------- */
int tp_mlp_fwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
               const void* X, const void* W1, const void* W2,
               void* A, void* H, void* Z);

/* ---------------------------------------------------------------------------
 * tp_mlp_bwd — GeLU MLP shard backward.  g is the identity backward, so dY
 * is the full upstream gradient ([JY] f/g table; [BM] Megatron_g):
 *   dA  = (dY W2^T) * GeLU'(A)     (GeLU' fused into the dgrad epilogue)
 *   dW2 = H^T dY                   (fp32, [f x d])
 *   dX  = dA W1^T                  (this shard's summand; f sums them, [HC] 3.4)
 *   dW1 = X^T dA                   (fp32, [d x f])
 * A, H are the forward's saved outputs.  dX [M x d] has dtype dt; dW1, dW2
 * are always fp32.  ws: device workspace of at least
 * tp_mlp_bwd_workspace_bytes(dt, M, d, f) bytes (holds dA and split-K
 * partials); it is scratch, contents undefined after the call.
 * ------------------------------------------------------------------------- */
int tp_mlp_bwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
               const void* X, const void* W1, const void* W2,
               const void* A, const void* H, const void* dY,
               void* dX, float* dW1, float* dW2, void* ws, size_t ws_bytes);
size_t tp_mlp_bwd_workspace_bytes(tp_dtype_t dt, int64_t M, int64_t d, int64_t f);

/* ---------------------------------------------------------------------------
 * tp_mlp_fwd_shards / tp_mlp_bwd_shards — every one of n_shards shards of the
 * GeLU MLP at once, for a layer whose shards are all held on this GPU (the
 * local stand-in for the TP group of [HC] 3.4: each shard's products depend
 * only on X forward and dY backward, so shard i computes exactly what
 * tp_mlp_fwd / tp_mlp_bwd compute for W1_i, W2_i).  Each product runs as one
 * launch over the shards.  Shard-stacked layouts (shard i's block follows
 * shard i-1's): W1s [n_shards x d x f] (shard i's column slice W1_i as its own
 * [d x f] matrix), W2s [n_shards x f x d]; A, H [n_shards x M x f]; Z, dX
 * [n_shards x M x d] (the partials that tp_shard_reduce sums); dW1s
 * [n_shards x d x f] and dW2s [n_shards x f x d], fp32.  X and dY [M x d] are
 * shared.  1 <= n_shards <= 64; other sizes, dtypes and errors as tp_mlp_fwd /
 * tp_mlp_bwd; ws: tp_mlp_bwd_shards_workspace_bytes(...) bytes.  Results equal
 * the per-shard calls' within rounding (the tile shapes may differ).
 * ------------------------------------------------------------------------- */
int tp_mlp_fwd_shards(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t M, int64_t d, int64_t f,
                      const void* X, const void* W1s, const void* W2s, void* A, void* H, void* Z);
int tp_mlp_bwd_shards(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t M, int64_t d, int64_t f,
                      const void* X, const void* W1s, const void* W2s, const void* A, const void* H,
                      const void* dY, void* dX, float* dW1s, float* dW2s, void* ws, size_t ws_bytes);
size_t tp_mlp_bwd_shards_workspace_bytes(tp_dtype_t dt, int64_t n_shards, int64_t M, int64_t d, int64_t f);

/* ---------------------------------------------------------------------------
 * tp_mlp_bwd_noalloc — tp_mlp_bwd for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving or training
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and
 * kernels as tp_mlp_bwd (bitwise the same outputs), without ws: its
 * workspace is a static device array of TP_MLP_BWD_NOALLOC_MAX_WORKSPACE
 * bytes (64 MiB) inside the library, one per GPU, held from the library's
 * first use on that GPU until the process ends.  Sizes whose
 * tp_mlp_bwd_workspace_bytes exceeds it return TP_E_WORKSPACE before any HIP
 * call (the 8192-token shards of a 8192 x 32768 layer at TP 8 and of a
 * 1024 x 4096 layer at TP 8 fit).  It calls no allocator.  The first call on
 * each GPU looks up that GPU's copy of the array (hipGetSymbolAddress, with
 * that GPU current); make it once outside graph capture.  Every call on a
 * GPU uses the same array, whatever its stream: calls that overlap in time
 * on one GPU (two streams, two threads) race on it, and it keeps the last
 * call's contents (nothing in it needs to start at zero).
 * ------------------------------------------------------------------------- */
#define TP_MLP_BWD_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
int tp_mlp_bwd_noalloc(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
                       const void* X, const void* W1, const void* W2,
                       const void* A, const void* H, const void* dY,
                       void* dX, float* dW1, float* dW2);

/* ---------------------------------------------------------------------------
 * tp_swiglu_fwd — SwiGLU MLP shard forward ([JY] FFN, SwiGLU part: W1 and
 * W3 split by columns, W2 by rows; the listing computes
 * w2(silu(w1(x)) * w3(x)), so W1 is the Swish'd gate and W3 the up projection):
 *   G = X W1, U = X W3  (one pass over X, both slices in the same tile)
 *   H = Swish(G) * U    (Swish(x) = x sigmoid(x), in the epilogue)
 *   Z = H W2
 * X [M x d], W1, W3 [d x f], W2 [f x d], G, U, H [M x f], Z [M x d].
 * G and U may both be NULL (not kept; then no backward is possible).
 * ------------------------------------------------------------------------- */
int tp_swiglu_fwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
                  const void* X, const void* W1, const void* W3, const void* W2,
                  void* G, void* U, void* H, void* Z);

/* ---------------------------------------------------------------------------
 * tp_swiglu_bwd — SwiGLU MLP shard backward (chain rule through the forward):
 *   dH = dY W2^T;  dU = dH * Swish(G);  dG = dH * U * Swish'(G)
 *   dW2 = H^T dY;  dW1 = X^T dG;  dW3 = X^T dU      (fp32)
 *   dX  = dG W1^T + dU W3^T                          (this shard's summand)
 * ws: at least tp_swiglu_bwd_workspace_bytes(dt, M, d, f) bytes.
 * ------------------------------------------------------------------------- */
int tp_swiglu_bwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
                  const void* X, const void* W1, const void* W3, const void* W2,
                  const void* G, const void* U, const void* H, const void* dY,
                  void* dX, float* dW1, float* dW3, float* dW2,
                  void* ws, size_t ws_bytes);
size_t tp_swiglu_bwd_workspace_bytes(tp_dtype_t dt, int64_t M, int64_t d, int64_t f);

/* ---------------------------------------------------------------------------
 * tp_attn_shard_fwd — head-group attention shard forward ([JY] Attention;
 * [BM] Megatron_MHA; [HC] Figure 3.5).  This shard owns h_local heads; local
 * head j uses columns [j*d_head, (j+1)*d_head) of Wq, Wk, Wv and rows
 * [j*d_head, (j+1)*d_head) of Wo.  For each batch row bi and head j:
 *   Q, K, V = X_bi W{q,k,v}[:, j]          written head-major [b, h_local, s, d_head]
 *   S[t,u]  = scale * Q_t . K_u, and -inf for u > t when causal
 *   o_j     = softmax_u(S) V              (online softmax, never stored as s x s)
 *   O       = [o_0 | ... | o_{h_local-1}] [b*s x h_local*d_head]
 *   Z       = O Wo                         this shard's partial [b*s x d]
 * X [b*s x d]; Wq, Wk, Wv [d x h_local*d_head]; Wo [h_local*d_head x d].
 *   L[bi,j,t] = log sum_u exp(S[t,u])     fp32 [b, h_local, s], natural log
 * Q, K, V, O and L are outputs (kept for inspection or the backward pass);
 * L may be NULL.
 * Supported: dt = TP_DT_BF16, d_head = 64 or 128, d a multiple of 8.
 * scale <= 0 selects 1/sqrt(d_head).  causal is 0 or 1.
 * ------------------------------------------------------------------------- */
int tp_attn_shard_fwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                      int64_t h_local, int64_t d_head, int causal, float scale,
                      const void* X, const void* Wq, const void* Wk, const void* Wv,
                      const void* Wo, void* Q, void* K, void* V, void* O, void* Z,
                      float* L);

/* ---------------------------------------------------------------------------
 * tp_attn_gqa_shard_fwd — grouped-query attention shard forward ([HC] 3.4,
 * the Llama-3 example: a GPU's query heads share its key/value heads).  As
 * tp_attn_shard_fwd, except that Wk and Wv are [d x h_kv_local*d_head], K and
 * V are [b, h_kv_local, s, d_head], and local query head j attends with
 * key/value head j / (h_local / h_kv_local).  h_kv_local must divide h_local
 * (TP_E_DIVIS); h_kv_local = h_local is tp_attn_shard_fwd.  When the K/V
 * projection is narrow and d long, its K split keeps fp32 partials in Z's
 * memory before Z itself is written (Z must be device memory of its full
 * size, as for every output).
 * ------------------------------------------------------------------------- */
int tp_attn_gqa_shard_fwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                          int64_t h_local, int64_t h_kv_local, int64_t d_head, int causal, float scale,
                          const void* X, const void* Wq, const void* Wk, const void* Wv,
                          const void* Wo, void* Q, void* K, void* V, void* O, void* Z,
                          float* L);

/* ---------------------------------------------------------------------------
 * tp_attn_shard_bwd — backward of the attention shard.  The input passes
 * [BM] Megatron_f (identity forward, all-reduce backward), so dX is this
 * shard's summand of the full dX (summed over shards by the f all-reduce,
 * [HC] 3.4); the output projection is row-parallel and g's backward is the
 * identity, so dY is the full upstream gradient [b*s x d].
 *   dO = dY Wo^T;  dWo = O^T dY
 *   per head, with P = exp(S - L) recomputed from Q, K and L:
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *     dQ = scale dS K,  dK = scale dS^T Q
 *   dX = dQ Wq^T + dK Wk^T + dV Wv^T  (dQ, dK, dV token-major like O)
 *   dWq = X^T dQ,  dWk = X^T dK,  dWv = X^T dV
 * Inputs are the forward's arguments and outputs (Q, K, V, O, L from the
 * same tp_attn_shard_fwd call).  dX is bf16 [b*s x d]; dWq, dWk, dWv
 * [d x h_local*d_head] and dWo [h_local*d_head x d] are fp32.  Supported:
 * dt = TP_DT_BF16, d_head = 128.  ws: device workspace of at least
 * tp_attn_shard_bwd_workspace_bytes(...) bytes, contents undefined on return.
 * ------------------------------------------------------------------------- */
int tp_attn_shard_bwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                      int64_t h_local, int64_t d_head, int causal, float scale,
                      const void* X, const void* Wq, const void* Wk, const void* Wv,
                      const void* Wo, const void* Q, const void* K, const void* V,
                      const void* O, const float* L, const void* dY,
                      void* dX, float* dWq, float* dWk, float* dWv, float* dWo,
                      void* ws, size_t ws_bytes);
size_t tp_attn_shard_bwd_workspace_bytes(tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                                         int64_t h_local, int64_t d_head);

/* ---------------------------------------------------------------------------
 * tp_attn_gqa_shard_bwd — backward of the grouped-query shard
 * (tp_attn_gqa_shard_fwd): tp_attn_shard_bwd's chain rule with local query
 * head j reading K/V head j / (h_local / h_kv_local).  A K/V head feeds every
 * query head of its group, so its dK and dV are the group's contributions
 * summed (in fp32, in head order).  Wk, Wv, dWk, dWv are [d x
 * h_kv_local*d_head]; K, V [b, h_kv_local, s, d_head]; everything else as
 * tp_attn_shard_bwd.  h_kv_local must divide h_local (TP_E_DIVIS); d_head =
 * 128; (h_local + 2 h_kv_local)*d_head <= 2^21.  ws: device workspace of at
 * least tp_attn_gqa_shard_bwd_workspace_bytes(...) bytes.
 * ------------------------------------------------------------------------- */
int tp_attn_gqa_shard_bwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                          int64_t h_local, int64_t h_kv_local, int64_t d_head, int causal,
                          float scale, const void* X, const void* Wq, const void* Wk,
                          const void* Wv, const void* Wo, const void* Q, const void* K,
                          const void* V, const void* O, const float* L, const void* dY,
                          void* dX, float* dWq, float* dWk, float* dWv, float* dWo,
                          void* ws, size_t ws_bytes);
size_t tp_attn_gqa_shard_bwd_workspace_bytes(tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                                             int64_t h_local, int64_t h_kv_local,
                                             int64_t d_head);

/* ---------------------------------------------------------------------------
 * tp_sp_reduce_scatter_ln — the sequence-parallel block end of one GPU ([HC]
 * 3.4, the sequence-parallelism paragraph and Figure 3.7; [BM] "Sharding
 * activations to reduce memory").  Sequence parallelism replaces g's
 * all-reduce by a reduce-scatter that sums the shards' partial outputs and
 * keeps this GPU's stripe of tokens; dropout, the residual add and the next
 * block's LayerNorm then run on that stripe only.  With k = rows / n_shards
 * and r0 = index * k (stripe `index`, as tp_shard_range), for r in [0, k):
 *   y[r]  = sum_{i=0}^{n_shards-1} partials[i*shard_stride + (r0+r)*cols + :]
 *           (+ bias, added once after the sum)
 *   y[r]  = y[r] * keep[r] / (1 - p_drop)          (only when keep != NULL)
 *   h[r]  = residual[r] + y[r]                     -> h_out  (dtype dt)
 *   x[r]  = (h[r] - mean) / sqrt(var + eps) * gamma + beta  -> x_out
 * with mean and the biased variance var over the row of h as stored in
 * h_out.  Sums and statistics in fp32, shard sum in order 0..n_shards-1.
 * partials: n_shards blocks of [rows x cols] (dtype dt), shard_stride
 * elements apart (>= rows*cols, a multiple of 8).  residual, h_out, x_out:
 * [k x cols]; keep: [k x cols] bytes, nonzero = kept (the caller draws the
 * mask: dropout's random numbers are an input); bias, gamma, beta: [cols].
 * bias and keep may be NULL.  cols must be a multiple of 8 (TP_E_DIVIS),
 * rows divisible by n_shards (TP_E_DIVIS), k <= 2^24, 0 <= p_drop < 1,
 * eps > 0.  Outputs may not overlap inputs or each other (TP_E_ALIAS).
 * ------------------------------------------------------------------------- */
int tp_sp_reduce_scatter_ln(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t rows,
                            int64_t cols, int64_t index, const void* partials,
                            int64_t shard_stride, const void* bias, const void* residual,
                            const uint8_t* keep, float p_drop, const void* gamma,
                            const void* beta, float eps, void* h_out, void* x_out);

/* ---------------------------------------------------------------------------
 * tp_sp_ln_bwd_reduce_scatter — backward of tp_sp_reduce_scatter_ln on one
 * stripe ([HC] Figure 3.7: the backward pass mirrors the forward, a
 * reduce-scatter where the forward gathered).  With k = rows / n_shards:
 *   dx[r]  = sum_i dx_partials[i*shard_stride + (index*k + r)*cols + :]
 *            (every shard's gradient of the next block's input, this stripe)
 *   dh[r]  = LayerNorm backward of dx[r] at h[r] (statistics recomputed from
 *            h as stored, biased variance, eps) + dres[r]     -> dh_out
 *   dy[r]  = dh[r] * keep[r] / (1 - p_drop)  (dh[r] when keep is NULL) -> dy_out
 *   dgamma = sum_r dx[r] * xhat[r],  dbeta = sum_r dx[r],  dbias = sum_r dy[r]
 * (fp32 [cols], this stripe's parts; summed in a fixed order).  dh_out is
 * the gradient of the previous residual stream; the all-gather of the
 * stripes' dy_out (tp_sp_all_gather) is the output gradient of every
 * shard's row-parallel product.  h, keep, dres, dh_out, dy_out: [k x cols];
 * dres and dbias may be NULL.  cols a multiple of 8 and <= 16384.  ws:
 * device workspace of tp_sp_ln_bwd_workspace_bytes(...) bytes.
 * ------------------------------------------------------------------------- */
int tp_sp_ln_bwd_reduce_scatter(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t rows,
                                int64_t cols, int64_t index, const void* dx_partials,
                                int64_t shard_stride, const void* h, const void* gamma, float eps,
                                const uint8_t* keep, float p_drop, const void* dres, void* dh_out,
                                void* dy_out, float* dgamma, float* dbeta, float* dbias, void* ws,
                                size_t ws_bytes);
size_t tp_sp_ln_bwd_workspace_bytes(tp_dtype_t dt, int64_t n_shards, int64_t rows, int64_t cols);

/* ---------------------------------------------------------------------------
 * tp_sp_all_gather — the all-gather that rebuilds the full input of the next
 * TP product from the n_shards token stripes ([HC] 3.2 collectives table and
 * Figure 3.2; 3.4, Figure 3.7):
 *   full[j*stripe_rows + r, :] = stripes[j][r, :]   for j < n_shards.
 * stripes: a HOST array of n_shards DEVICE pointers, each [stripe_rows x
 * cols] of dtype dt; full: [n_shards*stripe_rows x cols].  A stripe pointer
 * equal to its own place in full is in place and is not copied; any other
 * overlap of a stripe with full is TP_E_ALIAS.  1 <= n_shards <= 64, cols a
 * multiple of 8.  Together with tp_sp_reduce_scatter_ln's sum this is the
 * all-reduce: reduce-scatter followed by all-gather ([HC] 3.2).
 * ------------------------------------------------------------------------- */
int tp_sp_all_gather(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t stripe_rows,
                     int64_t cols, const void* const* stripes, void* full);

/* ---------------------------------------------------------------------------
 * tp_vocab_embed_fwd — one shard's partial of the vocabulary-parallel input
 * embedding ([JY] Embedding: the table is split by vocabulary rows and the
 * shards' results are all-reduced; Implementation, ParallelEmbedding).  The
 * shard holds rows [vocab_start, vocab_start + vocab_local) of the table as
 * E_local [vocab_local x d]:
 *   Y[t, :] = E_local[ids[t] - vocab_start, :]  if the id is in that range,
 *   Y[t, :] = 0                                 otherwise.
 * The embedding is the SUM of the shards' Y (tp_shard_reduce on one GPU);
 * an id outside [0, V) is in no shard and embeds as a zero row.  ids: int64
 * [n_tokens] on the device; Y: [n_tokens x d] of dtype dt.  d and
 * vocab_local multiples of 8 (TP_E_DIVIS), each <= 2^21; n_tokens <= 2^24.
 * Token-id arrays need 8-byte and per-token fp32 arrays (stats, loss, lse,
 * dloss) 4-byte alignment; tables and matrices 16 bytes.
 * ------------------------------------------------------------------------- */
int tp_vocab_embed_fwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d,
                       int64_t vocab_local, int64_t vocab_start, const int64_t* ids,
                       const void* E_local, void* Y);

/* ---------------------------------------------------------------------------
 * tp_vocab_embed_bwd — backward of tp_vocab_embed_fwd: the table gradient of
 * the shard's rows.  The forward's all-reduce has an identity backward, so
 * the shard receives the whole output gradient dY [n_tokens x d] (dtype dt):
 *   dE_local[v, :] = sum over tokens t with ids[t] == vocab_start + v of dY[t, :]
 * summed in token order (bitwise deterministic; no atomics); rows no token
 * hits are zero.  dE_local: fp32 [vocab_local x d], overwritten.  Sizes as
 * tp_vocab_embed_fwd.
 * ------------------------------------------------------------------------- */
int tp_vocab_embed_bwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d,
                       int64_t vocab_local, int64_t vocab_start, const int64_t* ids,
                       const void* dY, float* dE_local);

/* ---------------------------------------------------------------------------
 * tp_vocab_ce_fwd — one shard of the output embedding fused with the
 * cross-entropy ([JY] Embedding: fusing the loss into the output embedding
 * leaves only per-token values to exchange instead of [bs x V] logits).
 *   logits = X E_local^T                  [n_tokens x vocab_local], dtype dt
 *   stats[t] = (m, s, z_t):  m = max_v logits[t, v],
 *                            s = sum_v exp(logits[t, v] - m),
 *                            z_t = logits[t, targets[t] - vocab_start] when
 *                                  the target is one of the shard's rows, else 0
 * with the statistics taken from the logits as stored (fp32 arithmetic); in
 * the bf16 path the product's epilogue computes them as it stores the logits.
 * X: [n_tokens x d]; E_local: [vocab_local x d] (the same table slice as the
 * input embedding's); targets: int64 [n_tokens]; stats: fp32 [n_tokens x 3].
 * logits is kept for tp_vocab_ce_bwd.  ws: device workspace of
 * tp_vocab_ce_fwd_workspace_bytes(...) bytes (0 for TP_DT_F32: ws may then be
 * NULL).  Sizes as tp_vocab_embed_fwd.
 * ------------------------------------------------------------------------- */
int tp_vocab_ce_fwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d,
                    int64_t vocab_local, int64_t vocab_start, const void* X,
                    const void* E_local, const int64_t* targets, void* logits, float* stats,
                    void* ws, size_t ws_bytes);
size_t tp_vocab_ce_fwd_workspace_bytes(tp_dtype_t dt, int64_t n_tokens, int64_t d,
                                       int64_t vocab_local);

/* ---------------------------------------------------------------------------
 * tp_vocab_ce_combine — the exchange of the fused cross-entropy on one GPU:
 * the n_shards stats blocks (shard i at stats + i * shard_stride floats,
 * shard_stride >= 3 * n_tokens) are merged per token, in shard order:
 *   M = max_i m_i,  S = sum_i s_i exp(m_i - M),
 *   lse[t] = M + log S,  loss[t] = lse[t] - sum_i z_t,i.
 * A target outside [0, V) has no logit and its loss is lse.  loss, lse:
 * fp32 [n_tokens].
 * ------------------------------------------------------------------------- */
int tp_vocab_ce_combine(void* stream, int64_t n_shards, int64_t n_tokens, const float* stats,
                        int64_t shard_stride, float* loss, float* lse);

/* ---------------------------------------------------------------------------
 * tp_vocab_ce_bwd — backward of one shard of the fused output embedding and
 * cross-entropy, given lse from tp_vocab_ce_combine and dloss[t] = dL/dloss[t]
 * (fp32 [n_tokens]; a loss mask or the mean's 1/n_tokens goes here):
 *   dz = (exp(logits - lse) - onehot(targets - vocab_start)) * dloss
 *   dX = dz E_local     [n_tokens x d], dtype dt: this shard's summand of dX
 *                        (summed over shards by the backward all-reduce)
 *   dE = dz^T X          [vocab_local x d], fp32
 * logits: tp_vocab_ce_fwd's output.  ws: device workspace of at least
 * tp_vocab_ce_bwd_workspace_bytes(...) bytes, contents undefined on return.
 * ------------------------------------------------------------------------- */
int tp_vocab_ce_bwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d,
                    int64_t vocab_local, int64_t vocab_start, const void* X,
                    const void* E_local, const int64_t* targets, const void* logits,
                    const float* lse, const float* dloss, void* dX, float* dE,
                    void* ws, size_t ws_bytes);
size_t tp_vocab_ce_bwd_workspace_bytes(tp_dtype_t dt, int64_t n_tokens, int64_t d,
                                       int64_t vocab_local);

/* ---------------------------------------------------------------------------
 * tp_shard_reduce — the local stand-in for the g (forward) and f (backward)
 * all-reduce SUM of [JY] f/g table, [HC] 3.4 and [DW] 8.4.2, over the
 * partials of n_shards shards resident on this GPU:
 *   out[e] = sum_{i=0}^{n_shards-1} partials[i*shard_stride + e]
 *            (+ bias[e % bias_len], added once, after the sum: [BM]
 *             Megatron_FeedForward adds the row-parallel bias after g)
 * for e in [0, numel).  Sums in fp32 in shard order 0..n_shards-1 (bitwise
 * deterministic).  dt_in is the dtype of partials and bias, dt_out of out.
 * bias may be NULL (bias_len ignored), else bias_len > 0.
 * shard_stride >= numel (elements).  out may alias partials block 0 exactly
 * (in-place); any other overlap is TP_E_ALIAS.
 * ------------------------------------------------------------------------- */
int tp_shard_reduce(void* stream, tp_dtype_t dt_in, tp_dtype_t dt_out,
                    int64_t n_shards, int64_t numel,
                    const void* partials, int64_t shard_stride,
                    const void* bias, int64_t bias_len, void* out);

/* ---------------------------------------------------------------------------
 * Kernel-timing hook for measurement tools (no effect on results).
 * tp_profile_begin arms it on the calling thread: the i-th kernel that later
 * entry-point calls on this thread launch (i counting from 0, up to
 * `capacity`) is launched with hipExtLaunchKernelGGL so that it records the
 * caller's hipEvent_t start_events[i] before it runs and stop_events[i] after
 * it.  The events are created and owned by the caller and must belong to the
 * device the kernels run on.  tp_profile_end disarms the hook and returns the
 * number of kernels that recorded events; tp_profile_label(i) names kernel i
 * (static text such as "mlp_fwd.xw1_gelu"; "" out of range).  Launches past
 * `capacity` run untimed.  Returns TP_E_NULL / TP_E_DIM on bad arguments.
 * tp_profile_only(label) restricts the armed hook on the calling thread to
 * launches whose label equals `label` (copied): the others launch without
 * events and do not count.  NULL lifts the restriction; tp_profile_end also
 * lifts it.  Each event pair costs the launch a few microseconds, so a
 * measurement that needs one kernel's duration arms only that kernel.
 * ------------------------------------------------------------------------- */
int tp_profile_begin(void* const* start_events, void* const* stop_events, int capacity);
int tp_profile_only(const char* label);
int tp_profile_end(void);
const char* tp_profile_label(int i);

/* Human-readable text for a status code (static storage). */
const char* tp_strerror(int status);
/* Thread-local text describing the last failure on this thread ("" if none). */
const char* tp_last_error_detail(void);
/* TP_ABI_VERSION of the loaded library. */
int tp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TP_SHARD_H */
