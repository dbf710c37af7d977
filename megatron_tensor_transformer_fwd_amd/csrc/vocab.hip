// Vocabulary-parallel embeddings ([JY] Embedding and Implementation).
//
// Input embedding.  Shard i holds rows [vocab_start, vocab_start + V_local)
// of the table E.  A token whose id falls in that range reads its row; every
// other token gets a zero row; the all-reduce SUM over shards (the
// shard-reduce on one GPU) then yields E[id] for every token.  HBM-bound
// gather: each 16-byte chunk of an output row is one thread's copy (or zero
// fill), so a row is written by consecutive lanes.
//
// Output embedding fused with the cross-entropy.  The shard's logits
// z = X E_local^T come from the bf16 MFMA GEMM, whose epilogue also reduces
// each output tile's rows to (max, sum exp) pairs; a small per-token kernel
// merges a row's tile pairs and reads the target's logit, giving every
// token's three numbers, m = max z, s = sum exp(z - m) and the target's logit
// when the target is one of the shard's rows.  (The fp32 path keeps a
// separate row pass.)  Only these
// 3 * n_tokens values per shard cross GPUs (the combine kernel is the
// exchange), not the [n_tokens x V] logits.  The statistics are taken from the
// logits as stored (bf16 in the bf16 path), the values the backward reads.
// Backward: dz = (exp(z - lse) - onehot(target)) dloss per row, then
// dX_i = dz E_local (this shard's summand of dX) and dE_local = dz^T X.
#include <cfloat>

#include "epilogues.hpp"
#include "gemm_dispatch.hpp"

namespace tpk {

// ----------------------------------------------------------- input embedding

// Y[t, :] = E_local[ids[t] - vstart, :] when the id is in the shard, else 0.
// `rowvec` 16-byte vectors per row.
__global__ void __launch_bounds__(256)
vocab_embed_kernel(const int64_t* __restrict__ ids, int64_t n_tokens, int64_t rowvec, int64_t vstart,
                   int64_t vlocal, const u32x4* __restrict__ E, u32x4* __restrict__ Y) {
  const int64_t total = n_tokens * rowvec;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < total; v += step) {
    const int64_t t = v / rowvec, c = v - t * rowvec;
    const int64_t local = ids[t] - vstart;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (local >= 0 && local < vlocal) w = E[local * rowvec + c];
    st16<kNtOut>(Y + v, w);
  }
}

// ---------------------------------------------------------- input embedding backward

// dE_local[v, :] = sum of dY[t, :] over the tokens t whose id is vstart + v.
// A workgroup owns EB_R table rows, so no two workgroups write the same row
// and no atomics are needed.  It scans the ids in windows of EB_W tokens and
// compacts the window's hits on its rows into LDS in token order (a
// block-wide prefix sum of per-thread hit counts).  Threads own 8 columns
// each; when a row has fewer 8-column chunks than the workgroup has
// threads, HL groups of threads ("hit lanes") take every HL-th hit, each
// keeping per-row register accumulators and issuing eight (then four) hits'
// loads at a time.  The lanes' sums are added in lane order at the end, so the
// summation order is fixed (bitwise deterministic).  Rows wider than the
// workgroup's columns take several column passes over the same windows.
constexpr int EB_R = 8, EB_NT = 256, EB_W = 4096;

template <class T>
__global__ void __launch_bounds__(EB_NT)
vocab_embed_bwd_kernel(const int64_t* __restrict__ ids, int64_t n_tokens, const T* __restrict__ dY, int64_t d,
                       int64_t vstart, int64_t vlocal, float* __restrict__ dE, int HL) {
  __shared__ int hits[EB_W];
  __shared__ int wave_base[EB_NT / 64 + 1];
  __shared__ float red[EB_NT * 8];
  constexpr int PER = EB_W / EB_NT;                // tokens per thread per window
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t v0 = vstart + (int64_t)blockIdx.x * EB_R;
  const int rows = (int)std::min<int64_t>(EB_R, vlocal - (int64_t)blockIdx.x * EB_R);
  const int cols_t = EB_NT / HL;                    // threads per hit lane
  const int hl = tid / cols_t, ct = tid % cols_t;

  for (int64_t cp = 0; cp < d; cp += (int64_t)cols_t * 8) {
    const int64_t c = cp + (int64_t)ct * 8;
    const bool mine = c < d;
    float acc[EB_R][8];
#pragma unroll
    for (int r = 0; r < EB_R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

    for (int64_t w0 = 0; w0 < n_tokens; w0 += EB_W) {
      // ordered compaction of this window's hits: entry = token * EB_R + row
      const int64_t t0 = w0 + (int64_t)tid * PER;
      int cnt = 0;
      uint32_t rowbits[PER / 8];                   // 4 bits per token: row, 0xF = no hit
#pragma unroll
      for (int j = 0; j < PER / 8; ++j) rowbits[j] = 0xFFFFFFFFu;
      // the thread's PER ids: all loads in flight before the first compare
      // (unconditional where the whole run is inside the tokens)
      int64_t idv[PER];
      if (t0 + PER <= n_tokens) {
#pragma unroll
        for (int j = 0; j < PER; ++j) idv[j] = ids[t0 + j];
      } else {
#pragma unroll
        for (int j = 0; j < PER; ++j) idv[j] = t0 + j < n_tokens ? ids[t0 + j] : v0 - 1;
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        {
          const int64_t r = idv[j] - v0;
          if (r >= 0 && r < rows) {
            rowbits[j >> 3] = (rowbits[j >> 3] & ~(0xFu << (4 * (j & 7)))) | ((uint32_t)r << (4 * (j & 7)));
            ++cnt;
          }
        }
      }
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      __syncthreads();                              // hits[] and wave_base[] free from the previous window
      if (lane == 63) wave_base[wv + 1] = incl;
      if (tid == 0) wave_base[0] = 0;
      __syncthreads();
      if (tid == 0)
        for (int k = 1; k <= EB_NT / 64; ++k) wave_base[k] += wave_base[k - 1];
      __syncthreads();
      int pos = wave_base[wv] + incl - cnt;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const uint32_t r = (rowbits[j >> 3] >> (4 * (j & 7))) & 0xFu;
        if (r != 0xFu) hits[pos++] = (int)((t0 + j - w0) * EB_R + r);
      }
      const int nh = wave_base[EB_NT / 64];
      __syncthreads();
      if (mine) {
        int k = hl;
        for (; k + 7 * HL < nh; k += 8 * HL) {      // eight hits' loads in flight
          float v[8][8];
          int rr8[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int e = hits[k + u * HL];
            rr8[u] = e % EB_R;
            Vec8<T>::template load<kNtIn>(dY + (w0 + e / EB_R) * d + c, v[u]);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int rr = 0; rr < EB_R; ++rr)
              if (rr == rr8[u]) {
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[rr][q] += v[u][q];
              }
        }
        for (; k + 3 * HL < nh; k += 4 * HL) {      // four hits' loads in flight
          float v[4][8];
          int rr4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int e = hits[k + u * HL];
            rr4[u] = e % EB_R;
            Vec8<T>::template load<kNtIn>(dY + (w0 + e / EB_R) * d + c, v[u]);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rr = 0; rr < EB_R; ++rr)
              if (rr == rr4[u]) {
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[rr][q] += v[u][q];
              }
        }
        for (; k < nh; k += HL) {
          const int e = hits[k];
          const int r = e % EB_R;
          float v[8];
          Vec8<T>::template load<kNtIn>(dY + (w0 + e / EB_R) * d + c, v);
#pragma unroll
          for (int rr = 0; rr < EB_R; ++rr)
            if (rr == r) {
#pragma unroll
              for (int q = 0; q < 8; ++q) acc[rr][q] += v[q];
            }
        }
      }
    }
    // the hit lanes' sums, added in lane order
#pragma unroll
    for (int r = 0; r < EB_R; ++r) {
      if (r >= rows) break;                         // uniform
      if (HL > 1) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) red[tid * 8 + q] = acc[r][q];
        __syncthreads();
        if (hl == 0) {
          for (int l = 1; l < HL; ++l)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[r][q] += red[(l * cols_t + ct) * 8 + q];
        }
      }
      if (hl == 0 && mine) Vec8<float>::template store<kNtOut>(dE + ((int64_t)blockIdx.x * EB_R + r) * d + c, acc[r]);
    }
    __syncthreads();
  }
}

hipError_t launch_vocab_embed_bwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                                  int64_t vstart, const int64_t* ids, const void* dY, float* dE) {
  const dim3 grid((unsigned)cdiv(vlocal, EB_R));
  const int64_t chunks = d / 8;
  const int HL = chunks >= EB_NT ? 1 : (chunks >= EB_NT / 2 ? 2 : 4);   // hit lanes
  if (dt == DT_BF16)
    return launch("vocab.embed_bwd", vocab_embed_bwd_kernel<bf16>, grid, dim3(EB_NT), st, ids, n_tokens,
                  static_cast<const bf16*>(dY), d, vstart, vlocal, dE, HL);
  return launch("vocab.embed_bwd", vocab_embed_bwd_kernel<float>, grid, dim3(EB_NT), st, ids, n_tokens,
                static_cast<const float*>(dY), d, vstart, vlocal, dE, HL);
}

// ------------------------------------------------------ cross-entropy rows

// (m, s) pairs with s = sum exp(z - m), merged without overflow.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

// One workgroup per token row of the shard's logits [n_tokens x vlocal].
template <class T>
__global__ void __launch_bounds__(256)
ce_row_stats_kernel(const T* __restrict__ logits, int64_t vlocal, const int64_t* __restrict__ targets,
                    int64_t vstart, float* __restrict__ stats) {
  __shared__ float red_m[4], red_s[4];
  const int64_t t = blockIdx.x;
  const T* row = logits + t * vlocal;
  float m = -FLT_MAX, s = 0.f;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < vlocal; c += 256 * 8) {
    float z[8];
    Vec8<T>::template load<kNtIn>(row + c, z);
    float cm = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, z[e]);
    if (cm > m) {
      s *= __expf(m - cm);
      m = cm;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s += __expf(z[e] - m);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    ms_merge(m, s, m2, s2);
  }
  if ((threadIdx.x & 63) == 0) {
    red_m[threadIdx.x >> 6] = m;
    red_s[threadIdx.x >> 6] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = red_m[0];
    s = red_s[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) ms_merge(m, s, red_m[w], red_s[w]);
    const int64_t local = targets[t] - vstart;
    const float zt = (local >= 0 && local < vlocal) ? to_f32(row[local]) : 0.f;
    stats[t * 3 + 0] = m;
    stats[t * 3 + 1] = s;
    stats[t * 3 + 2] = zt;
  }
}

// The exchange: per token, the shards' (m, s, z_t) -> log-sum-exp and loss.
// Shards are merged in order 0..n-1.
__global__ void __launch_bounds__(256)
ce_combine_kernel(const float* __restrict__ stats, int64_t shard_stride, int n, int64_t n_tokens,
                  float* __restrict__ loss, float* __restrict__ lse) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tokens) return;
  float M = -FLT_MAX;
  for (int i = 0; i < n; ++i) M = fmaxf(M, stats[i * shard_stride + t * 3]);
  float S = 0.f, zt = 0.f;
  for (int i = 0; i < n; ++i) {
    const float* p = stats + i * shard_stride + t * 3;
    S += p[1] * __expf(p[0] - M);
    zt += p[2];
  }
  const float l = M + __logf(S);
  lse[t] = l;
  loss[t] = l - zt;
}

// dz[t, v] = (exp(z[t, v] - lse[t]) - [v == target - vstart]) * dloss[t].
template <class T>
__global__ void __launch_bounds__(256)
ce_dlogits_kernel(const T* __restrict__ logits, int64_t n_tokens, int64_t vlocal,
                  const int64_t* __restrict__ targets, int64_t vstart, const float* __restrict__ lse,
                  const float* __restrict__ dloss, T* __restrict__ dz) {
  const int64_t rowvec = vlocal / 8, total = n_tokens * rowvec;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < total; v += step) {
    const int64_t t = v / rowvec, c = (v - t * rowvec) * 8;
    const float l = lse[t], g = dloss[t];
    const int64_t hit = targets[t] - vstart - c;   // in [0, 8) when the target is in this chunk
    float z[8];
    Vec8<T>::template load<kNtIn>(logits + t * vlocal + c, z);
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__expf(z[e] - l) - (hit == e ? 1.f : 0.f)) * g;
    Vec8<T>::store(dz + t * vlocal + c, z);
  }
}

// The logits product's epilogue: stores the bf16 logits and, from the
// staged tile (the values as stored), each row's max and sum of exp over the
// tile's columns, written as one (m, s) pair per (token, tile column).  The
// loss is thereby fused into the output-embedding product: the logits are
// not read back for the forward statistics.
struct EpiCeLogits {
  static constexpr int NOUT = 1;
  static constexpr bool ROW_REDUCE = true;
  template <int O> using OutT = bf16;
  bf16* C;
  int64_t ldc;
  f32x2* part;      // [M x tiles_n]
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ bf16* out_ptr(int64_t m, int64_t n, int, int) const {
    return C + m * ldc + n;
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const { return v; }
  template <int O, int NT, int PASS, int CPR, int BNL>
  __device__ __forceinline__ void row_reduce(const char* smem, int r_base, int64_t m0, int64_t n0,
                                             const GemmParams& p, int tid) const {
    constexpr int TPR = NT >= PASS ? NT / PASS : 1;     // threads per staged row
    constexpr int RPT = PASS > NT ? PASS / NT : 1;      // staged rows per thread
    const int ncv = (int)std::min<int64_t>(CPR, (p.N - n0) / 8);   // chunks of 8 valid columns
    const int part_idx = tid % TPR;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int r = tid / TPR + rr * (NT / TPR);
      float mx = -FLT_MAX, sm = 0.f;
      for (int c = part_idx; c < ncv; c += TPR) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(smem + r * (CPR * 16) + ((c ^ (r & (CPR - 1))) * 16));
        float z[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[2 * i] = bf16_lo(w[i]);
          z[2 * i + 1] = bf16_hi(w[i]);
        }
        float cm = z[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) cm = fmaxf(cm, z[e]);
        if (cm > mx) {
          sm *= __expf(mx - cm);
          mx = cm;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sm += __expf(z[e] - mx);
      }
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        const float m2 = __shfl_xor(mx, o), s2 = __shfl_xor(sm, o);
        const float M = fmaxf(mx, m2);
        sm = sm * __expf(mx - M) + s2 * __expf(m2 - M);
        mx = M;
      }
      const int64_t m = m0 + r_base + r;
      if (part_idx == 0 && m < p.M) part[m * p.tiles_n + n0 / BNL] = f32x2{mx, sm};
    }
  }
};

// Per token: the tile columns' (m, s) pairs merged in order, and the target's
// logit when the target is one of the shard's rows.
__global__ void __launch_bounds__(256)
ce_tile_stats_kernel(const f32x2* __restrict__ part, int ntn, const bf16* __restrict__ logits, int64_t vlocal,
                     const int64_t* __restrict__ targets, int64_t vstart, int64_t n_tokens,
                     float* __restrict__ stats) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tokens) return;
  float m = -FLT_MAX, s = 0.f;
  for (int j = 0; j < ntn; ++j) {
    const f32x2 q = part[t * ntn + j];
    const float M = fmaxf(m, q[0]);
    s = s * __expf(m - M) + q[1] * __expf(q[0] - M);
    m = M;
  }
  const int64_t local = targets[t] - vstart;
  stats[t * 3 + 0] = m;
  stats[t * 3 + 1] = s;
  stats[t * 3 + 2] = (local >= 0 && local < vlocal) ? to_f32(logits[t * vlocal + local]) : 0.f;
}

// ------------------------------------------------------------------ launchers

static size_t up256v(size_t x) { return (x + 255) & ~(size_t)255; }

static unsigned flat_blocks(int64_t work) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(work, 256), 256 * 16));
}

hipError_t launch_vocab_embed_fwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                                  int64_t vstart, const int64_t* ids, const void* E, void* Y) {
  const int64_t rowvec = d * (dt == DT_BF16 ? 2 : 4) / 16;
  return launch("vocab.embed", vocab_embed_kernel, dim3(flat_blocks(n_tokens * rowvec)), dim3(256), st, ids,
                n_tokens, rowvec, vstart, vlocal, static_cast<const u32x4*>(E), static_cast<u32x4*>(Y));
}

size_t vocab_ce_fwd_ws_bytes(int dt, int64_t n_tokens, int64_t vlocal) {
  return dt == DT_BF16 ? (size_t)n_tokens * (size_t)cdiv(vlocal, 128) * 8 : 0;
}

hipError_t launch_vocab_ce_fwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                               int64_t vstart, const void* X, const void* E, const int64_t* targets,
                               void* logits, float* stats, void* ws) {
  if (dt == DT_BF16) {  // z = X E^T:  B(k, n) = E[n][k]; row statistics fused into the epilogue
    GemmParams p = make_params(n_tokens, vlocal, make_seg(X, d, n_tokens * d, E, d, vlocal * d, d));
    const GemmPlan plan = plan_gemm(n_tokens, vlocal, d, false, false);
    const int ntn = (int)cdiv(vlocal, plan.cfg == CFG_L ? 256 : 128);
    f32x2* part = static_cast<f32x2*>(ws);
    EpiCeLogits e{static_cast<bf16*>(logits), vlocal, part};
    TPK_TRY((launch_gemm<true, true, false>(st, "vocab_ce.xet", p, e, plan)));
    return launch("vocab_ce.tile_stats", ce_tile_stats_kernel, dim3((unsigned)cdiv(n_tokens, 256)), dim3(256), st,
                  (const f32x2*)part, ntn, static_cast<const bf16*>(logits), vlocal, targets, vstart, n_tokens,
                  stats);
  }
  GemmParamsF32 p = make_params_f32(n_tokens, vlocal, make_seg_f32(X, d, n_tokens, E, d, vlocal, d));
  EpiStore<float> e{static_cast<float*>(logits), vlocal, 0};
  TPK_TRY((launch_gemm_f32<true, true, false>(st, "vocab_ce_f32.nt", p, e)));
  return launch("vocab_ce.row_stats", ce_row_stats_kernel<float>, dim3((unsigned)n_tokens), dim3(256), st,
                static_cast<const float*>(logits), vlocal, targets, vstart, stats);
}

hipError_t launch_vocab_ce_combine(hipStream_t st, int n, int64_t n_tokens, const float* stats,
                                   int64_t shard_stride, float* loss, float* lse) {
  return launch("vocab_ce.combine", ce_combine_kernel, dim3((unsigned)cdiv(n_tokens, 256)), dim3(256), st, stats,
                shard_stride, n, n_tokens, loss, lse);
}

struct VocabBwdPlan {
  GemmPlan dE;
  size_t dz_bytes, split_bytes;
};

static VocabBwdPlan vocab_bwd_plan(int dt, int64_t n_tokens, int64_t d, int64_t vlocal) {
  VocabBwdPlan pl;
  pl.dz_bytes = up256v((size_t)n_tokens * vlocal * (dt == DT_BF16 ? 2 : 4));
  pl.dE = dt == DT_BF16 ? plan_gemm(vlocal, d, n_tokens, false, true) : GemmPlan{CFG_S, 1};
  pl.split_bytes = pl.dE.split > 1 ? up256v((size_t)pl.dE.split * vlocal * d * 4) : 0;
  return pl;
}

size_t vocab_ce_bwd_ws_bytes(int dt, int64_t n_tokens, int64_t d, int64_t vlocal) {
  const VocabBwdPlan pl = vocab_bwd_plan(dt, n_tokens, d, vlocal);
  return pl.dz_bytes + pl.split_bytes;
}

hipError_t launch_vocab_ce_bwd(hipStream_t st, int dt, int64_t n_tokens, int64_t d, int64_t vlocal,
                               int64_t vstart, const void* X, const void* E, const int64_t* targets,
                               const void* logits, const float* lse, const float* dloss, void* dX, float* dE,
                               void* ws) {
  const VocabBwdPlan pl = vocab_bwd_plan(dt, n_tokens, d, vlocal);
  const dim3 grid(flat_blocks(n_tokens * vlocal / 8));
  if (dt == DT_BF16) {
    bf16* dz = static_cast<bf16*>(ws);
    float* split_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.dz_bytes);
    TPK_TRY(launch("vocab_ce.dlogits", ce_dlogits_kernel<bf16>, grid, dim3(256), st,
                   static_cast<const bf16*>(logits), n_tokens, vlocal, targets, vstart, lse, dloss, dz));
    {  // dX = dz E:  B(k, n) = E[k][n]
      GemmParams p = make_params(n_tokens, d, make_seg(dz, vlocal, n_tokens * vlocal, E, d, vlocal * d, vlocal));
      EpiStore<bf16> e{static_cast<bf16*>(dX), d, 0};
      TPK_TRY((launch_gemm<true, false, false>(st, "vocab_ce.dze", p, e, plan_gemm(n_tokens, d, vlocal, false, false))));
    }
    {  // dE = dz^T X:  A(m, k) = dz[k][m], B(k, n) = X[k][n]
      GemmParams p = make_params(vlocal, d, make_seg(dz, vlocal, n_tokens * vlocal, X, d, n_tokens * d, n_tokens));
      return wgrad_f32_out(st, pl.dE, vlocal, d, dE, split_ws, [&](const EpiStore<float>& e, GemmPlan g) {
        return launch_gemm<false, false, false>(st, "vocab_ce.dztx", p, e, g);
      });
    }
  }
  float* dz = static_cast<float*>(ws);
  TPK_TRY(launch("vocab_ce.dlogits", ce_dlogits_kernel<float>, grid, dim3(256), st,
                 static_cast<const float*>(logits), n_tokens, vlocal, targets, vstart, lse, dloss, dz));
  {
    GemmParamsF32 p = make_params_f32(n_tokens, d, make_seg_f32(dz, vlocal, n_tokens, E, d, d, vlocal));
    EpiStore<float> e{static_cast<float*>(dX), d, 0};
    TPK_TRY((launch_gemm_f32<true, false, false>(st, "vocab_ce_f32.nn", p, e)));
  }
  GemmParamsF32 p = make_params_f32(vlocal, d, make_seg_f32(dz, vlocal, vlocal, X, d, d, n_tokens));
  EpiStore<float> e{dE, d, 0};
  return launch_gemm_f32<false, false, false>(st, "vocab_ce_f32.tn", p, e);
}

}  // namespace tpk
