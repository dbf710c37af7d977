// Sequence-parallel form of the block boundary ([HC] 3.4 and Figure 3.7;
// [BM] "Sharding activations to reduce memory").  With sequence parallelism
// the all-reduce at g becomes a reduce-scatter that sums the shards' partial
// outputs and leaves each GPU one contiguous stripe of tokens; dropout and
// the residual add run on that stripe, then the LayerNorm that opens the
// next block, and an all-gather rebuilds the full input of the next TP
// product.  An all-reduce is a reduce-scatter followed by an all-gather
// ([HC] Figure 3.2).
//
// sp_rs_ln_kernel: one workgroup per token row of this GPU's stripe.  Pass
// one sums the row over every shard in shard order (fp32, 16-byte loads,
// eight shards' loads in flight), adds the bias once, applies inverted
// dropout with the caller's keep mask, adds the residual and stores the new
// residual stream h in the output dtype.  LayerNorm then reads h as stored
// (rounded to the output dtype): two block reductions give the mean and the
// variance around it.  Rows of up to 8192 values stay in registers between
// the passes; longer rows re-read h, each thread its own writes.
// HBM-bound: (n_shards + 1) row reads plus 2 row writes per token, and the
// keep mask at one byte per value when dropout is on; the streamed rows use
// nontemporal accesses (bias, gamma and beta, shared by every row, do not).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace tpk {

constexpr int SP_NT = 256;        // threads per row
constexpr int SP_REG_CHUNKS = 4;  // 8-value chunks per thread kept in registers

__device__ __forceinline__ float round_to(float v, bf16*) { return (float)(bf16)v; }
__device__ __forceinline__ float round_to(float v, float*) { return v; }

__device__ __forceinline__ float sp_block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();  // red[] is free from its previous use
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Calls f(k, c) for this thread's chunks: c is the first column of chunk k.
// With REG the chunk loop is unrolled so that k indexes registers.
template <bool REG, class F>
__device__ __forceinline__ void sp_for_chunks(int64_t cols, F&& f) {
  if constexpr (REG) {
#pragma unroll
    for (int k = 0; k < SP_REG_CHUNKS; ++k) {
      const int64_t c = (int64_t)threadIdx.x * 8 + (int64_t)k * SP_NT * 8;
      if (c < cols) f(k, c);
    }
  } else {
    for (int64_t c = (int64_t)threadIdx.x * 8; c < cols; c += SP_NT * 8) f(0, c);
  }
}

template <class T, bool REG>
__global__ void __launch_bounds__(SP_NT)
sp_rs_ln_kernel(const T* __restrict__ P, int64_t stride, int n, int64_t row0, int64_t cols,
                const T* __restrict__ bias, const T* __restrict__ residual,
                const uint8_t* __restrict__ keep, float keep_scale,
                const T* __restrict__ gamma, const T* __restrict__ beta, float eps,
                T* __restrict__ h_out, T* __restrict__ x_out) {
  __shared__ float red[4];
  const int64_t src = (row0 + blockIdx.x) * cols;  // this row in every shard's partial
  const int64_t dst = (int64_t)blockIdx.x * cols;   // this row in the stripe buffers
  float hv[REG ? SP_REG_CHUNKS : 1][8];
  float sum = 0.f;

  sp_for_chunks<REG>(cols, [&](int k, int64_t c) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const T* p = P + src + c;
    int i = 0;
    for (; i + 8 <= n; i += 8) {
      float t[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) Vec8<T>::template load<kNtIn>(p + (int64_t)(i + u) * stride, t[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += t[u][e];
    }
    for (; i < n; ++i) {
      float t[8];
      Vec8<T>::template load<kNtIn>(p + (int64_t)i * stride, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += t[e];
    }
    if (bias) {
      float b[8];
      Vec8<T>::load(bias + c, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += b[e];
    }
    if (keep) {
      const u32x2 m = ld16<kNtIn>(reinterpret_cast<const u32x2*>(keep + dst + c));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t byte = (m[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        s[e] = byte ? s[e] * keep_scale : 0.f;
      }
    }
    float res[8];
    Vec8<T>::template load<kNtIn>(residual + dst + c, res);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] = round_to(s[e] + res[e], (T*)nullptr);
      sum += s[e];
    }
    Vec8<T>::template store<REG && kNtOut>(h_out + dst + c, s);   // re-read below when !REG
    if constexpr (REG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[k][e] = s[e];
    }
  });

  auto row_chunk = [&](int k, int64_t c, float* h) {
    if constexpr (REG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = hv[k][e];
    } else {
      Vec8<T>::load(h_out + dst + c, h);
    }
  };

  const float mean = sp_block_sum(sum, red) / (float)cols;
  float sq = 0.f;
  sp_for_chunks<REG>(cols, [&](int k, int64_t c) {
    float h[8];
    row_chunk(k, c, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += (h[e] - mean) * (h[e] - mean);
  });
  const float rstd = rsqrtf(sp_block_sum(sq, red) / (float)cols + eps);

  sp_for_chunks<REG>(cols, [&](int k, int64_t c) {
    float h[8], g[8], b[8], x[8];
    row_chunk(k, c, h);
    Vec8<T>::load(gamma + c, g);
    Vec8<T>::load(beta + c, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (h[e] - mean) * rstd * g[e] + b[e];
    Vec8<T>::template store<kNtOut>(x_out + dst + c, x);
  });
}

// All-gather on one GPU: block row j of `full` becomes a copy of stripe j
// (a NULL entry is a stripe already in place).
struct SpStripes {
  const void* p[kSpMaxShards];
};

__global__ void __launch_bounds__(256)
sp_all_gather_kernel(SpStripes s, int64_t nvec, u32x4* __restrict__ full) {
  const u32x4* src = static_cast<const u32x4*>(s.p[blockIdx.y]);
  if (!src) return;  // the stripe already sits at its place in `full`
  u32x4* dst = full + (int64_t)blockIdx.y * nvec;
  const int64_t step = (int64_t)gridDim.x * 256;
  // Streaming reads; ordinary stores, since the next TP product reads the
  // gathered tensor right away and finds it in the Infinity Cache.
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += step)
    st16<false>(dst + v, ld16<kNtIn>(src + v));
}

hipError_t launch_sp_reduce_scatter_ln(hipStream_t st, int dt, int n, int64_t rows, int64_t cols,
                                       int64_t index, const void* P, int64_t stride, const void* bias,
                                       const void* residual, const uint8_t* keep, float p_drop,
                                       const void* gamma, const void* beta, float eps, void* h_out,
                                       void* x_out) {
  const int64_t k = rows / n;
  const float ks = keep ? 1.0f / (1.0f - p_drop) : 1.0f;
  const bool reg = cols <= (int64_t)SP_NT * 8 * SP_REG_CHUNKS;
  auto go = [&](auto kern, auto* tag) {
    using T = std::remove_pointer_t<decltype(tag)>;
    return launch("sp.rs_ln", kern, dim3((unsigned)k), dim3(SP_NT), st, static_cast<const T*>(P), stride, n,
                  index * k, cols, static_cast<const T*>(bias), static_cast<const T*>(residual), keep, ks,
                  static_cast<const T*>(gamma), static_cast<const T*>(beta), eps, static_cast<T*>(h_out),
                  static_cast<T*>(x_out));
  };
  if (dt == DT_BF16)
    return reg ? go(sp_rs_ln_kernel<bf16, true>, (bf16*)nullptr) : go(sp_rs_ln_kernel<bf16, false>, (bf16*)nullptr);
  return reg ? go(sp_rs_ln_kernel<float, true>, (float*)nullptr) : go(sp_rs_ln_kernel<float, false>, (float*)nullptr);
}

hipError_t launch_sp_all_gather(hipStream_t st, int dt, int n, int64_t stripe_rows, int64_t cols,
                                const void* const* stripes, void* full) {
  SpStripes s{};
  for (int j = 0; j < n; ++j) s.p[j] = stripes[j];
  const int64_t nvec = stripe_rows * cols * (dt == DT_BF16 ? 2 : 4) / 16;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((nvec + 255) / 256, 2048 / n + 1));
  return launch("sp.all_gather", sp_all_gather_kernel, dim3((unsigned)blocks, (unsigned)n), dim3(256), st, s, nvec,
                static_cast<u32x4*>(full));
}

// ---------------------------------------------------------------------------
// Backward of the block end on one stripe ([HC] Figure 3.7: the backward
// mirrors the forward, a reduce-scatter where the forward gathered).  dx is
// the stripe of the sum of every shard's gradient of the next block's input;
// LayerNorm's backward (statistics recomputed from h as stored) plus the
// gradient arriving on h through the skip path gives dh, the previous
// residual stream's gradient; dropout's backward gives dy, the gradient of
// the reduce-scattered sum, which the all-gather hands to every shard's
// row-parallel product.  R rows per workgroup; each thread owns CH 8-column
// chunks of a row and accumulates its columns' gamma, beta and bias
// gradients over the workgroup's rows; a second kernel sums the workgroups'
// partials in order (deterministic, no atomics).
template <int NW>
__device__ __forceinline__ f32x2 sp_block_sum2(float a, float b, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  __syncthreads();  // red[] is free from its previous use
  if ((threadIdx.x & 63) == 0) {
    red[2 * (threadIdx.x >> 6)] = a;
    red[2 * (threadIdx.x >> 6) + 1] = b;
  }
  __syncthreads();
  f32x2 t = {0.f, 0.f};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    t[0] += red[2 * w];
    t[1] += red[2 * w + 1];
  }
  return t;
}

template <class T, int NTH, int CH>
__global__ void __launch_bounds__(NTH)
sp_ln_bwd_kernel(const T* __restrict__ P, int64_t stride, int n, int64_t row0, int64_t cols, int64_t k_rows,
                 int R, const T* __restrict__ h, const T* __restrict__ gamma, float eps,
                 const uint8_t* __restrict__ keep, float keep_scale, const T* __restrict__ dres,
                 T* __restrict__ dh_out, T* __restrict__ dy_out, float* __restrict__ part) {
  constexpr int NW = NTH / 64;
  __shared__ float red[2 * NW];
  float agam[CH][8], abet[CH][8], abias[CH][8];
#pragma unroll
  for (int k = 0; k < CH; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) agam[k][e] = abet[k][e] = abias[k][e] = 0.f;
  const float inv_cols = 1.0f / (float)cols;
  // With two chunks per thread (rows up to 8192 values) gamma is read once
  // per workgroup and a row's residual gradient and mask loads go out with
  // its partials', although they are used only after the row's three
  // reductions.  With four chunks the registers are not there (the fp32
  // variant would spill), and they are read where they are used.
  constexpr bool EARLY = CH <= 2;
  float gam[EARLY ? CH : 1][8];
  if constexpr (EARLY) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t c = ((int64_t)k * NTH + threadIdx.x) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[k][e] = 0.f;
      if (c < cols) Vec8<T>::load(gamma + c, gam[k]);
    }
  }

  for (int rr = 0; rr < R; ++rr) {
    const int64_t r = (int64_t)blockIdx.x * R + rr;
    if (r >= k_rows) break;                          // uniform over the workgroup
    const int64_t src = (row0 + r) * cols, dst = r * cols;
    float dx[CH][8], hv[CH][8], dr[EARLY ? CH : 1][8];
    u32x2 km[EARLY ? CH : 1];
    float hsum = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t c = ((int64_t)k * NTH + threadIdx.x) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) dx[k][e] = hv[k][e] = 0.f;
      if constexpr (EARLY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dr[k][e] = 0.f;
        km[k] = u32x2{0x01010101u, 0x01010101u};
        if (c < cols) {
          if (dres) Vec8<T>::template load<kNtIn>(dres + dst + c, dr[k]);
          if (keep) km[k] = ld16<kNtIn>(reinterpret_cast<const u32x2*>(keep + dst + c));
        }
      }
      if (c < cols) {
        const T* p = P + src + c;
        constexpr int SB = sizeof(T) == 2 ? 8 : 4;      // shards' loads in flight
        int i = 0;
        for (; i + SB <= n; i += SB) {
          float t[SB][8];
#pragma unroll
          for (int u = 0; u < SB; ++u) Vec8<T>::template load<kNtIn>(p + (int64_t)(i + u) * stride, t[u]);
#pragma unroll
          for (int u = 0; u < SB; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) dx[k][e] += t[u][e];
        }
        for (; i < n; ++i) {
          float t[8];
          Vec8<T>::template load<kNtIn>(p + (int64_t)i * stride, t);
#pragma unroll
          for (int e = 0; e < 8; ++e) dx[k][e] += t[e];
        }
        Vec8<T>::template load<kNtIn>(h + dst + c, hv[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) hsum += hv[k][e];
      }
    }
    const float mean = sp_block_sum2<NW>(hsum, 0.f, red)[0] * inv_cols;
    float sq = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t c = ((int64_t)k * NTH + threadIdx.x) * 8;
      if (c < cols) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sq += (hv[k][e] - mean) * (hv[k][e] - mean);
      }
    }
    const float rstd = rsqrtf(sp_block_sum2<NW>(sq, 0.f, red)[0] * inv_cols + eps);
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t c = ((int64_t)k * NTH + threadIdx.x) * 8;
      if (c < cols) {
        float g[8];
        if constexpr (EARLY) {
#pragma unroll
          for (int e = 0; e < 8; ++e) g[e] = gam[k][e];
        } else {
          Vec8<T>::load(gamma + c, g);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (hv[k][e] - mean) * rstd;
          const float gx = dx[k][e] * g[e];
          s1 += gx;
          s2 += gx * xh;
        }
      }
    }
    const f32x2 s12 = sp_block_sum2<NW>(s1, s2, red);
    const float m1 = s12[0] * inv_cols, m2 = s12[1] * inv_cols;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t c = ((int64_t)k * NTH + threadIdx.x) * 8;
      if (c < cols) {
        float g[8], r8[8], dh[8], dy[8];
        u32x2 m = {0x01010101u, 0x01010101u};
        if constexpr (EARLY) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            g[e] = gam[k][e];
            r8[e] = dr[k][e];
          }
          m = km[k];
        } else {
          Vec8<T>::load(gamma + c, g);
          if (dres) Vec8<T>::template load<kNtIn>(dres + dst + c, r8);
          if (keep) m = ld16<kNtIn>(reinterpret_cast<const u32x2*>(keep + dst + c));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (hv[k][e] - mean) * rstd;
          dh[e] = rstd * (dx[k][e] * g[e] - m1 - xh * m2) + (dres ? r8[e] : 0.f);
          const uint32_t byte = (m[e >> 2] >> (8 * (e & 3))) & 0xFFu;
          dy[e] = keep ? (byte ? dh[e] * keep_scale : 0.f) : dh[e];
          agam[k][e] += dx[k][e] * xh;
          abet[k][e] += dx[k][e];
          abias[k][e] += dy[e];
        }
        Vec8<T>::template store<kNtOut>(dh_out + dst + c, dh);
        Vec8<T>::template store<kNtOut>(dy_out + dst + c, dy);
      }
    }
  }
  float* pb = part + (int64_t)blockIdx.x * 3 * cols;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = ((int64_t)k * NTH + threadIdx.x) * 8;
    if (c < cols) {
      Vec8<float>::store(pb + c, agam[k]);
      Vec8<float>::store(pb + cols + c, abet[k]);
      Vec8<float>::store(pb + 2 * cols + c, abias[k]);
    }
  }
}

// dgamma, dbeta, dbias: the workgroups' partials summed in a fixed order.  A
// workgroup covers 32 consecutive entries of [dgamma | dbeta | dbias]; its 8
// thread rows each sum the partials of workgroups j, j + 8, j + 16, ..., and
// the 8 row sums are then added in row order.
__global__ void __launch_bounds__(256)
sp_param_grad_kernel(const float* __restrict__ part, int nblocks, int64_t cols, float* __restrict__ dgamma,
                     float* __restrict__ dbeta, float* __restrict__ dbias) {
  __shared__ float red[8][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t i = (int64_t)blockIdx.x * 32 + tx;   // entry of [dgamma | dbeta | dbias]
  const bool live = i < 3 * cols;
  const int q = live ? (int)(i / cols) : 0;
  const int64_t c = live ? i % cols : 0;
  float acc = 0.f;
  if (live) {
    const float* src = part + (int64_t)q * cols + c;
    const int64_t bstride = 3 * cols;
    int b = ty;
    for (; b + 24 < nblocks; b += 32) {              // four loads in flight
      const float v0 = src[(int64_t)b * bstride], v1 = src[(int64_t)(b + 8) * bstride];
      const float v2 = src[(int64_t)(b + 16) * bstride], v3 = src[(int64_t)(b + 24) * bstride];
      acc += v0;
      acc += v1;
      acc += v2;
      acc += v3;
    }
    for (; b < nblocks; b += 8) acc += src[(int64_t)b * bstride];
  }
  red[ty][tx] = acc;
  __syncthreads();
  if (ty == 0 && live) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) t += red[r][tx];
    float* out = q == 0 ? dgamma : (q == 1 ? dbeta : dbias);
    if (out) out[c] = t;
  }
}

static int sp_bwd_rows_per_block(int64_t k_rows) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(16, k_rows / 256));
}

size_t sp_ln_bwd_ws_bytes(int64_t rows, int64_t cols, int n) {
  const int64_t k = rows / n;
  const int R = sp_bwd_rows_per_block(k);
  return (size_t)((k + R - 1) / R) * 3 * (size_t)cols * 4;
}

hipError_t launch_sp_ln_bwd(hipStream_t st, int dt, int n, int64_t rows, int64_t cols, int64_t index,
                            const void* P, int64_t stride, const void* h, const void* gamma, float eps,
                            const uint8_t* keep, float p_drop, const void* dres, void* dh_out, void* dy_out,
                            float* dgamma, float* dbeta, float* dbias, void* ws) {
  const int64_t k = rows / n;
  const int R = sp_bwd_rows_per_block(k);
  const int nblocks = (int)((k + R - 1) / R);
  const float ks = keep ? 1.0f / (1.0f - p_drop) : 1.0f;
  float* part = static_cast<float*>(ws);
  const bool wide = cols > 512 * 8 * 2;              // 512 threads x 2 chunks up to 8192 values, else x 4
  auto go = [&](auto kern, int nth, auto* tag) {
    using T = std::remove_pointer_t<decltype(tag)>;
    return launch("sp.ln_bwd", kern, dim3((unsigned)nblocks), dim3(nth), st, static_cast<const T*>(P), stride, n,
                  index * k, cols, k, R, static_cast<const T*>(h), static_cast<const T*>(gamma), eps, keep, ks,
                  static_cast<const T*>(dres), static_cast<T*>(dh_out), static_cast<T*>(dy_out), part);
  };
  hipError_t e;
  if (dt == DT_BF16)
    e = wide ? go(sp_ln_bwd_kernel<bf16, 512, 4>, 512, (bf16*)nullptr) : go(sp_ln_bwd_kernel<bf16, 512, 2>, 512, (bf16*)nullptr);
  else
    e = wide ? go(sp_ln_bwd_kernel<float, 512, 4>, 512, (float*)nullptr) : go(sp_ln_bwd_kernel<float, 512, 2>, 512, (float*)nullptr);
  if (e != hipSuccess) return e;
  return launch("sp.param_grad", sp_param_grad_kernel, dim3((unsigned)((3 * cols + 31) / 32)), dim3(256), st,
                (const float*)part, nblocks, cols, dgamma, dbeta, dbias);
}

}  // namespace tpk
