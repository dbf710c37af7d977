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

}  // namespace tpk
