// Local shard-reduce: the on-GPU stand-in for the all-reduce SUM that g
// performs on the partial outputs in the forward pass and f on the dX
// summands in the backward pass ([JY] f/g table; [HC] 3.4, Z = sum_k Z_k;
// [DW] 8.4.2 all_reduce SUM).  HBM-bound: each thread owns 8 consecutive
// elements, reads them from every shard with 16-byte loads (all shards'
// loads in flight before the first add), sums in fp32 in shard order, adds
// the optional bias once ([BM] Megatron_FeedForward adds it after g) and
// writes 8 outputs with one or two 16-byte stores.  Partials are read and
// the result written with streaming (nontemporal) accesses: each byte is
// touched once, and ordinary accesses run at about half the HBM rate when
// the caches hold the producing products' dirty lines.
#include "common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace tpk {

// Vector path: numel_vec chunks of 8 elements; every shard base and the
// output are 16-byte aligned.  `out` may be partials block 0: each element is
// read by the thread that writes it, before the write.
template <class Tin, class Tout>
__global__ void __launch_bounds__(256)
shard_reduce_vec8(const Tin* P, int64_t stride, int n, int64_t nvec,
                  const Tin* bias, int64_t bias_len, Tout* out) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += step) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const Tin* p = P + v * 8;
    int i = 0;
    for (; i + 8 <= n; i += 8) {     // eight shards' loads in flight at once
      float t[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) Vec8<Tin>::template load<kNtIn>(p + (int64_t)(i + u) * stride, t[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += t[u][e];
    }
    for (; i < n; ++i) {
      float t[8];
      Vec8<Tin>::template load<kNtIn>(p + (int64_t)i * stride, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += t[e];
    }
    if (bias) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += to_f32(bias[(v * 8 + e) % bias_len]);
    }
    Vec8<Tout>::template store<kNtOut>(out + v * 8, s);
  }
}

// Scalar path for tails and for strides that break 16-byte alignment.
template <class Tin, class Tout>
__global__ void __launch_bounds__(256)
shard_reduce_scalar(const Tin* P, int64_t stride, int n, int64_t begin, int64_t numel,
                    const Tin* bias, int64_t bias_len, Tout* out) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < numel; e += step) {
    float s = 0.f;
    for (int i = 0; i < n; ++i) s += to_f32(P[(int64_t)i * stride + e]);
    if (bias) s += to_f32(bias[e % bias_len]);
    out[e] = (Tout)s;
  }
}

template <class Tin, class Tout>
static hipError_t reduce_impl(hipStream_t st, int n, int64_t numel, const void* P, int64_t stride,
                              const void* bias, int64_t bias_len, void* out) {
  const Tin* p = static_cast<const Tin*>(P);
  const Tin* b = static_cast<const Tin*>(bias);
  Tout* o = static_cast<Tout*>(out);
  const bool vec_ok = (stride % 8) == 0;   // base and out are 16-byte aligned (checked by the ABI)
  int64_t done = 0;
  if (vec_ok) {
    const int64_t nvec = numel / 8;
    if (nvec > 0) {
      const int64_t blocks = std::min<int64_t>((nvec + 255) / 256, 256 * 16);
      const hipError_t e = launch("shard_reduce.vec8", shard_reduce_vec8<Tin, Tout>, dim3((unsigned)blocks),
                                  dim3(256), st, p, stride, n, nvec, b, bias_len, o);
      if (e != hipSuccess) return e;
    }
    done = nvec * 8;
  }
  if (done < numel) {
    const int64_t rem = numel - done;
    const int64_t blocks = std::min<int64_t>((rem + 255) / 256, 256 * 16);
    return launch("shard_reduce.scalar", shard_reduce_scalar<Tin, Tout>, dim3((unsigned)blocks), dim3(256), st,
                  p, stride, n, done, numel, b, bias_len, o);
  }
  return hipSuccess;
}

hipError_t launch_shard_reduce(hipStream_t st, int dt_in, int dt_out, int n, int64_t numel,
                               const void* P, int64_t stride, const void* bias, int64_t bias_len,
                               void* out) {
  if (dt_in == DT_BF16 && dt_out == DT_BF16) return reduce_impl<bf16, bf16>(st, n, numel, P, stride, bias, bias_len, out);
  if (dt_in == DT_BF16 && dt_out == DT_F32) return reduce_impl<bf16, float>(st, n, numel, P, stride, bias, bias_len, out);
  if (dt_in == DT_F32 && dt_out == DT_BF16) return reduce_impl<float, bf16>(st, n, numel, P, stride, bias, bias_len, out);
  return reduce_impl<float, float>(st, n, numel, P, stride, bias, bias_len, out);
}

}  // namespace tpk
