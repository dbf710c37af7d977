// Head-group attention shard ([JY] Attention: o_i = softmax(Q_i K_i^T / sqrt(d_h)) V_i,
// O = [o_1..o_h] W_O; [BM] Megatron_MHA: Q/K/V column-parallel by heads,
// causal softmax local to the shard, row-parallel output projection;
// [HC] Figure 3.5: a contiguous group of heads per GPU).
//
// Three launches: (1) the Q/K/V projection, one batched MFMA product whose
// epilogue scatters straight into head-major [b, h_local, s, d_head];
// (2) a fused causal attention core; (3) the output projection, a plain
// MFMA product giving this shard's partial Z.
//
// Attention core, per workgroup: one (batch, head, 128-query tile), four
// waves of 32 queries.  Key/value tiles of 64 stream through double-buffered
// LDS (K as rows of d_head, V transposed to rows of keys so both products
// read 16-byte k-packed fragments).  A wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, so each lane owns one query column and 32 of the
// tile's keys: the row max and row sum need only one cross-lane exchange
// (lane l with lane l^32).  The running max/sum rescale the fp32 O^T
// accumulator (online softmax); P is packed to bf16 straight from the S^T
// registers and multiplied with V^T in the same key order, so the s x s
// matrix never leaves registers.  The causal mask keeps key u <= query t;
// tiles entirely above a wave's diagonal are skipped; the heaviest query
// tiles are dispatched first.
#include "epilogues.hpp"
#include "gemm_dispatch.hpp"
#include "stage_regs.hpp"

namespace tpk {

template <int D>
__global__ void __launch_bounds__(256)
flash_attn_fwd_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                      const bf16* __restrict__ V, bf16* __restrict__ O,
                      int nb, int hl, int s, int causal, float scale_log2) {
  constexpr int BQ = 128, BKV = 64, NT = 256;
  constexpr int LDK = D + 8;     // K tile: BKV rows of D
  constexpr int LDV = BKV + 8;   // V^T tile: D rows of BKV
  constexpr int STAGE = BKV * LDK + D * LDV;
  using KStage = KMajorStage<BKV, D, NT, LDK>;
  using VStage = MNMajorStage<D, BKV, NT, LDV>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int nqt = (s + BQ - 1) / BQ;
  const int nbh = nb * hl;
  const int qt = nqt - 1 - (int)(blockIdx.x / nbh);   // heaviest tiles first
  const int bh = (int)(blockIdx.x % nbh);
  const int bi = bh / hl, h = bh % hl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, g = lane >> 5;
  const int64_t head = (int64_t)bh * s * D;
  const bf16* Qh = Q + head;
  const bf16* Kh = K + head;
  const bf16* Vh = V + head;
  const int q0 = qt * BQ;
  const int qw = q0 + w * 32;       // first query of this wave
  const int qme = qw + lq;          // this lane's query

  bf16x8 qf[D / 16];
  {
    const rsrc_t rq = make_rsrc(Qh, (uint64_t)s * D * 2);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(((int64_t)qme * D + kk * 16 + g * 8) * 2)));
  }

  const int kv_end = causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;

  KStage sk;
  VStage sv;
  auto load_kv = [&](int t) {
    const int64_t kv0 = (int64_t)t * BKV;
    const uint64_t rem = (uint64_t)(s - kv0) * D * 2;
    sk.load(make_rsrc(Kh + kv0 * D, rem), D * 2, D, tid);
    sv.load(make_rsrc(Vh + kv0 * D, rem), D * 2, tid);
  };
  auto store_kv = [&](int buf) {
    bf16* Ks = smem + buf * STAGE;
    sk.store(Ks, tid);
    sv.store(Ks + BKV * LDK, tid);
  };

  f32x16 acc_o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc_o[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  load_kv(0);
  store_kv(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_kv(t + 1);

    const int kv0 = t * BKV;
    if (!(causal && kv0 > qw + 31)) {
      const bf16* Ks = smem + buf * STAGE;
      const bf16* Vs = Ks + BKV * LDK;
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + lq) * LDK + kk * 16 + g * 8);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sc[kb], 0, 0, 0);
        }
      }
      // sc[kb][r] is the score of query qme against key kv0 + kb*32 + 8*(r/4) + 4*g + r%4
      const bool need_mask = (causal && kv0 + BKV - 1 > qw) || (kv0 + BKV > s);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[kb][r] * scale_log2;
          if (need_mask) {
            const int kv = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if ((causal && kv > qme) || kv >= s) x = -INFINITY;
          }
          sc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sc[kb][r] - m_new);
          sc[kb][r] = pv;
          rs += pv;
        }
      rs += __shfl_xor(rs, 32);
      l_run = l_run * corr + rs;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc_o[i] *= corr;

      bf16x8 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 wv;
#pragma unroll
          for (int e = 0; e < 4; ++e) wv[e] = pack_bf16x2(sc[kb][8 * hh + 2 * e], sc[kb][8 * hh + 2 * e + 1]);
          pf[kb][hh] = __builtin_bit_cast(bf16x8, wv);
        }
      // O^T[d][q] += V^T[d][kv] P^T[kv][q] with the keys of pf[kb][hh]:
      // kv0 + kb*32 + 16*hh + {4g..4g+3, 8+4g..8+4g+3}
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const bf16* vr = Vs + (db * 32 + lq) * LDV + kb * 32 + hh * 16 + 4 * g;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
            const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
            acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[kb][hh],
                                                                acc_o[db], 0, 0, 0);
          }
    }
    if (more) store_kv(buf ^ 1);
    __syncthreads();
  }

  if (qme < s) {
    const float inv = 1.0f / l_run;
    bf16* orow = O + ((int64_t)bi * s + qme) * ((int64_t)hl * D) + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const f32x4 v = {acc_o[db][4 * b4] * inv, acc_o[db][4 * b4 + 1] * inv,
                         acc_o[db][4 * b4 + 2] * inv, acc_o[db][4 * b4 + 3] * inv};
        Quad<bf16>::store(orow + db * 32 + 8 * b4 + 4 * g, v);
      }
  }
}

hipError_t launch_attn_fwd(hipStream_t st, int64_t b, int64_t s, int64_t d, int64_t h_local,
                           int64_t d_head, int causal, float scale,
                           const void* X, const void* Wq, const void* Wk, const void* Wv,
                           const void* Wo, void* Q, void* K, void* V, void* O, void* Z) {
  const int64_t M = b * s, N = h_local * d_head;
  {  // Q, K, V = X W{q,k,v}, scattered to [b, h_local, s, d_head]
    GemmParams p = make_params(M, N, make_seg(X, d, M * d, Wq, N, d * N, d));
    p.Bz[0] = static_cast<const bf16*>(Wq);
    p.Bz[1] = static_cast<const bf16*>(Wk);
    p.Bz[2] = static_cast<const bf16*>(Wv);
    EpiHeadScatter<bf16> e{{static_cast<bf16*>(Q), static_cast<bf16*>(K), static_cast<bf16*>(V)},
                           (int)s, (int)h_local, (int)d_head};
    TPK_TRY((launch_gemm<true, false, false>(st, "attn.x_wqkv_scatter", p, e, plan_gemm(M, 3 * N, d, false, false), 3)));
  }
  {
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d_head);
    const float sl2 = sc * 1.4426950408889634f;
    const int64_t nqt = (s + 127) / 128;
    const dim3 grid((unsigned)(nqt * b * h_local));
    const bf16* q = static_cast<const bf16*>(Q);
    const bf16* k = static_cast<const bf16*>(K);
    const bf16* v = static_cast<const bf16*>(V);
    bf16* o = static_cast<bf16*>(O);
    if (d_head == 128)
      TPK_TRY(launch("attn.core_d128", flash_attn_fwd_kernel<128>, grid, dim3(256), st, q, k, v, o, (int)b,
                     (int)h_local, (int)s, causal, sl2));
    else
      TPK_TRY(launch("attn.core_d64", flash_attn_fwd_kernel<64>, grid, dim3(256), st, q, k, v, o, (int)b,
                     (int)h_local, (int)s, causal, sl2));
  }
  {  // Z = O Wo (this shard's partial)
    GemmParams p = make_params(M, d, make_seg(O, N, M * N, Wo, d, N * d, N));
    EpiStore<bf16> e{static_cast<bf16*>(Z), d, 0};
    TPK_TRY((launch_gemm<true, false, false>(st, "attn.o_wo", p, e, plan_gemm(M, d, N, false, false))));
  }
  return hipSuccess;
}

}  // namespace tpk
