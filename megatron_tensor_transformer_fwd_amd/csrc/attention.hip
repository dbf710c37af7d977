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
// LDS.  A wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each
// lane owns one query column and 32 of the tile's keys: the row max and row
// sum need only one cross-lane exchange (lane l with lane l^32).  The running
// max/sum rescale the fp32 O^T accumulator (online softmax); P is packed to
// bf16 straight from the S^T registers and multiplied with V^T in the same
// key order, so the s x s matrix never leaves registers.  The causal mask
// keeps key u <= query t; tiles entirely above a wave's diagonal are skipped;
// the heaviest query tiles are dispatched first.
//
// d_head 128 (the workloads' head size): K and V arrive by LDS DMA in their
// natural row-major layout (K rows of 256 bytes with an XOR chunk swizzle, V
// as [keys][d] rows read back transposed with ds_read_b64_tr_b16 in the key
// order the P registers hold), no staging registers or register transposes;
// at most 256 registers per wave, so two waves share each SIMD (two 4-wave
// workgroups per CU, or one 8-wave workgroup holding two query heads of a
// group) and one wave's softmax overlaps another's matrix products.  Within a
// wave the loop is software-pipelined: the next key tile's score MFMAs are issued
// before this tile's softmax, so both kinds of work are in flight (K and V
// have separate two-stage LDS rings for that).  The subtracted running max
// may lag a row's true max by up to 2^8, so O^T and the sum are rescaled only
// when a row of the wave moves past that (not each time a max moves, which
// with random scores is nearly every tile).  d_head 64 uses the
// register-staged variant.
#include "epilogues.hpp"
#include "gemm_dispatch.hpp"
#include "stage_regs.hpp"

namespace tpk {

template <int D>
__global__ void __launch_bounds__(256)
flash_attn_fwd_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                      const bf16* __restrict__ V, bf16* __restrict__ O, float* __restrict__ L,
                      int nb, int hl, int group, int s, int causal, float scale_log2) {
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
  // grouped-query attention: query head h reads key/value head h / group
  const int64_t kvhead = ((int64_t)bi * (hl / group) + h / group) * s * D;
  const bf16* Qh = Q + head;
  const bf16* Kh = K + kvhead;
  const bf16* Vh = V + kvhead;
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
    // log-sum-exp of the query's scaled scores, natural log (m_run is in log2 units)
    if (L && g == 0) L[(int64_t)bh * s + qme] = (m_run + __log2f(l_run)) * 0.69314718055994531f;
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

// ----------------------------------------------------------------------------
// d_head = 128 core with LDS-DMA staging.
// ----------------------------------------------------------------------------
namespace attn128 {
constexpr int D = 128, BQ = 128, BKV = 64, NT = 256, NW = 4;
constexpr int K_BYTES = BKV * D * 2, V_BYTES = BKV * D * 2;
constexpr int NK = K_BYTES / 1024 / NW, NV = V_BYTES / 1024 / NW;   // DMA instructions per wave
constexpr float kLazyMax = 8.0f;                  // lag allowed to the subtracted running max, log2 units
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kBf16One2 = {(__bf16)1.0f, (__bf16)1.0f};

// K tile: row r (key) of 256 bytes, logical 16-byte chunk c at c ^ (r % 16).
// V tile: row r (key) of 256 bytes (128 d values), chunk c at c ^ 4 (r & 3).
template <int NWV = NW>
__device__ __forceinline__ void dma_k(desc_t rk, uint32_t lds, int wave, int lane) {
  constexpr int NKW = K_BYTES / 1024 / NWV;
#pragma unroll
  for (int j = 0; j < NKW; ++j) {
    const int ins = wave * NKW + j;
    const int row = ins * 4 + (lane >> 4);
    const int lc = (lane & 15) ^ (row & 15);
    dma16(rk, lds + ins * 1024, (uint32_t)row * (D * 2) + (uint32_t)lc * 16u);
  }
}

template <int NWV = NW>
__device__ __forceinline__ void dma_v(desc_t rv, uint32_t lds, int wave, int lane) {
  constexpr int NVW = V_BYTES / 1024 / NWV;
#pragma unroll
  for (int j = 0; j < NVW; ++j) {
    const int ins = wave * NVW + j;
    const int row = ins * 4 + (lane >> 4);
    const int lc = (lane & 15) ^ (4 * (row & 3));
    dma16(rv, lds + ins * 1024, (uint32_t)row * (D * 2) + (uint32_t)lc * 16u);
  }
}

// K fragment (first MFMA operand of S^T = K Q^T): lane l holds key row0 + l%32,
// d values kk*16 + 8 (l/32) .. +8.
__device__ __forceinline__ bf16x8 frag_k(const char* kt, int row0, int kk, int lane) {
  const int row = row0 + (lane & 31);
  const int pc = (kk * 2 + (lane >> 5)) ^ (row & 15);
  return *reinterpret_cast<const bf16x8*>(kt + row * (D * 2) + pc * 16);
}

// V^T fragment (first MFMA operand of O^T += V^T P^T): lane l holds d value
// d0 + l%32 for the keys kvb + 4 (l/32) + {0..3} and kvb + 8 + 4 (l/32) + {0..3},
// the key order of the P registers.  Two transposing reads: within each
// 16-lane group, lane i addresses key row base + i/4, d columns 4 (i%4)..+3,
// and lane q receives the four keys of d column q.
__device__ __forceinline__ bf16x8 frag_v(const char* vt, int d0, int kvb, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int col = d0 + 16 * (G & 1) + 4 * (i & 3);
  const int k = kvb + 4 * (G >> 1) + (i >> 2);
  const int pc = (col >> 3) ^ (4 * (k & 3));
  const char* p = vt + k * (D * 2) + pc * 16 + (col & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * (D * 2)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}
}  // namespace attn128

// d_head 128.  Software-pipelined: a wave computes the next key tile's scores
// S^T_{t+1} = K_{t+1} Q^T (MFMA) while it turns tile t's scores into
// probabilities (VALU) and multiplies them with V_t, so the matrix cores and
// the vector units work on independent data.  K and V have separate
// two-stage rings: at the top of iteration t (one barrier) K_{t+1} and V_t
// have landed, and the DMAs of K_{t+2} and V_{t+1} go into the stages that
// held K_t (consumed at iteration t-1) and V_{t-1}.
//
// HPW = 1: four waves (128 queries of one head), two workgroups per CU,
// causal tiles in heavy/light pairs over the CU's two slots.
// HPW = 2 (grouped-query attention, an even group): eight waves take the same
// query tile of two query heads of one group, which read the same K/V head,
// so each K/V tile goes into LDS once for both (G1 185 -> 163 us); one
// workgroup per CU, heaviest tiles first.  Deeper rings, which its LDS would
// allow, were slower here (four stages: 170 us).
template <int HPW>
__global__ void __launch_bounds__(256 * HPW, 2 / HPW)
flash_attn_fwd_d128_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                              const bf16* __restrict__ V, bf16* __restrict__ O, float* __restrict__ L,
                              int nb, int hl, int group, int s, int causal, float scale_log2) {
  using namespace attn128;
  constexpr int NWV = NW * HPW, NS = 2;
  constexpr int NKW = K_BYTES / 1024 / NWV, NVW = V_BYTES / 1024 / NWV;   // DMA instructions per wave
  __shared__ __attribute__((aligned(1024))) char smem[NS * K_BYTES + NS * V_BYTES];

  const int nqt = (s + BQ - 1) / BQ;
  const int ngrp = nb * hl / HPW;
  const int bid = (int)blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int qt, bh;
  if (HPW == 1) {
    const int half = (int)(gridDim.x / 2);
    const bool light = (nqt % 2 == 0) && bid >= half;
    const int rank = light ? bid - half : bid;
    qt = light ? rank / ngrp : nqt - 1 - rank / ngrp;
    bh = rank % ngrp;
  } else {
    qt = nqt - 1 - bid / ngrp;                      // heaviest tiles first
    bh = (bid % ngrp) * HPW + wave / NW;
  }
  const int bi = bh / hl, h = bh % hl;
  const int wq = wave % NW;                         // wave within its head
  const int lq = lane & 31, g = lane >> 5;
  const int64_t head = (int64_t)bh * s * D;
  const int64_t kvhead = ((int64_t)bi * (hl / group) + h / group) * s * D;
  const bf16* Kh = K + kvhead;
  const bf16* Vh = V + kvhead;
  const int q0 = qt * BQ;
  const int qw = q0 + wq * 32;
  const int qme = qw + lq;
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t kring = lds0, vring = lds0 + NS * K_BYTES;

  const int kv_end = causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  // last key tile this wave needs (every tile for non-causal attention)
  const int wlast = causal ? min(ntiles - 1, (qw + 31) / BKV) : ntiles - 1;
  auto desc_of = [&](const bf16* base, int t) {
    const int64_t kv0 = (int64_t)t * BKV;
    const int64_t rb = (int64_t)(s - kv0) * D * 2;
    return make_desc(base + kv0 * D, rb < 0x7FFFFFFF ? (uint32_t)rb : 0x7FFFFFFFu);
  };
  auto issue_k = [&](int t) { dma_k<NWV>(desc_of(Kh, t), kring + (t % NS) * K_BYTES, wave, lane); };
  auto issue_v = [&](int t) { dma_v<NWV>(desc_of(Vh, t), vring + (t % NS) * V_BYTES, wave, lane); };

  bf16x8 qf[D / 16];
  {
    const rsrc_t rq = make_rsrc(Q + head, (uint64_t)s * D * 2);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(((int64_t)qme * D + kk * 16 + g * 8) * 2)));
  }
  // the tiles before the loop's first issues: K_0 .. K_{NS-1}, V_0 .. V_{NS-2}
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    if (j < ntiles) issue_k(j);
    if (j + 1 < NS && j < ntiles) issue_v(j);
  }

  auto scores = [&](int t, f32x16 (&sc)[2]) {
    const char* Ks = smem + (t % NS) * K_BYTES;
    sc[0] = f32x16{};
    sc[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_k(Ks, kb * 32, kk, lane), qf[kk], sc[kb], 0, 0, 0);
  };

  f32x16 acc_o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc_o[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // Top of iteration t: K_{t+1} and V_t have landed for every wave; every
  // wave is done with K_t and V_{t-1}, whose stages take the next DMAs.
  auto sync = [&](int t) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + NS - 1 < ntiles) issue_v(t + NS - 1);
    if (t + NS < ntiles) issue_k(t + NS);
  };
  // One key tile: sc holds its scores; the next tile's go into sn.
  auto step = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    sync(t);
    if (t + 1 <= wlast) scores(t + 1, sn);          // next tile's scores, independent of this softmax

    const int kv0 = t * BKV;
    if ((causal && kv0 + BKV - 1 > qw) || (kv0 + BKV > s)) {
      const int lim = (causal ? min(qme, s - 1) : s - 1) - (kv0 + 4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) <= lim) ? sc[kb][r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    // The subtracted max m_run may lag the row's true running max by up to
    // kLazyMax (log2 units), so P <= 2^kLazyMax: any m_run gives the same O and
    // L, and the lag only bounds P's range.  O^T and the sum are rescaled when
    // a row of the wave moves past it (with random scores, after the first few
    // tiles almost never), not each time a running max moves.
    if (__builtin_amdgcn_read_exec() & __ballot(m_new > m_run + kLazyMax)) {
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int j = 0; j < D / 32; ++j) acc_o[j] *= corr;
      m_run = m_new;
    }
    // the row sum is taken over the bf16 probabilities the P V product uses
    float rs = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * hh + 2 * e], scale_log2, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * hh + 2 * e + 1], scale_log2, -m_run));
          const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
          wv[e] = __builtin_bit_cast(uint32_t, pk);
          rs = __builtin_amdgcn_fdot2_f32_bf16(pk, kBf16One2, rs, false);
        }
        pf[kb][hh] = __builtin_bit_cast(bf16x8, wv);
      }
    rs += __shfl_xor(rs, 32);
    l_run += rs;

    const char* Vs = smem + NS * K_BYTES + (t % NS) * V_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_v(Vs, db * 32, kb * 32 + hh * 16, lane),
                                                              pf[kb][hh], acc_o[db], 0, 0, 0);
  };
  // The tiles this wave computes on (causal: up to its last query's
  // diagonal), two per iteration so the score registers alternate without
  // copies; then the workgroup's remaining tiles only pass the barriers.
  f32x16 sa[2], sb[2];
  scores(0, sa);
  int t = 0;
  for (; t + 1 <= wlast; t += 2) {
    step(t, sa, sb);
    step(t + 1, sb, sa);
  }
  if (t <= wlast) step(t++, sa, sb);
  for (; t < ntiles; ++t) sync(t);

  if (qme < s) {
    const float inv = 1.0f / l_run;
    if (L && g == 0) L[(int64_t)bh * s + qme] = (m_run + __log2f(l_run)) * 0.69314718055994531f;
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

// fp32 split-K partials of a z-batched product: split s, batch z at
// C + s * split_stride + z * z_stride + m * ldc + n.
struct EpiSplitZ {
  static constexpr int NOUT = 1;
  template <int O> using OutT = float;
  float* C;
  int64_t ldc, split_stride, z_stride;
  template <int O> __device__ __forceinline__ bool has_out() const { return true; }
  template <int O> __device__ __forceinline__ float* out_ptr(int64_t m, int64_t n, int split, int z) const {
    return C + split * split_stride + z * z_stride + m * ldc + n;
  }
  template <int O> __device__ __forceinline__ f32x4 value(int64_t, int64_t, f32x4 v) const { return v; }
};

// Sum of the split partials (in split order) of the K (z = 0) and V (z = 1)
// projections, scattered to head-major [b, h_kv, s, d_head] bf16.  One
// thread per 8 outputs.
__global__ void __launch_bounds__(256)
attn_kv_split_sum_kernel(const float* __restrict__ P, int splits, int64_t M, int64_t nkv, int s, int h_kv,
                         int d_head, bf16* __restrict__ Kout, bf16* __restrict__ Vout) {
  const int64_t per_z = M * nkv / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * per_z) return;
  const int z = (int)(i / per_z);
  const int64_t e = (i % per_z) * 8;
  const int64_t m = e / nkv, n = e % nkv;
  const float* src = P + z * M * nkv + e;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < splits; ++k) {
    float t[8];
    Vec8<float>::load<kNtIn>(src + (int64_t)k * 2 * M * nkv, t);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += t[q];
  }
  const int64_t bi = m / s, t = m % s, j = n / d_head, c = n % d_head;
  bf16* out = (z == 0 ? Kout : Vout) + ((bi * h_kv + j) * s + t) * d_head + c;
  Vec8<bf16>::store(out, acc);
}

hipError_t launch_attn_fwd(hipStream_t st, int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t h_kv,
                           int64_t d_head, int causal, float scale,
                           const void* X, const void* Wq, const void* Wk, const void* Wv,
                           const void* Wo, void* Q, void* K, void* V, void* O, void* Z, float* L) {
  const int64_t M = b * s, N = h_local * d_head, Nkv = h_kv * d_head;
  if (h_kv == h_local) {  // Q, K, V = X W{q,k,v}, scattered to [b, h_local, s, d_head]
    // One batched product of the three, or Q and K batched and V on its own
    // (in its own tile shape) when the three leave a partly filled last round
    // of tiles that the two launches avoid, by the planner's estimates.
    const GemmPlan p3 = plan_gemm(M, 3 * N, d, false, false);
    const GemmPlan p2 = plan_gemm(M, 2 * N, d, false, false);
    const GemmPlan pv = plan_gemm(M, N, d, false, false);
    const bool split_v = p2.est + pv.est + kGemmLaunchS < 0.97 * p3.est;
    GemmParams p = make_params(M, N, make_seg(X, d, M * d, Wq, N, d * N, d));
    p.Bz[0] = static_cast<const bf16*>(Wq);
    p.Bz[1] = static_cast<const bf16*>(Wk);
    p.Bz[2] = static_cast<const bf16*>(Wv);
    EpiHeadScatter<bf16> e{{static_cast<bf16*>(Q), static_cast<bf16*>(K), static_cast<bf16*>(V)},
                           (int)s, (int)h_local, (int)d_head};
    if (split_v) {
      TPK_TRY((launch_gemm<true, false, false>(st, "attn.x_wqk_scatter", p, e, p2, 2)));
      GemmParams q = make_params(M, N, make_seg(X, d, M * d, Wv, N, d * N, d));
      EpiHeadScatter<bf16> ev{{static_cast<bf16*>(V), nullptr, nullptr}, (int)s, (int)h_local, (int)d_head};
      TPK_TRY((launch_gemm<true, false, false>(st, "attn.x_wv_scatter", q, ev, pv)));
    } else {
      TPK_TRY((launch_gemm<true, false, false>(st, "attn.x_wqkv_scatter", p, e, p3, 3)));
    }
  } else {  // grouped-query: Q over h_local heads, then K and V over h_kv heads
    GemmParams pq = make_params(M, N, make_seg(X, d, M * d, Wq, N, d * N, d));
    EpiHeadScatter<bf16> eq{{static_cast<bf16*>(Q), nullptr, nullptr}, (int)s, (int)h_local, (int)d_head};
    TPK_TRY((launch_gemm<true, false, false>(st, "attn.x_wq_scatter", pq, eq, plan_gemm(M, N, d, false, false), 1)));
    GemmParams pk = make_params(M, Nkv, make_seg(X, d, M * d, Wk, Nkv, d * Nkv, d));
    pk.Bz[0] = static_cast<const bf16*>(Wk);
    pk.Bz[1] = static_cast<const bf16*>(Wv);
    // K and V are narrow (h_kv * d_head columns) and K = d is long: split K
    // until the 128x128 tiles fill the CUs' 512 slots (two per CU), with fp32
    // partials in Z's memory (Z is written only by the output projection at
    // the end, and holds M * d bf16).  G1: 4 ways, 512 workgroups, 99 us;
    // 256x128 tiles (one per CU, 4 ways) took 123 us.
    const int64_t tiles = cdiv(M, 128) * cdiv(Nkv, 128) * 2;
    int split = 1;
    while (split < 16 && tiles * split * 2 <= 512 && d / (split * 2) >= 1024) split *= 2;
    if ((int64_t)split * 2 * M * Nkv * 4 > M * d * 2) split = 1;
    if (split > 1) {
      float* part = static_cast<float*>(Z);
      EpiSplitZ e{part, Nkv, 2 * M * Nkv, M * Nkv};
      TPK_TRY((launch_gemm<true, false, false>(st, "attn.x_wkv_split", pk, e, GemmPlan{CFG_S, split}, 2)));
      const int64_t n = 2 * M * Nkv / 8;
      TPK_TRY(launch("attn.kv_split_sum", attn_kv_split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st,
                     (const float*)part, split, M, Nkv, (int)s, (int)h_kv, (int)d_head, static_cast<bf16*>(K),
                     static_cast<bf16*>(V)));
    } else {
      EpiHeadScatter<bf16> ek{{static_cast<bf16*>(K), static_cast<bf16*>(V), nullptr}, (int)s, (int)h_kv,
                              (int)d_head};
      TPK_TRY((launch_gemm<true, false, false>(st, "attn.x_wkv_scatter", pk, ek,
                                                plan_gemm(M, 2 * Nkv, d, false, false), 2)));
    }
  }
  {
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d_head);
    const float sl2 = sc * 1.4426950408889634f;
    const int64_t nqt = (s + 127) / 128;
    const dim3 grid((unsigned)(nqt * b * h_local));
    const int group = (int)(h_local / h_kv);
    const bf16* q = static_cast<const bf16*>(Q);
    const bf16* k = static_cast<const bf16*>(K);
    const bf16* v = static_cast<const bf16*>(V);
    bf16* o = static_cast<bf16*>(O);
    if (d_head == 128 && group % 2 == 0 && h_local % 2 == 0)   // two query heads per workgroup
      TPK_TRY(launch("attn.core_d128", flash_attn_fwd_d128_kernel<2>, dim3(grid.x / 2), dim3(512), st, q, k, v, o,
                     L, (int)b, (int)h_local, group, (int)s, causal, sl2));
    else if (d_head == 128)
      TPK_TRY(launch("attn.core_d128", flash_attn_fwd_d128_kernel<1>, grid, dim3(256), st, q, k, v, o, L, (int)b,
                     (int)h_local, group, (int)s, causal, sl2));
    else
      TPK_TRY(launch("attn.core_d64", flash_attn_fwd_kernel<64>, grid, dim3(256), st, q, k, v, o, L, (int)b,
                     (int)h_local, group, (int)s, causal, sl2));
  }
  {  // Z = O Wo (this shard's partial)
    GemmParams p = make_params(M, d, make_seg(O, N, M * N, Wo, d, N * d, N));
    EpiStore<bf16> e{static_cast<bf16*>(Z), d, 0};
    TPK_TRY((launch_gemm<true, false, false>(st, "attn.o_wo", p, e, plan_gemm(M, d, N, false, false))));
  }
  return hipSuccess;
}

}  // namespace tpk
