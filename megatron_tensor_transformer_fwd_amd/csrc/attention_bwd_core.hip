// Backward of the head-group attention shard ([BM] Megatron_MHA: the input
// passes Megatron_f, identity forward and all-reduce backward, so this
// shard's dX is one summand of the full dX; the output projection is
// row-parallel and g's backward is the identity, so the shard receives the
// full upstream dY.  [HC] 3.4: f all-reduces dX in the backward pass.)
//
//   dO = dY W_O^T                         (product, bf16 [b*s x h_l*d_h])
//   dW_O = O^T dY                         (product, fp32)
//   D[t] = sum_c dO[t, c] O[t, c]         per (batch, head, query)
//   per head, with P = exp(S - L) recomputed from Q, K and the forward's
//   log-sum-exp L:
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//     dK = scale dS^T Q,  dQ = scale dS K
//   dX = [dQ | dK | dV] [W_Q | W_K | W_V]^T   (one product over K = 3 h_l d_h)
//   [dW_Q | dW_K | dW_V] = X^T [dQ | dK | dV]  (one product, columns split)
//
// The two flash kernels recompute P and dP (no s x s matrix in memory) and
// are deterministic: the key-tile kernel owns dK and dV of 128 keys (lanes
// index keys, so P arrives in the layout the dK/dV products consume), the
// query-tile kernel owns dQ of 128 queries (lanes index queries, as in the
// forward).  Tiles stream through LDS by DMA with a 16-byte-chunk swizzle
// (swz below) that keeps both the row-wise fragment reads and the
// transposing ds_read_b64_tr_b16 reads free of bank conflicts.
//
// This file holds the flash kernels and their launchers; the products and
// the workspace layout are in attention_bwd.hip.  It is compiled with the
// MFMA accumulators in architectural registers (see build.py).
#include "epilogues.hpp"
#include "gemm_dispatch.hpp"
#include "launch.hpp"

namespace tpk {

// K/V stages of the two-head query-tile kernel (one workgroup per CU, so the
// LDS has room): G1 225 us with two, 208 with three, 230 with four.
#ifndef TPK_DQ2_STAGES
#define TPK_DQ2_STAGES 3
#endif

namespace attnb {
constexpr int D = 128, NT = 256, NW = 4;
constexpr int ROWB = D * 2;                   // bytes per tile row
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte chunk c of tile row r is stored at chunk c ^ swz(r), swz a
// permutation of r's low four bits r3 r2 r1 r0 into (r3^r1^r0, r0, r1, r2).
// The row fragments read 8 (or 16) consecutive rows at one chunk; each
// 16-lane group of a transposing read reads 4 consecutive rows at 2 (or 4)
// adjacent aligned chunks.  Both then fall on distinct chunks modulo 8 and
// modulo 16, so neither pattern has bank conflicts whether the LDS serves
// 128 or 256 bytes per cycle.
__device__ __forceinline__ int swz(int row) {
  return ((row >> 2) & 1) | (row & 2) | ((row & 1) << 2) | ((((row >> 3) ^ (row >> 1) ^ row) & 1) << 3);
}

// DMA of `rows` rows of 128 bf16 (row pitch `ld_b` bytes in memory) into a
// swizzled LDS tile: 4 rows per 1 KiB instruction; NI instructions per wave.
template <int ROWS, int NWV = NW>
__device__ __forceinline__ void dma_rows(desc_t r, uint32_t ld_b, uint32_t lds, int wave, int lane) {
  constexpr int NI = ROWS / 4 / NWV;
  static_assert(NI * 4 * NWV == ROWS, "tile rows");
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int ins = wave * NI + j;
    const int row = ins * 4 + (lane >> 4);
    const int lc = (lane & 15) ^ swz(row);
    dma16(r, lds + ins * 1024, (uint32_t)row * ld_b + (uint32_t)lc * 16u);
  }
}

// One dword per lane (64 floats) into LDS.
__device__ __forceinline__ void dma_vec(desc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voff), "s"(r) : "memory", "m0");
}

// Row fragment: lane l holds row row0 + l%32, columns kk*16 + 8 (l/32) .. +8.
__device__ __forceinline__ bf16x8 frag_row(const char* t, int row0, int kk, int lane) {
  const int row = row0 + (lane & 31);
  const int pc = (kk * 2 + (lane >> 5)) ^ swz(row);
  return *reinterpret_cast<const bf16x8*>(t + row * ROWB + pc * 16);
}

// Transposed fragment: lane l holds column d0 + l%32 of the rows
// r0 + 4 (l/32) + {0..3} and r0 + 8 + 4 (l/32) + {0..3}: the order in which
// an accumulator (lanes = the other index, registers = these rows) packs its
// values.  Two ds_read_b64_tr_b16: in each 16-lane group lane i addresses
// row base + i/4, columns 4 (i%4)..+3, and lane q receives the four rows of
// column q.
__device__ __forceinline__ bf16x8 frag_col(const char* t, int d0, int r0, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int col = d0 + 16 * (G & 1) + 4 * (i & 3);
  const int k = r0 + 4 * (G >> 1) + (i >> 2);
  const char* plo = t + k * ROWB + (((col >> 3) ^ swz(k)) * 16) + (col & 7) * 2;
  const char* phi = t + (k + 8) * ROWB + (((col >> 3) ^ swz(k + 8)) * 16) + (col & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(plo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(phi));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int base) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(a[base + 2 * e], a[base + 2 * e + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ desc_t range_desc(const void* base, int64_t bytes) {
  return make_desc(base, bytes <= 0 ? 0u : (bytes < 0x7FFFFFFF ? (uint32_t)bytes : 0x7FFFFFFFu));
}
}  // namespace attnb

// D[bh, t] = sum_c dO[t, h*128 + c] * O[t, h*128 + c], stored negated (the
// flash kernels form dP - D, and the key-tile kernel starts its dP
// accumulators from -D); one thread per (t, h).  Also the forward's
// log-sum-exp in base 2, L2 = L log2(e), which the flash kernels subtract
// inside exp2 without a multiply per score.
__global__ void __launch_bounds__(256) attn_bwd_rowdot_kernel(const bf16* __restrict__ dO,
                                                              const bf16* __restrict__ O, const float* __restrict__ L,
                                                              float* __restrict__ Dv, float* __restrict__ L2,
                                                              int64_t rows, int hl, int s, int64_t ld) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * hl) return;
  const int64_t row = i / hl;
  const int h = (int)(i % hl);
  const bf16* a = dO + row * ld + h * attnb::D;
  const bf16* o = O + row * ld + h * attnb::D;
  float acc = 0.f;
#pragma unroll 4
  for (int c = 0; c < attnb::D; c += 8) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(a + c);
    const u32x4 y = *reinterpret_cast<const u32x4*>(o + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(x[e]) * bf16_lo(y[e]) + bf16_hi(x[e]) * bf16_hi(y[e]);
  }
  const int64_t bi = row / s, t = row % s;
  Dv[(bi * hl + h) * s + t] = -acc;
  L2[(bi * hl + h) * s + t] = L[(bi * hl + h) * s + t] * attnb::kLog2e;   // log-sum-exp in base 2
}

// acc[db] += B^T X over a 64-row chunk: B the four bf16x8 operand quarters
// (32 rows x 16 per quarter, rows qb*32 + hh*16..) in register order, X the
// chunk's rows read transposed from LDS tile T (four 32-column blocks).  The
// fragments of quarter i+1 are read before quarter i's MFMAs issue.
__device__ __forceinline__ void acc_cols(f32x16 (&acc)[attnb::D / 32], const char* T, const bf16x8 (&B)[2][2],
                                         int lane) {
  using namespace attnb;
  bf16x8 fc[2][D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) fc[0][db] = frag_col(T, db * 32, 0, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qb = i >> 1, hh = i & 1;
    if (i + 1 < 4)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        fc[(i + 1) & 1][db] = frag_col(T, db * 32, ((i + 1) >> 1) * 32 + ((i + 1) & 1) * 16, lane);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc[i & 1][db], B[qb][hh], acc[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Key-tile kernel: dK and dV of 128 keys of one (batch, query head),
// streaming 64-query chunks of Q and dO.  Lanes index keys: the accumulators
// of S = Q K^T and dP = dO V^T hold, per lane, one key and 16 queries,
// exactly the operand layout of dV += P^T dO and dK += dS^T Q.  With
// grouped-query attention (group > 1) the keys and values are those of K/V
// head h / group, and the outputs are this query head's fp32 contributions,
// summed over the group afterwards.
//
// Eight waves in two roles per block of 32 keys (two waves per SIMD):
//  * P waves (0-3) recompute S for chunk c, form P = exp2(S scale log2e - L2),
//    hand P (bf16, in their register order) to their partner through LDS and
//    accumulate dV += P^T dO;
//  * dS waves (4-7) run one chunk behind: in step c they form
//    dS = P (dP - D) for chunk c-1 from their partner's P and the dP they
//    computed in step c-1, accumulate dK += dS^T Q, then compute dP for chunk c.
// On every SIMD one role's softmax or dS arithmetic overlaps the other's
// MFMAs.  Chunks rotate through three LDS stages (the dS waves still read
// chunk c-1 while chunk c+1 is loading) and P through two buffers; one
// barrier per step orders them.
template <class TO>
__global__ void __launch_bounds__(512, 1)
attn_bwd_dkv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                    const bf16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dv,
                    TO* __restrict__ dK, TO* __restrict__ dV, int nb, int hl, int group, int s, int causal,
                    float scale, int64_t ld_o, int64_t ld_g) {
  using namespace attnb;
  constexpr int BKEY = 128, BQ = 64, NSTG = 3;
  constexpr int QT = BQ * ROWB, VEC = BQ * 4;
  constexpr int STAGE = 2 * QT + 2 * VEC;            // Q, dO, L, D
  constexpr int PWAVE = 64 * 64;                     // one P wave's chunk of P: 64 lanes x four bf16x8
  constexpr int PBUF = NW * PWAVE;
  __shared__ __attribute__((aligned(1024))) char smem[NSTG * STAGE + 2 * PBUF];

  const int nbh = nb * hl;
  const int kt = (int)(blockIdx.x / nbh);            // key tile 0 (most queries) first
  const int bh = (int)(blockIdx.x % nbh);
  const int bi = bh / hl, h = bh % hl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool prole = wave < NW;                       // uniform per wave
  const int kb = wave & (NW - 1);                     // this wave's block of 32 keys
  const int lk = lane & 31, g = lane >> 5;
  const int k0 = kt * BKEY, kw = k0 + kb * 32, key = kw + lk;
  const int64_t head = (int64_t)bh * s * D;
  const int64_t kvhead = ((int64_t)bi * (hl / group) + h / group) * s * D;
  const uint32_t lds0 = lds_addr(smem);
  char* pbuf = smem + NSTG * STAGE;
  const float sl2 = scale * kLog2e;

  // P waves hold their keys, dS waves their values, as row fragments (zero
  // past the sequence).
  bf16x8 kvf[D / 16];
  {
    const rsrc_t r = make_rsrc((prole ? K : V) + kvhead, (uint64_t)s * ROWB);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      kvf[kk] = __builtin_bit_cast(bf16x8, buf_load16(r, (uint32_t)(((int64_t)key * D + kk * 16 + g * 8) * 2)));
  }

  const int nqc = (s + BQ - 1) / BQ;
  const int c_begin = causal ? k0 / BQ : 0;
  // Q rows by the P waves, dO rows by the dS waves, L and D by one wave each.
  auto issue = [&](int c) {
    const int q0 = c * BQ;
    const uint32_t st = lds0 + (uint32_t)((c % NSTG) * STAGE);
    if (prole) {
      dma_rows<BQ>(range_desc(Q + head + (int64_t)q0 * D, (int64_t)(s - q0) * ROWB), ROWB, st, kb, lane);
      if (kb == 0) dma_vec(range_desc(L2 + (int64_t)bh * s + q0, (int64_t)(s - q0) * 4), st + 2 * QT, lane * 4u);
    } else {
      const bf16* dorow = dO + ((int64_t)bi * s + q0) * ld_o + (int64_t)h * D;
      dma_rows<BQ>(range_desc(dorow, (int64_t)(s - q0 - 1) * ld_o * 2 + ROWB), (uint32_t)(ld_o * 2), st + QT, kb,
                   lane);
      if (kb == 0) dma_vec(range_desc(Dv + (int64_t)bh * s + q0, (int64_t)(s - q0) * 4), st + 2 * QT + VEC, lane * 4u);
    }
  };
  // chunk c has a query at or after one of this block's keys
  auto live = [&](int c) { return c >= c_begin && c < nqc && !(causal && c * BQ + BQ - 1 < kw); };
  // the mask matters only where a pair can be past the sequence or (causal) a key after a query
  auto masked = [&](int c) { return c * BQ + BQ > s || (causal && kw + 31 > c * BQ); };

  f32x16 acc[D / 32];                                 // dV (P waves) or dK (dS waves)
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  // The two roles run separate loops with the same steps and one barrier per
  // step, so that each role's registers are allocated on their own.
  if (c_begin < nqc) issue(c_begin);
  if (prole) {
    for (int c = c_begin; c <= nqc; ++c) {
      // chunk c landed (own DMAs), every wave done with step c-1: chunk c-2's
      // stage and the P buffer of chunk c-2 are free again
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 1 < nqc) issue(c + 1);
      if (!live(c)) continue;
      const char* st = smem + (c % NSTG) * STAGE;
      const int q0 = c * BQ;
      const char* Qs = st;
      const char* dOs = st + QT;
      const float* Ls = reinterpret_cast<const float*>(st + 2 * QT);
      f32x16 sacc[2];
      {  // fragments of step kk+1 are read before step kk's MFMAs issue
        bf16x8 fr[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) fr[0][qb] = frag_row(Qs, qb * 32, 0, lane);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk + 1 < D / 16)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) fr[(kk + 1) & 1][qb] = frag_row(Qs, qb * 32, kk + 1, lane);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[kk & 1][qb], kvf[kk], kk ? sacc[qb] : f32x16{},
                                                               0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // register r of block qb: query q0 + qb*32 + 8 (r/4) + 4 g + r%4
      bf16x8 pf[2][2];
      auto softmax = [&]<bool MASK>() {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int ql = qb * 32 + 8 * r4 + 4 * g;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + ql);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * r4 + e, q = q0 + ql + e;
              float p = __builtin_amdgcn_exp2f(fmaf(sacc[qb][r], sl2, -l4[e]));
              if constexpr (MASK) p = (q < s && (!causal || key <= q)) ? p : 0.f;
              sacc[qb][r] = p;
            }
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) pf[qb][hh] = pack8(sacc[qb], 8 * hh);
        }
      };
      if (masked(c)) softmax.template operator()<true>();
      else softmax.template operator()<false>();
      char* pw = pbuf + (c & 1) * PBUF + kb * PWAVE;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) *reinterpret_cast<bf16x8*>(pw + (qb * 2 + hh) * 1024 + lane * 16) = pf[qb][hh];
      // dV[key][d] += P^T dO (four d blocks); each quarter's fragments are
      // read before the previous quarter's MFMAs issue
      acc_cols(acc, dOs, pf, lane);
    }
  } else {
    f32x16 dp[2];                                     // dP of the previous chunk
    dp[0] = dp[1] = f32x16{};
    for (int c = c_begin; c <= nqc; ++c) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 1 < nqc) issue(c + 1);
      if (live(c - 1)) {
        // dS = P (dP - D) for chunk c-1 (dp already holds dP - D), then
        // dK[key][d] += dS^T Q
        const char* sp = smem + ((c - 1) % NSTG) * STAGE;
        const char* Qp = sp;
        const char* pr = pbuf + ((c - 1) & 1) * PBUF + kb * PWAVE;
        bf16x8 sf[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const u32x4 pw = *reinterpret_cast<const u32x4*>(pr + (qb * 2 + hh) * 1024 + lane * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * hh + 2 * e;                     // registers r, r+1
              dp[qb][r] = bf16_lo(pw[e]) * dp[qb][r];
              dp[qb][r + 1] = bf16_hi(pw[e]) * dp[qb][r + 1];
            }
            sf[qb][hh] = pack8(dp[qb], 8 * hh);
          }
        }
        acc_cols(acc, Qp, sf, lane);
      }
      if (live(c)) {
        // dP - D for chunk c: the accumulators start from -D of the
        // chunk's queries (register r of block qb: query qb*32 + 8 (r/4) + 4 g + r%4)
        const char* dOs = smem + (c % NSTG) * STAGE + QT;
        const float* nDs = reinterpret_cast<const float*>(smem + (c % NSTG) * STAGE + 2 * QT + VEC);
        f32x16 nd[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(nDs + qb * 32 + 8 * r4 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) nd[qb][4 * r4 + e] = v[e];
          }
        bf16x8 fr[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) fr[0][qb] = frag_row(dOs, qb * 32, 0, lane);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk + 1 < D / 16)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) fr[(kk + 1) & 1][qb] = frag_row(dOs, qb * 32, kk + 1, lane);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[kk & 1][qb], kvf[kk], kk ? dp[qb] : nd[qb], 0,
                                                             0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // register r of block db: d = db*32 + 8 (r/4) + 4 g + r%4 of key `key`
  if (key < s) {
    TO* row = (prole ? dV : dK) + ((int64_t)bi * s + key) * ld_g + (int64_t)h * D;
    const float f = prole ? 1.0f : scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int c = db * 32 + 8 * b4 + 4 * g;
        const f32x4 v = {acc[db][4 * b4] * f, acc[db][4 * b4 + 1] * f, acc[db][4 * b4 + 2] * f,
                         acc[db][4 * b4 + 3] * f};
        Quad<TO>::store(row + c, v);
      }
  }
}

// Query-tile kernel: dQ of 128 queries (four waves of 32) of one (batch,
// head), streaming 64-key chunks of K and V.  Lanes index queries, as in the
// forward: S^T = K Q^T and dP^T = V dO^T need row fragments of K and V, and
// dQ += dS K needs K transposed in the key order of the dS registers.
//
// HPW = 2 (grouped-query attention, an even group): one workgroup of eight
// waves takes the same query tile of two query heads of one group, which read
// the same K/V head, so each K/V chunk goes into LDS once for both (half the
// DMA bytes per FLOP; both heads have the same causal extent, so the waves
// stay in step).  Alone on its CU, it loads the chunks two steps ahead
// through three LDS stages; with one step of look-ahead its waits for the
// DMA cost about 8%.
template <int HPW>
__global__ void __launch_bounds__(256 * HPW, 2 / HPW)
attn_bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                   const bf16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dv,
                   bf16* __restrict__ dQ, int nb, int hl, int group, int s, int causal, float scale,
                   int64_t ld_o, int64_t ld_g) {
  using namespace attnb;
  constexpr int BQ = 128, BKV = 64, NWV = NW * HPW;
  constexpr int KT = BKV * ROWB, STAGE = 2 * KT;
  // one workgroup per CU with two heads: the LDS holds a deeper ring
  constexpr int NSTG = HPW == 2 ? TPK_DQ2_STAGES : 2;
  constexpr int DMA_PER_CHUNK = 2 * (BKV / 4 / NWV);    // K and V instructions per wave
  __shared__ __attribute__((aligned(1024))) char smem[NSTG * STAGE];

  const int nqt = (s + BQ - 1) / BQ;
  const int ngrp = nb * hl / HPW;                     // (batch, head set) pairs
  // Several rounds of workgroups: heaviest tiles first.  One round (at most
  // two workgroups per CU on 256 CUs, causal, an even tile count): the first
  // half of the grid takes the heavy tiles in falling order and the second
  // half the light ones in rising order, so the two workgroups that share a
  // CU carry nqt + 1 chunks between them.
  const int bid = (int)blockIdx.x, half = (int)(gridDim.x / 2);
  const bool light = HPW == 1 && causal && nqt % 2 == 0 && gridDim.x <= 2 * 256 && bid >= half;
  const int rank = light ? bid - half : bid;
  const int qt = light ? rank / ngrp : nqt - 1 - rank / ngrp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave % NW;                           // wave within its head
  const int bh = (rank % ngrp) * HPW + wave / NW;
  const int bi = bh / hl, h = bh % hl;
  const int lq = lane & 31, g = lane >> 5;
  const int q0 = qt * BQ, qw = q0 + wq * 32, qme = qw + lq;
  const int64_t head = (int64_t)bh * s * D;
  const int64_t kvhead = ((int64_t)bi * (hl / group) + h / group) * s * D;
  const uint32_t lds0 = lds_addr(smem);
  const float sl2 = scale * kLog2e;

  bf16x8 qf[D / 16], of[D / 16];
  {
    const rsrc_t rq = make_rsrc(Q + head, (uint64_t)s * ROWB);
    const bf16* dorow = dO + (int64_t)bi * s * ld_o + (int64_t)h * D;
    const rsrc_t ro = make_rsrc(dorow, (uint64_t)((int64_t)(s - 1) * ld_o * 2 + ROWB));
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(((int64_t)qme * D + kk * 16 + g * 8) * 2)));
      of[kk] = __builtin_bit_cast(bf16x8,
                                  buf_load16(ro, (uint32_t)(((int64_t)qme * ld_o + kk * 16 + g * 8) * 2)));
    }
  }
  const bool live = qme < s;
  const float l2 = live ? L2[(int64_t)bh * s + qme] : 0.f;
  const float ndq = live ? Dv[(int64_t)bh * s + qme] : 0.f;   // -D

  const int kv_end = causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  auto issue = [&](int t) {
    const int kv0 = t * BKV;
    const uint32_t st = lds0 + (uint32_t)((t % NSTG) * STAGE);
    const int64_t rem = (int64_t)(s - kv0) * ROWB;
    dma_rows<BKV, NWV>(range_desc(K + kvhead + (int64_t)kv0 * D, rem), ROWB, st, wave, lane);
    dma_rows<BKV, NWV>(range_desc(V + kvhead + (int64_t)kv0 * D, rem), ROWB, st + KT, wave, lane);
  };

  f32x16 adq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) adq[i] = f32x16{};

#pragma unroll
  for (int t = 0; t < NSTG - 1; ++t)
    if (t < ntiles) issue(t);
  if constexpr (NSTG > 2) {   // the fragment loads above are retired here, so no wait inside the loop drains the ring
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      settle(qf[kk]);
      settle(of[kk]);
    }
    settle(l2);
    settle(ndq);
  }
  // chunk t landed; the DMAs of up to NSTG - 2 later chunks may still be in
  // flight; then the DMA of chunk t + NSTG - 1 into the stage step t-1 read
  auto step_sync = [&](int t) {
    if constexpr (NSTG > 2) {
      const int ahead = min(NSTG - 2, ntiles - 1 - t);
      static_assert(NSTG <= 4 && DMA_PER_CHUNK == 4, "the barrier's vmcnt immediates");
      if (ahead >= 2) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (ahead == 1) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (t + NSTG - 1 < ntiles) issue(t + NSTG - 1);
  };
  // The chunks this wave computes on come first (causal: up to its last
  // query's diagonal); the rest of the workgroup's chunks only pass through
  // the barriers.  Keeping the skip out of the computing loop keeps a single
  // path through the dQ accumulation, whose registers then stay in place.
  const int wend = causal ? min(ntiles, (qw + 31) / BKV + 1) : ntiles;
  for (int t = 0; t < wend; ++t) {
    step_sync(t);
    const int kv0 = t * BKV;
    const char* Ks = smem + (t % NSTG) * STAGE;
    const char* Vs = Ks + KT;
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_row(Ks, kb * 32, kk, lane), qf[kk],
                                                           kk ? sacc[kb] : f32x16{}, 0, 0, 0);
        pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_row(Vs, kb * 32, kk, lane), of[kk],
                                                           kk ? pacc[kb] : f32x16{}, 0, 0, 0);
      }
    // register r of block kb: key kv0 + kb*32 + 8 (r/4) + 4 g + r%4 of query
    // qme.  The mask is evaluated only where a key of the chunk can be past
    // the sequence or (causal) after a query of the wave.
    bf16x8 sf[2][2];
    auto softmax = [&]<bool MASK>() {
      const int lim = (causal ? min(qme, s - 1) : s - 1) - (kv0 + 4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -l2));
          if constexpr (MASK) p = (kb * 32 + 8 * (r >> 2) + (r & 3) <= lim) ? p : 0.f;
          pacc[kb][r] = p * (pacc[kb][r] + ndq);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) sf[kb][hh] = pack8(pacc[kb], 8 * hh);
      }
    };
    if (kv0 + BKV > s || (causal && kv0 + BKV - 1 > qw)) softmax.template operator()<true>();
    else softmax.template operator()<false>();
    // dQ[q][d] += dS K (four d blocks, interleaved)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          adq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_col(Ks, db * 32, kb * 32 + hh * 16, lane),
                                                            sf[kb][hh], adq[db], 0, 0, 0);
  }
  for (int t = wend; t < ntiles; ++t) step_sync(t);

  if (live) {
    bf16* qrow = dQ + ((int64_t)bi * s + qme) * ld_g + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const f32x4 v = {adq[db][4 * b4] * scale, adq[db][4 * b4 + 1] * scale, adq[db][4 * b4 + 2] * scale,
                         adq[db][4 * b4 + 3] * scale};
        Quad<bf16>::store(qrow + db * 32 + 8 * b4 + 4 * g, v);
      }
  }
}

// [W_Q | W_K | W_V] side by side: row r of the result is the rows r of the
// three weights ([d x n0], [d x n1], [d x n1]), 16 bytes per thread.
__global__ void __launch_bounds__(256) attn_concat3_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B,
                                                           const bf16* __restrict__ C, bf16* __restrict__ out,
                                                           int64_t rows, int64_t n0, int64_t n1) {
  const int64_t c0 = n0 / 8, c1 = n1 / 8, cr = c0 + 2 * c1;   // widths are multiples of 8
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cr) return;
  const int64_t r = i / cr, j = i % cr;
  const bf16* src = j < c0 ? A + r * n0 + j * 8
                           : (j < c0 + c1 ? B + r * n1 + (j - c0) * 8 : C + r * n1 + (j - c0 - c1) * 8);
  *reinterpret_cast<u32x4*>(out + r * cr * 8 + j * 8) = *reinterpret_cast<const u32x4*>(src);
}

// Grouped-query attention: dK (or dV) of K/V head k is the sum, in order, of
// the fp32 contributions of query heads k*group .. k*group + group - 1
// (P [rows x hl*128]); written as bf16 into columns k*128.. of `out` (row
// pitch ld).  One thread per 8 outputs.
__global__ void __launch_bounds__(256) attn_bwd_group_sum_kernel(const float* __restrict__ P,
                                                                 bf16* __restrict__ out, int64_t rows, int hl,
                                                                 int group, int64_t ld) {
  constexpr int D = attnb::D;
  const int hkv = hl / group;
  const int64_t per_row = (int64_t)hkv * D / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * per_row) return;
  const int64_t r = i / per_row;
  const int64_t c = (i % per_row) * 8;                 // column within [0, hkv*128)
  const int k = (int)(c / D);
  const float* src = P + r * (int64_t)hl * D + (int64_t)k * group * D + (c % D);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < group; ++j) {
    float t[8];
    Vec8<float>::load<kNtIn>(src + (int64_t)j * D, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += t[e];
  }
  Vec8<bf16>::store(out + r * ld + c, acc);
}

// ------------------------------------------------------------------ launchers

hipError_t launch_attn_bwd_rowdot(hipStream_t st, const void* dO, const void* O, const float* L, float* Dv,
                                  float* L2, int64_t rows, int hl, int s, int64_t ld) {
  const int64_t n = rows * hl;
  return launch("attn_bwd.rowdot", attn_bwd_rowdot_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st,
                static_cast<const bf16*>(dO), static_cast<const bf16*>(O), L, Dv, L2, rows, hl, s, ld);
}

hipError_t launch_attn_bwd_flash(hipStream_t st, int b, int hl, int group, int s, int causal, float scale,
                                 const void* Qv, const void* Kv, const void* Vv, const void* dOv, const float* L2,
                                 const float* Dv, int64_t ld_o, void* dQKVv, int64_t ld_g, int64_t n_q,
                                 int64_t n_kv, float* part_k, float* part_v) {
  const bf16* Q = static_cast<const bf16*>(Qv);
  const bf16* K = static_cast<const bf16*>(Kv);
  const bf16* V = static_cast<const bf16*>(Vv);
  const bf16* dO = static_cast<const bf16*>(dOv);
  bf16* dQKV = static_cast<bf16*>(dQKVv);
  const int nbh = b * hl;
  const unsigned grid = (unsigned)(((s + 127) / 128) * nbh);
  if (group == 1) {  // dK, dV straight into their columns of [dQ | dK | dV]
    TPK_TRY(launch("attn_bwd.dkv", attn_bwd_dkv_kernel<bf16>, dim3(grid), dim3(512), st, Q, K, V, dO, L2, Dv,
                   dQKV + n_q, dQKV + n_q + n_kv, b, hl, 1, s, causal, scale, ld_o, ld_g));
  } else {  // per-query-head contributions, then the ordered sum over each group
    TPK_TRY(launch("attn_bwd.dkv", attn_bwd_dkv_kernel<float>, dim3(grid), dim3(512), st, Q, K, V, dO, L2, Dv,
                   part_k, part_v, b, hl, group, s, causal, scale, ld_o, n_q));
    const int64_t rows = (int64_t)b * s;
    const int64_t n = rows * n_kv / 8;
    const dim3 g2((unsigned)((n + 255) / 256));
    TPK_TRY(launch("attn_bwd.group_sum", attn_bwd_group_sum_kernel, g2, dim3(256), st, (const float*)part_k,
                   dQKV + n_q, rows, hl, group, ld_g));
    TPK_TRY(launch("attn_bwd.group_sum", attn_bwd_group_sum_kernel, g2, dim3(256), st, (const float*)part_v,
                   dQKV + n_q + n_kv, rows, hl, group, ld_g));
  }
  if (group % 2 == 0 && hl % 2 == 0)   // two query heads of a group per workgroup, K/V chunks shared
    return launch("attn_bwd.dq", attn_bwd_dq_kernel<2>, dim3(grid / 2), dim3(512), st, Q, K, V, dO, L2, Dv, dQKV,
                  b, hl, group, s, causal, scale, ld_o, ld_g);
  return launch("attn_bwd.dq", attn_bwd_dq_kernel<1>, dim3(grid), dim3(256), st, Q, K, V, dO, L2, Dv, dQKV, b, hl,
                group, s, causal, scale, ld_o, ld_g);
}

hipError_t launch_attn_concat3(hipStream_t st, const void* A, const void* B, const void* C, void* out, int64_t rows,
                               int64_t n0, int64_t n1) {
  const int64_t n = rows * ((n0 + 2 * n1) / 8);
  return launch("attn_bwd.concat_w", attn_concat3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st,
                static_cast<const bf16*>(A), static_cast<const bf16*>(B), static_cast<const bf16*>(C),
                static_cast<bf16*>(out), rows, n0, n1);
}

}  // namespace tpk
