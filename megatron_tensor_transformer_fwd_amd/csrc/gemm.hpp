// bf16 MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) B(k,n), fp32 accumulate,
// with a fused epilogue.
//
// Design (CDNA4-first):
//  * Workgroup tile BM x BN x BK computed by WM x WN wavefronts of 64 lanes;
//    every wave owns a (BM/WM) x (BN/WN) sub-tile of v_mfma_f32_32x32x16_bf16
//    blocks, accumulators in AGPRs.
//  * Operand tiles go global -> LDS with buffer_load ... lds (LDS DMA): no
//    staging registers and no ds_write.  Each wave instruction fills 1 KiB of
//    LDS, lane L writing bytes [16L, 16L+16); the lane picks which 16-byte
//    chunk of the tile it fetches, which is how the tiles get their bank
//    swizzle.  Reads past the end of an operand return zero (buffer range),
//    which pads ragged k tails; k tails inside a row are sent out of range.
//  * NSTAGE LDS stages in a ring: right after the one barrier of iteration t
//    the DMA of k-tile t+NSTAGE-1 is issued into the stage tile t-1 used, so
//    NSTAGE-1 tiles are in flight while tile t is multiplied; explicit
//    s_waitcnt vmcnt + s_barrier (no fences) order the ring.
//  * A K-major operand (k contiguous in memory) is kept as rows of 64 k
//    (128 B) with 16-byte chunk c of row r stored at c ^ ((r >> 1) & 7); MFMA
//    fragments are single ds_read_b128s, bank-conflict free for 16 rows.
//  * An M/N-major operand (m or n contiguous: the weights of the forward
//    products, both operands of the weight-gradient products) is kept as it
//    is in memory, k rows of 128 m/n values (256 B) per sub-tile, chunk c of
//    row r stored at c ^ (4 (r & 3)), and its fragments are read with two
//    ds_read_b64_tr_b16 (the gfx950 LDS transpose read): within each 16-lane
//    group lane q receives element q%4 of the rows addressed by lanes q/4 +
//    4e, so pointing lane i at row k0 + i/4, columns n0 + 4 (i%4) hands lane q
//    the four k values of column n0 + q.  No register transposes.
//  * The MFMA's first operand is the B fragment and its second the A
//    fragment, so each lane's accumulator holds 4 consecutive n of one m:
//    epilogues work on (m, n..n+3) quads.
//  * Workgroup ids are remapped so the tiles one XCD (of 8) runs are
//    contiguous, then grouped along m for L2 reuse.
#pragma once
#include <utility>

#include "common.hpp"
#include "epilogues.hpp"

namespace tpk {

struct GemmSeg {
  const bf16* A;       // A(m,k) at A[m*lda + k] (K-major) or A[k*lda + m] (M-major)
  const bf16* B;       // B(k,n) at B[n*ldb + k] (K-major) or B[k*ldb + n] (N-major)
  const bf16* B2;      // dual-B products only: second right operand, same layout as B
  int64_t lda, ldb;
  int64_t a_elems;     // readable elements from A (the buffer range)
  int64_t b_elems;     // readable elements from B (and from B2)
  int K;
};

struct GemmParams {
  int M, N;            // output extent (for dual-B products N counts the shared columns)
  int nseg;            // 1 or 2 K segments, summed into one accumulator
  GemmSeg seg[2];
  const bf16* Bz[3];   // batched products: per-batch right operand of segment 0 (or NULL)
  int tiles_m, tiles_n;
  int split_k;         // K-tile ranges over blockIdx.y
};

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64, int NSTAGE_ = 2>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NSTAGE = NSTAGE_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int SMEM_BYTES = NSTAGE * STAGE;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "M/N-major tiles are 128-wide sub-tiles");
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(NSTAGE >= 2 && SMEM_BYTES <= 160 * 1024, "LDS stages");
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every tile range

// Buffer descriptor words (gfx9 layout: base, stride 0, num_records, flags),
// kept in SGPRs.
typedef i32x4 desc_t;

__device__ __forceinline__ desc_t make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  desc_t d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xFFFFu));
  d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  d[3] = 0x00020000;
  return d;
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One 16-byte-per-lane LDS DMA: lane L's 16 bytes from buffer offset voff
// land at LDS byte lds + 16 L.  Issued as inline assembly so that the
// compiler does not serialise later LDS reads behind it; the kernel orders
// it with explicit s_waitcnt vmcnt and s_barrier.
__device__ __forceinline__ void dma16(desc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voff), "s"(r) : "memory", "m0");
}

// Buffer descriptor for an operand tile starting at (row0 in the m/n
// dimension, k0).  K-major: element (r, k) at base[r*ld + k]; M/N-major:
// base[k*ld + r].  The range ends at the operand's end (clamped below 2 GiB;
// a tile never spans more, see the ABI limits), so kOOB is always out of
// range.
template <bool KM>
__device__ __forceinline__ desc_t tile_desc(const bf16* base, int64_t ld, int64_t elems,
                                            int64_t row0, int64_t k0) {
  const int64_t off = KM ? row0 * ld + k0 : k0 * ld + row0;
  const int64_t rem = (elems - off) * 2;
  const uint32_t n = rem > 0 ? (rem < 0x7FFFFFFF ? (uint32_t)rem : 0x7FFFFFFFu) : 0u;
  return make_desc(base + off, n);
}

// K-major tiles: rows of BK k values (RB = 2 BK bytes); a 256-byte bank
// window holds RPW = 256 / RB rows, and 16-byte chunk c of row r is stored at
// c ^ ((r / RPW) % CPR), so 16 consecutive rows read at one logical chunk hit
// 16 distinct 16-byte bank slots.
template <int BK>
__device__ __forceinline__ int kswz(int row, int c) {
  constexpr int RPW = 256 / (2 * BK), CPR = BK / 8;
  return c ^ ((row / RPW) % CPR);
}

// DMA of one K-major tile (ROWS x BK; 1024 / (2 BK) rows per 1 KiB instruction).
template <int ROWS, int BK, int NW>
__device__ __forceinline__ void dma_kmajor(desc_t r, uint32_t ld_bytes, int kvalid, uint32_t lds,
                                           int wave, int lane) {
  constexpr int CPR = BK / 8, RPI = 64 / CPR;           // chunks per row, rows per instruction
  constexpr int INS = ROWS / RPI, PER = INS / NW;
  static_assert(INS % NW == 0, "K-major DMA split");
  const int rl = lane / CPR, pc = lane % CPR;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int ins = wave * PER + j;
    const int row = ins * RPI + rl;
    const int lc = kswz<BK>(row, pc);
    const uint32_t voff = lc * 8 < kvalid ? (uint32_t)row * ld_bytes + (uint32_t)lc * 16u : kOOB;
    dma16(r, lds + ins * 1024, voff);
  }
}

// DMA of one M/N-major tile: BK k rows of ROWS m/n values, stored as
// ROWS/128 sub-tiles of [BK][128]; 4 rows of one sub-tile per instruction.
// With two resources (dual-B), sub-tile s comes from r[s] at the same columns.
template <int ROWS, int BK, int NW, bool DUAL>
__device__ __forceinline__ void dma_mnmajor(desc_t r0, desc_t r1, uint32_t ld_bytes, uint32_t lds,
                                            int wave, int lane) {
  constexpr int IPS = BK / 4;                        // instructions per sub-tile
  constexpr int INS = ROWS / 128 * IPS, PER = INS / NW;
  static_assert(INS % NW == 0, "M/N-major DMA split");
  const int kr = lane >> 4, pc = lane & 15;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int ins = wave * PER + j;
    const int sub = ins / IPS;
    const int k = (ins % IPS) * 4 + kr;
    const int lc = pc ^ (4 * (k & 3));
    const int col = DUAL ? lc * 8 : sub * 128 + lc * 8;
    const uint32_t voff = (uint32_t)k * ld_bytes + (uint32_t)col * 2u;
    dma16((DUAL && sub) ? r1 : r0, lds + ins * 1024, voff);
  }
}

// Fragment of a K-major tile: rows row..(32 rows by lane), k-substep kk.
template <int BK>
__device__ __forceinline__ bf16x8 frag_kmajor(const char* tile, int row, int kk, int g) {
  const int pc = kswz<BK>(row, kk * 2 + g);
  return *reinterpret_cast<const bf16x8*>(tile + row * (2 * BK) + pc * 16);
}

// Fragment of an M/N-major tile for the 32 columns starting at col0.
template <int BK>
__device__ __forceinline__ bf16x8 frag_mnmajor(const char* tile, int col0, int kk, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int col = col0 + 16 * (G & 1) + 4 * (i & 3);
  const int k = kk * 16 + 8 * (G >> 1) + (i >> 2);
  const int sub = col >> 7, c = col & 127;
  const int pc = (c >> 3) ^ (4 * (k & 3));
  const char* p = tile + sub * (BK * 256) + k * 256 + pc * 16 + (c & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 256));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <bool KM, int BK>
__device__ __forceinline__ bf16x8 frag(const char* tile, int rowcol0, int lane, int kk) {
  if constexpr (KM) return frag_kmajor<BK>(tile, rowcol0 + (lane & 31), kk, lane >> 5);
  else return frag_mnmajor<BK>(tile, rowcol0, kk, lane);
}

// Own DMAs older than the newest N instructions landed, own LDS reads
// returned, then the workgroup barrier (no memory fence: the DMAs of later
// stages stay in flight).
template <int N>
__device__ __forceinline__ void dma_lds_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ----------------------------------------------------------------------------
// Workgroup -> output tile: XCD-contiguous, then grouped along m.
// ----------------------------------------------------------------------------
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n,
                                            int& tm, int& tn) {
  constexpr int NXCD = 8, GROUP = 8;
  const int q = nblocks / NXCD, r = nblocks % NXCD;
  const int xcd = bid % NXCD, local = bid / NXCD;
  const int t = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
  const int per_group = GROUP * tiles_n;
  const int g = t / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int w = t % per_group;
  tm = first_m + w % gsize;
  tn = w / gsize;
}

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f.template operator()<I>(), ...); }(
      std::make_integer_sequence<int, N>{});
}

// Epilogue.  acc[i][j][4*b + q] is C(m, n) with
//   m = m0 + wm*WTM + i*32 + (lane & 31)
//   n = n0 + <wave column of block j> + 8*b + 4*(lane >> 5) + q
// Each output of the epilogue is staged through the (now idle) LDS as a
// row-major tile, 16-byte chunk c of staged row r at c ^ (r % chunks-per-row),
// then written back one whole row segment at a time with 16-byte stores, so
// every store instruction covers full contiguous rows.  fp32 outputs that do
// not fit the LDS in one go are written in row passes.
template <class Cfg, bool DUAL, class Epi>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[Cfg::TM][Cfg::TN], const GemmParams& p,
                                           const Epi& epi, int64_t m0, int64_t n0, int wm, int wn,
                                           int lane, int zb, char* smem, int tid) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WTM = Cfg::WTM, WTN = Cfg::WTN, BM = Cfg::BM;
  constexpr int BNL = DUAL ? Cfg::BN / 2 : Cfg::BN;
  const int lrow = lane & 31;
  const int g4 = (lane >> 5) * 4;
  const int split = (int)blockIdx.y;
  static_for<Epi::NOUT>([&]<int O>() {
    if (!epi.template has_out<O>()) return;
    using TO = typename Epi::template OutT<O>;
    constexpr int ES = sizeof(TO);
    constexpr int ROWB = BNL * ES;                 // staged row bytes
    constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
    constexpr int FIT = Cfg::SMEM_BYTES / ROWB;
    constexpr int PASS = FIT >= BM ? BM : (FIT >= 128 ? 128 : (FIT >= 64 ? 64 : 32));
    static_assert(CPR >= 8 && (CPR & (CPR - 1)) == 0, "staged row width");
    static_assert(PASS * ROWB <= Cfg::SMEM_BYTES && BM % PASS == 0, "staging pass fits the LDS");
#pragma unroll
    for (int pass = 0; pass < BM / PASS; ++pass) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // LDS free
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rl = wm * WTM + i * 32;           // first tile row of block i (uniform)
        if (rl < pass * PASS || rl >= (pass + 1) * PASS) continue;
        const int r = rl + lrow - pass * PASS;
        const int64_t m = m0 + rl + lrow;
        char* rowp = smem + r * ROWB;
#pragma unroll
        for (int j = 0; j < (DUAL ? TN / 2 : TN); ++j)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int nl = (DUAL ? wn * (WTN / 2) : wn * WTN) + j * 32 + 8 * b + g4;
            const int64_t n = n0 + nl;
            if (m < p.M && n < p.N) {
              f32x4 v;
              if constexpr (DUAL) {
                const int jj = j + TN / 2;
                const f32x4 g = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]};
                const f32x4 u = {acc[i][jj][4 * b], acc[i][jj][4 * b + 1], acc[i][jj][4 * b + 2], acc[i][jj][4 * b + 3]};
                v = epi.template value2<O>(m, n, g, u);
              } else {
                const f32x4 a = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]};
                v = epi.template value<O>(m, n, a);
              }
              const int byte = nl * ES;
              const int pc = (byte >> 4) ^ (r & (CPR - 1));
              Quad<TO>::store(reinterpret_cast<TO*>(rowp + pc * 16 + (byte & 15)), v);
            }
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // staged tile complete
      constexpr int TOTAL = PASS * CPR;
#pragma unroll 4
      for (int idx = tid; idx < TOTAL; idx += Cfg::NT) {
        const int r = idx / CPR, c = idx % CPR;
        const int64_t m = m0 + pass * PASS + r;
        const int64_t n = n0 + c * (16 / ES);
        if (m < p.M && n < p.N) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(smem + r * ROWB + ((c ^ (r & (CPR - 1))) * 16));
          *reinterpret_cast<u32x4*>(epi.template out_ptr<O>(m, n, split, zb)) = w;
        }
      }
    }
  });
}

// DMA of k-tile kt of a product into one LDS stage, by the NWL waves
// numbered wl = 0..NWL-1 (each issues its share of the 1 KiB instructions).
template <class Cfg, bool A_KM, bool B_KM, bool DUAL, int NWL>
__device__ __forceinline__ void issue_tile(const GemmParams& p, int kt, int kt_seg0, uint32_t As,
                                           int64_t m0, int64_t n0, int zb, int wl, int lane) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  const int s = kt < kt_seg0 ? 0 : 1;
  const GemmSeg& g = p.seg[s];
  const int64_t k0 = (int64_t)(kt - (s ? kt_seg0 : 0)) * BK;
  const bf16* Bp = (s == 0 && p.Bz[zb]) ? p.Bz[zb] : g.B;
  const uint32_t Bs = As + Cfg::A_BYTES;
  const int kvalid = (int)(g.K - k0);
  const desc_t ra = tile_desc<A_KM>(g.A, g.lda, g.a_elems, m0, k0);
  if constexpr (A_KM) dma_kmajor<BM, BK, NWL>(ra, (uint32_t)(g.lda * 2), kvalid, As, wl, lane);
  else dma_mnmajor<BM, BK, NWL, false>(ra, ra, (uint32_t)(g.lda * 2), As, wl, lane);
  const desc_t rb = tile_desc<B_KM>(Bp, g.ldb, g.b_elems, n0, k0);
  if constexpr (B_KM) {
    dma_kmajor<BN, BK, NWL>(rb, (uint32_t)(g.ldb * 2), kvalid, Bs, wl, lane);
  } else if constexpr (DUAL) {
    const desc_t rb2 = tile_desc<false>(g.B2, g.ldb, g.b_elems, n0, k0);
    dma_mnmajor<BN, BK, NWL, true>(rb, rb2, (uint32_t)(g.ldb * 2), Bs, wl, lane);
  } else {
    dma_mnmajor<BN, BK, NWL, false>(rb, rb, (uint32_t)(g.ldb * 2), Bs, wl, lane);
  }
}

// Column (within the B tile) of wave column wn's n-block j.
template <class Cfg, bool DUAL>
__device__ __forceinline__ int bcol_of(int wn, int j) {
  constexpr int TN = Cfg::TN, WTN = Cfg::WTN;
  if constexpr (DUAL)
    return (j < TN / 2) ? wn * (WTN / 2) + j * 32 : 128 + wn * (WTN / 2) + (j - TN / 2) * 32;
  else
    return wn * WTN + j * 32;
}

// ----------------------------------------------------------------------------
// The kernel.  DUAL: the B tile's first BN/2 columns come from seg.B and the
// last BN/2 from seg.B2 for the same BN/2 output columns; wave (wm, wn) owns
// n-blocks j < TN/2 from B and j >= TN/2 from B2 of the same columns, so an
// epilogue sees both products of an (m, n) in one lane.
// ----------------------------------------------------------------------------
template <class Cfg, bool A_KM, bool B_KM, bool DUAL, class Epi>
__global__ void __launch_bounds__(Cfg::NT)
gemm_bf16_kernel(const GemmParams p, const Epi epi) {
  constexpr int BK = Cfg::BK, NW = Cfg::NW;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WTM = Cfg::WTM;
  constexpr int BNL = DUAL ? Cfg::BN / 2 : Cfg::BN;   // output columns per tile
  constexpr int NS = Cfg::NSTAGE;
  constexpr int NDMA = (Cfg::BM + Cfg::BN) * BK / 512 / NW;  // DMA instructions per wave per stage
  static_assert(!DUAL || !B_KM, "dual-B products take N-major right operands");
  static_assert(!DUAL || Cfg::BN == 256, "dual-B tiles hold two 128-column sub-tiles");

  __shared__ __attribute__((aligned(1024))) char smem[Cfg::SMEM_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * Cfg::BM;
  const int64_t n0 = (int64_t)tn * BNL;
  const int zb = blockIdx.z;

  const int kt_seg0 = (p.seg[0].K + BK - 1) / BK;
  const int kt_total = kt_seg0 + (p.nseg > 1 ? (p.seg[1].K + BK - 1) / BK : 0);
  const int kt_begin = (int)(((int64_t)kt_total * blockIdx.y) / p.split_k);
  const int kt_end = (int)(((int64_t)kt_total * (blockIdx.y + 1)) / p.split_k);
  const int T = kt_end - kt_begin;
  const uint32_t lds0 = lds_addr(smem);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // Prologue: the first NS-1 k-tiles in flight.
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < T)
      issue_tile<Cfg, A_KM, B_KM, DUAL, NW>(p, kt_begin + s, kt_seg0, lds0 + s * Cfg::STAGE, m0, n0, zb, wave, lane);

  for (int t = 0; t < T; ++t) {
    // Wait for tile t's DMA (the newer tiles' DMAs stay in flight), then the
    // barrier: tile t is in LDS everywhere and every wave has finished
    // multiplying tile t-1, whose stage now takes tile t+NS-1.
    const int newer = min(NS - 2, T - 1 - t);
    if constexpr (NS >= 4) {
      if (newer >= 2) dma_lds_barrier<2 * NDMA>();
      else if (newer == 1) dma_lds_barrier<NDMA>();
      else dma_lds_barrier<0>();
    } else if constexpr (NS == 3) {
      if (newer >= 1) dma_lds_barrier<NDMA>();
      else dma_lds_barrier<0>();
    } else {
      dma_lds_barrier<0>();
    }
    if (t + NS - 1 < T)
      issue_tile<Cfg, A_KM, B_KM, DUAL, NW>(p, kt_begin + t + NS - 1, kt_seg0,
                                            lds0 + ((t + NS - 1) % NS) * Cfg::STAGE, m0, n0, zb, wave, lane);

    const char* As = smem + (t % NS) * Cfg::STAGE;
    const char* Bs = As + Cfg::A_BYTES;

    bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = frag<A_KM, BK>(As, wm * WTM + i * 32, lane, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = frag<B_KM, BK>(Bs, bcol_of<Cfg, DUAL>(wn, j), lane, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[nxt][i] = frag<A_KM, BK>(As, wm * WTM + i * 32, lane, kk + 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[nxt][j] = frag<B_KM, BK>(Bs, bcol_of<Cfg, DUAL>(wn, j), lane, kk + 1);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  }

  store_tile<Cfg, DUAL>(acc, p, epi, m0, n0, wm, wn, lane, zb, smem, tid);
}

}  // namespace tpk
