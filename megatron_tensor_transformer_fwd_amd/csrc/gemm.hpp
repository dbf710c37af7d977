// bf16 MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) B(k,n), fp32 accumulate,
// with a fused epilogue.
//
// Design (CDNA4-first):
//  * Workgroup tile BM x BN x BK, WM x WN wavefronts of 64 lanes; every wave
//    owns a (BM/WM) x (BN/WN) sub-tile computed with v_mfma_f32_32x32x16_bf16.
//  * Both operands are staged through LDS as rows of BK contiguous k values
//    (pitch BK+8 bf16, which keeps 16-lane groups of 16-byte reads and
//    writes on distinct banks), double-buffered: the global loads of tile
//    t+1 are in flight while the MFMAs of tile t run, and one barrier per
//    k-tile separates the two buffers.
//  * An operand whose k index is contiguous in memory (K-major) is loaded in
//    16-byte chunks along k.  An operand whose m/n index is contiguous
//    (M- or N-major: the weights of the forward products, and both operands
//    of the weight-gradient products) is loaded as R x 8 blocks with 16-byte
//    row loads and transposed in registers with v_perm_b32 before the LDS
//    write, so global loads stay 16-byte and coalesced in every layout.
//  * Global loads go through buffer resources: reads past the end of an
//    operand return zero, which pads the ragged k tail; K-major tails inside a
//    row are masked explicitly.
//  * The MFMA's first operand is the B tile and its second the A tile, so the
//    32x32 accumulator hands each lane 4 consecutive n for one m: epilogues
//    work on (m, n..n+3) quads and store 8 or 16 bytes at a time.
//  * Workgroup ids are remapped so that the tiles one XCD (of 8) runs are
//    contiguous, then grouped along m for L2 reuse of the B panels.
#pragma once
#include "common.hpp"

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

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int LDK = BK + 8;
  static constexpr int SMEM_BYTES = 2 * (BM + BN) * LDK * 2;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 16 == 0, "tile shape");
};

// ----------------------------------------------------------------------------
// Operand staging (global -> registers -> LDS)
// ----------------------------------------------------------------------------

// K-major: 16-byte chunks along k.  Chunk q of the tile is row q / (BK/8),
// chunk q % (BK/8); eight lanes cover one 128-byte row segment.
template <int ROWS, int BK, int NT, int LDK>
struct KMajorStage {
  static constexpr int CPR = BK / 8;
  static constexpr int N = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "K-major staging split");
  u32x4 v[N];

  __device__ __forceinline__ void load(rsrc_t r, uint32_t ld_bytes, int kvalid, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT;
      const int row = q / CPR, kc = q % CPR;
      u32x4 x = buf_load16(r, (uint32_t)row * ld_bytes + (uint32_t)kc * 16u);
      if (kc * 8 >= kvalid) x = u32x4{0u, 0u, 0u, 0u};
      v[i] = x;
    }
  }
  __device__ __forceinline__ void store(bf16* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT;
      const int row = q / CPR, kc = q % CPR;
      *reinterpret_cast<u32x4*>(lds + row * LDK + kc * 8) = v[i];
    }
  }
};

// M/N-major: each thread loads R consecutive k rows of 8 consecutive m/n
// values (R 16-byte loads), transposes the R x 8 block in registers and
// writes 8 LDS rows of R k values.  Lanes kb = tid % (BK/R) share a column
// chunk, so every wave load instruction reads 128-byte row segments and every
// LDS write instruction covers whole 128-byte row segments.
template <int ROWS, int BK, int NT, int LDK>
struct MNMajorStage {
  static constexpr int R = ROWS * BK / 8 / NT;
  static constexpr int KB = BK / R;
  static_assert(R == 2 || R == 4 || R == 8, "M/N-major staging split");
  static_assert((ROWS / 8) * KB == NT, "M/N-major staging covers the tile");
  u32x4 v[R];

  __device__ __forceinline__ void load(rsrc_t r, uint32_t ld_bytes, int tid) {
    const int kb = tid % KB, nb = tid / KB;
#pragma unroll
    for (int j = 0; j < R; ++j)
      v[j] = buf_load16(r, (uint32_t)(kb * R + j) * ld_bytes + (uint32_t)nb * 16u);
  }

  __device__ __forceinline__ void store(bf16* lds, int tid) const {
    const int kb = tid % KB, nb = tid / KB;
    // element c of row j sits in half (c & 1) of dword c >> 1 of v[j]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      bf16* dst = lds + (nb * 8 + c) * LDK + kb * R;
      if constexpr (R == 8) {
        u32x4 o;
        o[0] = __builtin_amdgcn_perm(v[1][c >> 1], v[0][c >> 1], sel);
        o[1] = __builtin_amdgcn_perm(v[3][c >> 1], v[2][c >> 1], sel);
        o[2] = __builtin_amdgcn_perm(v[5][c >> 1], v[4][c >> 1], sel);
        o[3] = __builtin_amdgcn_perm(v[7][c >> 1], v[6][c >> 1], sel);
        *reinterpret_cast<u32x4*>(dst) = o;
      } else if constexpr (R == 4) {
        u32x2 o;
        o[0] = __builtin_amdgcn_perm(v[1][c >> 1], v[0][c >> 1], sel);
        o[1] = __builtin_amdgcn_perm(v[3][c >> 1], v[2][c >> 1], sel);
        *reinterpret_cast<u32x2*>(dst) = o;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(v[1][c >> 1], v[0][c >> 1], sel);
      }
    }
  }
};

template <bool KM, int ROWS, int BK, int NT, int LDK>
struct StageOf;
template <int ROWS, int BK, int NT, int LDK>
struct StageOf<true, ROWS, BK, NT, LDK> { using type = KMajorStage<ROWS, BK, NT, LDK>; };
template <int ROWS, int BK, int NT, int LDK>
struct StageOf<false, ROWS, BK, NT, LDK> { using type = MNMajorStage<ROWS, BK, NT, LDK>; };

// Buffer resource for the tile of an operand starting at (row0 in the m/n
// dimension, k0).  K-major: element (r, k) at base[r*ld + k]; M/N-major:
// element (r, k) at base[k*ld + r].  The resource starts at the tile origin
// so that in-tile byte offsets stay small for any operand size.
template <bool KM>
__device__ __forceinline__ rsrc_t tile_rsrc(const bf16* base, int64_t ld, int64_t elems,
                                            int64_t row0, int64_t k0) {
  const int64_t off = KM ? row0 * ld + k0 : k0 * ld + row0;
  const int64_t rem = elems - off;
  return make_rsrc(base + off, rem > 0 ? (uint64_t)rem * 2u : 0u);
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

// ----------------------------------------------------------------------------
// The kernel.  DUAL: the B tile's first BN/2 rows come from seg.B and the
// last BN/2 from seg.B2 for the same BN/2 output columns; wave (wm, wn) owns
// n-blocks j < TN/2 from B and j >= TN/2 from B2 of the same columns, so an
// epilogue sees both products of an (m, n) in one lane.
// ----------------------------------------------------------------------------
template <class Cfg, bool A_KM, bool B_KM, bool DUAL, class Epi>
__global__ void __launch_bounds__(Cfg::NT)
gemm_bf16_kernel(const GemmParams p, const Epi epi) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
  constexpr int LDK = Cfg::LDK, TM = Cfg::TM, TN = Cfg::TN;
  constexpr int WTM = Cfg::WTM, WTN = Cfg::WTN;
  constexpr int BNL = DUAL ? BN / 2 : BN;          // output columns per tile
  constexpr int BROWS = DUAL ? BN / 2 : BN;        // B rows per staged matrix
  using AStage = typename StageOf<A_KM, BM, BK, NT, LDK>::type;
  using BStage = typename StageOf<B_KM, BROWS, BK, NT, LDK>::type;

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BN) * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BNL;
  const int zb = blockIdx.z;

  // K-tiles of every segment, split over blockIdx.y
  int kt_seg0 = (p.seg[0].K + BK - 1) / BK;
  int kt_total = kt_seg0 + (p.nseg > 1 ? (p.seg[1].K + BK - 1) / BK : 0);
  const int kt_begin = (int)(((int64_t)kt_total * blockIdx.y) / p.split_k);
  const int kt_end = (int)(((int64_t)kt_total * (blockIdx.y + 1)) / p.split_k);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  AStage sa;
  BStage sb, sb2;

  auto load_tile = [&](int kt) {
    const int s = kt < kt_seg0 ? 0 : 1;
    const GemmSeg& g = p.seg[s];
    const int64_t k0 = (int64_t)(kt - (s ? kt_seg0 : 0)) * BK;
    const bf16* Bp = (s == 0 && p.Bz[zb]) ? p.Bz[zb] : g.B;
    const rsrc_t ra = tile_rsrc<A_KM>(g.A, g.lda, g.a_elems, m0, k0);
    const rsrc_t rb = tile_rsrc<B_KM>(Bp, g.ldb, g.b_elems, n0, k0);
    const int kvalid = (int)(g.K - k0);
    if constexpr (A_KM) sa.load(ra, (uint32_t)(g.lda * 2), kvalid, tid);
    else sa.load(ra, (uint32_t)(g.lda * 2), tid);
    if constexpr (B_KM) sb.load(rb, (uint32_t)(g.ldb * 2), kvalid, tid);
    else sb.load(rb, (uint32_t)(g.ldb * 2), tid);
    if constexpr (DUAL) {
      const rsrc_t rb2 = tile_rsrc<B_KM>(g.B2, g.ldb, g.b_elems, n0, k0);
      if constexpr (B_KM) sb2.load(rb2, (uint32_t)(g.ldb * 2), kvalid, tid);
      else sb2.load(rb2, (uint32_t)(g.ldb * 2), tid);
    }
  };
  auto store_tile = [&](int buf) {
    bf16* As = smem + buf * (BM + BN) * LDK;
    bf16* Bs = As + BM * LDK;
    sa.store(As, tid);
    sb.store(Bs, tid);
    if constexpr (DUAL) sb2.store(Bs + BROWS * LDK, tid);
  };

  if (kt_begin < kt_end) {
    load_tile(kt_begin);
    store_tile(0);
  }
  __syncthreads();

  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    if (more) load_tile(kt + 1);

    const bf16* As = smem + buf * (BM + BN) * LDK;
    const bf16* Bs = As + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * WTM + i * 32 + lrow) * LDK + kk + lk);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int brow;
        if constexpr (DUAL)
          brow = (j < TN / 2) ? wn * (WTN / 2) + j * 32 : BROWS + wn * (WTN / 2) + (j - TN / 2) * 32;
        else
          brow = wn * WTN + j * 32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (brow + lrow) * LDK + kk + lk);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: acc[i][j][4*b + q] is C(m, n) with
  //   m = m0 + wm*WTM + i*32 + (lane & 31)
  //   n = n0 + <wave column of block j> + 8*b + 4*(lane >> 5) + q
  const int g4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm * WTM + i * 32 + lrow;
    if constexpr (DUAL) {
#pragma unroll
      for (int j = 0; j < TN / 2; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t n = n0 + wn * (WTN / 2) + j * 32 + 8 * b + g4;
          const f32x4 vg = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]};
          const int jj = j + TN / 2;
          const f32x4 vu = {acc[i][jj][4 * b], acc[i][jj][4 * b + 1], acc[i][jj][4 * b + 2], acc[i][jj][4 * b + 3]};
          if (m < p.M && n < p.N) epi.apply2(m, n, vg, vu);
        }
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t n = n0 + wn * WTN + j * 32 + 8 * b + g4;
          const f32x4 v = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]};
          if (m < p.M && n < p.N) epi.apply(m, n, v, (int)blockIdx.y, zb);
        }
    }
  }
}

}  // namespace tpk
