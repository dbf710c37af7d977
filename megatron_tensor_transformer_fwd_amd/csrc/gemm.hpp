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
//  * A and B tiles stream through two LDS rings (NSA and NSB slots) with one
//    barrier per k-tile (pipeline at the kernel); explicit s_waitcnt vmcnt +
//    s_barrier (no fences) order the rings.
//  * A K-major operand (k contiguous in memory) is kept as rows of BK k with
//    a 16-byte-chunk XOR swizzle (kswz); MFMA fragments are single
//    ds_read_b128s, bank-conflict free for 16 rows.
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
#include <type_traits>
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
  // Strided batches (grid z = batch, e.g. the shards of a TP layer held on one
  // GPU): batch z reads segment 0's A at A + z*a_zs and B (B2) at B + z*b_zs,
  // and its outputs are row-stacked: the epilogue sees row m + z*z_rows.
  int64_t a_zs, b_zs;
  int z_rows;
  int tiles_m, tiles_n;
  int split_k;         // K-tile ranges (grid y)
  int tile_base;       // the grid covers tiles tile_base .. tile_base + gridDim.x - 1 of the grouped order
};

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64, int NSA_ = 2, int NSB_ = 2, int SPA_ = 1,
          int SPB_ = 1, int ROT_ = 0, int BARQ_ = -1>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int NSA = NSA_, NSB = NSB_;          // LDS stages of the A and B rings
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int KK = BK / 16;                   // MFMA k-steps per k-tile
  static constexpr int SPA = SPA_, SPB = SPB_;         // k-steps each ring's DMA is spread over
  static constexpr bool ROT = ROT_ != 0;               // per-XCD rotation of the k-tile order
  static constexpr int BARQ = BARQ_ < 0 ? TM * TN / 2 : BARQ_;   // last-k-step MFMAs before the barrier
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int B_RING = NSA * A_BYTES;         // LDS offset of the B ring
  static constexpr int SMEM_BYTES = NSA * A_BYTES + NSB * B_BYTES;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "M/N-major tiles are 128-wide sub-tiles");
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(KK % 2 == 0, "fragment double buffer parity");
  // A ring with one tile of look-ahead must land by this k-tile's barrier,
  // so its DMA is issued before the last k-step; with more look-ahead it
  // may spread over the whole k-tile.
  static_assert(SPA >= 1 && SPA <= KK && (NSA > 2 || SPA < KK), "A DMA spread");
  static_assert(SPB >= 1 && SPB <= KK && (NSB > 2 || SPB < KK), "B DMA spread");
  static_assert(BARQ >= 0 && BARQ < TM * TN, "barrier position");
  static_assert(NSA >= 2 && NSB >= 2 && SMEM_BYTES <= 160 * 1024, "LDS stages");
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
constexpr int kTileGroup = 8;

// Tile at position t of the grouped order: groups of 8 m-tiles, and inside a
// group the 8 m-tiles of one n-tile after another.
__host__ __device__ inline void tile_of(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kTileGroup * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kTileGroup;
  const int gsize = min(tiles_m - first_m, kTileGroup);
  const int w = t % per_group;
  tm = first_m + w % gsize;
  tn = w / gsize;
}

// Position of tile (tm, tn) in the grouped order (the inverse of tile_of).
__host__ __device__ inline int position_of(int tm, int tn, int tiles_m, int tiles_n) {
  const int g = tm / kTileGroup;
  const int first_m = g * kTileGroup;
  const int gsize = min(tiles_m - first_m, kTileGroup);
  return g * kTileGroup * tiles_n + tn * gsize + (tm - first_m);
}

// Workgroup -> (tile position lx, K split ly, batch lz) and its XCD.  The
// hardware hands consecutive workgroup ids (x fastest, then y, then z) to
// the 8 XCDs in turn; the whole grid is remapped so that each XCD runs one
// contiguous range of the logical order (split slowest, then batch, then the
// grouped tile order).  The tiles an XCD runs together then share operand
// slices in its L2: the same K range of a split product, the same batch.
// A one-dimensional grid keeps the plain XCD-contiguous tile order.
__device__ __forceinline__ void grid_coords(int& lx, int& ly, int& lz, int& xcd) {
  constexpr int NXCD = 8;
  const int nx = (int)gridDim.x, ny = (int)gridDim.y, nz = (int)gridDim.z;
  const int total = nx * ny * nz;
  const int lin = (int)blockIdx.x + nx * ((int)blockIdx.y + ny * (int)blockIdx.z);
  const int q = total / NXCD, r = total % NXCD;
  xcd = lin % NXCD;
  const int local = lin / NXCD;
  const int t = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
  lx = t % nx;
  const int t2 = t / nx;
  lz = t2 % nz;
  ly = t2 / nz;
}

// The same remap for workgroup lin of a one-dimensional range of `total`.
__device__ __forceinline__ void coords_1d(int lin, int total, int& lx, int& xcd) {
  constexpr int NXCD = 8;
  const int q = total / NXCD, r = total % NXCD;
  xcd = lin % NXCD;
  const int local = lin / NXCD;
  lx = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f.template operator()<I>(), ...); }(
      std::make_integer_sequence<int, N>{});
}

// An epilogue may also reduce each staged output row of the tile (its values
// as stored) by defining ROW_REDUCE and row_reduce<O, NT, PASS, CPR, BNL>().
template <class E, class = void> struct epi_row_reduce : std::false_type {};
template <class E> struct epi_row_reduce<E, std::void_t<decltype(E::ROW_REDUCE)>> : std::true_type {};

// An epilogue whose output O the next product reads at once defines
// keep<O>() true: that output is stored without the streaming hint.
template <class E, int O> constexpr bool epi_keep() {
  if constexpr (requires { E::template keep<O>(); }) return E::template keep<O>();
  else return false;
}

// An epilogue that reads other tensors at the output positions (a saved
// activation) defines Aux, aux_load<O>(m, n) and value_aux<O>(m, n, v, aux):
// the staging loop then issues one 32-row block's loads together before
// using any of them, instead of one load-and-wait per quad.
template <class E, class = void> struct epi_aux : std::false_type {};
template <class E> struct epi_aux<E, std::void_t<typename E::Aux>> : std::true_type {};
template <class E, bool = epi_aux<E>::value> struct epi_aux_type { struct type {}; };
template <class E> struct epi_aux_type<E, true> { using type = typename E::Aux; };

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
                                           int lane, int zb, int split, char* smem, int tid) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WTM = Cfg::WTM, WTN = Cfg::WTN, BM = Cfg::BM;
  constexpr int BNL = DUAL ? Cfg::BN / 2 : Cfg::BN;
  const int lrow = lane & 31;
  const int g4 = (lane >> 5) * 4;
  const int64_t zrow = (int64_t)zb * p.z_rows;     // row offset of this batch's outputs
  // A tile wholly inside the output (every tile but the ragged last ones)
  // takes a copy of the staging without bounds checks: each check is a branch
  // that cuts the staging loop into one block per quad, so the activation
  // math of different quads could not be interleaved.
  const bool inside = m0 + BM <= p.M && n0 + BNL <= p.N;
  // The main loop's trailing DMAs (issued past the last k-tile into slots no
  // one reads) must land before the LDS is reused; after that, each pass
  // waits only for the LDS reads of the one before, so its activation math
  // runs while the previous pass's stores drain.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  auto stage_all = [&](auto guard) {
    constexpr bool G = decltype(guard)::value;
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
          constexpr int JN = DUAL ? TN / 2 : TN;
          using AuxT = typename epi_aux_type<Epi>::type;
          [[maybe_unused]] AuxT ax[JN][4];
          if constexpr (epi_aux<Epi>::value) {
#pragma unroll
            for (int j = 0; j < JN; ++j)
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                const int64_t n = n0 + wn * WTN + j * 32 + 8 * b + g4;
                if (!G || (m < p.M && n < p.N)) ax[j][b] = epi.template aux_load<O>(m + zrow, n);
              }
          }
#pragma unroll
          for (int j = 0; j < JN; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int nl = (DUAL ? wn * (WTN / 2) : wn * WTN) + j * 32 + 8 * b + g4;
              const int64_t n = n0 + nl;
              if (!G || (m < p.M && n < p.N)) {
                f32x4 v;
                if constexpr (epi_aux<Epi>::value) {
                  static_assert(!DUAL, "auxiliary inputs in single-B products only");
                  const f32x4 a = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]};
                  v = epi.template value_aux<O>(m + zrow, n, a, ax[j][b]);
                } else if constexpr (DUAL) {
                  const int jj = j + TN / 2;
                  const f32x4 g = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]};
                  const f32x4 u = {acc[i][jj][4 * b], acc[i][jj][4 * b + 1], acc[i][jj][4 * b + 2], acc[i][jj][4 * b + 3]};
                  v = epi.template value2<O>(m + zrow, n, g, u);
                } else {
                  const f32x4 a = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]};
                  v = epi.template value<O>(m + zrow, n, a);
                }
                const int byte = nl * ES;
                const int pc = (byte >> 4) ^ (r & (CPR - 1));
                Quad<TO>::store(reinterpret_cast<TO*>(rowp + pc * 16 + (byte & 15)), v);
              }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // staged tile complete
        if constexpr (epi_row_reduce<Epi>::value)     // per-row statistics of the staged (stored) values
          epi.template row_reduce<O, Cfg::NT, PASS, CPR, BNL>(smem, pass * PASS, m0, n0, p, tid);
        constexpr int TOTAL = PASS * CPR;
#pragma unroll 4
        for (int idx = tid; idx < TOTAL; idx += Cfg::NT) {
          const int r = idx / CPR, c = idx % CPR;
          const int64_t m = m0 + pass * PASS + r;
          const int64_t n = n0 + c * (16 / ES);
          if (!G || (m < p.M && n < p.N)) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(smem + r * ROWB + ((c ^ (r & (CPR - 1))) * 16));
            // streaming store: the tile is not read again by this product, and
            // its dirty lines would otherwise compete with the operand stream
            // (plain stores for an output the epilogue keeps for its next reader)
            u32x4* dst = reinterpret_cast<u32x4*>(epi.template out_ptr<O>(m + zrow, n, split, zb));
            if constexpr (epi_keep<Epi, O>()) *dst = w;
            else __builtin_nontemporal_store(w, dst);
          }
        }
      }
    });
  };
  if (inside) stage_all(std::false_type{});
  else stage_all(std::true_type{});
}

// Operand description kept in registers for the whole kernel (the kernel
// argument block is read once).
struct SegRegs {
  const bf16* A;
  const bf16* B;
  const bf16* B2;
  int64_t lda, ldb, a_elems, b_elems;
  int K;
};

__device__ __forceinline__ SegRegs seg_regs(const GemmSeg& g) {
  return SegRegs{g.A, g.B, g.B2, g.lda, g.ldb, g.a_elems, g.b_elems, g.K};
}

// The LDS DMA of one operand's k-tile into one slot of its ring, as N
// instructions per wave; issue<J0, J1>() sends instructions [J0, J1), so a
// tile's loads can be spread over several MFMA k-steps.  IS_A selects the
// left operand (ROWS = BM, layout A_KM) or the right one (ROWS = BN, layout
// B_KM; dual-B products take their two 128-column halves from B and B2).
template <class Cfg, bool KM, bool IS_A, bool DUAL>
struct OperandDma {
  static constexpr int BK = Cfg::BK, NW = Cfg::NW;
  static constexpr int ROWS = IS_A ? Cfg::BM : Cfg::BN;
  static constexpr int N = ROWS * BK * 2 / 1024 / NW;
  static constexpr bool TWO = !IS_A && DUAL;
  static_assert(N * NW * 1024 == ROWS * BK * 2, "DMA split");
  desc_t r0, r1;
  uint32_t ld_b;
  uint32_t lds;
  int kvalid;

  // k-tile kt (counted over both K segments) at tile-local row row0.
  __device__ __forceinline__ OperandDma(const SegRegs& g0, const SegRegs& g1, const bf16* bz, int kt,
                                        int kt_seg0, uint32_t lds_slot, int64_t row0) {
    const bool hi = kt >= kt_seg0;
    const SegRegs& g = hi ? g1 : g0;
    const int64_t k0 = (int64_t)(kt - (hi ? kt_seg0 : 0)) * BK;
    kvalid = (int)(g.K - k0);
    lds = lds_slot;
    if constexpr (IS_A) {
      ld_b = (uint32_t)(g.lda * 2);
      r0 = tile_desc<KM>(g.A, g.lda, g.a_elems, row0, k0);
      r1 = r0;
    } else {
      const bf16* Bp = (!hi && bz) ? bz : g.B;
      ld_b = (uint32_t)(g.ldb * 2);
      r0 = tile_desc<KM>(Bp, g.ldb, g.b_elems, row0, k0);
      if constexpr (TWO) r1 = tile_desc<false>(g.B2, g.ldb, g.b_elems, row0, k0);
      else r1 = r0;
    }
  }

  // Instruction j of the wave: its buffer offset, resource and LDS block.
  __device__ __forceinline__ uint32_t voff_of(int j, int wave, int lane) const {
    const int ins = wave * N + j;
    if constexpr (KM) {
      // K-major: 1 KiB = 1024 / (2 BK) rows of BK k values.
      constexpr int CPR = BK / 8, RPI = 64 / CPR;
      const int row = ins * RPI + lane / CPR;
      const int lc = kswz<BK>(row, lane % CPR);
      return lc * 8 < kvalid ? (uint32_t)row * ld_b + (uint32_t)lc * 16u : kOOB;
    } else {
      // M/N-major: 4 k rows of one [BK][128] sub-tile.
      constexpr int IPS = BK / 4;
      const int sub = ins / IPS;
      const int k = (ins % IPS) * 4 + (lane >> 4);
      const int lc = (lane & 15) ^ (4 * (k & 3));
      const int col = TWO ? lc * 8 : sub * 128 + lc * 8;
      return (uint32_t)k * ld_b + (uint32_t)col * 2u;
    }
  }
  __device__ __forceinline__ desc_t rsrc_of(int j, int wave) const {
    if constexpr (TWO) return ((wave * N + j) / (BK / 4)) ? r1 : r0;
    else return r0;
  }
  __device__ __forceinline__ uint32_t lds_of(int j, int wave) const {
    return lds + (uint32_t)((wave * N + j) * 1024);
  }

  template <int J0, int J1>
  __device__ __forceinline__ void issue(int wave, int lane) const {
    static_for<J1 - J0>([&]<int I>() {
      constexpr int J = J0 + I;
      dma16(rsrc_of(J, wave), lds_of(J, wave), voff_of(J, wave, lane));
    });
  }
};

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
//
// Pipeline.  A and B tiles live in two LDS rings of NSA and NSB slots; the
// DMA of A k-tile t+NSA-1 and of B k-tile t+NSB-1 is issued during k-tile t,
// so each operand has NS-1 tiles in flight (with the 160 KiB of LDS a
// 256 x 256 tile affords three A slots and two B slots).  Every k-tile is KK
// MFMA k-steps of TM x TN MFMAs whose instruction stream is written out in
// groups the compiler may not reorder across (sched_barrier): after each
// MFMA, its share of the next k-step's fragment reads and of the DMA
// (each ring's spread over its first SPA / SPB k-steps, the operand with
// fewer slots first).  In the last k-step, after BARQ MFMAs, the wave waits until its
// DMAs of tile t+1 have landed and its LDS reads have returned, then the
// workgroup barrier; the remaining MFMAs carry the reads of tile t+1's first
// k-step.  After that barrier no wave reads tile t's slots again, so later
// DMAs may refill them.  DMAs are issued for every t, past the last tile
// with an empty or out-of-range source (into slots never read again), which
// keeps the number of loads in flight, and so every vmcnt, static.  With ROT
// the k-tile order of a workgroup starts at an offset set by its XCD, so the
// eight XCDs stream different k-columns of the operands at any moment
// (deterministic: each tile always sums in the same order).
// ----------------------------------------------------------------------------
template <class Cfg, bool A_KM, bool B_KM, bool DUAL, class Epi>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const Epi& epi, int lx, int split, int zb, int xcd,
                                          char* smem) {
  constexpr int BK = Cfg::BK;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WTM = Cfg::WTM;
  constexpr int BNL = DUAL ? Cfg::BN / 2 : Cfg::BN;   // output columns per tile
  constexpr int NSA = Cfg::NSA, NSB = Cfg::NSB, KK = Cfg::KK, BARQ = Cfg::BARQ;
  constexpr int LA = NSA - 1, LB = NSB - 1;           // tiles of look-ahead per ring
  constexpr int Q = TM * TN;                          // MFMAs per k-step
  constexpr int NRD = TM + TN;                        // fragments per k-step
  using DmaA = OperandDma<Cfg, A_KM, true, DUAL>;
  using DmaB = OperandDma<Cfg, B_KM, false, DUAL>;
  constexpr int NA = DmaA::N, NB = DmaB::N, ND = NA + NB;
  constexpr bool B_FIRST = LB <= LA;                  // per tile, the nearer tile's DMA first
  // Issue plan: ring X's N instructions spread evenly over its first SP
  // k-steps, and within a k-step over the Q MFMAs (after MFMA q).
  constexpr auto upto = [](int n, int sp, int kk, int q) {   // issued at or before (kk, q)
    if (kk < 0) return 0;
    if (kk >= sp) return n;
    const int c0 = kk * n / sp, c1 = (kk + 1) * n / sp;
    return c0 + (q + 1) * (c1 - c0) / Q;
  };
  constexpr auto before = [upto](int n, int sp, int kk, int q) {   // issued before (kk, q)
    return q > 0 ? upto(n, sp, kk, q - 1) : upto(n, sp, kk - 1, Q - 1);
  };
  // At this k-tile's barrier (before MFMA BARQ of the last k-step) the ring
  // with one tile of look-ahead must have landed; the own DMAs issued after
  // its last instruction (the other ring's) may still be in flight.  In the
  // prologue, whole tiles were issued: the later tiles of each ring.
  constexpr int VM_PRO = (LA - 1) * NA + (LB - 1) * NB;
  // At k-tile t's barrier the DMAs of tile t+1 must have landed: the own DMAs
  // allowed in flight are those issued after the last one of tile t+1.  Found
  // by walking the issue order of a steady-state k-tile and its predecessors.
  constexpr int VM_SIM = [=]() {
    constexpr int L = LA > LB ? LA : LB;
    const int t = L + 1;                         // a steady-state k-tile
    int count = 0, after = -1;                   // instructions so far; position after tile t+1's last
    for (int u = t + 1 - L; u <= t; ++u)
      for (int kk = 0; kk < KK; ++kk)
        for (int q = 0; q < Q; ++q) {
          if (u == t && kk == KK - 1 && q == BARQ) return count - after;
          for (int r = 0; r < 2; ++r) {
            const bool is_b = (r == 0) == B_FIRST;
            const int n = is_b ? NB : NA, sp = is_b ? Cfg::SPB : Cfg::SPA, look = is_b ? LB : LA;
            const int k = upto(n, sp, kk, q) - before(n, sp, kk, q);
            count += k;
            if (k > 0 && u + look == t + 1) after = count;
          }
        }
    return -1;
  }();
  constexpr int VM_LOOP_OLD = [=]() {
    const int NN = B_FIRST ? NB : NA, SN = B_FIRST ? Cfg::SPB : Cfg::SPA;   // near ring
    const int NF = B_FIRST ? NA : NB, SF = B_FIRST ? Cfg::SPA : Cfg::SPB;   // far ring
    const bool far_deadline = (B_FIRST ? LA : LB) == 1;
    // position of the near ring's last instruction
    int lk = 0, lq = 0;
    for (int kk = 0; kk < KK; ++kk)
      for (int q = 0; q < Q; ++q)
        if (upto(NN, SN, kk, q) == NN && before(NN, SN, kk, q) < NN) { lk = kk; lq = q; }
    if (far_deadline) return 0;             // both rings due at this barrier
    // far-ring instructions after (lk, lq) (those at (lk, lq) come after it)
    // and before the barrier
    return upto(NF, SF, KK - 1, BARQ - 1) - before(NF, SF, lk, lq);
  }();
  static_assert(NSA != 2 && NSB != 2 || VM_SIM == VM_LOOP_OLD, "issue-order walk agrees with the one-ring rule");
  constexpr int VM_LOOP = VM_SIM;
  static_assert(VM_PRO <= 63 && VM_LOOP >= 0 && VM_LOOP <= 63, "vmcnt range");
  static_assert(!DUAL || !B_KM, "dual-B products take N-major right operands");
  static_assert(!DUAL || Cfg::BN == 256, "dual-B tiles hold two 128-column sub-tiles");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

  int tm, tn;
  tile_of(p.tile_base + lx, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * Cfg::BM;
  const int64_t n0 = (int64_t)tn * BNL;

  SegRegs g0 = seg_regs(p.seg[0]);
  const SegRegs g1 = seg_regs(p.seg[1]);
  g0.A += zb * p.a_zs;
  g0.B += zb * p.b_zs;
  if (g0.B2) g0.B2 += zb * p.b_zs;
  const bf16* bz = zb < 3 ? p.Bz[zb] : nullptr;
  const int kt_seg0 = (g0.K + BK - 1) / BK;
  const int kt_total = kt_seg0 + (p.nseg > 1 ? (g1.K + BK - 1) / BK : 0);
  const int kt_begin = (int)(((int64_t)kt_total * split) / p.split_k);
  const int kt_end = (int)(((int64_t)kt_total * (split + 1)) / p.split_k);
  const int T = kt_end - kt_begin;
  const uint32_t lds0 = lds_addr(smem);
  // k-tile processed at step t (t >= T: past the end, loads that are never read)
  const int rot = (Cfg::ROT && T > 0) ? (int)(((int64_t)xcd * T) / 8) : 0;
  auto kt_of = [&](int t) {
    const int u = t + rot;
    return kt_begin + (u >= T ? u - T : u);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  auto slot_a = [&](int t) { return (uint32_t)((t % NSA) * Cfg::A_BYTES); };
  auto slot_b = [&](int t) { return (uint32_t)(Cfg::B_RING + (t % NSB) * Cfg::B_BYTES); };
  auto dma_a = [&](int t) { return DmaA(g0, g1, bz, kt_of(t), kt_seg0, lds0 + slot_a(t), m0); };
  auto dma_b = [&](int t) { return DmaB(g0, g1, bz, kt_of(t), kt_seg0, lds0 + slot_b(t), n0); };
  // Fragment r of a k-step, in the order the MFMAs consume them:
  // A block 0, B blocks 0..TN-1, A blocks 1..TM-1.
  auto read_frag = [&]<int r>(bf16x8(&fa)[TM], bf16x8(&fb)[TN], const char* As, const char* Bs, int kk) {
    if constexpr (r == 0) fa[0] = frag<A_KM, BK>(As, wm * WTM, lane, kk);
    else if constexpr (r <= TN) fb[r - 1] = frag<B_KM, BK>(Bs, bcol_of<Cfg, DUAL>(wn, r - 1), lane, kk);
    else fa[r - TN] = frag<A_KM, BK>(As, wm * WTM + (r - TN) * 32, lane, kk);
  };

  bf16x8 fa[2][TM], fb[2][TN];
  if (T > 0) {
    // Prologue: A tiles 0..LA-1 and B tiles 0..LB-1 in flight, in the order
    // the loop keeps, then tile 0 visible to every wave.
#pragma unroll
    for (int s = 0; s < (LA > LB ? LA : LB); ++s) {
      if (B_FIRST) {
        if (s < LB) dma_b(s).template issue<0, NB>(wave, lane);
        if (s < LA) dma_a(s).template issue<0, NA>(wave, lane);
      } else {
        if (s < LA) dma_a(s).template issue<0, NA>(wave, lane);
        if (s < LB) dma_b(s).template issue<0, NB>(wave, lane);
      }
    }
    dma_lds_barrier<VM_PRO>();
    static_for<NRD>([&]<int r>() {
      read_frag.template operator()<r>(fa[0], fb[0], smem + slot_a(0), smem + slot_b(0), 0);
    });
  }

  for (int t = 0; t < T; ++t) {
    const DmaA da = dma_a(t + LA);
    const DmaB db = dma_b(t + LB);
    const char* a_cur = smem + slot_a(t);
    const char* b_cur = smem + slot_b(t);
    const char* a_next = smem + slot_a(t + 1);
    const char* b_next = smem + slot_b(t + 1);
    static_for<KK>([&]<int kk>() {
      constexpr int cur = kk & 1, nxt = cur ^ 1;
      constexpr bool last = kk + 1 == KK;
      constexpr int QS = last ? BARQ : 0;             // reads start after MFMA QS
      const char* ra = last ? a_next : a_cur;
      const char* rb = last ? b_next : b_cur;
      constexpr int rkk = last ? 0 : kk + 1;
      static_for<Q>([&]<int q>() {
        constexpr int i = q / TN, j = q % TN;
        if constexpr (last && q == BARQ) dma_lds_barrier<VM_LOOP>();
        // With two waves per SIMD the MFMA issue is raised above the other
        // wave's memory instructions; with one wave per SIMD it has no peer.
        if constexpr (Cfg::NW > 4) __builtin_amdgcn_s_setprio(1);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
        if constexpr (Cfg::NW > 4) __builtin_amdgcn_s_setprio(0);
        if constexpr (q >= QS) {
          constexpr int r0 = (q - QS) * NRD / (Q - QS), r1 = (q - QS + 1) * NRD / (Q - QS);
          static_for<r1 - r0>([&]<int rr>() {
            read_frag.template operator()<r0 + rr>(fa[nxt], fb[nxt], ra, rb, rkk);
          });
        }
        // This MFMA's share of the DMA: the nearer ring's first, then the
        // farther ring's.
        constexpr int b0 = before(NB, Cfg::SPB, kk, q), b1 = upto(NB, Cfg::SPB, kk, q);
        constexpr int a0 = before(NA, Cfg::SPA, kk, q), a1 = upto(NA, Cfg::SPA, kk, q);
        if constexpr (B_FIRST) {
          if constexpr (b1 > b0) db.template issue<b0, b1>(wave, lane);
          if constexpr (a1 > a0) da.template issue<a0, a1>(wave, lane);
        } else {
          if constexpr (a1 > a0) da.template issue<a0, a1>(wave, lane);
          if constexpr (b1 > b0) db.template issue<b0, b1>(wave, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }

  store_tile<Cfg, DUAL>(acc, p, epi, m0, n0, wm, wn, lane, zb, split, smem, tid);
}

template <class Cfg, bool A_KM, bool B_KM, bool DUAL, class Epi>
__global__ void __launch_bounds__(Cfg::NT)
gemm_bf16_kernel(const GemmParams p, const Epi epi) {
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::SMEM_BYTES];
  int lx, split, zb, xcd;
  grid_coords(lx, split, zb, xcd);
  gemm_tile<Cfg, A_KM, B_KM, DUAL, Epi>(p, epi, lx, split, zb, xcd, smem);
}

// Two independent products in one launch (one tile shape, no K split, no
// batches), so that the tiles of one fill the compute units the other's last
// round leaves idle.  Workgroups 0 .. n1-1 take the first product's tiles
// (the one with the longer K, dispatched first), the rest the second's; each
// range is remapped XCD-contiguous like a launch of its own.
template <class Cfg, bool A1, bool B1, class E1, bool A2, bool B2, class E2>
__global__ void __launch_bounds__(Cfg::NT)
gemm_pair_kernel(const GemmParams p1, const E1 e1, const GemmParams p2, const E2 e2, int n1) {
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::SMEM_BYTES];
  const int b = (int)blockIdx.x;
  const bool first = b < n1;
  int lx, xcd;
  coords_1d(first ? b : b - n1, first ? n1 : (int)gridDim.x - n1, lx, xcd);
  if (first) gemm_tile<Cfg, A1, B1, false, E1>(p1, e1, lx, 0, 0, xcd, smem);
  else gemm_tile<Cfg, A2, B2, false, E2>(p2, e2, lx, 0, 0, xcd, smem);
}

}  // namespace tpk
