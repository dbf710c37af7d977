// Register-staged LDS tile loads used by the attention core: a K-major tile
// is copied in 16-byte chunks along k; an M/N-major tile is loaded as R x 8
// blocks of 16-byte row loads and transposed in registers (v_perm_b32) before
// the LDS write, so the LDS tile always holds rows of contiguous k.
#pragma once
#include "common.hpp"

namespace tpk {

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

}  // namespace tpk
