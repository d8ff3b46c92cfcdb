// Chunk-level building blocks shared by the forward and backward kernels:
// swizzled LDS tiles, 16-byte operand fragments, direct global->LDS loads,
// the gate prefix, the A / P products and the blocked UT inverse.
//
// Row order of accumulator tiles.  An accumulator tile `mt` (16 logical rows)
// holds physical rows prow(mt, m) = 32(mt/2) + 8(m/4) + 4(mt%2) + m%4.  With
// this order, lane group g of the tile pair (2kb, 2kb+1) holds the 8
// consecutive physical rows 32kb + 8g .. 32kb + 8g + 7, so the pair is a B
// operand for a contraction over those rows, and the matching A operand is
// one contiguous 16-byte LDS read per lane.  Every tile whose rows index
// chunk tokens or d_k uses this order; tiles of the C x C products use the
// natural order 16t + m.
//
// LDS swizzle.  Matrices are stored without padding; the 16-byte unit u of
// row r sits at unit position u ^ swz(r).  The swizzle makes both the
// permuted-row and the natural-row fragment reads of 16 lanes hit 16
// distinct 4-bank groups.
#pragma once

#include "dn_device.h"

namespace dn {

__device__ __forceinline__ int prow(int mt, int m) {
  return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

template <int U>
__device__ __forceinline__ int swz(int r) {
  static_assert(U == 8 || U == 16, "rows of 8 or 16 units");
  if (U == 16) return (r & 3) | ((((r >> 2) ^ (r >> 4)) & 3) << 2);
  return ((r >> 1) & 1) | ((((r >> 2) ^ (r >> 4)) & 3) << 1);
}

// A swizzled LDS matrix of E with COLS columns.
template <typename E, int COLS>
struct Tile {
  static constexpr int EPU = 16 / sizeof(E);
  static constexpr int U = COLS / EPU;  // 16-byte units per row
  static_assert(U == 8 || U == 16, "unsupported tile width");
  __device__ static __forceinline__ int off(int r, int c) {  // element offset
    return r * COLS + (((c / EPU) ^ swz<U>(r)) * EPU) + (c % EPU);
  }
  __device__ static __forceinline__ int unit_off(int r, int u) {  // unit u of row r
    return r * COLS + ((u ^ swz<U>(r)) * EPU);
  }
};

// 32-index A fragment: 8 contiguous elements of row r starting at column 32kb + 8g
template <typename E, int COLS>
__device__ __forceinline__ F32<E> frag(const E *m, int r, int kb) {
  using TL = Tile<E, COLS>;
  const int g = lane_id() >> 4;
  if constexpr (sizeof(E) == 2) {
    return *reinterpret_cast<const F32<E> *>(m + TL::unit_off(r, 4 * kb + g));
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(m + TL::unit_off(r, 8 * kb + 2 * g));
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(m + TL::unit_off(r, 8 * kb + 2 * g + 1));
    F32<E> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = lo[i];
      f[4 + i] = hi[i];
    }
    return f;
  }
}

// wait for this wave's outstanding vector-memory operations (incl. LDS DMA)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Direct global -> LDS copy of 16 bytes per lane: lane l's 16 bytes land at
// lds_base + 16 l.  Lanes with `valid` false are masked off.
__device__ __forceinline__ void dma16(const void *gsrc, void *lds_base, bool valid) {
  if (valid)
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Copy a 64-row chunk of a [rows, H, D] tensor (row r of the chunk is global
// row row0 + r; columns col0 .. col0 + COLS) into a swizzled LDS tile with
// direct loads.  Rows >= L are not loaded.  Each wave issues its share.
template <typename E, int COLS>
__device__ __forceinline__ void dma_tile(E *lds, const E *g, size_t row0, int H, int h, int D,
                                         int col0, int L) {
  using TL = Tile<E, COLS>;
  constexpr int NU = CH * TL::U;   // units in the tile
  constexpr int NI = NU / 64;      // wave-instructions per tile
  const int w = wave_id(), l = lane_id();
  for (int j = w; j < NI; j += NTHR / 64) {
    const int p = j * 64 + l;      // destination unit
    const int r = p / TL::U, pos = p % TL::U;
    const int u = pos ^ swz<TL::U>(r);
    const E *src = g + ((row0 + r) * H + h) * (size_t)D + col0 + u * TL::EPU;
    dma16(src, lds + j * 64 * TL::EPU, r < L);
  }
}

// zero rows [L, 64) of a tile (partial chunk)
template <typename E, int COLS>
__device__ __forceinline__ void zero_rows(E *lds, int L) {
  u128 z = zero128();
  constexpr int EPU = 16 / sizeof(E);
  for (int i = L * (COLS / EPU) + threadIdx.x; i < CH * (COLS / EPU); i += NTHR)
    *reinterpret_cast<u128 *>(lds + i * EPU) = z;
}

// Per-chunk gate data (b = cumsum g, gamma = exp b, wl = exp(b_63 - b), beta)
struct Gates {
  float b[CH], gam[CH], wl[CH], beta[CH];
};

// Wave 0 (holding g of row lane) writes b, gamma, wl; wave 1 writes beta.
__device__ __forceinline__ void write_gates(Gates &G, float gval, float bval) {
  const int w = wave_id(), l = lane_id();
  if (w == 0) {
    const float b = wave_incl_scan(gval);
    const float blast = __shfl(b, 63, 64);
    G.b[l] = b;
    G.gam[l] = __expf(b);
    G.wl[l] = __expf(blast - b);
  } else if (w == 1) {
    G.beta[l] = bval;
  }
}

}  // namespace dn
