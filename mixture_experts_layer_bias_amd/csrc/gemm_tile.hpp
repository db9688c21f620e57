// Tile scheduling and LDS-ring helpers shared by the grouped GEMM kernels.
#pragma once

#include "kernels.hpp"

namespace moezc {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

struct TileCoord {
  int g;      // group (expert)
  int m0;     // first row of the tile
  int m_end;  // one past its last row
  int n0;     // first output column (SwiGLU: first hidden unit)
  int nt;     // weight panel index
};

// Logical tile -> (group, rows, output columns).  Returns false past the end.
// Grouped problems (tile_prefix set): tiles run expert by expert, then weight
// panel, then row part; an expert whose rows need several tiles is cut into
// near-equal parts of whole 32-row blocks (only the last part is ragged), so
// a split costs no more padded MFMA rows than an unsplit expert.  One group (tile_prefix null): `tile_rows` rows per tile.
// A panel is BN weight rows (SwiGLU: BN / 2 gate rows and as many up rows).
template <int BN, bool SWIGLU>
__device__ __forceinline__ bool map_tile(const GemmProblem& p, int n_tiles, int logical,
                                         int tile_rows, TileCoord& c) {
  if (p.tile_prefix) {
    const int total = p.tile_prefix[p.G] * n_tiles;
    if (logical >= total) return false;
    const int mt_all = logical / n_tiles;  // only to find the group
    int lo = 0, hi = p.G;  // tile_prefix[lo] <= mt_all < tile_prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_prefix[mid] <= mt_all) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int mtc = p.tile_prefix[g + 1] - p.tile_prefix[g];
    const int local = logical - p.tile_prefix[g] * n_tiles;
    const int nt = local / mtc;
    const int mt = local - nt * mtc;
    const int r0 = p.row_offsets[g], r1 = p.row_offsets[g + 1];
    const int rpt = ((r1 - r0 + mtc - 1) / mtc + 31) / 32 * 32;  // parts of whole 32-row blocks
    c.g = g;
    c.m0 = r0 + mt * rpt;
    c.m_end = min(c.m0 + rpt, r1);
    c.nt = nt;
  } else {
    const int mtiles = (p.M + tile_rows - 1) / tile_rows;
    if (logical >= mtiles * n_tiles) return false;
    const int nt = logical / mtiles;
    const int mt = logical - nt * mtiles;
    c.g = 0;
    c.m0 = mt * tile_rows;
    c.m_end = min(c.m0 + tile_rows, p.M);
    c.nt = nt;
  }
  c.n0 = SWIGLU ? c.nt * (BN / 2) : c.nt * BN;
  return true;
}

// XCD-aware order: workgroup b runs on XCD b % 8, and XCD x takes the logical
// range [x * per, (x + 1) * per) of the `total` live tiles, so neighbouring
// tiles (one expert's panels and row parts) share one XCD's L2.  Returns -1
// for a workgroup past the end.
__device__ __forceinline__ int xcd_logical_tile(int total) {
  const int per = (total + 7) >> 3;
  const int jx = blockIdx.x >> 3;
  if (jx >= per) return -1;
  return (blockIdx.x & 7) * per + jx;
}

// Workgroup barrier for an LDS ring filled by direct loads: this wavefront's
// vector-memory operations older than the newest n have completed (loads
// return in issue order) and all its LDS operations are done (s_waitcnt
// vmcnt(n) lgkmcnt(0), gfx9 encoding), then s_barrier.  No memory fence: a
// fence would wait for every load in flight and empty the ring.
template <int n>
__device__ __forceinline__ void ring_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((n >> 4) << 14) | 0x0070 | (n & 15));
  __builtin_amdgcn_s_barrier();
}

// Epilogue of a 256-thread MFMA tile with bf16 output: wavefront `wave` holds
// acc[i][j] for row block i and its column blocks j = 0, 1 of 32 columns; D of
// a 32 x 32 block sits in lane j + 32 ((i / 4) % 2), register 4 (i / 8) + i % 4.
// SwiGLU: column block 0 holds gate, 1 holds up of the same 32 hidden units,
// and the output is silu(gate) * up (32 columns per wavefront); otherwise 64
// columns.  Values go through a wavefront-private LDS tile (smem must hold
// 4 x 32 rows of padded columns), one 32-row block at a time, so that global
// stores are whole 16-byte row pieces.  SAVE (SwiGLU only) also stores the
// pre-activations gate and up (bf16) the same way, to p.C2 columns n and
// Nout + n.
template <int NA, bool SWIGLU, bool SAVE = false>
__device__ __forceinline__ void store_bf16_tile(const f32x16_t (&acc)[NA][2], char* smem,
                                                int wave, int lane, const TileCoord& c,
                                                const GemmProblem& p) {
  const int lrow4 = 4 * (lane >> 5);
  const int lcol = lane & 31;
  constexpr int OC = SWIGLU ? 32 : 64;  // output columns of this wavefront
  constexpr int OS = OC + 8;            // padded LDS row (elements)
  constexpr int CH = OC / 8;            // 16-byte pieces per row
  bf16_t* ot = reinterpret_cast<bf16_t*>(smem) + wave * (32 * OS);
  const int gcol0 = c.n0 + wave * OC;
  bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.C);
#pragma unroll
  for (int i = 0; i < NA; ++i) {
#pragma unroll
    for (int jj = 0; jj < OC / 32; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + lrow4 + (v & 3);
        float val;
        if (SWIGLU) {
          val = swiglu_fast(acc[i][0][v], acc[i][1][v]);
        } else {
          val = acc[i][jj][v];
        }
        ot[r * OS + jj * 32 + lcol] = f32_to_bf16(val);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes landed
    __builtin_amdgcn_wave_barrier();
    const int grow0 = c.m0 + i * 32;
#pragma unroll
    for (int q = lane; q < 32 * CH; q += 64) {
      const int r = q / CH, ch = q - r * CH;
      const int grow = grow0 + r;
      const int gcol = gcol0 + ch * 8;
      if (grow < c.m_end && gcol < p.Nout)
        *reinterpret_cast<u32x4_t*>(&Cout[(int64_t)grow * p.ldc + gcol]) =
            *reinterpret_cast<const u32x4_t*>(&ot[r * OS + ch * 8]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block overwrites
    __builtin_amdgcn_wave_barrier();
    if constexpr (SWIGLU && SAVE) {
      bf16_t* __restrict__ C2 = static_cast<bf16_t*>(p.C2);
#pragma unroll
      for (int part = 0; part < 2; ++part) {  // gate, then up
#pragma unroll
        for (int v = 0; v < 16; ++v)
          ot[(8 * (v >> 2) + lrow4 + (v & 3)) * OS + lcol] = f32_to_bf16(acc[i][part][v]);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = lane; q < 32 * CH; q += 64) {
          const int r = q / CH, ch = q - r * CH;
          const int grow = grow0 + r;
          const int gcol = gcol0 + ch * 8;
          if (grow < c.m_end && gcol < p.Nout)
            *reinterpret_cast<u32x4_t*>(&C2[(int64_t)grow * p.ldc2 + part * p.Nout + gcol]) =
                *reinterpret_cast<const u32x4_t*>(&ot[r * OS + ch * 8]);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

}  // namespace moezc
