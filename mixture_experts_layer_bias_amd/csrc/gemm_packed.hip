// Grouped GEMM on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16, fp32 accumulate)
// with the weights in a packed, fragment-ordered layout:
//
//   C[rows of group g, :] = A[rows, :] * B_g^T        (router, expert down)
//   H[rows of group g, :] = silu(A B_gate_g^T) * (A B_up_g^T)   (expert gate/up)
//
// Same products, tile schedule and per-element accumulation order (k in
// stages of 64, MFMA substeps of 16) as the row-major kernel, so the two give
// bitwise equal results; only the way operands reach the matrix cores differs.
//
// Packed layout.  The weights of one group are cut into panels of 256 weight
// rows (output columns; for SwiGLU 128 gate rows and the 128 up rows of the
// same hidden units) and each panel into stages of 64 k.  One (group, panel,
// stage) block is 32 KB: four 8 KB quarters, one per wavefront w; quarter w
// holds eight 1 KB pieces q = 2 ks + j (MFMA substep ks, column block j), and
// piece q holds for lane l the 16 bytes that lane feeds to the MFMA:
//   B[row][64 stage + 16 ks + 8 (l / 32) + 0..7],   row = r(w, j, l % 32),
//   r = panel * 256 + 64 w + 32 j + c             (plain; zero past the end)
//   r = gate (j = 0) or up (j = 1) row panel * 128 + 32 w + c   (SwiGLU).
// Blocks are ordered group, panel, stage, so a tile streams one contiguous
// range and every load instruction reads 1 KB of consecutive bytes.
//
// Kernel.  A 256-thread workgroup (one wavefront per SIMD) computes up to 256
// rows by one 256-column panel; wavefront w owns columns [64 w, 64 w + 64) of
// every row (up to 8 x 2 MFMA blocks, 256 accumulators).  Weights go from
// global memory straight into registers: each wavefront loads only its own
// quarter, nothing is loaded twice and nothing passes through LDS.
// Activations, which all four wavefronts share, stream into an LDS ring by
// direct loads.  Both operands are loaded CFG::DIST stages ahead of the MFMAs.
#include "gemm_tile.hpp"

namespace moezc {

namespace {

constexpr int PK_WAVES = 4;                          // one wavefront per SIMD
constexpr int PK_BKS = 64;                           // k per stage
constexpr int PK_ROWB = PK_BKS * 2;                  // LDS bytes of one activation row
constexpr int PK_BLOCK = kPackedPanel * PK_BKS * 2;  // 32 KB of weights per stage
constexpr int PK_QUARTER = PK_BLOCK / PK_WAVES;      // one wavefront's share
static_assert(PK_QUARTER == 8 * 1024, "eight 1 KB pieces per wavefront");

// Kernel configuration: MAXRB = most 32-row blocks per tile, DEPTH = stages
// in the pipeline (DEPTH - 1 loaded ahead of use), OCC = workgroups per CU.
//   gate/up, router: 256-row tiles, three stages, one workgroup per CU (256
//     accumulators per wavefront leave room for no second workgroup);
//   down: 128-row tiles, three stages, two workgroups per CU - its tiles are
//     short (K = I), and a second workgroup covers each tile's pipeline fill
//     and epilogue (128 accumulators and three weight register sets fit the
//     256 registers each of two wavefronts per SIMD may hold).
template <int MAXRB_, int DEPTH_, int OCC_>
struct PkCfg {
  static constexpr int MAXRB = MAXRB_, DEPTH = DEPTH_, OCC = OCC_;
  static constexpr int DIST = DEPTH - 1;
  static constexpr int SLOT = MAXRB * 32 * PK_ROWB;  // bytes of one activation stage
};
using PkWide = PkCfg<kPackedMaxTileRows / 32, 3, 1>;
using PkHalf = PkCfg<kPackedMaxTileRows / 64, 3, 2>;

// NA = live 32-row blocks of the tile (1..CFG::MAXRB).
template <typename CFG, int EPI, int NA>
__device__ __forceinline__ void run_packed(const GemmProblem& p, const TileCoord& c,
                                           int n_tiles, int split, char* __restrict__ smem) {
  constexpr int PK_DEPTH = CFG::DEPTH, PK_DIST = CFG::DIST, PK_SLOT = CFG::SLOT;
  constexpr bool SWIGLU = is_swiglu_bf16(EPI);
  const int tid = threadIdx.x;
  // the wavefront index is uniform: keep it in a scalar register, so LDS
  // destinations of the direct loads (M0) need no per-load readfirstlane
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // split-K (fp32 output only): this tile covers stages [k_base, k_base + nk)
  // of the nk_all of its panel; the other epilogues always take the whole range
  const int nk_all = p.K / PK_BKS;
  const int nsplit = (EPI == kStoreF32 && p.k_splits > 1) ? p.k_splits : 1;
  const int nk = nk_all / nsplit;
  const int k_base = (EPI == kStoreF32) ? split * nk : 0;
  const int rows = c.m_end - c.m0;

  // ---- activation direct loads: LDS rows of 128 bytes, chunk c of row r at
  // position c ^ ((r >> 1) & 7) (conflict-free fragment reads).  Instruction
  // t of wavefront w fills rows 8 (w + 4 t) .. + 7 (lane l: row + l / 8,
  // position l % 8); rows past the tile repeat its last row (their products
  // reach accumulator rows that are never stored).  These are buffer loads
  // with the LDS bit (MUBUF), not global_load_lds: the compiler treats a
  // FLAT-encoded load that writes LDS as making both wait counters unordered
  // while it is in flight, and would then turn every wait it needs into a
  // full drain of the pipeline.
  // k-blocked A (a_plane != 0): stage kt of the tile is rows m0.. of plane kt,
  // one contiguous block of 128-byte rows; row-major A: 128 bytes of each
  // row, rows lda apart.
  const bool kblk = p.a_plane != 0;
  // gathered A (a_rows): GEMM row s reads row a_rows[s] of A, so offsets are
  // taken from the start of A; otherwise from the tile's first row
  const int32_t* __restrict__ a_rows = p.a_rows;
  const char* A_tile = static_cast<const char*>(p.A) +
                       (a_rows ? (int64_t)0
                               : (int64_t)c.m0 * (kblk ? (int64_t)PK_ROWB : p.lda * 2));
  const int a_row_bytes = kblk ? PK_ROWB : (int)p.lda * 2;
  // bytes from one stage to the next, and the stage at which the A column
  // wraps back to 0 (router: A = x is read twice, once per weight term)
  const int64_t a_step = kblk ? p.a_plane : (int64_t)PK_ROWB;
  const int a_wrap = kblk ? nk : p.a_kwrap / PK_BKS;
  uint32_t a_src[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    const int r = 8 * (wave + PK_WAVES * t) + (lane >> 3);  // LDS row filled
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    const int rs = min(r, rows - 1);                          // tile row read
    const uint32_t arow = a_rows ? (uint32_t)a_rows[c.m0 + rs] : (uint32_t)rs;
    a_src[t] = arow * (uint32_t)a_row_bytes + (uint32_t)(lc * 16);
  }
  char* const a_dst = smem + wave * 1024;  // + slot + 4096 t

  // ---- this wavefront's quarter of each weight block of the panel
  const char* B_pan = static_cast<const char*>(p.B0) +
                      (((int64_t)c.g * n_tiles + c.nt) * (int64_t)nk_all + k_base) * PK_BLOCK;
  const uint32_t b_off = (uint32_t)(wave * PK_QUARTER + lane * 16);

  // ---- fragment reads: lane l reads row 32 i + l % 32, logical chunk
  // 2 ks + l / 32 (the swizzle depends on the lane only)
  const int swz = ((lane & 31) >> 1) & 7;
  int fr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) fr[ks] = (lane & 31) * PK_ROWB + ((2 * ks + (lane >> 5)) ^ swz) * 16;

  f32x16_t acc[NA][2];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  bf16x8_t fa[2][NA];
  bf16x8_t fb[PK_DEPTH][8];

#define PK_LOAD_B(kt, u)                                                              \
  {                                                                                   \
    const char* b_ = B_pan + (int64_t)(kt) * PK_BLOCK + b_off;                        \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) fb[u][q] =                          \
        *reinterpret_cast<const bf16x8_t*>(b_ + q * 1024);                            \
  }
#define PK_DMA_A(kt, u)                                                               \
  {                                                                                   \
    const int ka_ = (kt) + k_base;                                                    \
    const int ks_ = ka_ >= a_wrap ? ka_ - a_wrap : ka_;                               \
    const char* a_ = A_tile + (int64_t)ks_ * a_step;                                  \
    const __amdgpu_buffer_rsrc_t r_ =                                                 \
        __builtin_amdgcn_make_buffer_rsrc((void*)a_, 0, 0x7fffffff, 0x00020000);      \
    _Pragma("unroll") for (int t = 0; t < NA; ++t)                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                     \
            r_, (lds_void_t*)(a_dst + (u) * PK_SLOT + t * 4096), 16, a_src[t], 0, 0, 0); \
  }
#define PK_LOADF(fs, u, ks)                                                           \
  {                                                                                   \
    const char* l_ = smem + (u) * PK_SLOT + fr[ks];                                   \
    _Pragma("unroll") for (int i = 0; i < NA; ++i) fa[fs][i] =                        \
        *reinterpret_cast<const bf16x8_t*>(l_ + i * 4096);                            \
  }
  // One substep ks of stage slot/register set u.  For each live row block g:
  // the LDS read of block g's fragment for the next substep (fragment set
  // 1 - fs, slot nu, substep nks; skipped when NEXT is false), the two MFMAs
  // of block g, and block g's share of the refill of stage KN into set NU
  // (VMK 1 / 2: weight pieces 0-3 / 4-7, spread over the blocks; VMK 3: the
  // activation rows of block g; VMK 0: none).  One wavefront per SIMD has no
  // other wavefront to cover a burst of memory instructions, so they are
  // spread between MFMAs; a scheduling fence after each group keeps that
  // order through both scheduler passes (without it, register reuse in the
  // second pass let the LDS reads and direct loads bunch up and the MFMAs
  // wait on them).
#define PK_SUB(fs, u, ks, NEXT, nu, nks, VMK, KN, NU)                                 \
  _Pragma("unroll") for (int g_ = 0; g_ < NA; ++g_) {                                 \
    if (NEXT) fa[1 - (fs)][g_] = *reinterpret_cast<const bf16x8_t*>(                  \
        smem + (nu) * PK_SLOT + fr[nks] + g_ * 4096);                                 \
    acc[g_][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fs][g_], fb[u][2 * (ks)], \
                                                         acc[g_][0], 0, 0, 0);        \
    acc[g_][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fs][g_], fb[u][2 * (ks) + 1], \
                                                         acc[g_][1], 0, 0, 0);        \
    if ((VMK) == 1 || (VMK) == 2) {                                                   \
      const char* b_ = B_pan + (int64_t)(KN) * PK_BLOCK + b_off;                      \
      _Pragma("unroll") for (int q = 4 * ((VMK) - 1) + (g_ * 4) / NA;                 \
                             q < 4 * ((VMK) - 1) + ((g_ + 1) * 4) / NA; ++q)          \
          fb[NU][q] = *reinterpret_cast<const bf16x8_t*>(b_ + q * 1024);              \
    } else if ((VMK) == 3) {                                                          \
      const int ka_ = (KN) + k_base;                                                  \
      const int ks_ = ka_ >= a_wrap ? ka_ - a_wrap : ka_;                             \
      const char* a_ = A_tile + (int64_t)ks_ * a_step;                                \
      const __amdgpu_buffer_rsrc_t r_ =                                               \
          __builtin_amdgcn_make_buffer_rsrc((void*)a_, 0, 0x7fffffff, 0x00020000);    \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                       \
          r_, (lds_void_t*)(a_dst + (NU) * PK_SLOT + g_ * 4096), 16, a_src[g_], 0, 0, 0); \
    }                                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                \
  }
  // Stage kt uses slot and register set u = kt % PK_DEPTH and refills the set
  // of stage kt-1 (every wavefront finished reading that slot before the last
  // barrier) with stage kt+PK_DIST: weight halves in substeps 0 and 1, the
  // activations in substep 2.  Before the last substep the wavefront waits for
  // its own loads of stage kt+1 (loads complete in issue order; the refill of
  // kt+PK_DIST stays in flight) and meets the others, so stage kt+1 is whole
  // in LDS and in registers; the last substep's MFMAs cover the first
  // fragment reads of kt+1.  In the steady loop, a refill past the last stage
  // repeats the last stage's addresses (those slots and registers are never
  // read), so every stage there keeps the same count of loads in flight and
  // the loop has no branches.  The stages after the loop (fewer than
  // PK_DEPTH) would only refill past the end, so they issue no loads and wait
  // for all of them: the compiler drops register loads whose results are
  // never read, and a dummy refill there would not be issued at all, leaving
  // a count-based wait short.
#define PK_STAGE(kt, u, REFILL)                                                       \
  {                                                                                   \
    const int kn_ = min((kt) + PK_DIST, nk - 1);                                      \
    const int un_ = ((u) + PK_DIST) % PK_DEPTH;                                       \
    PK_SUB(0, u, 0, true, u, 1, (REFILL) ? 1 : 0, kn_, un_);                          \
    PK_SUB(1, u, 1, true, u, 2, (REFILL) ? 2 : 0, kn_, un_);                          \
    PK_SUB(0, u, 2, true, u, 3, (REFILL) ? 3 : 0, kn_, un_);                          \
    ring_barrier<(REFILL) ? (PK_DIST - 1) * (8 + NA) : 0>();                          \
    __builtin_amdgcn_sched_barrier(0);                                                \
    PK_SUB(1, u, 3, true, ((u) + 1) % PK_DEPTH, 0, 0, 0, 0);                          \
  }

  // prologue: stages 0 .. PK_DIST-1 (repeating the last stage where nk is
  // smaller), weights then activations of each; wait for stage 0 only
  // (fenced, so that the loads are issued stage by stage, as the wait counts
  // assume)
#pragma unroll
  for (int u = 0; u < PK_DIST; ++u) {
    PK_LOAD_B(min(u, nk - 1), u);
    PK_DMA_A(min(u, nk - 1), u);
    __builtin_amdgcn_sched_barrier(0);
  }
  ring_barrier<(PK_DIST - 1) * (8 + NA)>();
  PK_LOADF(0, 0, 0);
  int kt = 0;
  for (; kt + PK_DEPTH <= nk; kt += PK_DEPTH) {
#pragma unroll
    for (int u = 0; u < PK_DEPTH; ++u) PK_STAGE(kt + u, u, true);
  }
#pragma unroll
  for (int u = 0; u + 1 < PK_DEPTH; ++u)
    if (kt + u < nk) PK_STAGE(kt + u, u, false);
#undef PK_LOAD_B
#undef PK_DMA_A
#undef PK_LOADF
#undef PK_STAGE
#undef PK_SUB
  ring_barrier<0>();  // every wavefront is done reading the ring before it is reused

  // ---- epilogue: D[i][j] of a 32 x 32 block sits in lane j + 32 ((i / 4) % 2),
  // register 4 (i / 8) + i % 4
  const int lrow4 = 4 * (lane >> 5);
  const int lcol = lane & 31;
  if (EPI == kStoreF32) {
    float* __restrict__ Cf = static_cast<float*>(p.C) + (int64_t)split * p.c_split_stride;
    if ((p.Nout & 3) == 0 && (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(Cf) & 15) == 0) {
      // through a wavefront-private LDS tile (the ring is free), one 32-row
      // block at a time, so that global stores are whole 16-byte row pieces
      constexpr int OS = 64 + 4;  // padded LDS row (floats)
      float* ot = reinterpret_cast<float*>(smem) + wave * (32 * OS);
      const int gcol0 = c.n0 + wave * 64;
#pragma unroll
      for (int i = 0; i < NA; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            ot[(8 * (v >> 2) + lrow4 + (v & 3)) * OS + j * 32 + lcol] = acc[i][j][v];
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes landed
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = lane; q < 32 * 16; q += 64) {
          const int r = q >> 4, ch = q & 15;
          const int grow = c.m0 + i * 32 + r, gcol = gcol0 + ch * 4;
          if (grow < c.m_end && gcol < p.Nout)
            *reinterpret_cast<f32x4_t*>(Cf + (int64_t)grow * p.ldc + gcol) =
                *reinterpret_cast<const f32x4_t*>(ot + r * OS + ch * 4);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block overwrites
        __builtin_amdgcn_wave_barrier();
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int gcol = c.n0 + wave * 64 + j * 32 + lcol;
        if (gcol >= p.Nout) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int grow = c.m0 + i * 32 + 8 * (v >> 2) + lrow4 + (v & 3);
          if (grow < c.m_end)
            static_cast<float*>(p.C)[split * p.c_split_stride + (int64_t)grow * p.ldc + gcol] =
                acc[i][j][v];
        }
      }
    return;
  }
  store_bf16_tile<NA, SWIGLU, EPI == kSwiGLU_BF16_ACT>(acc, smem, wave, lane, c, p);
}

template <typename CFG, int EPI>
__global__ __launch_bounds__(64 * PK_WAVES, CFG::OCC) void packed_gemm_kernel(GemmProblem p,
                                                                             int n_tiles,
                                                                             int total_bound,
                                                                             int tile_rows) {
  constexpr bool SWIGLU = is_swiglu_bf16(EPI);
  __shared__ __attribute__((aligned(16))) char smem[CFG::DEPTH * CFG::SLOT];
  int logical =
      xcd_logical_tile(p.tile_prefix ? p.tile_prefix[p.G] * n_tiles : total_bound);
  if (logical < 0) return;
  // split-K (fp32 output, one group): the parts of a tile are adjacent
  int split = 0;
  if (EPI == kStoreF32 && p.k_splits > 1) {
    split = logical % p.k_splits;
    logical /= p.k_splits;
  }
  TileCoord c;
  if (!map_tile<kPackedPanel, SWIGLU>(p, n_tiles, logical, tile_rows, c)) return;
  // at most CFG::MAXRB: the host checks tile_rows against the configuration
  const int nb = (c.m_end - c.m0 + 31) / 32;
  if (nb <= 0) return;
  constexpr int M = CFG::MAXRB;
  switch (nb) {
    case 1: run_packed<CFG, EPI, 1>(p, c, n_tiles, split, smem); break;
    case 2: run_packed<CFG, EPI, (M >= 2 ? 2 : M)>(p, c, n_tiles, split, smem); break;
    case 3: run_packed<CFG, EPI, (M >= 3 ? 3 : M)>(p, c, n_tiles, split, smem); break;
    case 4: run_packed<CFG, EPI, (M >= 4 ? 4 : M)>(p, c, n_tiles, split, smem); break;
    case 5: run_packed<CFG, EPI, (M >= 5 ? 5 : M)>(p, c, n_tiles, split, smem); break;
    case 6: run_packed<CFG, EPI, (M >= 6 ? 6 : M)>(p, c, n_tiles, split, smem); break;
    case 7: run_packed<CFG, EPI, (M >= 7 ? 7 : M)>(p, c, n_tiles, split, smem); break;
    default: run_packed<CFG, EPI, M>(p, c, n_tiles, split, smem); break;
  }
}

// ---- packing ------------------------------------------------------------------
// Byte offset o (multiple of 16) inside a 32 KB block -> the weight row and
// first k (relative to the block's panel and stage) of its 16 bytes.
__device__ __forceinline__ void packed_piece(int o, bool swiglu, int& row, int& k, bool& up) {
  const int w = o >> 13;         // 8 KB quarter: wavefront
  const int q = (o >> 10) & 7;   // 1 KB piece: 2 ks + j
  const int l = (o >> 4) & 63;   // lane
  const int ks = q >> 1, j = q & 1, cc = l & 31;
  k = 16 * ks + 8 * (l >> 5);
  if (swiglu) {
    row = 32 * w + cc;  // within the 128 hidden units of the panel
    up = (j == 1);
  } else {
    row = 64 * w + 32 * j + cc;  // within the 256 rows of the panel
    up = false;
  }
}

// One workgroup per 32 KB block (group, panel, stage), 2048 pieces of 16 bytes;
// consecutive threads write consecutive pieces.
__global__ __launch_bounds__(256) void pack_weights_kernel(const bf16_t* __restrict__ w0,
                                                           const bf16_t* __restrict__ w1,
                                                           bf16_t* __restrict__ out, int rows,
                                                           int K, int n_panels,
                                                           int64_t group_stride, int swiglu) {
  const int nk = K / PK_BKS;
  const int64_t b = blockIdx.x;
  const int64_t per_group = (int64_t)n_panels * nk;
  const int64_t g = b / per_group;
  const int rem = (int)(b - g * per_group);
  const int nt = rem / nk, kt = rem - nt * nk;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int o = (threadIdx.x + 256 * i) * 16;
    int row, k;
    bool up;
    packed_piece(o, swiglu != 0, row, k, up);
    row += swiglu ? nt * (kPackedPanel / 2) : nt * kPackedPanel;
    k += kt * PK_BKS;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row < rows) {
      const bf16_t* src = (up ? w1 : w0) + g * group_stride + (int64_t)row * K + k;
      v = *reinterpret_cast<const u32x4_t*>(src);
    }
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(out) + b * PK_BLOCK + o) = v;
  }
}

// The packed layout of a transposed operand, gathered from the untransposed
// weights: packed row r (an output column of the GEMM), reduction index k
// holds src[k][r] with src = w0 for k < k_split and w1 (at k - k_split)
// otherwise, rows src_ld elements long.  For the backward: W_gate | W_up as
// [d][2I] (k_split = I, src_ld = d) and W_down as [I][d] (k_split = d,
// src_ld = I).  Eight k of one row are eight strided loads; consecutive lanes
// take consecutive rows, so each load instruction reads whole row segments.
// One workgroup per 32 KB block, as pack_weights_kernel; runs once, at load.
__global__ __launch_bounds__(256) void pack_transposed_kernel(const bf16_t* __restrict__ w0,
                                                              const bf16_t* __restrict__ w1,
                                                              bf16_t* __restrict__ out, int rows,
                                                              int K, int k_split, int src_ld,
                                                              int n_panels,
                                                              int64_t group_stride) {
  const int nk = K / PK_BKS;
  const int64_t b = blockIdx.x;
  const int64_t per_group = (int64_t)n_panels * nk;
  const int64_t g = b / per_group;
  const int rem = (int)(b - g * per_group);
  const int nt = rem / nk, kt = rem - nt * nk;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int o = (threadIdx.x + 256 * i) * 16;
    int row, k;
    bool up;
    packed_piece(o, false, row, k, up);
    row += nt * kPackedPanel;
    k += kt * PK_BKS;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (row < rows) {
      const bool second = k >= k_split;  // eight k never straddle k_split (a multiple of 8)
      const bf16_t* src = (second ? w1 : w0) + g * group_stride +
                          (int64_t)(second ? k - k_split : k) * src_ld + row;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)src[(int64_t)(2 * e) * src_ld] |
               ((uint32_t)src[(int64_t)(2 * e + 1) * src_ld] << 16);
    }
    u32x4_t v = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(out) + b * PK_BLOCK + o) = v;
  }
}

// fp32 W_router [E, d] -> packed [E, 2d] bf16 split: k < d holds bf16(w),
// k >= d holds bf16(w - bf16(w)) of column k - d; rows past E are zero.
// w = hi + lo + r with |r| <= 2^-17 |w|, so x (bf16) times [hi | lo] on MFMA
// with fp32 accumulation (A columns wrap at d) gives the fp32 logits to about
// 1e-5 absolute at d = 6144 (one bf16 term alone: about 1e-3).
__global__ __launch_bounds__(256) void split_router_packed_kernel(const float* __restrict__ w,
                                                                  bf16_t* __restrict__ out,
                                                                  int E, int d) {
  const int nk = 2 * d / PK_BKS;
  const int b = blockIdx.x;
  const int nt = b / nk, kt = b - nt * nk;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int o = (threadIdx.x + 256 * i) * 16;
    int row, k;
    bool up;
    packed_piece(o, false, row, k, up);
    row += nt * kPackedPanel;
    k += kt * PK_BKS;
    uint32_t h[4] = {0u, 0u, 0u, 0u};
    if (row < E) {
      const bool lo = k >= d;
      const float* src = w + (int64_t)row * d + (lo ? k - d : k);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = src[e];
        const bf16_t hi = f32_to_bf16(v);
        const bf16_t r = lo ? f32_to_bf16(v - bf16_to_f32(hi)) : hi;
        h[e >> 1] |= (uint32_t)r << (16 * (e & 1));
      }
    }
    const u32x4_t v = {h[0], h[1], h[2], h[3]};
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(out) + (int64_t)b * PK_BLOCK + o) = v;
  }
}

}  // namespace

int64_t packed_bytes(int64_t rows, int64_t K, bool swiglu) {
  // SwiGLU: `rows` hidden units, gate and up together
  const int64_t panels = swiglu ? rows / (kPackedPanel / 2)
                                : (rows + kPackedPanel - 1) / kPackedPanel;
  return panels * (K / PK_BKS) * (int64_t)PK_BLOCK;
}

hipError_t launch_pack_transposed(const bf16_t* w0, const bf16_t* w1, bf16_t* out, int groups,
                                  int rows, int K, int k_split, int src_ld, int64_t group_stride,
                                  hipStream_t s) {
  if (K % PK_BKS != 0 || k_split % 8 != 0 || k_split <= 0) return hipErrorInvalidValue;
  const int n_panels = (rows + kPackedPanel - 1) / kPackedPanel;
  const int64_t blocks = (int64_t)groups * n_panels * (K / PK_BKS);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_transposed_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w0, w1, out,
                     rows, K, k_split, src_ld, n_panels, group_stride);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const bf16_t* w0, const bf16_t* w1, bf16_t* out, int groups,
                               int rows, int K, bool swiglu, hipStream_t s) {
  if (K % PK_BKS != 0 || (swiglu && rows % (kPackedPanel / 2) != 0)) return hipErrorInvalidValue;
  const int n_panels = swiglu ? rows / (kPackedPanel / 2) : (rows + kPackedPanel - 1) / kPackedPanel;
  const int64_t blocks = (int64_t)groups * n_panels * (K / PK_BKS);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w0, w1, out,
                     rows, K, n_panels, (int64_t)rows * K, swiglu ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_split_router_packed(const float* w, bf16_t* out, int E, int d, hipStream_t s) {
  if ((2 * d) % PK_BKS != 0) return hipErrorInvalidValue;
  const int n_panels = (E + kPackedPanel - 1) / kPackedPanel;
  const int blocks = n_panels * (2 * d / PK_BKS);
  hipLaunchKernelGGL(split_router_packed_kernel, dim3(blocks), dim3(256), 0, s, w, out, E, d);
  return hipGetLastError();
}

int packed_down_tile_rows(int ffn_tile_rows) {
  return ffn_tile_rows < 32 * PkHalf::MAXRB ? ffn_tile_rows : 32 * PkHalf::MAXRB;
}

hipError_t launch_packed_gemm(const GemmProblem& p, int epilogue, int tile_rows, int64_t max_rows,
                              hipStream_t s) {
  if (p.K < PK_BKS || p.K % PK_BKS != 0 || p.a_kwrap % PK_BKS != 0) return hipErrorInvalidValue;
  if (tile_rows < 32 || tile_rows > kPackedMaxTileRows || tile_rows % 32 != 0)
    return hipErrorInvalidValue;
  const bool swiglu = is_swiglu_bf16(epilogue);
  if (swiglu && p.Nout % (kPackedPanel / 2) != 0) return hipErrorInvalidValue;
  const int n_tiles = swiglu ? p.Nout / (kPackedPanel / 2) : (p.Nout + kPackedPanel - 1) / kPackedPanel;
  // the down GEMM runs the two-workgroups-per-CU configuration
  const bool half_cfg = (epilogue == kStoreBF16);
  if (tile_rows > 32 * (half_cfg ? PkHalf::MAXRB : PkWide::MAXRB)) return hipErrorInvalidValue;
  int64_t mt_bound;
  if (p.tile_prefix) {
    mt_bound = (max_rows + (int64_t)p.G * (tile_rows - 1)) / tile_rows;
    if (mt_bound > max_rows) mt_bound = max_rows;
  } else {
    mt_bound = (p.M + tile_rows - 1) / tile_rows;
  }
  // split-K: fp32 output of one group only, equal whole-stage parts
  const int splits = std::max(1, p.k_splits);
  if (splits > 1 && (epilogue != kStoreF32 || p.tile_prefix || (p.K / PK_BKS) % splits != 0))
    return hipErrorInvalidValue;
  int64_t blocks = mt_bound * n_tiles * splits;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0) return hipErrorInvalidValue;
  const int total = (int)blocks;
  blocks = (blocks + 7) / 8 * 8;
  const dim3 grid((unsigned)blocks), block(64 * PK_WAVES);
  switch (epilogue) {
    case kStoreF32:
      hipLaunchKernelGGL((packed_gemm_kernel<PkWide, kStoreF32>), grid, block, 0, s, p, n_tiles,
                         total, tile_rows);
      break;
    case kStoreBF16:
      hipLaunchKernelGGL((packed_gemm_kernel<PkHalf, kStoreBF16>), grid, block, 0, s, p, n_tiles,
                         total, tile_rows);
      break;
    case kSwiGLU_BF16:
      hipLaunchKernelGGL((packed_gemm_kernel<PkWide, kSwiGLU_BF16>), grid, block, 0, s, p, n_tiles,
                         total, tile_rows);
      break;
    case kSwiGLU_BF16_ACT:
      if (!p.C2) return hipErrorInvalidValue;
      hipLaunchKernelGGL((packed_gemm_kernel<PkWide, kSwiGLU_BF16_ACT>), grid, block, 0, s, p,
                         n_tiles, total, tile_rows);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moezc
