// Grouped GEMM on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
//   C[rows of group g, :] = A[rows, :] * B_g^T        (router, expert down)
//   H[rows of group g, :] = silu(A B_gate_g^T) * (A B_up_g^T)   (expert gate/up)
//
// Groups are the FFN experts; their rows are the grouped (token, expert) slots
// written by the permute kernel.  The device-side m-tile prefix from the scan
// tells each workgroup which expert, which rows and which weight panel it
// owns, so the grid is sized without reading any count back to the host and
// experts with no rows cost nothing.  Both operands are K-contiguous ([rows, K]
// activations, nn.Linear [out, in] weights), which is the per-lane layout the
// MFMA wants: lane l feeds row (l % 32) with the 8 consecutive k at 8*(l / 32).
//
// Prefill shape (about 256 rows per expert, K = 6144 or 2048): a 256 x 256
// tile per workgroup, so one workgroup holds every row of a typical expert and
// each weight panel is streamed from HBM once while it is used 256 times; four
// wavefronts each own a 128 x 128 block (16 MFMA blocks, 256 accumulators).
// An expert with more rows than the tile is split into equal parts whose
// workgroups run side by side on one XCD and so share the panel in L2.
// Row blocks of 32 that hold no rows are skipped by the wavefront that owns
// them (the K loop is instantiated per count of live row blocks).
//
// Tile order: expert, then weight panel, then row part.  Consecutive
// workgroups land on different XCDs (round robin), so each XCD is handed a
// contiguous range of this order: the workgroups of one expert run together
// on one XCD and share its L2 for the expert's activation rows.
//
// Pipeline: two LDS stages of BK = 64; the global loads of step k+1 are
// issued into registers before the MFMAs of step k.  LDS rows are padded to
// 72 bf16 so the 16-byte fragment reads of a wavefront hit distinct banks.
#include "kernels.hpp"

namespace moezc {

namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row

struct TileCoord {
  int g, m0, m_end, n0;
};

// Logical tile -> (group, rows, output columns).  Returns false past the end.
template <int BM, int BN, bool SWIGLU>
__device__ __forceinline__ bool map_tile(const GemmProblem& p, int n_tiles, int logical,
                                         TileCoord& c) {
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
    const int rpt = (r1 - r0 + mtc - 1) / mtc;  // equal parts
    c.g = g;
    c.m0 = r0 + mt * rpt;
    c.m_end = min(c.m0 + rpt, r1);
    c.n0 = SWIGLU ? nt * (BN / 2) : nt * BN;
  } else {
    const int mtiles = (p.M + BM - 1) / BM;
    if (logical >= mtiles * n_tiles) return false;
    const int nt = logical / mtiles;
    const int mt = logical - nt * mtiles;
    c.g = 0;
    c.m0 = mt * BM;
    c.m_end = min(c.m0 + BM, p.M);
    c.n0 = SWIGLU ? nt * (BN / 2) : nt * BN;
  }
  return true;
}

template <int EPI, int BM, int BN, int WAVES_M, int WAVES_N, int NA>
__device__ __forceinline__ void run_tile(const GemmProblem& p, const TileCoord& c,
                                         bf16_t* __restrict__ As, bf16_t* __restrict__ Bs) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M;
  constexpr int WTN = BN / WAVES_N;
  constexpr int CB = WTN / 32;
  constexpr bool SWIGLU = (EPI == kSwiGLU_BF16);
  constexpr int HB = CB / 2;
  constexpr int ROWS_PER_LD = NT / 8;           // tile rows covered by one load round
  constexpr int A_LD = BM / ROWS_PER_LD;        // 16-byte loads per thread per stage
  constexpr int B_LD = BN / ROWS_PER_LD;
  constexpr int B_GATE_LD = (BN / 2) / ROWS_PER_LD;
  constexpr int STAGE_A = BM * LDS_STRIDE, STAGE_B = BN * LDS_STRIDE;
  constexpr int NAc = NA > 0 ? NA : 1;

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  const bf16_t* __restrict__ B0 =
      static_cast<const bf16_t*>(p.B0) + (int64_t)c.g * p.b_group_stride;
  const bf16_t* __restrict__ B1 =
      SWIGLU ? static_cast<const bf16_t*>(p.B1) + (int64_t)c.g * p.b_group_stride : nullptr;

  const int tid = threadIdx.x;
  const int lrow = tid >> 3, lc = (tid & 7) * 8;
  // Uniform per-tile bases (scalar registers) plus constant 32-bit byte
  // offsets per thread, so each load is "scalar base + vector offset" and
  // needs one vector register.  Rows past the end are clamped to a valid row;
  // their products only reach accumulator rows that are never stored.
  const char* A_tile = reinterpret_cast<const char*>(A + (int64_t)c.m0 * p.lda);
  const char* B_gate = reinterpret_cast<const char*>(B0 + (int64_t)c.n0 * p.ldb);
  const char* B_up = SWIGLU ? reinterpret_cast<const char*>(B1 + (int64_t)c.n0 * p.ldb) : nullptr;
  uint32_t a_off[A_LD], b_off[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = min(lrow + ROWS_PER_LD * i, c.m_end - 1 - c.m0);
    a_off[i] = (uint32_t)((r * (int)p.lda + lc) * 2);
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = lrow + ROWS_PER_LD * i;
    int n;
    if (SWIGLU) n = (i < B_GATE_LD) ? r : r - BN / 2;
    else n = min(c.n0 + r, p.Nout - 1) - c.n0;
    b_off[i] = (uint32_t)((n * (int)p.ldb + lc) * 2);
  }

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // row block i of this wavefront starts at tile row (i * WAVES_M + wm) * 32:
  // interleaved so a partly filled tile keeps both wavefront rows busy
  int brow[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    if (SWIGLU)
      brow[j] = (j < HB) ? wn * HB * 32 + j * 32 : BN / 2 + wn * HB * 32 + (j - HB) * 32;
    else
      brow[j] = wn * WTN + j * 32;
  }
  const int frag_col = (lane >> 5) * 8;
  int a_frag[NAc], b_frag[CB];  // LDS element offsets of this lane's fragments
#pragma unroll
  for (int i = 0; i < NAc; ++i)
    a_frag[i] = ((i * WAVES_M + wm) * 32 + (lane & 31)) * LDS_STRIDE + frag_col;
#pragma unroll
  for (int j = 0; j < CB; ++j) b_frag[j] = (brow[j] + (lane & 31)) * LDS_STRIDE + frag_col;

  f32x16_t acc[NAc][CB];
#pragma unroll
  for (int i = 0; i < NAc; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Two register sets stage global loads two k-steps ahead (set k & 1 holds
  // k-step k); the k loop is unrolled by two so the set index is static (the
  // arrays must stay in registers: no lambdas, no dynamic indexing).
  u32x4_t ra[A_LD], rb[B_LD];
  bf16x8_t fa[2][NAc], fb[2][CB];

#define MOEZC_GLOAD_A(kt)                                                            \
  {                                                                                  \
    const char* a_k = A_tile + (((kt) * BK) % p.a_kwrap) * 2;                        \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) ra[i] =                         \
        *reinterpret_cast<const u32x4_t*>(a_k + a_off[i]);                           \
  }
#define MOEZC_GLOAD_B(RB, kt)                                                        \
  {                                                                                  \
    const char* bg_k = B_gate + (kt) * BK * 2;                                       \
    const char* bu_k = SWIGLU ? B_up + (kt) * BK * 2 : bg_k;                         \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) RB[i] =                         \
        *reinterpret_cast<const u32x4_t*>(((SWIGLU && i >= B_GATE_LD) ? bu_k : bg_k) + \
                                          b_off[i]);                                 \
  }
#define MOEZC_LSTORE(RB, buf)                                                    \
  {                                                                                  \
    bf16_t* as_w = As + (buf) * STAGE_A;                                             \
    bf16_t* bs_w = Bs + (buf) * STAGE_B;                                             \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i)                                 \
        *reinterpret_cast<u32x4_t*>(&as_w[(lrow + ROWS_PER_LD * i) * LDS_STRIDE + lc]) = \
        ra[i];                                                                       \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i)                                 \
        *reinterpret_cast<u32x4_t*>(&bs_w[(lrow + ROWS_PER_LD * i) * LDS_STRIDE + lc]) = \
        RB[i];                                                                       \
  }
  // this lane's MFMA fragments of substep ks (16 k) into register slot sl
#define MOEZC_LOADF(sl, as_r, bs_r, ks)                                              \
  {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < NAc; ++i) fa[sl][i] =                      \
        *reinterpret_cast<const bf16x8_t*>(&(as_r)[a_frag[i] + (ks) * 16]);          \
    _Pragma("unroll") for (int j = 0; j < CB; ++j) fb[sl][j] =                       \
        *reinterpret_cast<const bf16x8_t*>(&(bs_r)[b_frag[j] + (ks) * 16]);          \
  }
#define MOEZC_MMA(sl)                                                                \
  {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < NAc; ++i)                                  \
        _Pragma("unroll") for (int j = 0; j < CB; ++j) acc[i][j] =                   \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][i], fb[sl][j], acc[i][j], 0, 0, 0); \
  }
  // One k-step.  The global loads of k-step kt+1 are issued first; substep
  // ks then issues the fragment reads of ks+1 and its own MFMAs, so LDS
  // latency hides under MFMA work.  Before the last substep the data of kt+1
  // goes to the other LDS stage and the workgroup meets at its one barrier;
  // the last substep's MFMAs then cover the first fragment reads of kt+1.
#define MOEZC_KSTEP(kt)                                                              \
  {                                                                                  \
    const int buf_ = (kt) & 1;                                                       \
    const bf16_t* as_r = As + buf_ * STAGE_A;                                        \
    const bf16_t* bs_r = Bs + buf_ * STAGE_B;                                        \
    if ((kt) + 1 < nk) {                                                             \
      MOEZC_GLOAD_B(rb, (kt) + 1);                                                   \
      MOEZC_GLOAD_A((kt) + 1);                                                       \
    }                                                                                \
    _Pragma("unroll") for (int ks = 0; ks + 1 < KS; ++ks) {                          \
      if (NA > 0) {                                                                  \
        MOEZC_LOADF((ks + 1) & 1, as_r, bs_r, ks + 1);                               \
        __builtin_amdgcn_sched_barrier(0);                                           \
        MOEZC_MMA(ks & 1);                                                           \
        __builtin_amdgcn_sched_barrier(0);                                           \
      }                                                                              \
    }                                                                                \
    if ((kt) + 1 < nk) MOEZC_LSTORE(rb, buf_ ^ 1);                                   \
    __syncthreads();                                                                 \
    if (NA > 0) {                                                                    \
      if ((kt) + 1 < nk) MOEZC_LOADF(0, As + (buf_ ^ 1) * STAGE_A,                   \
                                     Bs + (buf_ ^ 1) * STAGE_B, 0);                  \
      __builtin_amdgcn_sched_barrier(0);                                             \
      MOEZC_MMA((KS - 1) & 1);                                                       \
      __builtin_amdgcn_sched_barrier(0);                                             \
    }                                                                                \
  }

  constexpr int KS = BK / 16;  // MFMA substeps per k-step (even)
  static_assert(KS % 2 == 0, "fragment slots alternate");
  const int nk = p.K / BK;
  MOEZC_GLOAD_A(0);
  MOEZC_GLOAD_B(rb, 0);
  MOEZC_LSTORE(rb, 0);
  __syncthreads();
  if (NA > 0) MOEZC_LOADF(0, As, Bs, 0);
  for (int kt = 0; kt < nk; ++kt) MOEZC_KSTEP(kt);
#undef MOEZC_GLOAD_A
#undef MOEZC_GLOAD_B
#undef MOEZC_LSTORE
#undef MOEZC_LOADF
#undef MOEZC_MMA
#undef MOEZC_KSTEP
  if (NA == 0) return;

  // epilogue: D[i][j] of a 32x32 block sits in lane j + 32*((i/4)%2),
  // register 4*(i/8) + i%4
  const int lrow4 = 4 * (lane >> 5);
  const int lcol = lane & 31;
  if (EPI == kStoreF32) {
#pragma unroll
    for (int i = 0; i < NAc; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int gcol = c.n0 + wn * WTN + j * 32 + lcol;
        if (gcol >= p.Nout) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int grow = c.m0 + (i * WAVES_M + wm) * 32 + 8 * (v >> 2) + lrow4 + (v & 3);
          if (grow < c.m_end)
            static_cast<float*>(p.C)[(int64_t)grow * p.ldc + gcol] = acc[i][j][v];
        }
      }
    return;
  }
  // bf16 outputs go through a wavefront-private LDS tile so that global
  // stores are whole 16-byte row pieces (the main loop is done with LDS:
  // every wavefront passed the last barrier before its final MFMAs)
  constexpr int OC = SWIGLU ? HB * 32 : CB * 32;  // output columns of this wavefront
  constexpr int OS = OC + 8;                      // padded LDS row
  constexpr int RBmax = BM / WAVES_M / 32;          // same stride for every wavefront
  bf16_t* ot = As + wave * (RBmax * 32 * OS);         // As and Bs are one LDS block
  static_assert(WAVES_M * WAVES_N * RBmax * 32 * OS <= 2 * BM * LDS_STRIDE + 2 * BN * LDS_STRIDE,
                "output staging must fit in the LDS stages");
#pragma unroll
  for (int i = 0; i < NAc; ++i)
#pragma unroll
    for (int j = 0; j < OC / 32; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = i * 32 + 8 * (v >> 2) + lrow4 + (v & 3);
        float val;
        if (SWIGLU) {
          const float a = acc[i][j][v];
          val = a / (1.0f + __expf(-a)) * acc[i][j + HB][v];
        } else {
          val = acc[i][j][v];
        }
        ot[r * OS + j * 32 + lcol] = f32_to_bf16(val);
        // one 32x32 block at a time keeps the epilogue's live registers small
        if (v == 15) __builtin_amdgcn_sched_barrier(0);
      }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this lane's LDS writes landed
  __builtin_amdgcn_wave_barrier();
  const int gcol0 = c.n0 + (SWIGLU ? wn * HB * 32 : wn * WTN);
  bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.C);
  constexpr int CH = OC / 8;  // 16-byte pieces per row
#pragma unroll
  for (int q = lane; q < NAc * 32 * CH; q += 64) {
    const int r = q / CH, ch = q - r * CH;
    const int i = r >> 5;
    const int grow = c.m0 + (i * WAVES_M + wm) * 32 + (r & 31);
    const int gcol = gcol0 + ch * 8;
    if (grow < c.m_end && gcol < p.Nout)
      *reinterpret_cast<u32x4_t*>(&Cout[(int64_t)grow * p.ldc + gcol]) =
          *reinterpret_cast<const u32x4_t*>(&ot[r * OS + ch * 8]);
  }
}

template <int EPI, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void mfma_gemm_kernel(GemmProblem p,
                                                                               int n_tiles,
                                                                               int total_bound) {
  constexpr int WTM = BM / WAVES_M;
  constexpr int RB = WTM / 32;
  constexpr bool SWIGLU = (EPI == kSwiGLU_BF16);
  static_assert((BM / WAVES_M) % 32 == 0 && (BN / WAVES_N) % 32 == 0, "wave tile");
  static_assert(!SWIGLU || ((BN / WAVES_N) / 32) % 2 == 0, "SwiGLU needs gate and up blocks");
  // one LDS block: two A stages, then two B stages (the epilogue reuses all)
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * LDS_STRIDE];
  bf16_t* As = smem;
  bf16_t* Bs = smem + 2 * BM * LDS_STRIDE;

  // XCD-aware order: workgroup b runs on XCD b % 8; XCD x takes the logical
  // range [x * per, (x + 1) * per) of the live tiles
  const int total = p.tile_prefix ? p.tile_prefix[p.G] * n_tiles : total_bound;
  const int per = (total + 7) >> 3;
  const int jx = blockIdx.x >> 3;
  if (jx >= per) return;
  const int logical = (blockIdx.x & 7) * per + jx;
  TileCoord c;
  if (!map_tile<BM, BN, SWIGLU>(p, n_tiles, logical, c)) return;

  // live 32-row blocks of the tile, and how many of them this wavefront owns
  // (row block i of wavefront row wm is tile block i * WAVES_M + wm)
  const int wm = (threadIdx.x >> 6) / WAVES_N;
  const int nb = (c.m_end - c.m0 + 31) / 32;
  int na = (nb - wm + WAVES_M - 1) / WAVES_M;
  na = na < 0 ? 0 : (na > RB ? RB : na);
  switch (na) {
    case 0: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, 0>(p, c, As, Bs); break;
    case 1: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 1 ? 1 : 0)>(p, c, As, Bs); break;
    case 2: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 2 ? 2 : 0)>(p, c, As, Bs); break;
    case 3: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 3 ? 3 : 0)>(p, c, As, Bs); break;
    default: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 4 ? 4 : 0)>(p, c, As, Bs); break;
  }
}

template <int EPI, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmProblem& p, int64_t max_rows, hipStream_t s) {
  static_assert(BM / WM / 32 <= 4, "at most four row blocks per wavefront");
  const int n_tiles = (EPI == kSwiGLU_BF16) ? p.Nout / (BN / 2) : (p.Nout + BN - 1) / BN;
  int64_t mt_bound;
  if (p.tile_prefix) {
    mt_bound = (max_rows + (int64_t)p.G * (BM - 1)) / BM;
    if (mt_bound > max_rows) mt_bound = max_rows;
  } else {
    mt_bound = (p.M + BM - 1) / BM;
  }
  int64_t blocks = mt_bound * n_tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0) return hipErrorInvalidValue;
  blocks = (blocks + 7) / 8 * 8;
  hipLaunchKernelGGL((mfma_gemm_kernel<EPI, BM, BN, WM, WN>), dim3((unsigned)blocks),
                     dim3(64 * WM * WN), 0, s, p, n_tiles, (int)(mt_bound * n_tiles));
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_epi(const GemmProblem& p, int epi, int64_t max_rows, hipStream_t s) {
  switch (epi) {
    case kStoreF32: return launch_cfg<kStoreF32, BM, BN, WM, WN>(p, max_rows, s);
    case kStoreBF16: return launch_cfg<kStoreBF16, BM, BN, WM, WN>(p, max_rows, s);
    case kSwiGLU_BF16: return launch_cfg<kSwiGLU_BF16, BM, BN, WM, WN>(p, max_rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int mfma_tile_rows(int64_t expected_rows_per_group) {
  if (expected_rows_per_group < 48) return 32;
  if (expected_rows_per_group < 160) return 128;
  return 256;
}

hipError_t launch_mfma_gemm(const GemmProblem& p, int epilogue, int tile_rows, int64_t max_rows,
                            hipStream_t s) {
  if (p.K % BK != 0 || p.a_kwrap % BK != 0) return hipErrorInvalidValue;
  if (epilogue == kSwiGLU_BF16 && tile_rows != 32 && p.Nout % 128 != 0) return hipErrorInvalidValue;
  if (tile_rows == 256) return launch_epi<256, 256, 2, 4>(p, epilogue, max_rows, s);
  if (tile_rows == 128) return launch_epi<128, 256, 2, 4>(p, epilogue, max_rows, s);
  if (tile_rows == 32) return launch_epi<32, 256, 1, 4>(p, epilogue, max_rows, s);
  return hipErrorInvalidValue;
}

}  // namespace moezc
