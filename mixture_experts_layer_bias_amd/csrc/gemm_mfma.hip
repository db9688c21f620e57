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
  // rows past the end are clamped to a valid row; their products only reach
  // accumulator rows that are never stored
  int64_t a_off[A_LD];
  int b_off[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = min(c.m0 + lrow + ROWS_PER_LD * i, c.m_end - 1);
    a_off[i] = (int64_t)r * p.lda + lc;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = lrow + ROWS_PER_LD * i;
    if (SWIGLU) {
      const int n = c.n0 + (i < B_GATE_LD ? r : r - BN / 2);
      b_off[i] = n * (int)p.ldb + lc;
    } else {
      const int n = min(c.n0 + r, p.Nout - 1);
      b_off[i] = n * (int)p.ldb + lc;
    }
  }

  u32x4_t ra[A_LD], rb[B_LD];

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int brow[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    if (SWIGLU)
      brow[j] = (j < HB) ? wn * HB * 32 + j * 32 : BN / 2 + wn * HB * 32 + (j - HB) * 32;
    else
      brow[j] = wn * WTN + j * 32;
  }

  f32x16_t acc[NAc][CB];
#pragma unroll
  for (int i = 0; i < NAc; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // global -> registers for k-step kt (no lambdas: the staging arrays must
  // stay in registers)
#define MOEZC_GLOAD(kt)                                                              \
  {                                                                                  \
    const int ka_ = ((kt) * BK) % p.a_kwrap;                                         \
    const int kb_ = (kt) * BK;                                                       \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) ra[i] =                         \
        *reinterpret_cast<const u32x4_t*>(A + a_off[i] + ka_);                         \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) rb[i] =                         \
        *reinterpret_cast<const u32x4_t*>(((SWIGLU && i >= B_GATE_LD) ? B1 : B0) +     \
                                        b_off[i] + kb_);                             \
  }
#define MOEZC_LSTORE(buf)                                                            \
  {                                                                                  \
    bf16_t* as_ = As + (buf) * STAGE_A;                                              \
    bf16_t* bs_ = Bs + (buf) * STAGE_B;                                              \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i)                                 \
        *reinterpret_cast<u32x4_t*>(&as_[(lrow + ROWS_PER_LD * i) * LDS_STRIDE + lc]) = \
        ra[i];                                                                       \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i)                                 \
        *reinterpret_cast<u32x4_t*>(&bs_[(lrow + ROWS_PER_LD * i) * LDS_STRIDE + lc]) = \
        rb[i];                                                                       \
  }

  const int nk = p.K / BK;
  MOEZC_GLOAD(0);
  MOEZC_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) MOEZC_GLOAD(kt + 1);
    if (NA > 0) {
      const bf16_t* as = As + buf * STAGE_A;
      const bf16_t* bs = Bs + buf * STAGE_B;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int col = ks * 16 + (lane >> 5) * 8;
        bf16x8_t af[NAc], bfrag[CB];
#pragma unroll
        for (int i = 0; i < NAc; ++i) {
          const int row = wm * WTM + i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8_t*>(&as[row * LDS_STRIDE + col]);
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          const int row = brow[j] + (lane & 31);
          bfrag[j] = *reinterpret_cast<const bf16x8_t*>(&bs[row * LDS_STRIDE + col]);
        }
#pragma unroll
        for (int i = 0; i < NAc; ++i)
#pragma unroll
          for (int j = 0; j < CB; ++j)
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfrag[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) MOEZC_LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef MOEZC_GLOAD
#undef MOEZC_LSTORE
  if (NA == 0) return;

  // epilogue: D[i][j] of a 32x32 block sits in lane j + 32*((i/4)%2),
  // register 4*(i/8) + i%4
  const int lrow4 = 4 * (lane >> 5);
  const int lcol = lane & 31;
  if (SWIGLU) {
    bf16_t* __restrict__ H = static_cast<bf16_t*>(p.C);
#pragma unroll
    for (int i = 0; i < NAc; ++i)
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int gcol = c.n0 + wn * HB * 32 + j * 32 + lcol;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int grow = c.m0 + wm * WTM + i * 32 + 8 * (v >> 2) + lrow4 + (v & 3);
          if (grow < c.m_end) {
            const float a = acc[i][j][v];
            const float u = acc[i][j + HB][v];
            H[(int64_t)grow * p.ldc + gcol] = f32_to_bf16(a / (1.0f + __expf(-a)) * u);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < NAc; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int gcol = c.n0 + wn * WTN + j * 32 + lcol;
        if (gcol >= p.Nout) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int grow = c.m0 + wm * WTM + i * 32 + 8 * (v >> 2) + lrow4 + (v & 3);
          if (grow < c.m_end) {
            if (EPI == kStoreF32)
              static_cast<float*>(p.C)[(int64_t)grow * p.ldc + gcol] = acc[i][j][v];
            else
              static_cast<bf16_t*>(p.C)[(int64_t)grow * p.ldc + gcol] =
                  f32_to_bf16(acc[i][j][v]);
          }
        }
      }
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
  __shared__ __attribute__((aligned(16))) bf16_t As[2 * BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2 * BN * LDS_STRIDE];

  // XCD-aware order: workgroup b runs on XCD b % 8; XCD x takes the logical
  // range [x * per, (x + 1) * per) of the live tiles
  const int total = p.tile_prefix ? p.tile_prefix[p.G] * n_tiles : total_bound;
  const int per = (total + 7) >> 3;
  const int jx = blockIdx.x >> 3;
  if (jx >= per) return;
  const int logical = (blockIdx.x & 7) * per + jx;
  TileCoord c;
  if (!map_tile<BM, BN, SWIGLU>(p, n_tiles, logical, c)) return;

  const int wm = (threadIdx.x >> 6) / WAVES_N;
  int na = (c.m_end - (c.m0 + wm * WTM) + 31) / 32;
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
  if (tile_rows == 256) return launch_epi<256, 256, 2, 2>(p, epilogue, max_rows, s);
  if (tile_rows == 128) return launch_epi<128, 256, 2, 2>(p, epilogue, max_rows, s);
  if (tile_rows == 32) return launch_epi<32, 256, 1, 4>(p, epilogue, max_rows, s);
  return hipErrorInvalidValue;
}

}  // namespace moezc
