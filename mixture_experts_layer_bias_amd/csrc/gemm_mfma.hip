// Grouped GEMM on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
//   C[rows of group g, :] = A[rows, :] * B_g^T        (router, expert down)
//   H[rows of group g, :] = silu(A B_gate_g^T) * (A B_up_g^T)   (expert gate/up)
//
// Groups are the FFN experts; their rows are the grouped (token, expert) slots
// written by the permute kernel, and the device-side m-tile prefix from the
// scan tells each workgroup which expert and which rows it owns, so the grid
// can be sized without reading any count back to the host and experts with no
// rows cost nothing.  Both operands are K-contiguous ([rows, K] activations,
// nn.Linear [out, in] weights), which is exactly the per-lane layout the MFMA
// wants: lane l feeds row (l % 32) with the 8 consecutive k at 8*(l / 32).
//
// Tiles: BM x BN outputs per workgroup, BK = 64, two LDS stages (global loads
// of step k+1 are issued before the MFMAs of step k).  LDS rows are padded to
// 72 bf16 so the 16-byte fragment reads of a wavefront hit distinct banks.
// Workgroup -> tile mapping is XCD-aware: consecutive workgroups land on
// different XCDs (round robin), so each XCD is given a contiguous range of
// logical tiles; tiles of one expert then share that XCD's L2 for the expert's
// activation rows and weight panel.
#include "kernels.hpp"

namespace moezc {

namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row

template <int EPI, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void mfma_gemm_kernel(GemmProblem p,
                                                                            int n_tiles) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M;
  constexpr int WTN = BN / WAVES_N;
  constexpr int RB = WTM / 32;
  constexpr int CB = WTN / 32;
  constexpr bool SWIGLU = (EPI == kSwiGLU_BF16);
  constexpr int HB = CB / 2;  // gate blocks per wave (SwiGLU)
  constexpr int A_LD = (BM * BK / 8) / NT;  // 16-byte chunks per thread
  constexpr int B_LD = (BN * BK / 8) / NT;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the workgroup");
  static_assert(!SWIGLU || (CB % 2 == 0), "SwiGLU needs gate and up blocks per wave");

  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDS_STRIDE];

  // ---- which tile ---------------------------------------------------------
  const int total_mt = p.tile_prefix ? p.tile_prefix[p.G] : (p.M + BM - 1) / BM;
  const int total = total_mt * n_tiles;
  const int xcd = blockIdx.x & 7;
  const int jx = blockIdx.x >> 3;
  const int per = (total + 7) >> 3;
  if (jx >= per) return;
  const int logical = xcd * per + jx;
  if (logical >= total) return;
  const int mt = logical / n_tiles;
  const int nt = logical - mt * n_tiles;
  int g = 0, m0, m_end;
  if (p.tile_prefix) {
    int lo = 0, hi = p.G;  // tile_prefix[lo] <= mt < tile_prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_prefix[mid] <= mt) lo = mid; else hi = mid;
    }
    g = lo;
    m0 = p.row_offsets[g] + (mt - p.tile_prefix[g]) * BM;
    m_end = p.row_offsets[g + 1];
  } else {
    m0 = mt * BM;
    m_end = p.M;
  }
  const int n0 = SWIGLU ? nt * (BN / 2) : nt * BN;

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  const bf16_t* __restrict__ B0 = static_cast<const bf16_t*>(p.B0) + (int64_t)g * p.b_group_stride;
  const bf16_t* __restrict__ B1 =
      SWIGLU ? static_cast<const bf16_t*>(p.B1) + (int64_t)g * p.b_group_stride : nullptr;

  const int tid = threadIdx.x;
  // per-thread global row offsets for the tile loads (rows past the end are
  // clamped to a valid row; their products land in rows that are not stored)
  int64_t a_off[A_LD], b_off[B_LD];
  const bf16_t* b_base[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + NT * i;
    int r = m0 + (q >> 3);
    if (r >= m_end) r = m_end - 1;
    a_off[i] = (int64_t)r * p.lda + (q & 7) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = tid + NT * i;
    const int r = q >> 3;
    if (SWIGLU) {
      const bool up = r >= BN / 2;
      b_base[i] = up ? B1 : B0;
      b_off[i] = (int64_t)(n0 + (up ? r - BN / 2 : r)) * p.ldb + (q & 7) * 8;
    } else {
      int n = n0 + r;
      if (n >= p.Nout) n = p.Nout - 1;
      b_base[i] = B0;
      b_off[i] = (int64_t)n * p.ldb + (q & 7) * 8;
    }
  }

  uint4 ra[A_LD], rb[B_LD];
  auto gload = [&](int kt) {
    const int ka = (kt * BK) % p.a_kwrap;
    const int kb = kt * BK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const uint4*>(A + a_off[i] + ka);
#pragma unroll
    for (int i = 0; i < B_LD; ++i)
      rb[i] = *reinterpret_cast<const uint4*>(b_base[i] + b_off[i] + kb);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + NT * i;
      *reinterpret_cast<uint4*>(&As[buf][(q >> 3) * LDS_STRIDE + (q & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int q = tid + NT * i;
      *reinterpret_cast<uint4*>(&Bs[buf][(q >> 3) * LDS_STRIDE + (q & 7) * 8]) = rb[i];
    }
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int brow[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (SWIGLU)
      brow[cb] = (cb < HB) ? wn * HB * 32 + cb * 32 : BN / 2 + wn * HB * 32 + (cb - HB) * 32;
    else
      brow[cb] = wn * WTN + cb * 32;
  }

  f32x16_t acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = p.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int col = ks * 16 + (lane >> 5) * 8;
      bf16x8_t af[RB], bfrag[CB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int row = wm * WTM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][row * LDS_STRIDE + col]);
      }
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int row = brow[j] + (lane & 31);
        bfrag[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][row * LDS_STRIDE + col]);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfrag[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D[i][j] of a 32x32 block sits in lane j + 32*((i/4)%2),
  // register 4*(i/8) + i%4 -------------------------------------------------
  const int lrow = 4 * (lane >> 5);
  const int lcol = lane & 31;
  if (SWIGLU) {
    bf16_t* __restrict__ H = static_cast<bf16_t*>(p.C);
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int gcol = n0 + wn * HB * 32 + j * 32 + lcol;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int grow = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + lrow + (v & 3);
          if (grow < m_end) {
            const float a = acc[i][j][v];
            const float u = acc[i][j + HB][v];
            H[(int64_t)grow * p.ldc + gcol] = f32_to_bf16(a / (1.0f + __expf(-a)) * u);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int gcol = n0 + wn * WTN + j * 32 + lcol;
        if (gcol >= p.Nout) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int grow = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + lrow + (v & 3);
          if (grow < m_end) {
            if (EPI == kStoreF32)
              static_cast<float*>(p.C)[(int64_t)grow * p.ldc + gcol] = acc[i][j][v];
            else
              static_cast<bf16_t*>(p.C)[(int64_t)grow * p.ldc + gcol] = f32_to_bf16(acc[i][j][v]);
          }
        }
      }
  }
}

template <int EPI, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmProblem& p, int64_t max_rows, hipStream_t s) {
  const int n_tiles = (EPI == kSwiGLU_BF16) ? p.Nout / (BN / 2) : (p.Nout + BN - 1) / BN;
  int64_t mt_bound;
  if (p.tile_prefix) {
    mt_bound = (max_rows + (int64_t)p.G * (BM - 1)) / BM;
    if (mt_bound > max_rows) mt_bound = max_rows;
  } else {
    mt_bound = (p.M + BM - 1) / BM;
  }
  int64_t blocks = mt_bound * n_tiles;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mfma_gemm_kernel<EPI, BM, BN, WM, WN>), dim3((unsigned)blocks),
                     dim3(64 * WM * WN), 0, s, p, n_tiles);
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
  return expected_rows_per_group >= 48 ? 128 : 32;
}

hipError_t launch_mfma_gemm(const GemmProblem& p, int epilogue, int tile_rows, int64_t max_rows,
                            hipStream_t s) {
  if (p.K % BK != 0 || p.a_kwrap % BK != 0) return hipErrorInvalidValue;
  if (tile_rows == 128) return launch_epi<128, 128, 2, 2>(p, epilogue, max_rows, s);
  if (tile_rows == 32) return launch_epi<32, 256, 1, 4>(p, epilogue, max_rows, s);
  return hipErrorInvalidValue;
}

}  // namespace moezc
