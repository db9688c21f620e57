// Grouped GEMM in fp32 on the vector ALUs (the fp32 storage path of the layer;
// small shapes).  Same problem description and device-side tile schedule as
// the MFMA path: C[rows of group g] = A[rows] * B_g^T, or for SwiGLU
// H = silu(A B_gate^T) * (A B_up^T).  64 x 64 outputs per workgroup of 256
// threads (4 x 4 each), BK = 16, operands staged through LDS transposed so
// the inner loop reads 16-byte vectors.
#include "kernels.hpp"

namespace moezc {

namespace {

constexpr int TM = 64, TN = 64, TK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void simt_gemm_kernel(GemmProblem p, int n_tiles) {
  constexpr bool SWIGLU = (EPI == kSwiGLU_F32);
  __shared__ __attribute__((aligned(16))) float As[TK][TM];
  __shared__ __attribute__((aligned(16))) float Bs[TK][TN];
  __shared__ float Cs[SWIGLU ? TM : 1][SWIGLU ? TN + 1 : 1];

  const int total_mt = p.tile_prefix ? p.tile_prefix[p.G] : (p.M + TM - 1) / TM;
  const int total = total_mt * n_tiles;
  const int logical = blockIdx.x;
  if (logical >= total) return;
  const int mt = logical / n_tiles, nt = logical - mt * n_tiles;
  int g = 0, m0, m_end;
  if (p.tile_prefix) {
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_prefix[mid] <= mt) lo = mid; else hi = mid;
    }
    g = lo;
    m0 = p.row_offsets[g] + (mt - p.tile_prefix[g]) * TM;
    m_end = p.row_offsets[g + 1];
  } else {
    m0 = mt * TM;
    m_end = p.M;
  }
  const int n0 = SWIGLU ? nt * (TN / 2) : nt * TN;
  const float* A = static_cast<const float*>(p.A);
  const float* B0 = static_cast<const float*>(p.B0) + (int64_t)g * p.b_group_stride;
  const float* B1 = SWIGLU ? static_cast<const float*>(p.B1) + (int64_t)g * p.b_group_stride : nullptr;

  const int tid = threadIdx.x;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;  // loader: one row, 4 k
  int ar = m0 + lrow;
  if (ar >= m_end) ar = m_end - 1;
  const float* a_ptr = A + (int64_t)ar * p.lda + lk;
  const float* b_ptr;
  if (SWIGLU) {
    b_ptr = (lrow < TN / 2 ? B0 + (int64_t)(n0 + lrow) * p.ldb
                           : B1 + (int64_t)(n0 + lrow - TN / 2) * p.ldb) + lk;
  } else {
    int n = n0 + lrow;
    if (n >= p.Nout) n = p.Nout - 1;
    b_ptr = B0 + (int64_t)n * p.ldb + lk;
  }

  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += TK) {
    const float4 av = *reinterpret_cast<const float4*>(a_ptr + (k0 % p.a_kwrap));
    const float4 bv = *reinterpret_cast<const float4*>(b_ptr + k0);
    As[lk + 0][lrow] = av.x; As[lk + 1][lrow] = av.y; As[lk + 2][lrow] = av.z; As[lk + 3][lrow] = av.w;
    Bs[lk + 0][lrow] = bv.x; Bs[lk + 1][lrow] = bv.y; Bs[lk + 2][lrow] = bv.z; Bs[lk + 3][lrow] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      const float4 a4 = *reinterpret_cast<const float4*>(&As[k][ty * 4]);
      const float4 b4 = *reinterpret_cast<const float4*>(&Bs[k][tx * 4]);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w}, b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  if (SWIGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) Cs[ty * 4 + i][tx * 4 + j] = acc[i][j];
    __syncthreads();
    float* H = static_cast<float*>(p.C);
    for (int q = tid; q < TM * (TN / 2); q += 256) {
      const int r = q / (TN / 2), c = q % (TN / 2);
      const int grow = m0 + r;
      if (grow < m_end) {
        const float a = Cs[r][c], u = Cs[r][c + TN / 2];
        H[(int64_t)grow * p.ldc + n0 + c] = a / (1.0f + expf(-a)) * u;
      }
    }
  } else {
    float* C = static_cast<float*>(p.C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int grow = m0 + ty * 4 + i;
      if (grow >= m_end) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gcol = n0 + tx * 4 + j;
        if (gcol < p.Nout) C[(int64_t)grow * p.ldc + gcol] = acc[i][j];
      }
    }
  }
}

}  // namespace

hipError_t launch_simt_gemm(const GemmProblem& p, int epilogue, int64_t max_rows, hipStream_t s) {
  if (p.K % TK != 0 || p.a_kwrap % TK != 0) return hipErrorInvalidValue;
  const bool sw = (epilogue == kSwiGLU_F32);
  if (sw && p.Nout % (TN / 2) != 0) return hipErrorInvalidValue;
  const int n_tiles = sw ? p.Nout / (TN / 2) : (p.Nout + TN - 1) / TN;
  int64_t mt_bound;
  if (p.tile_prefix) {
    mt_bound = (max_rows + (int64_t)p.G * (TM - 1)) / TM;
    if (mt_bound > max_rows) mt_bound = max_rows;
  } else {
    mt_bound = (p.M + TM - 1) / TM;
  }
  const int64_t blocks = mt_bound * n_tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (sw)
    hipLaunchKernelGGL(simt_gemm_kernel<kSwiGLU_F32>, dim3((unsigned)blocks), dim3(256), 0, s, p,
                       n_tiles);
  else if (epilogue == kStoreF32)
    hipLaunchKernelGGL(simt_gemm_kernel<kStoreF32>, dim3((unsigned)blocks), dim3(256), 0, s, p,
                       n_tiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moezc
