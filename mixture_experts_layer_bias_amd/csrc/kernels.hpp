// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moezc {

// Rows of tokens handled by one histogram chunk (one wavefront: one bit each).
constexpr int kChunk = 64;
constexpr int kMaxExperts = 2048;
constexpr int kMaxTopK = 32;

// ---- routing (route.hip) ----------------------------------------------------
// fp64 softmax, fp32 bias key, top-K with lowest-index tie-break.  With
// nsplit > 1, `logits` holds nsplit partial products split_stride apart: the
// logits are their sum in part order, written to logits_out.
hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int E, int K,
                       int32_t* idx, float* gate, hipStream_t s, int nsplit = 1,
                       int64_t split_stride = 0, float* logits_out = nullptr);
// loads[e] = slots of idx [T, K] routed to expert e (zeroed first).
hipError_t launch_count_loads(const int32_t* idx, int64_t T, int K, int E, int32_t* loads,
                              hipStream_t s);
// Per 64-token chunk: expert counts [C, E] and each FFN slot's rank among the
// chunk's earlier tokens (written to rank[T, K], -1 for zero experts).
hipError_t launch_chunk_hist(const int32_t* idx, int64_t T, int K, int E, int N,
                             int32_t* counts, int32_t* rank, hipStream_t s);
// counts [C, E] -> exclusive per-expert chunk bases (in place); loads [E];
// offsets [N+1]; m-tile prefix [N+1] for tiles of `bm` rows, and another for
// tiles of `bm2` rows when tile_prefix2 is not null.
hipError_t launch_scan(int32_t* counts, int C, int E, int N, int32_t* loads,
                       int32_t* offsets, int bm, int32_t* tile_prefix, int bm2,
                       int32_t* tile_prefix2, hipStream_t s);
// Grouped rows: pos (rank -> row), perm, and xp[row] = x[token] (the row
// copy only when xp is not null).
template <typename T>
hipError_t launch_permute(const T* x, const int32_t* idx, const int32_t* chunk_base,
                          const int32_t* offsets, int32_t* pos, int32_t* perm, T* xp,
                          int64_t Tn, int d, int K, int E, int N, hipStream_t s);
// y = r + sum_k g * (FFN row or x).
template <typename T>
hipError_t launch_combine(const T* x, const T* o, const T* res, const int32_t* idx,
                          const float* gate, const int32_t* pos, T* y, int64_t Tn,
                          int d, int K, int N, hipStream_t s);
hipError_t launch_pid(const int32_t* loads, const float* target, float* bias, float* e1,
                      float* e2, int E, float kp, float ki, float kd, hipStream_t s);

// ---- grouped GEMMs ------------------------------------------------------------
// C[rows of group g, :] = A[rows, :K] * B_g[:, :K]^T.  Groups are the FFN
// experts (rows = their grouped slots) or one group of M rows (router).
struct GemmProblem {
  const void* A;           // [rows, K] (row stride lda), or k-blocked (a_plane)
  int64_t lda;
  int a_kwrap;             // A column = k % a_kwrap (router: d; else K)
  int64_t a_plane;         // k-blocked A: bytes between planes of 64 k, each
                           // [rows][64] (row stride 128 B); 0 = row-major A
  const int32_t* a_rows;   // row-major A only: GEMM row s reads A row
                           // a_rows[s] (gather), or null: A row s
  const void* B0;          // [G][Nout or I][K] weights (gate or plain)
  const void* B1;          // up weights for SwiGLU, else null
  int64_t ldb;             // row stride of B
  int64_t b_group_stride;  // elements between groups of B
  void* C;                 // output
  int64_t ldc;
  int K;                   // reduction length
  int Nout;                // output columns (SwiGLU: I)
  const int32_t* row_offsets;  // [G+1] device, or null: one group of M rows
  const int32_t* tile_prefix;  // [G+1] device m-tile prefix, or null
  int G;
  int M;
  const uint8_t* a_scales;  // block-FP8 A only: [rows][K / 32] scale bytes
  int64_t a_scale_ld;       // scale bytes per A row (K / 32)
  // packed fp32-output GEMM only (the router): the K range is cut into
  // k_splits equal parts and part s writes its partial product to
  // C + s * c_split_stride (0 or 1: one part, C itself)
  int k_splits;
  int64_t c_split_stride;
  // kSwiGLU_BF16_ACT (and the block-FP8 GEMM when set): the pre-activations
  // in bf16, a = x W_gate^T to C2[row][col] and u = x W_up^T to C2[row][Nout + col]
  void* C2;
  int64_t ldc2;
  // kSwiGLU_FP8 (block-FP8 GEMM only): h quantized in blocks of 32 columns,
  // E4M3 codes to C (ldc bytes per row) and scale bytes to
  // c_scales[row * c_scale_ld + col / 32]
  uint8_t* c_scales;
  int64_t c_scale_ld;
};

// kSwiGLU_BF16_ACT: kSwiGLU_BF16 that also stores the pre-activations to C2
// (a separate instantiation, so the plain SwiGLU kernels are unchanged).
enum Epilogue { kStoreF32 = 0, kStoreBF16 = 1, kSwiGLU_BF16 = 2, kSwiGLU_F32 = 3,
                kSwiGLU_BF16_ACT = 4, kSwiGLU_FP8 = 5 };
constexpr bool is_swiglu_bf16(int epi) { return epi == kSwiGLU_BF16 || epi == kSwiGLU_BF16_ACT; }

// bf16 MFMA path (gemm_mfma.hip).  `tile_rows` selects the row-tile variant
// (128 for many rows per expert, 32 for a few); the scan must have used it.
hipError_t launch_mfma_gemm(const GemmProblem& p, int epilogue, int tile_rows,
                            int64_t max_rows, hipStream_t s);
int mfma_tile_rows(int64_t expected_rows_per_group);

// bf16 MFMA path on packed weights (gemm_packed.hip).  Panels of
// kPackedPanel weight rows (SwiGLU: half gate, half up rows), stages of 64 k,
// one 32 KB block per (group, panel, stage); tiles of at most
// kPackedMaxTileRows rows, any multiple of 32.
constexpr int kPackedPanel = 256;
constexpr int kPackedMaxTileRows = 256;
// Bytes of one group's packed weights: `rows` weight rows (SwiGLU: hidden
// units, gate and up together) by K.
int64_t packed_bytes(int64_t rows, int64_t K, bool swiglu);
// Row-major [groups][rows][K] (gate w0 and up w1 for SwiGLU) -> packed.
// Packed layout (non-SwiGLU panels) of a transposed operand, gathered from the
// untransposed weights: row r, reduction index k <- (k < k_split ? w0[k] :
// w1[k - k_split])[r], source rows src_ld elements long.
hipError_t launch_pack_transposed(const bf16_t* w0, const bf16_t* w1, bf16_t* out, int groups,
                                  int rows, int K, int k_split, int src_ld, int64_t group_stride,
                                  hipStream_t s);
hipError_t launch_pack_weights(const bf16_t* w0, const bf16_t* w1, bf16_t* out, int groups,
                               int rows, int K, bool swiglu, hipStream_t s);
// W_router fp32 [E, d] -> packed two-term bf16 split [E, 2d].
hipError_t launch_split_router_packed(const float* w, bf16_t* out, int E, int d, hipStream_t s);
// B0 = packed weights; B1, ldb and b_group_stride are unused.  The down GEMM
// (kStoreBF16) runs tiles of at most packed_down_tile_rows() rows.
hipError_t launch_packed_gemm(const GemmProblem& p, int epilogue, int tile_rows,
                              int64_t max_rows, hipStream_t s);
int packed_down_tile_rows(int ffn_tile_rows);

// Block-FP8 path (gemm_fp8.hip): E4M3 codes with one power-of-two scale per
// 32 values along k; gate/up always, the down projection optionally.
// Bytes of one group's packed FP8 gate/up weights (I hidden units by d), and
// of its packed FP8 down weights (d rows by I).
int64_t fp8_packed_bytes(int64_t I, int64_t d);
int64_t fp8_packed_down_bytes(int64_t d, int64_t I);
// x [rows][d] bf16 -> codes [rows][d] and scale bytes [rows][d / 32].
hipError_t launch_quantize_mx(const bf16_t* x, uint8_t* xq, uint8_t* xs, int64_t rows, int64_t d,
                              hipStream_t s);
// W_gate, W_up [groups][I][d] bf16 -> packed FP8 gate/up blocks.
hipError_t launch_pack_weights_fp8(const bf16_t* wg, const bf16_t* wu, uint8_t* out, int groups,
                                   int I, int d, hipStream_t s);
// W_down [groups][d][I] bf16 -> packed FP8 down blocks.
hipError_t launch_pack_down_fp8(const bf16_t* wd, uint8_t* out, int groups, int d, int I,
                                hipStream_t s);
// Grouped GEMM on FP8 operands: A = FP8 codes (row stride lda bytes, optional
// gather a_rows), a_scales / a_scale_ld its scales, B0 = packed FP8 weights.
// epilogue kSwiGLU_BF16 (or _ACT with C2): C = h bf16 from gate/up blocks;
// kSwiGLU_FP8 (C2 optional, as _ACT): h quantized from its fp32 values in
// blocks of 32 hidden units, codes to C and scales to c_scales;
// kStoreBF16: C = A B^T bf16 from down blocks.  Tiles of at most
// kPackedMaxTileRows rows, as the bf16 packed path.
hipError_t launch_fp8_gemm(const GemmProblem& p, int epilogue, int tile_rows, int64_t max_rows,
                           hipStream_t s);

// fp32 FMA path (gemm_simt.hip).
hipError_t launch_simt_gemm(const GemmProblem& p, int epilogue, int64_t max_rows,
                            hipStream_t s);
constexpr int kSimtTileRows = 64;

}  // namespace moezc
