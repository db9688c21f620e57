// Launchers of the backward's kernels (backward.hip), for the C ABI.
#pragma once

#include "kernels.hpp"

namespace moezc {

// Backward (backward.hip).
// tile_prefix (row tiles of bm) and kofs (rows rounded up to 32) of the groups.
hipError_t launch_bwd_prefix(const int32_t* offsets, int N, int bm, int32_t* tile_prefix,
                             int32_t* kofs, hipStream_t s);
// colrow[c]: grouped row held by padded column c, or -1.
hipError_t launch_bwd_colrow(const int32_t* offsets, const int32_t* kofs, int N, int32_t* colrow,
                             int ncols, hipStream_t s);
// row_gate[pos[i]] = gate[i] for the FFN slots.
hipError_t launch_bwd_rowgate(const int32_t* pos, const float* gate, int64_t slots,
                              float* row_gate, hipStream_t s);
// Tiled transpose: dst[j][dst_col0 + c] = scale(s) src[row(s)][src_col0 + j],
// s = colrow ? colrow[c] : (c < ncols_valid ? c : -1) (zeros where s < 0),
// row(s) = rowidx ? rowidx[s] : s, scale = rowscale ? rowscale[s] : 1.
struct TrArgsHost {
  const void* src;
  int64_t src_ld, src_col0, src_bstride;
  const int32_t* rowidx;
  const float* rowscale;
  const int32_t* colrow;
  int64_t ncols_valid;
  void* dst;
  int64_t dst_ld, dst_col0, dst_bstride;
  int dim;
  int64_t ncols;
  int batch;
  bool src_f32, dst_f32;
  // non-null: expert-blocked, k-blocked destination (group g's columns
  // [kofs[g], kofs[g+1]) from element offset kofs[g] * dim as slabs of 32
  // columns: column k of the group, row j at (k / 32) * dim * 32 + j * 32 +
  // k % 32; dst_ld unused; batch 1, dst_col0 0)
  const int32_t* kofs;
  int ngroups;
};
hipError_t launch_transpose(const TrArgsHost& a, hipStream_t s);
hipError_t launch_swiglu_bwd(const void* A, const void* U, int64_t ld_au, bool au_bf16,
                             const float* Q, const float* row_gate, const int32_t* offsets, int N,
                             int I, int64_t max_rows, bf16_t* dau, bf16_t* H, float* row_dg,
                             hipStream_t s);
// Per token: gate gradients and the router softmax backward dl [T][ldl] bf16.
hipError_t launch_token_route_bwd(const bf16_t* x, const bf16_t* dy, const float* logits,
                                  const int32_t* idx, const int32_t* pos, const float* row_dg,
                                  int64_t T, int d, int E, int K, int N, bf16_t* dl, int ldl,
                                  hipStream_t s);
// dx = bf16(sum over slots of the expert row's dx or g dy, plus dx_r).
hipError_t launch_dx_sum(const bf16_t* dy, const int32_t* idx, const float* gate,
                         const int32_t* pos, const float* dxg, const float* dx_r, int64_t T, int d,
                         int K, int N, bf16_t* dx, hipStream_t s);
hipError_t launch_set_range(int32_t* out, int a, int b, hipStream_t s);
// C[g] = A_g B_g^T, fp32 [G][M][N], with A_g [M][R_g] and B_g [N][R_g] the
// expert-blocked operands in the transposes' k-blocked layout (slabs of 32
// columns; R_g = kofs[g+1] - kofs[g]).
// With 8 or more groups each XCD owns whole groups, as the plan that
// launch_wgrad_plan writes into xcd_groups (8 * wgrad_xcd_cap(G) int32, device)
// assigns them; the plan depends only on kofs and G, so one serves every
// launch with the same groups.
hipError_t launch_wgrad(const bf16_t* A, const bf16_t* B, const int32_t* kofs, int G, int M,
                        int N, float* C, const int32_t* xcd_groups, hipStream_t s);
int wgrad_xcd_cap(int G);
constexpr int kWgradMaxGroups = 2048;  // the most experts the library accepts
constexpr int kWgradMaxCap = (kWgradMaxGroups + 7) / 8 + (kWgradMaxGroups + 63) / 64;
hipError_t launch_wgrad_plan(const int32_t* kofs, int G, int32_t* xcd_groups, hipStream_t s);

}  // namespace moezc
