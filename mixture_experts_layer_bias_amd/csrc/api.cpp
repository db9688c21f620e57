// C ABI of the MoE layer with zero-computation experts: argument checks,
// workspace plan and the stream-ordered launch sequence.  See
// include/moe_zc.h for the contract of each entry point.
#include "../../include/moe_zc.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "backward.hpp"
#include "kernels.hpp"

using namespace moezc;

static_assert(kWgradMaxGroups >= MOE_ZC_MAX_EXPERTS, "the weight-gradient plan covers every expert");

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Shape {
  int64_t T, d, I;
  int32_t N, Z, K, E;
  moe_zc_dtype dt;
  int64_t smax;  // T * min(K, N): most (token, FFN expert) rows possible
  int64_t chunks;
  size_t es;     // element size of dt
  int ffn_tile_rows;
  // the bf16 expert GEMMs gather their rows of x through perm (byte offsets
  // into x below 2^31); otherwise the permute stage copies them into xp
  bool gather;
};

// Host-side shape validation shared by every entry point that takes sizes.
moe_zc_status check_shape(int64_t T, int64_t d, int64_t I, int32_t N, int32_t Z, int32_t K,
                          moe_zc_dtype dt, Shape* s) {
  if (dt != MOE_ZC_F32 && dt != MOE_ZC_BF16) return MOE_ZC_ERR_INVALID;
  if (T < 0 || d <= 0 || I <= 0 || N < 0 || Z < 0 || K < 1) return MOE_ZC_ERR_INVALID;
  const int64_t E = (int64_t)N + Z;
  if (E < 1 || K > E) return MOE_ZC_ERR_INVALID;
  if (E > MOE_ZC_MAX_EXPERTS || K > MOE_ZC_MAX_TOPK) return MOE_ZC_ERR_UNSUPPORTED;
  if (dt == MOE_ZC_BF16 ? (d % 64 != 0 || I % 128 != 0) : (d % 32 != 0 || I % 32 != 0))
    return MOE_ZC_ERR_UNSUPPORTED;
  if (d * I >= (int64_t(1) << 31) || 2 * d * E >= (int64_t(1) << 31)) return MOE_ZC_ERR_UNSUPPORTED;
  const int64_t smax = T * std::min<int64_t>(K, N);
  if (smax >= (int64_t(1) << 31) || T * K >= (int64_t(1) << 31) || T >= (int64_t(1) << 31))
    return MOE_ZC_ERR_UNSUPPORTED;
  const int64_t widest = std::max<int64_t>(std::max<int64_t>(d, I), E);
  if (T > 0 && widest > (int64_t(1) << 40) / T) return MOE_ZC_ERR_UNSUPPORTED;
  // 32-bit byte offsets of up to 256 rows inside a GEMM tile
  if (d >= (int64_t(1) << 20) || I >= (int64_t(1) << 20)) return MOE_ZC_ERR_UNSUPPORTED;
  s->T = T; s->d = d; s->I = I; s->N = N; s->Z = Z; s->K = K; s->E = (int32_t)E; s->dt = dt;
  s->smax = smax;
  s->chunks = (T + kChunk - 1) / kChunk;
  s->es = (dt == MOE_ZC_BF16) ? 2 : 4;
  s->gather = (dt == MOE_ZC_BF16) && T * d * 2 < (int64_t(1) << 31);
  if (dt == MOE_ZC_BF16) {
    const int64_t expected = (N > 0) ? (T * K) / E : 0;  // rows per expert, symmetric routing
    s->ffn_tile_rows = mfma_tile_rows(expected);
  } else {
    s->ffn_tile_rows = kSimtTileRows;
  }
  return MOE_ZC_OK;
}

// Extra conditions of the block-FP8 forward: bf16 data, stages of 128 k,
// and byte offsets into the FP8 copy of x below 2^31 (rows are gathered).
moe_zc_status check_fp8_shape(const Shape& s) {
  if (s.dt != MOE_ZC_BF16) return MOE_ZC_ERR_UNSUPPORTED;
  if (s.d % 128 != 0 || s.T * s.d >= (int64_t(1) << 31)) return MOE_ZC_ERR_UNSUPPORTED;
  // the FP8 copy of h (down projection in FP8): 32-bit row byte offsets
  if (s.smax * s.I >= (int64_t(1) << 31)) return MOE_ZC_ERR_UNSUPPORTED;
  return MOE_ZC_OK;
}

struct Plan {
  size_t logits, idx, gate, pos, loads, offsets, perm, counts, tiles, tiles2, wr2, xp, h, o;
  size_t xq, xs;    // FP8 codes and scales of x (block-FP8 forward only)
  size_t hq, hs;    // FP8 codes and scales of h (block-FP8 down projection)
  size_t lsplit;    // partial router products of a split-K router
  int splits;       // parts of the router's K range (1: not split)
  size_t total;
};

int router_tile_rows(int64_t T, int E);
int router_splits(int64_t T, int E, int64_t d);

Plan make_plan(const Shape& s, bool fp8 = false) {
  Plan p{};
  p.splits = (s.dt == MOE_ZC_BF16) ? router_splits(s.T, s.E, s.d) : 1;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += align_up(bytes);
    return here;
  };
  p.logits = take((size_t)s.T * s.E * 4);
  p.idx = take((size_t)s.T * s.K * 4);
  p.gate = take((size_t)s.T * s.K * 4);
  p.pos = take((size_t)s.T * s.K * 4);
  p.loads = take((size_t)s.E * 4);
  p.offsets = take((size_t)(s.N + 1) * 4);
  p.perm = take((size_t)std::max<int64_t>(s.smax, 1) * 4);
  p.counts = take((size_t)s.chunks * s.E * 4);
  p.tiles = take((size_t)(s.N + 1) * 4);
  p.tiles2 = take((size_t)(s.N + 1) * 4);
  p.wr2 = take(s.dt == MOE_ZC_BF16 ? (size_t)packed_bytes(s.E, 2 * s.d, false) : 0);
  p.xp = take(s.gather ? 0 : (size_t)s.smax * s.d * s.es);
  p.h = take((size_t)s.smax * s.I * s.es);
  p.o = take((size_t)s.smax * s.d * s.es);
  p.xq = take(fp8 ? (size_t)s.T * s.d : 0);
  p.xs = take(fp8 ? (size_t)s.T * (s.d / 32) : 0);
  p.hq = take(fp8 ? (size_t)s.smax * s.I : 0);
  p.hs = take(fp8 ? (size_t)s.smax * (s.I / 32) : 0);
  p.lsplit = take(p.splits > 1 ? (size_t)p.splits * s.T * s.E * 4 : 0);
  p.total = at;
  return p;
}

#define MOE_ZC_TRY(expr)                          \
  do {                                            \
    if ((expr) != hipSuccess) return MOE_ZC_ERR_HIP; \
  } while (0)

// Rows per router tile: enough tiles to cover the 256 CUs once where T allows
// (the router is one group of T rows by E columns in 256-column panels).
int router_tile_rows(int64_t T, int E) {
  const int64_t panels = (E + kPackedPanel - 1) / kPackedPanel;
  const int64_t tiles_m = std::max<int64_t>(1, 256 / panels);
  int64_t rows = (T + tiles_m - 1) / tiles_m;
  rows = (rows + 31) / 32 * 32;
  return (int)std::min<int64_t>(std::max<int64_t>(rows, 32), kPackedMaxTileRows);
}

// Parts of the bf16 router's K range (2d in stages of 64).  Few tokens give
// few row tiles (T = 128: 12 tiles of 192 stages each, on 256 CUs), and each
// tile then walks a long K range alone; splitting K into equal parts of at
// least four stages brings the tile count near one per CU.  More than 128
// row tiles are left whole.
int router_splits(int64_t T, int E, int64_t d) {
  if (T <= 0) return 1;
  const int64_t panels = (E + kPackedPanel - 1) / kPackedPanel;
  const int64_t rows = router_tile_rows(T, E);
  const int64_t tiles = (T + rows - 1) / rows * panels;
  if (tiles > 128) return 1;
  const int64_t nk = 2 * d / 64;
  const int64_t target = (256 + tiles - 1) / tiles;
  int best = 1;
  for (int64_t sp = 2; sp <= target; ++sp)
    if (nk % sp == 0 && nk / sp >= 4) best = (int)sp;
  return best;
}

enum Layout { kRowMajor = 0, kPacked = 1, kPackedFp8 = 2 };

// The forward on one of the weight layouts.  kPacked: bf16 expert weights as
// written by moe_zc_pack_expert_weights (gate_up and down point there);
// kPackedFp8: the gate/up weights as written by moe_zc_pack_expert_weights_fp8
// and the down weights packed bf16 (or FP8 with down_fp8); x is quantized per
// forward, and h too when the down projection runs in FP8.
moe_zc_status forward_impl(const void* x, const float* w_router, const float* bias,
                           const void* w_gate, const void* w_up, const void* w_down,
                           Layout layout, const void* residual, void* y, int64_t T, int64_t d,
                           int64_t I, int32_t N, int32_t Z, int32_t K, moe_zc_dtype dt,
                           moe_zc_aux* aux, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, bool down_fp8 = false) {
  Shape s;
  const moe_zc_status st = check_shape(T, d, I, N, Z, K, dt, &s);
  if (st != MOE_ZC_OK) return st;
  const bool packed = layout != kRowMajor;
  const bool fp8 = layout == kPackedFp8;
  if (packed && dt != MOE_ZC_BF16) return MOE_ZC_ERR_UNSUPPORTED;
  if (fp8) {
    const moe_zc_status s8 = check_fp8_shape(s);
    if (s8 != MOE_ZC_OK) return s8;
  }
  if (T == 0) return MOE_ZC_OK;
  if (!x || !w_router || !bias || !y) return MOE_ZC_ERR_INVALID;
  if (N > 0 && (!w_gate || !w_down || (!packed && !w_up))) return MOE_ZC_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y) || !aligned16(w_router) || (residual && !aligned16(residual)))
    return MOE_ZC_ERR_INVALID;
  if (N > 0 && (!aligned16(w_gate) || !aligned16(w_down) || (!packed && !aligned16(w_up))))
    return MOE_ZC_ERR_INVALID;
  void* act = aux ? aux->act : nullptr;  // pre-activations, saved for the backward
  if (act && dt != MOE_ZC_BF16) return MOE_ZC_ERR_UNSUPPORTED;
  if (act && !aligned16(act)) return MOE_ZC_ERR_INVALID;
  const Plan pl = make_plan(s, fp8);
  if (!workspace || workspace_bytes < pl.total) return MOE_ZC_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_ZC_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  float* logits = (aux && aux->logits) ? aux->logits : reinterpret_cast<float*>(ws + pl.logits);
  int32_t* idx = (aux && aux->topk_idx) ? aux->topk_idx : reinterpret_cast<int32_t*>(ws + pl.idx);
  float* gate = (aux && aux->topk_gate) ? aux->topk_gate : reinterpret_cast<float*>(ws + pl.gate);
  int32_t* pos = (aux && aux->pos) ? aux->pos : reinterpret_cast<int32_t*>(ws + pl.pos);
  int32_t* loads = (aux && aux->loads) ? aux->loads : reinterpret_cast<int32_t*>(ws + pl.loads);
  int32_t* offsets =
      (aux && aux->offsets) ? aux->offsets : reinterpret_cast<int32_t*>(ws + pl.offsets);
  int32_t* perm = (aux && aux->perm) ? aux->perm : reinterpret_cast<int32_t*>(ws + pl.perm);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + pl.counts);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + pl.tiles);
  // the packed down GEMM runs shorter row tiles, with a schedule of its own
  int32_t* tiles2 = packed ? reinterpret_cast<int32_t*>(ws + pl.tiles2) : nullptr;
  const int down_rows = packed ? packed_down_tile_rows(s.ffn_tile_rows) : s.ffn_tile_rows;
  hipEvent_t* ev = (aux && aux->stage_events) ? aux->stage_events : nullptr;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };

  const bool bf = (dt == MOE_ZC_BF16);
  const bool gather = s.gather;
  void* xp = ws + pl.xp;
  void* h = ws + pl.h;
  void* o = ws + pl.o;
  const int E = s.E;

  // stage 0: router logits
  MOE_ZC_TRY(mark(0));
  {
    GemmProblem p{};
    p.A = x; p.lda = d; p.a_kwrap = (int)d;
    p.C = logits; p.ldc = E; p.Nout = E;
    p.G = 1; p.M = (int)T;
    if (bf) {
      bf16_t* wr2 = reinterpret_cast<bf16_t*>(ws + pl.wr2);
      MOE_ZC_TRY(launch_split_router_packed(w_router, wr2, E, (int)d, stream));
      p.B0 = wr2; p.K = (int)(2 * d);
      if (pl.splits > 1) {  // partial products, summed by the top-K stage
        p.C = ws + pl.lsplit;
        p.k_splits = pl.splits;
        p.c_split_stride = T * E;
      }
      MOE_ZC_TRY(launch_packed_gemm(p, kStoreF32, router_tile_rows(T, E), T, stream));
    } else {
      p.B0 = w_router; p.ldb = d; p.K = (int)d;
      MOE_ZC_TRY(launch_simt_gemm(p, kStoreF32, T, stream));
    }
  }
  // stage 1: softmax, bias key, top-K
  MOE_ZC_TRY(mark(1));
  if (bf && pl.splits > 1)
    MOE_ZC_TRY(launch_topk(reinterpret_cast<const float*>(ws + pl.lsplit), bias, T, E, K, idx,
                           gate, stream, pl.splits, T * E, logits));
  else
    MOE_ZC_TRY(launch_topk(logits, bias, T, E, K, idx, gate, stream));
  // stage 2: per-chunk histogram and in-chunk ranks (into pos)
  MOE_ZC_TRY(mark(2));
  MOE_ZC_TRY(launch_chunk_hist(idx, T, K, E, N, counts, pos, stream));
  // stage 3: loads, offsets, tile schedule
  MOE_ZC_TRY(mark(3));
  MOE_ZC_TRY(launch_scan(counts, (int)s.chunks, E, N, loads, offsets, s.ffn_tile_rows, tiles,
                         down_rows, tiles2, stream));
  // stage 4: grouping permutation and row gather
  MOE_ZC_TRY(mark(4));
  if (bf)
    MOE_ZC_TRY(launch_permute<bf16_t>(static_cast<const bf16_t*>(x), idx, counts, offsets, pos,
                                      perm, gather ? nullptr : static_cast<bf16_t*>(xp), T,
                                      (int)d, K, E, N, stream));
  else
    MOE_ZC_TRY(launch_permute<float>(static_cast<const float*>(x), idx, counts, offsets, pos,
                                     perm, static_cast<float*>(xp), T, (int)d, K, E, N, stream));
  // stages 5, 6: expert FFNs as grouped GEMMs
  MOE_ZC_TRY(mark(5));
  if (N > 0) {
    GemmProblem p{};
    p.A = gather ? x : xp; p.lda = d; p.a_kwrap = (int)d; p.K = (int)d;
    p.a_rows = gather ? perm : nullptr;
    p.B0 = w_gate; p.B1 = w_up; p.ldb = d; p.b_group_stride = I * d;
    p.C = h; p.ldc = I; p.Nout = (int)I;
    p.row_offsets = offsets; p.tile_prefix = tiles; p.G = N; p.M = 0;
    p.C2 = act; p.ldc2 = 2 * I;
    const int swiglu_epi = act ? kSwiGLU_BF16_ACT : kSwiGLU_BF16;
    if (fp8) {
      // block-FP8 gate/up: x quantized once, its code rows gathered through perm
      uint8_t* xq = reinterpret_cast<uint8_t*>(ws + pl.xq);
      uint8_t* xs = reinterpret_cast<uint8_t*>(ws + pl.xs);
      MOE_ZC_TRY(launch_quantize_mx(static_cast<const bf16_t*>(x), xq, xs, T, d, stream));
      p.A = xq; p.a_rows = perm;
      p.a_scales = xs; p.a_scale_ld = d / 32;
      if (down_fp8) {
        // h leaves the epilogue already quantized for the FP8 down projection
        // (from its fp32 values), instead of as bf16
        p.C = ws + pl.hq; p.ldc = I;
        p.c_scales = reinterpret_cast<uint8_t*>(ws + pl.hs); p.c_scale_ld = I / 32;
        MOE_ZC_TRY(launch_fp8_gemm(p, kSwiGLU_FP8, s.ffn_tile_rows, s.smax, stream));
      } else {
        MOE_ZC_TRY(launch_fp8_gemm(p, swiglu_epi, s.ffn_tile_rows, s.smax, stream));
      }
    } else if (packed)
      MOE_ZC_TRY(launch_packed_gemm(p, swiglu_epi, s.ffn_tile_rows, s.smax, stream));
    else if (bf)
      MOE_ZC_TRY(launch_mfma_gemm(p, swiglu_epi, s.ffn_tile_rows, s.smax, stream));
    else
      MOE_ZC_TRY(launch_simt_gemm(p, kSwiGLU_F32, s.smax, stream));
  }
  MOE_ZC_TRY(mark(6));
  if (N > 0) {
    GemmProblem p{};
    p.A = h; p.lda = I; p.a_kwrap = (int)I; p.K = (int)I;
    p.B0 = w_down; p.ldb = I; p.b_group_stride = d * I;
    p.C = o; p.ldc = d; p.Nout = (int)d;
    p.row_offsets = offsets; p.tile_prefix = packed ? tiles2 : tiles; p.G = N; p.M = 0;
    if (fp8 && down_fp8) {
      // block-FP8 down projection on the codes and scales of h that the
      // gate/up epilogue wrote, on the gate/up tile schedule
      uint8_t* hq = reinterpret_cast<uint8_t*>(ws + pl.hq);
      uint8_t* hs = reinterpret_cast<uint8_t*>(ws + pl.hs);
      p.A = hq; p.lda = I;
      p.a_scales = hs; p.a_scale_ld = I / 32;
      p.tile_prefix = tiles;
      MOE_ZC_TRY(launch_fp8_gemm(p, kStoreBF16, s.ffn_tile_rows, s.smax, stream));
    } else if (packed)
      MOE_ZC_TRY(launch_packed_gemm(p, kStoreBF16, down_rows, s.smax, stream));
    else if (bf)
      MOE_ZC_TRY(launch_mfma_gemm(p, kStoreBF16, s.ffn_tile_rows, s.smax, stream));
    else
      MOE_ZC_TRY(launch_simt_gemm(p, kStoreF32, s.smax, stream));
  }
  // stage 7: combine with the identity experts and the residual
  MOE_ZC_TRY(mark(7));
  if (bf)
    MOE_ZC_TRY(launch_combine<bf16_t>(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(o),
                                      static_cast<const bf16_t*>(residual), idx, gate, pos,
                                      static_cast<bf16_t*>(y), T, (int)d, K, N, stream));
  else
    MOE_ZC_TRY(launch_combine<float>(static_cast<const float*>(x), static_cast<const float*>(o),
                                     static_cast<const float*>(residual), idx, gate, pos,
                                     static_cast<float*>(y), T, (int)d, K, N, stream));
  MOE_ZC_TRY(mark(8));
  return MOE_ZC_OK;
}

// ---- backward -------------------------------------------------------------------
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct BwdPlan {
  int64_t Sp, T64, E64;  // padded grouped columns, padded tokens, padded experts
  size_t tiles, kofs, kofs_r, xg, colrow, row_gate, row_dg, A, U, Q, dau, H, dxg, XT, ET, DAT, DUT,
      HT, dl, dlT, xT, wrT, wrP, dx_r, total;
};

BwdPlan make_bwd_plan(const Shape& s) {
  BwdPlan p{};
  p.Sp = round_up(s.smax + 64 * (int64_t)s.N, 64);
  p.T64 = round_up(s.T, 64);
  p.E64 = round_up(s.E, 64);
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += align_up(bytes);
    return here;
  };
  const size_t S = (size_t)std::max<int64_t>(s.smax, 1), I = (size_t)s.I, d = (size_t)s.d;
  p.tiles = take((size_t)(s.N + 1) * 4);
  p.kofs = take((size_t)(s.N + 1) * 4);
  p.kofs_r = take(2 * 4);
  p.xg = take((size_t)8 * wgrad_xcd_cap(s.N) * 4);
  p.colrow = take((size_t)p.Sp * 4);
  p.row_gate = take(S * 4);
  p.row_dg = take(S * 4);
  p.A = take(S * I * 4);
  p.U = take(S * I * 4);
  p.Q = take(S * I * 4);
  p.dau = take(S * 2 * I * 2);
  p.H = take(S * I * 2);
  p.dxg = take(S * d * 4);
  p.XT = take(d * (size_t)p.Sp * 2);
  p.ET = take(d * (size_t)p.Sp * 2);
  p.DAT = take(I * (size_t)p.Sp * 2);
  p.DUT = take(I * (size_t)p.Sp * 2);
  p.HT = take(I * (size_t)p.Sp * 2);
  p.dl = take((size_t)s.T * p.E64 * 2);
  p.dlT = take((size_t)s.E * p.T64 * 2);
  p.xT = take(d * (size_t)p.T64 * 2);
  p.wrT = take(d * (size_t)p.E64 * 2);
  p.wrP = take((size_t)packed_bytes(s.d, p.E64, false));
  p.dx_r = take((size_t)s.T * d * 4);
  p.total = at;
  return p;
}

// Conditions of the backward beyond the forward's: bf16, grouped rows of x and
// dy gathered with 32-bit byte offsets, padded group columns below 2^31.
moe_zc_status check_bwd_shape(int64_t T, int64_t d, int64_t I, int32_t N, int32_t Z, int32_t K,
                              Shape* s) {
  const moe_zc_status st = check_shape(T, d, I, N, Z, K, MOE_ZC_BF16, s);
  if (st != MOE_ZC_OK) return st;
  if (!s->gather) return MOE_ZC_ERR_UNSUPPORTED;
  if (round_up(s->smax + 64 * (int64_t)N, 64) >= (int64_t(1) << 31)) return MOE_ZC_ERR_UNSUPPORTED;
  return MOE_ZC_OK;
}

TrArgsHost tr(const void* src, int64_t src_ld, void* dst, int64_t dst_ld, int dim, int64_t ncols,
              int64_t ncols_valid, bool src_f32 = false, bool dst_f32 = false) {
  TrArgsHost a{};
  a.src = src; a.src_ld = src_ld; a.dst = dst; a.dst_ld = dst_ld; a.dim = dim; a.ncols = ncols;
  a.ncols_valid = ncols_valid; a.batch = 1; a.src_f32 = src_f32; a.dst_f32 = dst_f32;
  return a;
}

// Shape checks of the packing entry points (bf16 only; the forward's limits).
moe_zc_status check_pack_shape(int64_t d, int64_t I, moe_zc_dtype dt) {
  if (dt != MOE_ZC_F32 && dt != MOE_ZC_BF16) return MOE_ZC_ERR_INVALID;
  if (d <= 0 || I <= 0) return MOE_ZC_ERR_INVALID;
  if (dt != MOE_ZC_BF16) return MOE_ZC_ERR_UNSUPPORTED;
  Shape s;
  return check_shape(0, d, I, 1, 0, 1, dt, &s);
}

}  // namespace

// ---- the forward without allocation -----------------------------------------
// Scratch of moe_zc_forward_packed_noalloc: one fixed array per GPU, alive
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host it is only a stand-in for the device symbol); it uses
// the device address that hipGetSymbolAddress returns for the current device,
// looked up once per device and kept in g_scratch.
static __device__ __align__(256) char scratch[MOE_ZC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call there).
moe_zc_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ZC_ERR_HIP;
  if (dev >= kMaxDevices) return MOE_ZC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return MOE_ZC_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MOE_ZC_OK;
}
}  // namespace

extern "C" {

int32_t moe_zc_abi_version(void) { return MOE_ZC_ABI_VERSION; }

const char* moe_zc_status_string(moe_zc_status s) {
  switch (s) {
    case MOE_ZC_OK: return "ok";
    case MOE_ZC_ERR_INVALID: return "invalid argument";
    case MOE_ZC_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ZC_ERR_UNSUPPORTED: return "sizes outside what the kernels support";
    case MOE_ZC_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

size_t moe_zc_workspace_size(int64_t T, int64_t d, int64_t I, int32_t N, int32_t Z, int32_t K,
                             moe_zc_dtype dt) {
  Shape s;
  if (check_shape(T, d, I, N, Z, K, dt, &s) != MOE_ZC_OK) return 0;
  return make_plan(s).total;
}

moe_zc_status moe_zc_forward(const void* x, const float* w_router, const float* bias,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* residual, void* y, int64_t T, int64_t d, int64_t I,
                             int32_t N, int32_t Z, int32_t K, moe_zc_dtype dt, moe_zc_aux* aux,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(x, w_router, bias, w_gate, w_up, w_down, kRowMajor, residual, y, T, d, I,
                      N, Z, K, dt, aux, workspace, workspace_bytes, stream);
}

moe_zc_status moe_zc_forward_packed_noalloc(const void* x, const float* w_router,
                                            const float* bias, const void* gate_up_packed,
                                            const void* down_packed, const void* residual,
                                            void* y, int64_t T, int64_t d, int64_t I, int32_t N,
                                            int32_t Z, int32_t K, moe_zc_dtype dt,
                                            moe_zc_aux* aux, hipStream_t stream) {
  Shape s;
  const moe_zc_status st = check_shape(T, d, I, N, Z, K, dt, &s);
  if (st != MOE_ZC_OK) return st;
  if (dt != MOE_ZC_BF16) return MOE_ZC_ERR_UNSUPPORTED;
  const size_t need = make_plan(s).total;
  if (need > (size_t)MOE_ZC_NOALLOC_SCRATCH_BYTES) return MOE_ZC_ERR_WORKSPACE;
  if (T == 0) return MOE_ZC_OK;
  // the stream must belong to the current device: that device's scratch is used
  if (stream) {
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
      return MOE_ZC_ERR_HIP;
    if (sdev != cur) return MOE_ZC_ERR_INVALID;
  }
  void* ws = nullptr;
  const moe_zc_status ss = noalloc_scratch(&ws);
  if (ss != MOE_ZC_OK) return ss;
  return forward_impl(x, w_router, bias, gate_up_packed, nullptr, down_packed, kPacked, residual,
                      y, T, d, I, N, Z, K, dt, aux, ws, (size_t)MOE_ZC_NOALLOC_SCRATCH_BYTES,
                      stream);
}

moe_zc_status moe_zc_forward_packed(const void* x, const float* w_router, const float* bias,
                                    const void* gate_up_packed, const void* down_packed,
                                    const void* residual, void* y, int64_t T, int64_t d,
                                    int64_t I, int32_t N, int32_t Z, int32_t K, moe_zc_dtype dt,
                                    moe_zc_aux* aux, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return forward_impl(x, w_router, bias, gate_up_packed, nullptr, down_packed, kPacked, residual,
                      y, T, d, I, N, Z, K, dt, aux, workspace, workspace_bytes, stream);
}

size_t moe_zc_workspace_size_fp8(int64_t T, int64_t d, int64_t I, int32_t N, int32_t Z,
                                 int32_t K) {
  Shape s;
  if (check_shape(T, d, I, N, Z, K, MOE_ZC_BF16, &s) != MOE_ZC_OK) return 0;
  if (check_fp8_shape(s) != MOE_ZC_OK) return 0;
  return make_plan(s, true).total;
}

moe_zc_status moe_zc_forward_packed_fp8(const void* x, const float* w_router, const float* bias,
                                        const void* gate_up_fp8, const void* down,
                                        int32_t down_fp8, const void* residual, void* y,
                                        int64_t T, int64_t d, int64_t I, int32_t N, int32_t Z,
                                        int32_t K, moe_zc_aux* aux, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (down_fp8 != 0 && down_fp8 != 1) return MOE_ZC_ERR_INVALID;
  return forward_impl(x, w_router, bias, gate_up_fp8, nullptr, down, kPackedFp8, residual, y, T,
                      d, I, N, Z, K, MOE_ZC_BF16, aux, workspace, workspace_bytes, stream,
                      down_fp8 == 1);
}

moe_zc_status moe_zc_packed_fp8_expert_bytes(int64_t d, int64_t I, size_t* gate_up_bytes,
                                             size_t* down_bytes) {
  if (!gate_up_bytes) return MOE_ZC_ERR_INVALID;
  const moe_zc_status st = check_pack_shape(d, I, MOE_ZC_BF16);
  if (st != MOE_ZC_OK) return st;
  if (d % 128 != 0) return MOE_ZC_ERR_UNSUPPORTED;
  *gate_up_bytes = (size_t)fp8_packed_bytes(I, d);
  if (down_bytes) *down_bytes = (size_t)fp8_packed_down_bytes(d, I);
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_pack_expert_weights_fp8(const void* w_gate, const void* w_up,
                                             const void* w_down, int32_t n_experts, int64_t d,
                                             int64_t I, void* gate_up_fp8, void* down_fp8,
                                             hipStream_t stream) {
  const moe_zc_status st = check_pack_shape(d, I, MOE_ZC_BF16);
  if (st != MOE_ZC_OK) return st;
  if (d % 128 != 0) return MOE_ZC_ERR_UNSUPPORTED;
  if (n_experts < 0) return MOE_ZC_ERR_INVALID;
  if (!w_down != !down_fp8) return MOE_ZC_ERR_INVALID;  // both or neither
  if (n_experts == 0) return MOE_ZC_OK;
  if (!w_gate || !w_up || !gate_up_fp8) return MOE_ZC_ERR_INVALID;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(gate_up_fp8)) return MOE_ZC_ERR_INVALID;
  if (w_down && (!aligned16(w_down) || !aligned16(down_fp8))) return MOE_ZC_ERR_INVALID;
  MOE_ZC_TRY(launch_pack_weights_fp8(static_cast<const bf16_t*>(w_gate),
                                     static_cast<const bf16_t*>(w_up),
                                     static_cast<uint8_t*>(gate_up_fp8), n_experts, (int)I,
                                     (int)d, stream));
  if (w_down)
    MOE_ZC_TRY(launch_pack_down_fp8(static_cast<const bf16_t*>(w_down),
                                    static_cast<uint8_t*>(down_fp8), n_experts, (int)d, (int)I,
                                    stream));
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_quantize_mx(const void* x, int64_t rows, int64_t d, void* codes,
                                 void* scales, hipStream_t stream) {
  if (rows < 0 || d <= 0) return MOE_ZC_ERR_INVALID;
  if (d % 32 != 0 || rows * d >= (int64_t(1) << 40)) return MOE_ZC_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_ZC_OK;
  if (!x || !codes || !scales) return MOE_ZC_ERR_INVALID;
  if (!aligned16(x) || !aligned16(codes)) return MOE_ZC_ERR_INVALID;
  MOE_ZC_TRY(launch_quantize_mx(static_cast<const bf16_t*>(x), static_cast<uint8_t*>(codes),
                                static_cast<uint8_t*>(scales), rows, d, stream));
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_packed_expert_bytes(int64_t d, int64_t I, moe_zc_dtype dt,
                                         size_t* gate_up_bytes, size_t* down_bytes) {
  if (!gate_up_bytes || !down_bytes) return MOE_ZC_ERR_INVALID;
  const moe_zc_status st = check_pack_shape(d, I, dt);
  if (st != MOE_ZC_OK) return st;
  *gate_up_bytes = (size_t)packed_bytes(I, d, true);
  *down_bytes = (size_t)packed_bytes(d, I, false);
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_pack_expert_weights(const void* w_gate, const void* w_up,
                                         const void* w_down, int32_t n_experts, int64_t d,
                                         int64_t I, moe_zc_dtype dt, void* gate_up_packed,
                                         void* down_packed, hipStream_t stream) {
  const moe_zc_status st = check_pack_shape(d, I, dt);
  if (st != MOE_ZC_OK) return st;
  if (n_experts < 0) return MOE_ZC_ERR_INVALID;
  if (n_experts == 0) return MOE_ZC_OK;
  if (!w_gate || !w_up || !w_down || !gate_up_packed || !down_packed) return MOE_ZC_ERR_INVALID;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(gate_up_packed) ||
      !aligned16(down_packed))
    return MOE_ZC_ERR_INVALID;
  MOE_ZC_TRY(launch_pack_weights(static_cast<const bf16_t*>(w_gate),
                                 static_cast<const bf16_t*>(w_up),
                                 static_cast<bf16_t*>(gate_up_packed), n_experts, (int)I, (int)d,
                                 true, stream));
  MOE_ZC_TRY(launch_pack_weights(static_cast<const bf16_t*>(w_down), nullptr,
                                 static_cast<bf16_t*>(down_packed), n_experts, (int)d, (int)I,
                                 false, stream));
  return MOE_ZC_OK;
}

size_t moe_zc_backward_workspace_size(int64_t T, int64_t d, int64_t I, int32_t N, int32_t Z,
                                      int32_t K) {
  Shape s;
  if (check_bwd_shape(T, d, I, N, Z, K, &s) != MOE_ZC_OK) return 0;
  return make_bwd_plan(s).total;
}

moe_zc_status moe_zc_transpose_expert_weights(const void* w_gate, const void* w_up,
                                              const void* w_down, int32_t n_experts, int64_t d,
                                              int64_t I, void* w_gate_up_t, void* w_down_t,
                                              hipStream_t stream) {
  const moe_zc_status st = check_pack_shape(d, I, MOE_ZC_BF16);
  if (st != MOE_ZC_OK) return st;
  if (n_experts < 0) return MOE_ZC_ERR_INVALID;
  if (n_experts == 0) return MOE_ZC_OK;
  if (!w_gate || !w_up || !w_down || !w_gate_up_t || !w_down_t) return MOE_ZC_ERR_INVALID;
  if (!aligned16(w_gate_up_t) || !aligned16(w_down_t)) return MOE_ZC_ERR_INVALID;
  const bf16_t* wg = static_cast<const bf16_t*>(w_gate);
  const bf16_t* wu = static_cast<const bf16_t*>(w_up);
  const bf16_t* wd = static_cast<const bf16_t*>(w_down);
  // [W_gate; W_up]^T as rows j < d over k < 2I; W_down^T as rows i < I over k < d
  MOE_ZC_TRY(launch_pack_transposed(wg, wu, static_cast<bf16_t*>(w_gate_up_t), n_experts, (int)d,
                                    (int)(2 * I), (int)I, (int)d, I * d, stream));
  MOE_ZC_TRY(launch_pack_transposed(wd, wd, static_cast<bf16_t*>(w_down_t), n_experts, (int)I,
                                    (int)d, (int)d, (int)I, d * I, stream));
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_transposed_expert_bytes(int64_t d, int64_t I, size_t* gate_up_t_bytes,
                                             size_t* down_t_bytes) {
  if (!gate_up_t_bytes || !down_t_bytes) return MOE_ZC_ERR_INVALID;
  const moe_zc_status st = check_pack_shape(d, I, MOE_ZC_BF16);
  if (st != MOE_ZC_OK) return st;
  *gate_up_t_bytes = (size_t)packed_bytes(d, 2 * I, false);
  *down_t_bytes = (size_t)packed_bytes(I, d, false);
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_backward(const void* x, const float* w_router, const void* w_gate,
                              const void* w_up, const void* w_gate_up_t, const void* w_down_t,
                              const moe_zc_aux* fwd, const void* dy, void* dx, float* dw_router,
                              float* dw_gate, float* dw_up, float* dw_down, int64_t T, int64_t d,
                              int64_t I, int32_t N, int32_t Z, int32_t K, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  const moe_zc_status st = check_bwd_shape(T, d, I, N, Z, K, &s);
  if (st != MOE_ZC_OK) return st;
  if (T == 0) return MOE_ZC_OK;
  if (!x || !w_router || !dy || !dx || !dw_router || !fwd) return MOE_ZC_ERR_INVALID;
  if (!fwd->logits || !fwd->topk_idx || !fwd->topk_gate || !fwd->pos || !fwd->perm ||
      !fwd->offsets)
    return MOE_ZC_ERR_INVALID;
  // a and u: from the forward's saved pre-activations, else recomputed
  const void* act = fwd->act;
  if (N > 0 && (!w_gate_up_t || !w_down_t || !dw_gate || !dw_up || !dw_down))
    return MOE_ZC_ERR_INVALID;
  if (N > 0 && !act && (!w_gate || !w_up)) return MOE_ZC_ERR_INVALID;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(w_router) ||
      !aligned16(dw_router) ||
      (N > 0 && (!aligned16(dw_gate) || !aligned16(dw_up) || !aligned16(dw_down))) ||
      (N > 0 && (!aligned16(w_gate_up_t) || !aligned16(w_down_t))) ||
      (N > 0 && (act ? !aligned16(act) : (!aligned16(w_gate) || !aligned16(w_up)))))
    return MOE_ZC_ERR_INVALID;
  const BwdPlan pl = make_bwd_plan(s);
  if (!workspace || workspace_bytes < pl.total) return MOE_ZC_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_ZC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  auto F = [&](size_t o) { return reinterpret_cast<float*>(ws + o); };
  auto B = [&](size_t o) { return reinterpret_cast<bf16_t*>(ws + o); };
  auto Ix = [&](size_t o) { return reinterpret_cast<int32_t*>(ws + o); };
  const int E = s.E;
  const int32_t* offsets = fwd->offsets;
  const int32_t* perm = fwd->perm;
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* dyb = static_cast<const bf16_t*>(dy);
  float* dxg = F(pl.dxg);
  float* row_dg = F(pl.row_dg);

  if (N > 0) {
    int32_t* tiles = Ix(pl.tiles);
    int32_t* kofs = Ix(pl.kofs);
    int32_t* colrow = Ix(pl.colrow);
    float* row_gate = F(pl.row_gate);
    MOE_ZC_TRY(launch_bwd_prefix(offsets, N, s.ffn_tile_rows, tiles, kofs, stream));
    int32_t* xg = Ix(pl.xg);
    MOE_ZC_TRY(launch_wgrad_plan(kofs, N, xg, stream));
    MOE_ZC_TRY(launch_bwd_colrow(offsets, kofs, N, colrow, (int)pl.Sp, stream));
    MOE_ZC_TRY(launch_bwd_rowgate(fwd->pos, fwd->topk_gate, T * K, row_gate, stream));
    // a = W_gate x and u = W_up x of every grouped row (fp32; unless the
    // forward saved them), q = W_down^T dy
    GemmProblem p{};
    p.A = x; p.lda = d; p.a_kwrap = (int)d; p.K = (int)d; p.a_rows = perm;
    p.ldb = d; p.b_group_stride = I * d;
    p.ldc = I; p.Nout = (int)I;
    p.row_offsets = offsets; p.tile_prefix = tiles; p.G = N; p.M = 0;
    if (!act) {
      p.B0 = w_gate; p.C = F(pl.A);
      MOE_ZC_TRY(launch_mfma_gemm(p, kStoreF32, s.ffn_tile_rows, s.smax, stream));
      p.B0 = w_up; p.C = F(pl.U);
      MOE_ZC_TRY(launch_mfma_gemm(p, kStoreF32, s.ffn_tile_rows, s.smax, stream));
    }
    // q on the packed kernel: B = the packed W_down^T (rows i < I over k < d)
    p.A = dy; p.B0 = w_down_t; p.C = F(pl.Q); p.ldb = 0; p.b_group_stride = 0;
    MOE_ZC_TRY(launch_packed_gemm(p, kStoreF32, s.ffn_tile_rows, s.smax, stream));
    // SwiGLU backward: da | du, h, and the gate gradient of every grouped row
    if (act)
      MOE_ZC_TRY(launch_swiglu_bwd(act, static_cast<const bf16_t*>(act) + I, 2 * I, true,
                                   F(pl.Q), row_gate, offsets, N, (int)I, s.smax, B(pl.dau),
                                   B(pl.H), row_dg, stream));
    else
      MOE_ZC_TRY(launch_swiglu_bwd(F(pl.A), F(pl.U), I, false, F(pl.Q), row_gate, offsets, N,
                                   (int)I, s.smax, B(pl.dau), B(pl.H), row_dg, stream));
    // rows of dx from the experts: [da | du] [W_gate ; W_up]
    // (packed [W_gate; W_up]^T: rows j < d over k < 2I)
    GemmProblem q{};
    q.A = B(pl.dau); q.lda = 2 * I; q.a_kwrap = (int)(2 * I); q.K = (int)(2 * I);
    q.B0 = w_gate_up_t;
    q.C = dxg; q.ldc = d; q.Nout = (int)d;
    q.row_offsets = offsets; q.tile_prefix = tiles; q.G = N; q.M = 0;
    MOE_ZC_TRY(launch_packed_gemm(q, kStoreF32, s.ffn_tile_rows, s.smax, stream));
    // weight gradients: operands transposed into expert blocks of rows_e
    // rounded up to 32 columns (zeros in the padding columns), stored as slabs
    // of 32 columns
    auto blocked = [&](const void* src, int64_t src_ld, void* dst, int64_t dim) {
      TrArgsHost a = tr(src, src_ld, dst, 0, (int)dim, pl.Sp, 0);
      a.colrow = colrow;
      a.kofs = kofs;
      a.ngroups = N;
      return a;
    };
    TrArgsHost a = blocked(x, d, B(pl.XT), d);
    a.rowidx = perm;
    MOE_ZC_TRY(launch_transpose(a, stream));
    a = blocked(dy, d, B(pl.ET), d);
    a.rowidx = perm; a.rowscale = row_gate;
    MOE_ZC_TRY(launch_transpose(a, stream));
    a = blocked(B(pl.dau), 2 * I, B(pl.DAT), I);
    MOE_ZC_TRY(launch_transpose(a, stream));
    a.dst = B(pl.DUT); a.src_col0 = I;
    MOE_ZC_TRY(launch_transpose(a, stream));
    a = blocked(B(pl.H), I, B(pl.HT), I);
    MOE_ZC_TRY(launch_transpose(a, stream));
    MOE_ZC_TRY(launch_wgrad(B(pl.ET), B(pl.HT), kofs, N, (int)d, (int)I, dw_down, xg, stream));
    MOE_ZC_TRY(launch_wgrad(B(pl.DAT), B(pl.XT), kofs, N, (int)I, (int)d, dw_gate, xg, stream));
    MOE_ZC_TRY(launch_wgrad(B(pl.DUT), B(pl.XT), kofs, N, (int)I, (int)d, dw_up, xg, stream));
  }
  // per token: gate gradients, router softmax backward, dx from expert rows and
  // identity slots
  bf16_t* dl = B(pl.dl);
  MOE_ZC_TRY(launch_token_route_bwd(xb, dyb, fwd->logits, fwd->topk_idx, fwd->pos, row_dg, T,
                                    (int)d, E, K, N, dl, (int)pl.E64, stream));
  // router: dx += dl W_r on the packed kernel (bf16 dl and W_r, fp32
  // accumulation; W_r^T [d][E rounded up to 64] packed on every call),
  // dW_r = dl^T x
  TrArgsHost a = tr(w_router, d, B(pl.wrT), pl.E64, (int)d, pl.E64, E, true, false);
  MOE_ZC_TRY(launch_transpose(a, stream));
  MOE_ZC_TRY(launch_pack_weights(B(pl.wrT), nullptr, B(pl.wrP), 1, (int)d, (int)pl.E64, false,
                                 stream));
  GemmProblem r{};
  r.A = dl; r.lda = pl.E64; r.a_kwrap = (int)pl.E64; r.K = (int)pl.E64;
  r.B0 = B(pl.wrP);
  r.C = F(pl.dx_r); r.ldc = d; r.Nout = (int)d; r.G = 1; r.M = (int)T;
  MOE_ZC_TRY(launch_packed_gemm(r, kStoreF32, router_tile_rows(T, (int)d), T, stream));
  // dx: the slots' expert rows and identity terms in slot order, then the router term
  MOE_ZC_TRY(launch_dx_sum(dyb, fwd->topk_idx, fwd->topk_gate, fwd->pos, dxg, F(pl.dx_r), T,
                           (int)d, K, N, static_cast<bf16_t*>(dx), stream));
  // dl^T and x^T as one group of T rows (rounded up to 64), in the
  // weight-gradient kernel's k-blocked layout
  int32_t* kofs_r = Ix(pl.kofs_r);
  MOE_ZC_TRY(launch_set_range(kofs_r, 0, (int)pl.T64, stream));
  a = tr(dl, pl.E64, B(pl.dlT), pl.T64, E, pl.T64, T);
  a.kofs = kofs_r; a.ngroups = 1;
  MOE_ZC_TRY(launch_transpose(a, stream));
  a = tr(x, d, B(pl.xT), pl.T64, (int)d, pl.T64, T);
  a.kofs = kofs_r; a.ngroups = 1;
  MOE_ZC_TRY(launch_transpose(a, stream));
  MOE_ZC_TRY(launch_wgrad(B(pl.dlT), B(pl.xT), kofs_r, 1, E, (int)d, dw_router, nullptr, stream));
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_route(const float* logits, const float* bias, int64_t T, int32_t E,
                           int32_t K, int32_t* topk_idx, float* topk_gate, int32_t* loads,
                           hipStream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E) return MOE_ZC_ERR_INVALID;
  if (E > MOE_ZC_MAX_EXPERTS || K > MOE_ZC_MAX_TOPK) return MOE_ZC_ERR_UNSUPPORTED;
  if (T * K >= (int64_t(1) << 31) || T >= (int64_t(1) << 33)) return MOE_ZC_ERR_UNSUPPORTED;
  if (T == 0) {  // no slots: every load is zero
    if (loads) MOE_ZC_TRY(launch_count_loads(nullptr, 0, K, E, loads, stream));
    return MOE_ZC_OK;
  }
  if (!logits || !bias || !topk_idx || !topk_gate) return MOE_ZC_ERR_INVALID;
  MOE_ZC_TRY(launch_topk(logits, bias, T, E, K, topk_idx, topk_gate, stream));
  if (loads) MOE_ZC_TRY(launch_count_loads(topk_idx, T, K, E, loads, stream));
  return MOE_ZC_OK;
}

moe_zc_status moe_zc_bias_update(const int32_t* loads, const float* target, float* bias,
                                 const moe_zc_pid* pid, int32_t E, hipStream_t stream) {
  if (!loads || !target || !bias || !pid || !pid->e_prev || !pid->e_prev2)
    return MOE_ZC_ERR_INVALID;
  if (E < 1) return MOE_ZC_ERR_INVALID;
  if (E > MOE_ZC_MAX_EXPERTS) return MOE_ZC_ERR_UNSUPPORTED;
  MOE_ZC_TRY(launch_pid(loads, target, bias, pid->e_prev, pid->e_prev2, E, pid->kp, pid->ki,
                        pid->kd, stream));
  return MOE_ZC_OK;
}

}  // extern "C"
