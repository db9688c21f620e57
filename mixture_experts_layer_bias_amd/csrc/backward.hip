// Backward of the MoE layer with zero-computation experts (bf16 data, fp32
// arithmetic, fixed reduction orders: two runs give identical bits).
//
// With routing fixed by the forward (top-K and gates), upstream gradient dy
// and, for a slot (t, k) on FFN expert e, a = W_gate x, u = W_up x,
// s = sigmoid(a), h = a s u, g the gate:
//   q    = W_down^T dy_t            (so dh = g q and the gate's gradient is <q, h>)
//   da   = g q u s (1 + a (1 - s)),  du = g q a s
//   dx_t += W_gate^T da + W_up^T du
//   dW_down += (g dy_t) h^T,  dW_gate += da x_t^T,  dW_up += du x_t^T
// for a slot on an identity expert: gate gradient <dy_t, x_t>, dx_t += g dy_t;
// router: dl_t = p_t * (dp_t - <p_t, dp_t>) with dp_t the gate gradients at the
// chosen experts, dx_t += W_r^T dl_t, dW_r += dl_t x_t^T.
//
// Kernels here: bookkeeping (tile prefix, 64-padded group columns, column ->
// row map, slot of each grouped row), a tiled transpose that gathers, scales
// and zero-pads rows into expert-blocked [dim][rows] operands, the per-row
// SwiGLU backward, the per-token router-softmax backward, the sum of each
// token's dx contributions, and the weight-gradient GEMM: groups (experts)
// with their own reduction range over the padded rows, both operands
// K-contiguous, fp32 output.  The other products (q, the rows of dx, the
// router's dx term, and a and u when the forward did not save them) run on
// the bf16 MFMA grouped GEMMs.
#include "backward.hpp"
#include "gemm_tile.hpp"

namespace moezc {

namespace {

// ---- bookkeeping --------------------------------------------------------------
// tile_prefix[g] = sum over f < g of ceil(rows_f / bm); kofs[g] = sum over f < g
// of rows_f rounded up to 32 (each group's reduction range in the padded
// operands).  One wave: lane l sums a contiguous segment of ceil(N / 64)
// groups, a shuffle scan over the 64 lane sums gives each segment its start,
// then every lane writes its own segment.
__global__ __launch_bounds__(64) void bwd_prefix_kernel(const int32_t* __restrict__ offsets,
                                                        int N, int bm,
                                                        int32_t* __restrict__ tile_prefix,
                                                        int32_t* __restrict__ kofs) {
  const int lane = threadIdx.x;
  const int seg = (N + 63) / 64;
  const int e0 = min(N, lane * seg);
  const int e1 = min(N, e0 + seg);
  int st = 0, sk = 0;
  for (int e = e0; e < e1; ++e) {
    const int rows = offsets[e + 1] - offsets[e];
    st += (rows + bm - 1) / bm;
    sk += (rows + 31) / 32 * 32;
  }
  int it = st, ik = sk;  // inclusive scan over lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(it, off), b = __shfl_up(ik, off);
    if (lane >= off) {
      it += a;
      ik += b;
    }
  }
  int t = it - st, k = ik - sk;
  for (int e = e0; e < e1; ++e) {
    tile_prefix[e] = t;
    kofs[e] = k;
    const int rows = offsets[e + 1] - offsets[e];
    t += (rows + bm - 1) / bm;
    k += (rows + 31) / 32 * 32;
  }
  if (lane == 63) {
    tile_prefix[N] = it;
    kofs[N] = ik;
  }
}

// colrow[c] = grouped row s held by padded column c, or -1 for padding and
// for c >= kofs[N]
__global__ __launch_bounds__(256) void bwd_colrow_kernel(const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ kofs, int N,
                                                         int32_t* __restrict__ colrow, int ncols) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ncols) return;
  int r = -1;
  if (N > 0 && c < kofs[N]) {
    int lo = 0, hi = N;  // kofs[lo] <= c < kofs[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (kofs[mid] <= c) lo = mid; else hi = mid;
    }
    const int s = offsets[lo] + (c - kofs[lo]);
    r = s < offsets[lo + 1] ? s : -1;
  }
  colrow[c] = r;
}

// the gate of each grouped row (slot (t, k) with pos[t, k] = s)
__global__ __launch_bounds__(256) void bwd_rowgate_kernel(const int32_t* __restrict__ pos,
                                                          const float* __restrict__ gate,
                                                          int64_t slots,
                                                          float* __restrict__ row_gate) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= slots) return;
  const int s = pos[i];
  if (s >= 0) row_gate[s] = gate[i];
}

// ---- transpose ----------------------------------------------------------------
// dst[j][dst_col0 + c] = scale(s) * src[row(s)][src_col0 + j] for the 64 x 64
// tile of (c, j); s = colrow ? colrow[c] : (c < ncols_valid ? c : -1), row(s) =
// rowidx ? rowidx[s] : s, scale = rowscale ? rowscale[s] : 1; columns with s < 0
// get zeros.  Batched over blockIdx.z with the given strides.
struct TrArgs {
  const void* src;
  int64_t src_ld, src_col0, src_bstride;
  const int32_t* rowidx;
  const float* rowscale;
  const int32_t* colrow;
  int64_t ncols_valid;
  void* dst;
  int64_t dst_ld, dst_col0, dst_bstride;
  int dim;        // destination rows (source columns)
  int64_t ncols;  // destination columns (multiple of 64)
  // non-null: expert-blocked, k-blocked destination.  Group g owns columns
  // [kofs[g], kofs[g+1]) (multiples of 32), stored from element offset
  // kofs[g] * dim as slabs of 32 columns: column k of the group, row j at
  // (k / 32) * dim * 32 + j * 32 + k % 32.  One slab holds every row's 32
  // consecutive columns (64 bytes for bf16) back to back, so a weight-gradient
  // stage reads one contiguous block.  Columns at or past kofs[ngroups] are
  // not written.
  const int32_t* kofs;
  int ngroups;
};

__device__ __forceinline__ float ld_elem(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void st_elem(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void st_elem(float* p, int64_t i, float v) { p[i] = v; }

// 16 consecutive elements through 16-byte accesses (the address is 16-byte
// aligned: every row stride and column offset is a multiple of 8 elements)
__device__ __forceinline__ void ld16(const bf16_t* p, float (&v)[16]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 u = reinterpret_cast<const uint4*>(p)[h];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[8 * h + 2 * q] = __uint_as_float(w[q] << 16);
      v[8 * h + 2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  }
}
__device__ __forceinline__ void ld16(const float* p, float (&v)[16]) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float4 f = reinterpret_cast<const float4*>(p)[h];
    v[4 * h] = f.x; v[4 * h + 1] = f.y; v[4 * h + 2] = f.z; v[4 * h + 3] = f.w;
  }
}
__device__ __forceinline__ void st16(bf16_t* p, const float (&v)[16]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = f32x2_to_bf16x2(v[8 * h + 2 * q], v[8 * h + 2 * q + 1]);
    reinterpret_cast<uint4*>(p)[h] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}
__device__ __forceinline__ void st16(float* p, const float (&v)[16]) {
#pragma unroll
  for (int h = 0; h < 4; ++h)
    reinterpret_cast<float4*>(p)[h] = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
}

// 64 x 64 tiles: thread (row, 16-element chunk) reads a source row segment
// and writes a destination row segment with 16-byte accesses; the LDS tile
// (padded rows) turns one into the other.  Partial chunks at the edges
// (dim or ncols not a multiple of 16) go element by element.
template <typename SRC, typename DST>
__global__ __launch_bounds__(256) void transpose_kernel(TrArgs a) {
  __shared__ float tile[64][65];
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int j0 = blockIdx.y * 64;
  const SRC* src = static_cast<const SRC*>(a.src) + (int64_t)blockIdx.z * a.src_bstride;
  DST* dst = static_cast<DST*>(a.dst) + (int64_t)blockIdx.z * a.dst_bstride;
  const int64_t dst_ld = a.dst_ld;  // destination row stride
  const bool kslab = a.kofs != nullptr;
  // k-blocked destination: the tile's two 32-column halves may belong to
  // different groups (groups are 32-column aligned); for each half, the
  // group's block and the half's first column in it (-1: past the groups)
  DST* hdst[2] = {dst, dst};
  int64_t hk[2] = {c0, c0 + 32};
  if (kslab) {
    const int64_t kend = a.kofs[a.ngroups];
    if (c0 >= kend) return;
    int g = 0;  // the group of each half: kofs[g] <= column < kofs[g + 1]
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t ch = c0 + 32 * h;
      if (ch >= kend) {
        hk[h] = -1;
        continue;
      }
      // the second half searches only when a group ends inside the tile
      if (h == 0 || a.kofs[g + 1] <= ch) {
        int lo = g, hi = a.ngroups;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (a.kofs[mid] <= ch) lo = mid; else hi = mid;
        }
        g = lo;
      }
      hdst[h] = dst + (int64_t)a.kofs[g] * a.dim;
      hk[h] = ch - a.kofs[g];
    }
  }
  const int tid = threadIdx.x;
  {
    const int cl = tid >> 2, jc = (tid & 3) * 16;  // column c0 + cl, 16 source columns
    const int64_t c = c0 + cl;
    int64_t s = -1;
    if (c < a.ncols) s = a.colrow ? (int64_t)a.colrow[c] : (c < a.ncols_valid ? c : -1);
    float v[16];
    if (s < 0) {
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = 0.f;
    } else {
      const float sc = a.rowscale ? a.rowscale[s] : 1.f;
      const int64_t row = a.rowidx ? (int64_t)a.rowidx[s] : s;
      const SRC* p = src + row * a.src_ld + a.src_col0 + j0 + jc;
      if (j0 + jc + 16 <= a.dim) {
        ld16(p, v);
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = (j0 + jc + q < a.dim) ? ld_elem(p, q) : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] *= sc;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) tile[jc + q][cl] = v[q];
  }
  __syncthreads();
  {
    const int jl = tid >> 2, cc = (tid & 3) * 16;
    const int j = j0 + jl;
    if (j < a.dim) {
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = tile[jl][cc + q];
      // 16 columns from a multiple of 16: inside one 32-column slab
      const int h = cc >> 5;
      if (kslab && hk[h] < 0) return;  // this half is past the last group (so is the rest)
      const int64_t k = kslab ? hk[h] + (cc & 31) : c0 + cc;
      DST* p = kslab ? hdst[h] + (k >> 5) * ((int64_t)a.dim * 32) + (int64_t)j * 32 + (k & 31)
                     : dst + (int64_t)j * dst_ld + a.dst_col0 + k;
      if (c0 + cc + 16 <= a.ncols) {
        st16(p, v);
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (c0 + cc + q < a.ncols) st_elem(p, q, v[q]);
      }
    }
  }
}

// ---- per-row SwiGLU backward --------------------------------------------------
// Row s of expert rows: a, u (row stride ld_au: fp32 [S][I] recomputed, or
// the forward's bf16 pre-activations [S][2I]) and q [S][I] fp32 -> dau [S][2I]
// bf16 (da | du), h [S][I] bf16, row_dg[s] = <q, h> (the gate gradient of
// the row's slot).  One workgroup of 256 threads per row; the dot product
// reduces in a fixed tree.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T* __restrict__ A,
                                                         const T* __restrict__ U, int64_t ld_au,
                                                         const float* __restrict__ Q,
                                                         const float* __restrict__ row_gate,
                                                         const int32_t* __restrict__ offsets,
                                                         int N, int I, bf16_t* __restrict__ dau,
                                                         bf16_t* __restrict__ H,
                                                         float* __restrict__ row_dg) {
  __shared__ float red[256];
  const int64_t s = blockIdx.x;
  if (s >= offsets[N]) return;
  const float g = row_gate[s];
  float dot = 0.f;
  for (int i = threadIdx.x; i < I; i += 256) {
    const int64_t o = s * I + i;
    const float a = ld_elem(A, s * ld_au + i), u = ld_elem(U, s * ld_au + i), q = Q[o];
    const float sg = sigmoid_fast(a);
    const float h = a * sg * u;
    dot += q * h;
    const float dh = g * q;
    dau[s * 2 * I + i] = f32_to_bf16(dh * u * sg * (1.0f + a * (1.0f - sg)));
    dau[s * 2 * I + I + i] = f32_to_bf16(dh * a * sg);
    H[o] = f32_to_bf16(h);
  }
  red[threadIdx.x] = dot;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) row_dg[s] = red[0];
}

// ---- per-token backward ---------------------------------------------------------
// Sum over the 64 lanes of a wavefront, in a fixed butterfly order (every lane
// ends with the same value).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Token t, one wavefront per token: the gate gradients of its K slots (FFN:
// row_dg of the slot's grouped row; identity: <dy_t, x_t>) and the router's
// softmax backward dl_t = p_t * (dp_t - <p_t, dp_t>) (p = softmax of the fp32
// logits, dp_t = the gate gradients at the chosen experts) into dl [T][ldl]
// bf16, zeros past E.
__global__ __launch_bounds__(256) void token_route_bwd_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy, const float* __restrict__ logits,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ pos,
    const float* __restrict__ row_dg, int64_t T, int d, int E, int K, int N,
    bf16_t* __restrict__ dl, int ldl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int32_t* it = idx + t * K;
  const int32_t* pt = pos + t * K;
  // <dy_t, x_t>: lane l takes the 8-element pieces l, l + 64, ...
  float xy = 0.f;
  for (int j = lane * 8; j < d; j += 512) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + t * d + j);
    const uint4 yv = *reinterpret_cast<const uint4*>(dy + t * d + j);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xy += __uint_as_float(xw[q] << 16) * __uint_as_float(yw[q] << 16);
      xy += __uint_as_float(xw[q] & 0xffff0000u) * __uint_as_float(yw[q] & 0xffff0000u);
    }
  }
  xy = wave_sum(xy);
  // softmax statistics of the fp32 logits
  const float* lt = logits + t * E;
  float mx = -INFINITY;
  for (int i = lane; i < E; i += 64) mx = fmaxf(mx, lt[i]);
  mx = wave_max(mx);
  float se = 0.f;
  for (int i = lane; i < E; i += 64) se += __expf(lt[i] - mx);
  const float inv = 1.0f / wave_sum(se);
  // <p, dp>: only the chosen experts have dp != 0 (every lane the same)
  float c = 0.f;
  for (int k = 0; k < K; ++k) {
    const float dg = it[k] < N ? row_dg[pt[k]] : xy;
    c += __expf(lt[it[k]] - mx) * inv * dg;
  }
  for (int i = lane; i < ldl; i += 64) {  // padding columns E .. ldl - 1 get zeros
    float v = 0.f;
    if (i < E) {
      float dp = 0.f;
      for (int k = 0; k < K; ++k)
        if (it[k] == i) dp = it[k] < N ? row_dg[pt[k]] : xy;
      v = __expf(lt[i] - mx) * inv * (dp - c);
    }
    dl[t * ldl + i] = f32_to_bf16(v);
  }
}

// dx[t][j .. j+7] = bf16(sum over the slots of t, in slot order, of the
// expert row's dx (FFN slot) or g dy_t (identity slot), plus the router term
// dx_r[t]).  One thread per 8 elements: a pure stream over the rows.
__global__ __launch_bounds__(256) void dx_sum_kernel(const bf16_t* __restrict__ dy,
                                                     const int32_t* __restrict__ idx,
                                                     const float* __restrict__ gate,
                                                     const int32_t* __restrict__ pos,
                                                     const float* __restrict__ dxg,
                                                     const float* __restrict__ dx_r, int64_t T,
                                                     int d, int K, int N,
                                                     bf16_t* __restrict__ dx) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_t = d / 8;
  if (q >= T * per_t) return;
  const int64_t t = q / per_t;
  const int j = (int)(q - t * per_t) * 8;
  float yv[8], acc[8];
  {
    const uint4 u = *reinterpret_cast<const uint4*>(dy + t * d + j);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      yv[2 * e] = __uint_as_float(w[e] << 16);
      yv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int k = 0; k < K; ++k) {
    const int e_k = idx[t * K + k];
    if (e_k < N) {
      const float* r = dxg + (int64_t)pos[t * K + k] * d + j;
      const float4 a0 = *reinterpret_cast<const float4*>(r);
      const float4 a1 = *reinterpret_cast<const float4*>(r + 4);
      acc[0] += a0.x; acc[1] += a0.y; acc[2] += a0.z; acc[3] += a0.w;
      acc[4] += a1.x; acc[5] += a1.y; acc[6] += a1.z; acc[7] += a1.w;
    } else {
      const float g = gate[t * K + k];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += g * yv[e];
    }
  }
  const float* rr = dx_r + t * d + j;
  const float4 r0 = *reinterpret_cast<const float4*>(rr);
  const float4 r1 = *reinterpret_cast<const float4*>(rr + 4);
  const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = f32x2_to_bf16x2(acc[2 * e] + rv[2 * e], acc[2 * e + 1] + rv[2 * e + 1]);
  *reinterpret_cast<uint4*>(dx + t * d + j) = make_uint4(o[0], o[1], o[2], o[3]);
}

// out[0] = a, out[1] = b (a one-group reduction range)
__global__ void set_range_kernel(int32_t* out, int a, int b) {
  if (threadIdx.x == 0) {
    out[0] = a;
    out[1] = b;
  }
}

// ---- weight-gradient GEMM --------------------------------------------------------
// C[g][m][n] = sum over k < R_g of A_g[m][k] B_g[n][k], R_g = kofs[g+1] - kofs[g]
// (a multiple of 32); A_g and B_g bf16 start at element offsets kofs[g] * M
// and kofs[g] * N in the k-blocked layout of the transposes above (slabs of
// 32 k: A_g[m][k] at (k / 32) * M * 32 + m * 32 + k % 32); C fp32 [G][M][N].
// 128 x 128 tiles, four wavefronts (2 x 2, 64 x 64 each), stages of 32 k
// double-buffered in LDS by direct loads: a stage of a tile is 128 rows of
// 64 bytes, consecutive in its slab.
constexpr int WG_BKS = 32, WG_ROWB = 64;

struct WgradProblem {
  const bf16_t* A;
  const bf16_t* B;
  const int32_t* kofs;
  int G, M, N;
  float* C;
  // XCD x owns groups xcd_groups[x * cap + j], j < cap (-1: none); null: the
  // groups are spread over the XCDs tile by tile
  const int32_t* xcd_groups;
  int cap;
};

// The XCD plan.  A weight-gradient tile's time is about its group's
// reduction stages plus a fixed store phase (measured at prefill: nine 32-k
// stages of about 2.2 us against a 9.5 us epilogue, so the epilogue counts as
// kWgradEpiUnits stages).  Groups differ by their rows only, so with skewed
// loads (one expert holding a tenth of all rows) an XCD that owns whole
// groups by index gets far more work than the others.  The plan gives each
// XCD whole groups by longest processing time first: groups in order of
// descending work (ties: lower index), each to the XCD with the least work so
// far (ties: lower XCD) among those holding fewer than cap groups.
constexpr int kWgradEpiUnits = 4;

__global__ __launch_bounds__(1024) void wgrad_plan_kernel(const int32_t* __restrict__ kofs, int G,
                                                         int cap,
                                                         int32_t* __restrict__ xcd_groups) {
  __shared__ uint64_t key[kWgradMaxGroups];
  __shared__ int32_t tab[8 * kWgradMaxCap];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < G) P <<= 1;
  // key: work above, complemented index below, so that a descending sort puts
  // more work first and, on equal work, the lower index; padding (0) sorts last
  for (int i = tid; i < P; i += 1024) {
    uint64_t k = 0;
    if (i < G) {
      const uint32_t w = (uint32_t)((kofs[i + 1] - kofs[i]) / WG_BKS) + kWgradEpiUnits;
      k = ((uint64_t)w << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
    }
    key[i] = k;
  }
  for (int i = tid; i < 8 * cap; i += 1024) tab[i] = -1;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t a = key[i], b = key[j];
          const bool desc = (i & size) == 0;
          if (desc ? (a < b) : (a > b)) {
            key[i] = b;
            key[j] = a;
          }
        }
      }
      __syncthreads();
    }
  // greedy assignment by the first wavefront: lane x < 8 holds XCD x's key
  // (work << 3 | x, or all ones once it holds cap groups) and group count;
  // per group the least key, read lane by lane into scalar registers, names
  // the XCD that takes it (8 cap >= G, so one is always below cap).  The
  // sorted keys arrive 64 at a time, one per lane.
  if (tid < 64) {
    uint32_t kx = (uint32_t)tid;  // work 0
    int cnt = 0;
    for (int base = 0; base < G; base += 64) {
      const uint64_t kk = key[min(base + tid, P - 1)];
      const int klo = (int)(uint32_t)kk, khi = (int)(uint32_t)(kk >> 32);
      const int n = min(64, G - base);
      // the keys are in registers before the loop, so the loop itself never
      // waits on its table writes
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      for (int j = 0; j < n; ++j) {
        const uint32_t wk = (uint32_t)__builtin_amdgcn_readlane(khi, j);
        const int e = (int)(0xffffffffu - (uint32_t)__builtin_amdgcn_readlane(klo, j));
        uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)kx, 0);
#pragma unroll
        for (int x = 1; x < 8; ++x) m = min(m, (uint32_t)__builtin_amdgcn_readlane((int)kx, x));
        if (tid == (int)(m & 7u)) {
          tab[tid * cap + cnt] = e;
          ++cnt;
          kx = cnt == cap ? 0xffffffffu : kx + (wk << 3);
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < 8 * cap; i += 1024) xcd_groups[i] = tab[i];
}

// Tiles of 64 RB rows (of A) by 64 CB columns (of B): 128 x 128 (32 KB of
// LDS, five workgroups per CU) for few groups, 256 x 128 (48 KB, three per
// CU) for the experts' gradients, where the taller tile reads 25% fewer
// operand bytes per output.  Four wavefronts as 2 x 2, each RB x CB MFMA
// blocks of 32 x 32.
// Tile order.  With 8 or more groups, workgroup i (dispatched to XCD i % 8)
// takes a tile of a group that the XCD plan gave XCD i % 8: each XCD owns
// whole groups, so a group's operands are fetched into one L2 only, and the
// XCDs' shares of the work are balanced.  Within a group the faster
// index runs over the smaller operand's tiles (m_inner: over A's), which
// keeps the tiles in flight on an XCD to a few of the larger operand's.
// Several workgroups share a CU, so the loads of one hide behind the others.
template <int RB, int CB>
constexpr int wg_slot() { return 64 * (RB + CB) * WG_ROWB; }  // bytes of one stage

// (the body is a device function: the host pass of a kernel template
// instantiates its body, where the gfx950 buffer builtins do not exist)
template <int RB, int CB>
__device__ __forceinline__ void wgrad_tile(const WgradProblem& p, int mtiles, int ntiles,
                                           int xcd_major, int m_inner, char* smem) {
  constexpr int TM = 64 * RB;                  // tile rows (of A)
  constexpr int SLOT_A = TM * WG_ROWB;         // bytes of one A stage
  constexpr int TN = 64 * CB;                  // tile columns (rows of B)
  constexpr int SLOT = wg_slot<RB, CB>();
  constexpr int NLA = TM / 64, NLB = TN / 64;  // direct loads per wavefront and stage
  constexpr int PITCH = TN;                    // fp32 epilogue rows in LDS
  static_assert(64 * PITCH * 4 <= 2 * SLOT, "a 64-row part of the tile fits");
  const int per_g = mtiles * ntiles;
  int g, rem;
  if (xcd_major) {
    const int q = blockIdx.x >> 3;
    const int j = q / per_g;  // the XCD's j-th group, in plan order
    if (j >= p.cap) return;
    g = p.xcd_groups[(blockIdx.x & 7) * p.cap + j];
    rem = q - j * per_g;
  } else {
    g = blockIdx.x / per_g;
    rem = blockIdx.x % per_g;
  }
  if (g < 0 || g >= p.G) return;
  const int mt = m_inner ? rem % mtiles : rem / ntiles;
  const int nt = m_inner ? rem / mtiles : rem % ntiles;
  const int m0 = mt * TM, n0 = nt * TN;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t k0 = p.kofs[g];
  const int nk = (int)((p.kofs[g + 1] - k0) / WG_BKS);
  // direct loads: instruction t of wavefront w fills rows 16 (w + 4 t) .. + 15
  // of the operand's tile (lane l: row + l / 4, position l % 4 holding chunk
  // (l % 4) ^ ((row >> 2) & 3)); rows past M or N repeat the last one
  const char* A_base = reinterpret_cast<const char*>(p.A + k0 * p.M + (int64_t)m0 * WG_BKS);
  const char* B_base = reinterpret_cast<const char*>(p.B + k0 * p.N + (int64_t)n0 * WG_BKS);
  const int64_t a_slab = (int64_t)p.M * WG_ROWB, b_slab = (int64_t)p.N * WG_ROWB;  // bytes
  uint32_t a_src[NLA], b_src[NLB];
#pragma unroll
  for (int t = 0; t < NLA; ++t) {
    const int r = 16 * (wave + 4 * t) + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 2) & 3);
    a_src[t] = (uint32_t)(min(r, p.M - 1 - m0) * WG_ROWB + lc * 16);
  }
#pragma unroll
  for (int t = 0; t < NLB; ++t) {
    const int r = 16 * (wave + 4 * t) + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 2) & 3);
    b_src[t] = (uint32_t)(min(r, p.N - 1 - n0) * WG_ROWB + lc * 16);
  }
  char* const dstA = smem + wave * 1024;
  char* const dstB = smem + SLOT_A + wave * 1024;
#define WG_LOAD_STAGE(kt, slot)                                                       \
  {                                                                                   \
    const __amdgpu_buffer_rsrc_t ra_ = __builtin_amdgcn_make_buffer_rsrc(             \
        (void*)(A_base + (int64_t)(kt) * a_slab), 0, 0x7fffffff, 0x00020000);         \
    const __amdgpu_buffer_rsrc_t rb_ = __builtin_amdgcn_make_buffer_rsrc(             \
        (void*)(B_base + (int64_t)(kt) * b_slab), 0, 0x7fffffff, 0x00020000);         \
    _Pragma("unroll") for (int t = 0; t < NLA; ++t)                                   \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                     \
            ra_, (lds_void_t*)(dstA + (slot) * SLOT + t * 4096), 16, a_src[t], 0, 0, 0); \
    _Pragma("unroll") for (int t = 0; t < NLB; ++t)                                   \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                     \
            rb_, (lds_void_t*)(dstB + (slot) * SLOT + t * 4096), 16, b_src[t], 0, 0, 0); \
  }
  const int swz = ((lane & 31) >> 2) & 3;
  f32x16_t acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if (nk > 0) WG_LOAD_STAGE(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt & 1;
    if (kt + 1 < nk) {
      WG_LOAD_STAGE(kt + 1, slot ^ 1);
      ring_barrier<NLA + NLB>();  // this stage's loads are older than the next stage's
    } else {
      ring_barrier<0>();
    }
    const char* As = smem + slot * SLOT;
    const char* Bs = As + SLOT_A;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ((2 * ks + (lane >> 5)) ^ swz) * 16;
      bf16x8_t fa[RB], fb[CB];
#pragma unroll
      for (int i = 0; i < RB; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(
            As + (wm * (TM / 2) + 32 * i + (lane & 31)) * WG_ROWB + ch);
#pragma unroll
      for (int j = 0; j < CB; ++j)
        fb[j] = *reinterpret_cast<const bf16x8_t*>(
            Bs + (wn * (TN / 2) + 32 * j + (lane & 31)) * WG_ROWB + ch);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    // every wavefront is done reading this slot before it is refilled (its LDS
    // reads have landed; the next stage's loads may stay in flight)
    ring_barrier<63>();
  }
#undef WG_LOAD_STAGE
  // D[i][j] of a 32 x 32 block: lane j + 32 ((i / 4) % 2), register 4 (i / 8) + i % 4.
  // The tile leaves through LDS in parts of 64 rows (part h: wavefronts with
  // wm = h / (RB / 2), their row blocks 2 (h % (RB / 2)) and the next), as
  // 16-byte stores of whole 512-byte row segments.  The stores are
  // non-temporal: the gradients are written once and never read here, and
  // through L2 they would evict the expert's operand slices that the next
  // tiles read again (the operands were then fetched 2.4 times, now once).
  float* Cs = reinterpret_cast<float*>(smem);
  float* Cg = p.C + (int64_t)g * p.M * p.N;
  const int lrow4 = 4 * (lane >> 5), lcol = lane & 31;
#pragma unroll
  for (int h = 0; h < TM / 64; ++h) {
    if (wm == h / (RB / 2)) {
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int i = 2 * (h % (RB / 2)) + i2;
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ml = 32 * i2 + 8 * (v >> 2) + lrow4 + (v & 3);
            const int nl = wn * (TN / 2) + 32 * j + lcol;
            Cs[ml * PITCH + nl] = acc[i][j][v];
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < TN / 16; ++q) {
      const int idx = q * 256 + tid;  // TN / 4 chunks of 4 floats per row
      const int ml = idx / (TN / 4), nc = (idx % (TN / 4)) * 4;
      const int m = m0 + 64 * h + ml, n = n0 + nc;
      if (m < p.M && n < p.N) {
        const f32x4_t val = *reinterpret_cast<const f32x4_t*>(Cs + ml * PITCH + nc);
        __builtin_nontemporal_store(val, reinterpret_cast<f32x4_t*>(Cg + (int64_t)m * p.N + n));
      }
    }
    __syncthreads();
  }
}

template <int RB, int CB>
__global__ __launch_bounds__(256) void wgrad_kernel(WgradProblem p, int mtiles, int ntiles,
                                                     int xcd_major, int m_inner) {
  __shared__ __attribute__((aligned(16))) char smem[2 * wg_slot<RB, CB>()];
  wgrad_tile<RB, CB>(p, mtiles, ntiles, xcd_major, m_inner, smem);
}

}  // namespace

hipError_t launch_bwd_prefix(const int32_t* offsets, int N, int bm, int32_t* tile_prefix,
                             int32_t* kofs, hipStream_t s) {
  hipLaunchKernelGGL(bwd_prefix_kernel, dim3(1), dim3(64), 0, s, offsets, N, bm, tile_prefix, kofs);
  return hipGetLastError();
}

hipError_t launch_bwd_colrow(const int32_t* offsets, const int32_t* kofs, int N, int32_t* colrow,
                             int ncols, hipStream_t s) {
  if (ncols <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_colrow_kernel, dim3((ncols + 255) / 256), dim3(256), 0, s, offsets, kofs,
                     N, colrow, ncols);
  return hipGetLastError();
}

hipError_t launch_bwd_rowgate(const int32_t* pos, const float* gate, int64_t slots,
                              float* row_gate, hipStream_t s) {
  if (slots <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_rowgate_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, s,
                     pos, gate, slots, row_gate);
  return hipGetLastError();
}

hipError_t launch_transpose(const TrArgsHost& h, hipStream_t s) {
  if (h.ncols <= 0 || h.dim <= 0 || h.batch <= 0) return hipSuccess;
  // 16-byte accesses: strides and column offsets in multiples of 8 elements
  // (of 4 for fp32 would do; 8 keeps one rule), bases 16-byte aligned
  const bool ok = h.src_ld % 8 == 0 && h.src_col0 % 8 == 0 && h.src_bstride % 8 == 0 &&
                  h.dst_ld % 8 == 0 && h.dst_col0 % 8 == 0 && h.dst_bstride % 8 == 0 &&
                  (reinterpret_cast<uintptr_t>(h.src) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(h.dst) & 15) == 0;
  if (!ok) return hipErrorInvalidValue;
  if (h.kofs && (h.dst_col0 != 0 || h.batch != 1 || h.ngroups < 1)) return hipErrorInvalidValue;
  TrArgs a{h.src, h.src_ld, h.src_col0, h.src_bstride, h.rowidx, h.rowscale, h.colrow,
           h.ncols_valid, h.dst, h.dst_ld, h.dst_col0, h.dst_bstride, h.dim, h.ncols,
           h.kofs, h.ngroups};
  const dim3 grid((unsigned)((h.ncols + 63) / 64), (unsigned)((h.dim + 63) / 64), (unsigned)h.batch);
  if (h.src_f32 && h.dst_f32)
    hipLaunchKernelGGL((transpose_kernel<float, float>), grid, dim3(256), 0, s, a);
  else if (h.src_f32)
    hipLaunchKernelGGL((transpose_kernel<float, bf16_t>), grid, dim3(256), 0, s, a);
  else if (h.dst_f32)
    hipLaunchKernelGGL((transpose_kernel<bf16_t, float>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((transpose_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* A, const void* U, int64_t ld_au, bool au_bf16,
                             const float* Q, const float* row_gate, const int32_t* offsets, int N,
                             int I, int64_t max_rows, bf16_t* dau, bf16_t* H, float* row_dg,
                             hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  if (au_bf16)
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16_t>, dim3((unsigned)max_rows), dim3(256), 0, s,
                       static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(U), ld_au, Q,
                       row_gate, offsets, N, I, dau, H, row_dg);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, dim3((unsigned)max_rows), dim3(256), 0, s,
                       static_cast<const float*>(A), static_cast<const float*>(U), ld_au, Q,
                       row_gate, offsets, N, I, dau, H, row_dg);
  return hipGetLastError();
}

hipError_t launch_token_route_bwd(const bf16_t* x, const bf16_t* dy, const float* logits,
                                  const int32_t* idx, const int32_t* pos, const float* row_dg,
                                  int64_t T, int d, int E, int K, int N, bf16_t* dl, int ldl,
                                  hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(token_route_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x,
                     dy, logits, idx, pos, row_dg, T, d, E, K, N, dl, ldl);
  return hipGetLastError();
}

hipError_t launch_dx_sum(const bf16_t* dy, const int32_t* idx, const float* gate,
                         const int32_t* pos, const float* dxg, const float* dx_r, int64_t T, int d,
                         int K, int N, bf16_t* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d % 8 != 0) return hipErrorInvalidValue;
  const int64_t n = T * (d / 8);
  if ((n + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dx_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dy, idx,
                     gate, pos, dxg, dx_r, T, d, K, N, dx);
  return hipGetLastError();
}

hipError_t launch_set_range(int32_t* out, int a, int b, hipStream_t s) {
  hipLaunchKernelGGL(set_range_kernel, dim3(1), dim3(64), 0, s, out, a, b);
  return hipGetLastError();
}

int wgrad_xcd_cap(int G) { return (G + 7) / 8 + (G + 63) / 64; }

hipError_t launch_wgrad_plan(const int32_t* kofs, int G, int32_t* xcd_groups, hipStream_t s) {
  if (G < 8) return hipSuccess;  // no plan: fewer groups than XCDs
  if (G > kWgradMaxGroups) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wgrad_plan_kernel, dim3(1), dim3(1024), 0, s, kofs, G, wgrad_xcd_cap(G),
                     xcd_groups);
  return hipGetLastError();
}

hipError_t launch_wgrad(const bf16_t* A, const bf16_t* B, const int32_t* kofs, int G, int M,
                        int N, float* C, const int32_t* xcd_groups, hipStream_t s) {
  if (G <= 0 || M <= 0 || N <= 0) return hipSuccess;
  if (N % 4 != 0) return hipErrorInvalidValue;  // 16-byte stores of C rows
  const int xcd_major = G >= 8;
  if (xcd_major && (!xcd_groups || G > kWgradMaxGroups)) return hipErrorInvalidValue;
  const int cap = xcd_major ? wgrad_xcd_cap(G) : 0;
  const int tm = xcd_major ? 256 : 128, tn = 128;  // taller tiles where there are many groups
  const int mt = (M + tm - 1) / tm, nt = (N + tn - 1) / tn;
  const int64_t tiles = (int64_t)(xcd_major ? 8 * cap : G) * mt * nt;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  WgradProblem p{A, B, kofs, G, M, N, C, xcd_major ? xcd_groups : nullptr, cap};
  if (tm == 256)
    hipLaunchKernelGGL((wgrad_kernel<4, 2>), dim3((unsigned)tiles), dim3(256), 0, s, p, mt, nt,
                       xcd_major, (int)(M <= N));
  else
    hipLaunchKernelGGL((wgrad_kernel<2, 2>), dim3((unsigned)tiles), dim3(256), 0, s, p, mt, nt,
                       xcd_major, (int)(M <= N));
  return hipGetLastError();
}

}  // namespace moezc
