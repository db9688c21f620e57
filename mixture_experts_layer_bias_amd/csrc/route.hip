// Routing-side kernels of the MoE layer with zero-computation experts (gfx950):
// softmax + bias key + top-K, expert histogram, scan, grouping permutation,
// combine and the PID bias update.
//
// Layer definition: LongCat-Flash pages, 『衝上熱搜！美團大模型，靠「快」火了』,
// section 零計算專家 (softmax router over N FFN + Z identity experts, bias b_i
// used for selection, K experts per token; PID tuning of the bias).
#include <math.h>

#include <algorithm>

#include "kernels.hpp"

namespace moezc {

// ---------------------------------------------------------------------------
// Softmax + bias key + top-K.  One wavefront per token; lane l holds experts
// l, l+64, ...  The softmax runs in fp64 from the fp32 logits (max, exp,
// sum, divide), its result is rounded once to fp32 (the gate), and the
// selection key is the fp32 sum fl32(p32 + b).  The K winners are the first K
// in the order (key descending, index ascending), so an exact tie goes to the
// lower expert index, and they are written in that order (the selection is
// described at its code below).  Reductions are xor butterflies: every lane
// ends with the same, run-to-run reproducible value.  A split router product
// arrives as nsplit partial logits; they are summed in part order (fixed, so
// reproducible) and the sums are stored as the logits.

// Bitonic sort of one (key, index, payload) triple per lane over the
// wavefront into the order (key descending, index ascending): lane 0 ends with
// the first.  Triples with equal keys and indices (the padding) compare equal
// and never swap.
__device__ __forceinline__ void wave_sort_desc(int lane, float& k, int& i, float& p) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float ok = __shfl_xor(k, stride);
      const int oi = __shfl_xor(i, stride);
      const float op = __shfl_xor(p, stride);
      const bool o_first = ok > k || (ok == k && oi < i);   // the partner's triple comes first
      const bool m_first = k > ok || (k == ok && i < oi);
      // the lower lane of a pair keeps the first triple in a descending run and
      // the second in an ascending one (runs alternate with lane & size)
      const bool lower = (lane & stride) == 0, desc = (lane & size) == 0;
      const bool take = (lower == desc) ? o_first : m_first;
      k = take ? ok : k;
      i = take ? oi : i;
      p = take ? op : p;
    }
}

template <int EPL, bool SPLIT>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias,
                                                   int64_t T, int E, int K,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ gate_out, int nsplit,
                                                   int64_t split_stride,
                                                   float* __restrict__ logits_out) {
  __shared__ float cand_k[4][64];
  __shared__ int cand_i[4][64];
  __shared__ float cand_p[4][64];
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;

  float l[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane + 64 * i;
    l[i] = j < E ? row[j] : -INFINITY;
  }
  // partial logits of a split router product: four parts of every element
  // in flight at a time (4 EPL loads), each element's parts added in part
  // order; past E the added zeros leave -inf
  for (int s = 1; SPLIT && s < nsplit; s += 4) {
    float q[4][EPL];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int j = lane + 64 * i;
        q[r][i] = (s + r < nsplit && j < E) ? row[(s + r) * split_stride + j] : 0.f;
      }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (s + r < nsplit) l[i] += q[r][i];
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane + 64 * i;
    if (SPLIT && j < E) logits_out[t * E + j] = l[i];
    m = fmaxf(m, l[i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));

  double ex[EPL];
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane + 64 * i;
    ex[i] = (j < E) ? exp((double)l[i] - (double)m) : 0.0;
    s += ex[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);

  float p32[EPL], key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane + 64 * i;
    p32[i] = (float)(ex[i] / s);
    key[i] = (j < E) ? __fadd_rn(p32[i], bias[j]) : -INFINITY;
  }

  // Selection in the total order (key descending, index ascending).  Every
  // lane's best element is a lower bound for the K-th best overall once K
  // lanes are counted, so with tau = the K-th best of the 64 lane bests, the
  // K winners are among the elements not worse than tau (tau itself
  // included): usually a dozen or two.  They are gathered into one element per
  // lane and sorted across the wavefront; lanes 0 .. K-1 then hold the winners
  // in order.  Should more than 64 elements qualify, K rounds of a wavefront
  // arg-max select the winners instead.  Both give the same result.
  int my_idx = 0;
  float my_gate = 0.f;
  float bk = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane + 64 * i;
    // j grows with i, so a strict '>' keeps the lower index on a tie
    const bool take = j < E && (key[i] > bk || bi == 0x7fffffff);
    bk = take ? key[i] : bk;
    bi = take ? j : bi;
  }
  float sk = bk;
  int si = bi;
  float sp = 0.f;
  wave_sort_desc(lane, sk, si, sp);
  const float tk = __shfl(sk, K - 1);
  const int ti = __shfl(si, K - 1);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane + 64 * i;
    cnt += (j < E && (key[i] > tk || (key[i] == tk && j <= ti))) ? 1 : 0;
  }
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int total = __shfl(incl, 63);
  if (total <= 64) {
    float* ck = cand_k[threadIdx.x >> 6];
    int* ci = cand_i[threadIdx.x >> 6];
    float* cp = cand_p[threadIdx.x >> 6];
    int at = incl - cnt;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int j = lane + 64 * i;
      if (j < E && (key[i] > tk || (key[i] == tk && j <= ti))) {
        ck[at] = key[i];
        ci[at] = j;
        cp[at] = p32[i];
        ++at;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes landed
    __builtin_amdgcn_wave_barrier();
    sk = lane < total ? ck[lane] : -INFINITY;
    si = lane < total ? ci[lane] : 0x7fffffff;
    sp = lane < total ? cp[lane] : 0.f;
    wave_sort_desc(lane, sk, si, sp);
    my_idx = si;
    my_gate = sp;
  } else {
    uint32_t taken = 0u;
    for (int r = 0; r < K; ++r) {
      float rk = -INFINITY, rp = 0.f;
      int ri = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int j = lane + 64 * i;
        const bool take = j < E && !((taken >> i) & 1u) && (key[i] > rk || ri == 0x7fffffff);
        rk = take ? key[i] : rk;
        rp = take ? p32[i] : rp;
        ri = take ? j : ri;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ok = __shfl_xor(rk, off);
        const int oi = __shfl_xor(ri, off);
        const bool take = ok > rk || (ok == rk && oi < ri);
        rk = take ? ok : rk;
        ri = take ? oi : ri;
      }
      const float gate = __shfl(rp, ri & 63);      // the winner's lane holds its gate
      taken |= ((ri & 63) == lane) ? (1u << (ri >> 6)) : 0u;
      my_idx = (lane == r) ? ri : my_idx;
      my_gate = (lane == r) ? gate : my_gate;
    }
  }
  if (lane < K) {
    idx_out[t * K + lane] = my_idx;
    gate_out[t * K + lane] = my_gate;
  }
}

// SPLIT: the instantiation that adds partial logits (more registers)
template <int EPL>
hipError_t launch_topk_epl(const float* logits, const float* bias, int64_t T, int E, int K,
                           int32_t* idx, float* gate, hipStream_t s, int nsplit,
                           int64_t split_stride, float* logits_out) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (nsplit > 1)
    hipLaunchKernelGGL((topk_kernel<EPL, true>), grid, block, 0, s, logits, bias, T, E, K, idx,
                       gate, nsplit, split_stride, logits_out);
  else
    hipLaunchKernelGGL((topk_kernel<EPL, false>), grid, block, 0, s, logits, bias, T, E, K, idx,
                       gate, 1, split_stride, logits_out);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int E, int K,
                       int32_t* idx, float* gate, hipStream_t s, int nsplit,
                       int64_t split_stride, float* logits_out) {
  const int epl = (E + 63) / 64;
  if (nsplit < 1 || (nsplit > 1 && !logits_out)) return hipErrorInvalidValue;
#define MOEZC_TOPK(n) \
  launch_topk_epl<n>(logits, bias, T, E, K, idx, gate, s, nsplit, split_stride, logits_out)
  if (epl <= 1) return MOEZC_TOPK(1);
  if (epl <= 2) return MOEZC_TOPK(2);
  if (epl <= 4) return MOEZC_TOPK(4);
  if (epl <= 8) return MOEZC_TOPK(8);
  if (epl <= 12) return MOEZC_TOPK(12);
  if (epl <= 16) return MOEZC_TOPK(16);
  if (epl <= 32) return MOEZC_TOPK(32);
#undef MOEZC_TOPK
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Expert loads from top-K indices alone (moe_zc_route): loads[e] = number of
// slots routed to e.  Integer counts, so the atomics below give the same
// result in any order.  The first launch zeroes loads (a kernel, not a
// memset, so the sequence can be captured in a graph); the second counts
// each workgroup's slots in LDS and adds its nonzero counts to loads.
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void count_loads_kernel(const int32_t* __restrict__ idx,
                                                          int64_t n, int E,
                                                          int32_t* __restrict__ loads) {
  __shared__ int32_t hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    atomicAdd(&hist[idx[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    if (hist[e]) atomicAdd(&loads[e], hist[e]);
}

hipError_t launch_count_loads(const int32_t* idx, int64_t T, int K, int E, int32_t* loads,
                              hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, loads,
                     E);
  const int64_t n = T * K;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  if (blocks > 0)
    hipLaunchKernelGGL(count_loads_kernel, dim3((unsigned)blocks), dim3(256), 0, s, idx, n, E,
                       loads);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-chunk expert histogram and stable in-chunk ranks.  One wavefront per
// chunk of 64 tokens: lane l (token c*64+l) sets bit l of the 64-bit mask of
// each expert it chose (an LDS OR, order independent).  A token's rank among
// the chunk's tokens routed to expert e is the popcount of the mask bits
// below its own; a token picks an expert at most once, so this orders the
// expert's rows by token.  counts[c][e] = popcount(mask[e]).
__global__ __launch_bounds__(64) void chunk_hist_kernel(const int32_t* __restrict__ idx,
                                                        int64_t T, int K, int E, int N,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ rank) {
  __shared__ unsigned long long mask[kMaxExperts];
  const int lane = threadIdx.x;
  const int64_t c = blockIdx.x;
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  const int64_t t = c * kChunk + lane;
  if (t < T) {
    for (int k = 0; k < K; ++k) atomicOr(&mask[idx[t * K + k]], 1ull << lane);
  }
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      rank[t * K + k] = (e < N) ? __popcll(mask[e] & below) : -1;
    }
  }
  for (int e = lane; e < E; e += 64) counts[c * E + e] = __popcll(mask[e]);
}

hipError_t launch_chunk_hist(const int32_t* idx, int64_t T, int K, int E, int N,
                             int32_t* counts, int32_t* rank, hipStream_t s) {
  const int64_t C = (T + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(chunk_hist_kernel, dim3((unsigned)C), dim3(64), 0, s, idx, T, K, E, N,
                     counts, rank);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scan of the chunk counts, in two launches (all sums are integer):
//   scan_chunks: counts[c][e] <- sum_{c' < c} counts[c'][e]  (exclusive, in
//     place) and loads[e] = sum_c counts[c][e].  One workgroup of 16
//     wavefronts per 64 experts (lane = expert); wave w owns the chunk range
//     [C*w/16, C*(w+1)/16).
//   scan_experts: offsets[e] = sum_{e' < e} loads[e'] over the N FFN experts
//     (offsets[N] = S), tile_prefix[e] = sum_{e' < e} ceil(loads[e'] / bm),
//     and tile_prefix2 the same for tiles of bm2 rows (optional).  One
//     wavefront; lane l owns a contiguous segment of experts.
constexpr int kScanWaves = 16;
__global__ __launch_bounds__(64 * kScanWaves) void scan_chunks_kernel(
    int32_t* __restrict__ counts, int C, int E, int32_t* __restrict__ loads) {
  __shared__ int32_t part[kScanWaves][64];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int e = blockIdx.x * 64 + lane;
  const bool live = e < E;
  const int c0 = (int)(((int64_t)C * w) / kScanWaves);
  const int c1 = (int)(((int64_t)C * (w + 1)) / kScanWaves);
  int s = 0;
  if (live) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) s += counts[(int64_t)c * E + e];
  }
  part[w][lane] = s;
  __syncthreads();
  if (w == 0) {
    int run = 0;
    for (int v = 0; v < kScanWaves; ++v) {
      const int x = part[v][lane];
      part[v][lane] = run;
      run += x;
    }
    if (live) loads[e] = run;
  }
  __syncthreads();
  if (live) {
    int run = part[w][lane];
    for (int c = c0; c < c1; ++c) {
      const int64_t q = (int64_t)c * E + e;
      const int x = counts[q];
      counts[q] = run;
      run += x;
    }
  }
}

__global__ __launch_bounds__(64) void scan_experts_kernel(const int32_t* __restrict__ loads,
                                                          int N, int32_t* __restrict__ offsets,
                                                          int bm, int32_t* __restrict__ tile_prefix,
                                                          int bm2,
                                                          int32_t* __restrict__ tile_prefix2) {
  const int lane = threadIdx.x;
  const int seg = (N + 63) / 64;
  const int e0 = lane * seg;
  const int e1 = min(N, e0 + seg);
  int sr = 0, st = 0, st2 = 0;
  for (int e = e0; e < e1; ++e) {
    const int l = loads[e];
    sr += l;
    st += (l + bm - 1) / bm;
    st2 += (l + bm2 - 1) / bm2;
  }
  int ir = sr, it = st, it2 = st2;  // inclusive scan over lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(ir, off), b = __shfl_up(it, off), b2 = __shfl_up(it2, off);
    if (lane >= off) {
      ir += a;
      it += b;
      it2 += b2;
    }
  }
  int rr = ir - sr, rt = it - st, rt2 = it2 - st2;
  for (int e = e0; e < e1; ++e) {
    const int l = loads[e];
    offsets[e] = rr;
    tile_prefix[e] = rt;
    if (tile_prefix2) tile_prefix2[e] = rt2;
    rr += l;
    rt += (l + bm - 1) / bm;
    rt2 += (l + bm2 - 1) / bm2;
  }
  if (lane == 63) {
    offsets[N] = ir;
    tile_prefix[N] = it;
    if (tile_prefix2) tile_prefix2[N] = it2;
  }
}

hipError_t launch_scan(int32_t* counts, int C, int E, int N, int32_t* loads, int32_t* offsets,
                       int bm, int32_t* tile_prefix, int bm2, int32_t* tile_prefix2,
                       hipStream_t s) {
  hipLaunchKernelGGL(scan_chunks_kernel, dim3((unsigned)((E + 63) / 64)), dim3(64 * kScanWaves),
                     0, s, counts, C, E, loads);
  hipLaunchKernelGGL(scan_experts_kernel, dim3(1), dim3(64), 0, s, loads, N, offsets, bm,
                     tile_prefix, bm2, tile_prefix2);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouping.  One workgroup per token: the first K threads turn each FFN slot's
// in-chunk rank into its grouped row offsets[e] + base[c][e] + rank, write
// pos and perm; then the whole workgroup copies the token's row of x into
// each of its FFN rows (x read once, 16-byte vector accesses).
template <typename T>
__global__ __launch_bounds__(256) void permute_kernel(const T* __restrict__ x,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ pos,
                                                      int32_t* __restrict__ perm,
                                                      T* __restrict__ xp, int d, int K,
                                                      int E, int N) {
  __shared__ int32_t rows[kMaxTopK];
  const int64_t t = blockIdx.x;
  const int64_t c = t / kChunk;
  if ((int)threadIdx.x < K) {
    const int k = threadIdx.x;
    const int e = idx[t * K + k];
    int row = -1;
    if (e < N) {
      row = offsets[e] + base[c * E + e] + pos[t * K + k];
      perm[row] = (int32_t)t;
    }
    pos[t * K + k] = row;
    rows[k] = row;
  }
  __syncthreads();
  constexpr int kVec = 16 / sizeof(T);  // elements per 16-byte access
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  for (int v = threadIdx.x; v < d / kVec; v += blockDim.x) {
    const uint4 val = src[v];
    for (int k = 0; k < K; ++k) {
      const int row = rows[k];
      if (row >= 0) reinterpret_cast<uint4*>(xp + (int64_t)row * d)[v] = val;
    }
  }
}

// Grouping without the row copy (the grouped GEMM gathers rows of x through
// perm itself): one thread per slot (t, k).
__global__ __launch_bounds__(256) void group_rows_kernel(const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ base,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ perm,
                                                         int64_t TK, int K, int E, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= TK) return;
  const int64_t t = i / K;
  const int e = idx[i];
  int row = -1;
  if (e < N) {
    row = offsets[e] + base[(t / kChunk) * E + e] + pos[i];
    perm[row] = (int32_t)t;
  }
  pos[i] = row;
}

template <typename T>
hipError_t launch_permute(const T* x, const int32_t* idx, const int32_t* chunk_base,
                          const int32_t* offsets, int32_t* pos, int32_t* perm, T* xp,
                          int64_t Tn, int d, int K, int E, int N, hipStream_t s) {
  if (xp) {
    hipLaunchKernelGGL(permute_kernel<T>, dim3((unsigned)Tn), dim3(256), 0, s, x, idx,
                       chunk_base, offsets, pos, perm, xp, d, K, E, N);
  } else {
    const int64_t TK = Tn * K;
    hipLaunchKernelGGL(group_rows_kernel, dim3((unsigned)((TK + 255) / 256)), dim3(256), 0, s,
                       idx, chunk_base, offsets, pos, perm, TK, K, E, N);
  }
  return hipGetLastError();
}
template hipError_t launch_permute<float>(const float*, const int32_t*, const int32_t*,
                                          const int32_t*, int32_t*, int32_t*, float*, int64_t,
                                          int, int, int, int, hipStream_t);
template hipError_t launch_permute<bf16_t>(const bf16_t*, const int32_t*, const int32_t*,
                                           const int32_t*, int32_t*, int32_t*, bf16_t*, int64_t,
                                           int, int, int, int, hipStream_t);

// ---------------------------------------------------------------------------
// Combine.  One workgroup per token; y_t = r_t + sum_k g[t,k] * src_k with
// src_k the grouped FFN output row pos[t,k] or, for a zero-computation
// expert, x_t itself (the identity expert is never materialised).  fp32
// accumulation in slot order, one rounding to the output type.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ x,
                                                      const T* __restrict__ o,
                                                      const T* __restrict__ res,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ pos,
                                                      T* __restrict__ y, int d, int K, int N) {
  __shared__ float g_s[kMaxTopK];
  __shared__ int32_t row_s[kMaxTopK];
  const int64_t t = blockIdx.x;
  if ((int)threadIdx.x < K) {
    const int k = threadIdx.x;
    g_s[k] = gate[t * K + k];
    row_s[k] = (idx[t * K + k] < N) ? pos[t * K + k] : -1;
  }
  __syncthreads();
  const T* xt = x + t * d;
  for (int v = threadIdx.x; v < d / 8; v += blockDim.x) {
    float acc[8];
    if (res) {
      load8(res + t * d + v * 8, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int k = 0; k < K; ++k) {
      const int row = row_s[k];
      const T* src = (row >= 0) ? o + (int64_t)row * d : xt;
      float vals[8];
      load8(src + v * 8, vals);
      const float g = g_s[k];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, vals[i], acc[i]);
    }
    store8(y + t * d + v * 8, acc);
  }
}

template <typename T>
hipError_t launch_combine(const T* x, const T* o, const T* res, const int32_t* idx,
                          const float* gate, const int32_t* pos, T* y, int64_t Tn, int d, int K,
                          int N, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel<T>, dim3((unsigned)Tn), dim3(256), 0, s, x, o, res, idx,
                     gate, pos, y, d, K, N);
  return hipGetLastError();
}
template hipError_t launch_combine<float>(const float*, const float*, const float*,
                                          const int32_t*, const float*, const int32_t*, float*,
                                          int64_t, int, int, int, hipStream_t);
template hipError_t launch_combine<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*,
                                           const int32_t*, const float*, const int32_t*, bf16_t*,
                                           int64_t, int, int, int, hipStream_t);

// ---------------------------------------------------------------------------
// PID step on the expert bias (velocity form; one workgroup).
//   e_i = (target_i - loads_i) / sum(target)
//   bias_i += kp (e_i - e1_i) + ki e_i + kd (e_i - 2 e1_i + e2_i)
// Sums and updates in fp64 with a fixed reduction tree; state stored in fp32.
__global__ __launch_bounds__(1024) void pid_kernel(const int32_t* __restrict__ loads,
                                                   const float* __restrict__ target,
                                                   float* __restrict__ bias,
                                                   float* __restrict__ e1,
                                                   float* __restrict__ e2, int E, double kp,
                                                   double ki, double kd) {
  __shared__ double red[1024];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int e = tid; e < E; e += 1024) s += (double)target[e];
  red[tid] = s;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const double total = red[0];
  for (int e = tid; e < E; e += 1024) {
    const double err = ((double)target[e] - (double)loads[e]) / total;
    const double p1 = (double)e1[e], p2 = (double)e2[e];
    const double db = kp * (err - p1) + ki * err + kd * (err - 2.0 * p1 + p2);
    bias[e] = (float)((double)bias[e] + db);
    e2[e] = (float)p1;
    e1[e] = (float)err;
  }
}

hipError_t launch_pid(const int32_t* loads, const float* target, float* bias, float* e1,
                      float* e2, int E, float kp, float ki, float kd, hipStream_t s) {
  hipLaunchKernelGGL(pid_kernel, dim3(1), dim3(1024), 0, s, loads, target, bias, e1, e2, E,
                     (double)kp, (double)ki, (double)kd);
  return hipGetLastError();
}

}  // namespace moezc
