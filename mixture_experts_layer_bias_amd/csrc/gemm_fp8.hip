// Block-FP8 expert projections (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4):
//
//   H[rows of expert g, :] = silu(A B_gate_g^T) * (A B_up_g^T)     (gate/up)
//   O[rows of expert g, :] = A B_down_g^T                          (down, optional)
//
// with A (the token rows of x, or of h for the down projection) and B (W_gate,
// W_up, W_down) in FP8 E4M3, each block of
// 32 consecutive values along k carrying one power-of-two scale (an 8-bit
// biased exponent, bias 127).  The matrix cores apply both operands' scales
// inside the MFMA and accumulate in fp32; the outputs h and o are bf16, as on
// the bf16 path; the down projection runs in FP8 or bf16, a per-layer choice.
// This is the fine-grained
// block quantization the LongCat pages adopt (same scheme family as
// DeepSeek-V3, mixed per layer: the down projection's inputs carry extreme
// activations), in the block-scaled form the MI355X matrix cores consume.
//
// Quantization of a block of 32 values v: s = the smallest integer with
// max|v| <= 448 * 2^s (clamped to [-127, 127]; an all-zero block takes -127),
// codes = E4M3(v / 2^s) rounded to nearest even, sign bit copied from v.
//
// MFMA operand layout (measured on the hardware with random codes and random
// scales): a 64-k step is two scale blocks of 32 k.  For row (A) or column (B)
// r, lane r holds 16 codes of block 0 (bytes 0-15) and 16 of block 1 (bytes
// 16-31), lane r + 32 the other 16 of each; the scale byte of lane r scales
// block 0 and that of lane r + 32 block 1, for both lanes' codes.  So lane
// (r, h = lane / 32) takes codes 16 h .. 16 h + 15 of each block.  op_sel n
// picks byte n of the 32-bit scale register.  The output layout is that of
// the bf16 32x32 MFMA.
//
// Packed gate/up weights: panels of 128 hidden units (their 128 gate rows and
// 128 up rows), stages of 128 k.  One (expert, panel, stage) block is 33 KB:
//   codes, 32 KB: quarter w (8 KB) = wavefront w; piece q = 4 ks + 2 j + half
//     (1 KB) holds for lane l the 16 codes of (substep ks, column block j
//     (0 gate, 1 up), scale block half):  row = panel * 128 + 32 w + l % 32,
//     k = 128 stage + 64 ks + 32 half + 16 (l / 32) + 0..15;
//   scales, 1 KB: 256 bytes per wavefront, 4 per lane; byte 2 ks + j of lane
//     l is the scale of row (j, l % 32), k block 4 stage + 2 ks + l / 32.
// Packed down weights: the same blocks over panels of 256 rows of W_down
// (output columns) and stages of 128 k along I, with column block j of
// wavefront w holding rows panel * 256 + 64 w + 32 j + l % 32 (zeros past d).
// Blocks are ordered expert, panel, stage: a tile streams one contiguous range.
//
// Activations: x is quantized once per forward into codes [T, d] and scales
// [T, d / 32] (row-major).  The GEMM gathers code rows through the grouping
// permutation into an LDS ring exactly as the bf16 kernel gathers bf16 rows
// (a stage of 128 codes is 128 bytes per row, the bf16 stage's size), and each
// lane loads the 4 scale bytes of its rows' stage directly.
#include "gemm_tile.hpp"

namespace moezc {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

constexpr int F8_WAVES = 4;
constexpr int F8_BKS = 128;                              // k per stage
constexpr int F8_DATA = kPackedPanel * F8_BKS;           // 32 KB of codes per stage
constexpr int F8_SCL = kPackedPanel * (F8_BKS / 32);     // 1 KB of scales per stage
constexpr int F8_BLOCK = F8_DATA + F8_SCL;
constexpr int F8_QUARTER = F8_DATA / F8_WAVES;           // one wavefront's codes
constexpr int F8_MAXRB = kPackedMaxTileRows / 32;        // 32-row blocks per tile
constexpr int F8_DEPTH = 3, F8_DIST = 2;                 // ring stages, loaded ahead
constexpr int F8_WLOADS = 9;                             // weight register loads per stage
// the wait between a stage's substeps counts only one refill's weight loads
static_assert(F8_DIST == 2, "one stage's refill in flight across the barrier");
constexpr int F8_SLOT = F8_MAXRB * 32 * F8_BKS;          // LDS bytes of one stage
static_assert(F8_QUARTER == 8 * 1024, "eight 1 KB pieces per wavefront");

// Four E4M3 codes of (a, b, c, d) (each |y| <= 448) in one dword, a in the
// low byte: round to nearest, ties to even, sign bit copied (negative values
// that round to zero give 0x80).  gfx950's v_cvt_pk_fp8_f32 converts to the
// OCP E4M3 format with exactly this rounding: on the device it agrees with
// the format's definition (grid step 2^-9 below 2^-6, else 2^(E-3) in binade
// E) on every fp32 value of that range.  The callers scale by powers of two
// first, which is exact.
__device__ __forceinline__ uint32_t e4m3_quad(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0, 1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);        // bytes 2, 3
  return (uint32_t)w;
}

// Smallest s with amax <= 448 * 2^s, clamped to [-127, 127]; 448 = 1.75 * 2^8,
// so with amax = f 2^E (1 <= f < 2): s = E - 8, plus 1 when f > 1.75.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ex = (int)((b >> 23) & 0xff);
  if (!(amax > 0.f) || ex == 0) return -127;  // zero, or below 2^-126: clamps
  const int s = ex - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// One block of 32 bf16 values: codes (4 per dword, lowest k first) and the
// scale byte.
__device__ __forceinline__ uint32_t mx_block(const bf16_t* __restrict__ src, uint32_t codes[8]) {
  u32x4_t raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = reinterpret_cast<const u32x4_t*>(src)[i];
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = raw[i >> 2][i & 3];
    v[2 * i] = __uint_as_float(w << 16);
    v[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int s = mx_scale_exp(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    codes[i] = e4m3_quad(ldexpf(v[4 * i], -s), ldexpf(v[4 * i + 1], -s),
                         ldexpf(v[4 * i + 2], -s), ldexpf(v[4 * i + 3], -s));
  }
  return (uint32_t)(s + 127);
}

// x [rows][d] bf16 -> codes [rows][d], scales [rows][d / 32]; one thread per
// block of 32 (consecutive threads, consecutive blocks).
__global__ __launch_bounds__(256) void quantize_mx_kernel(const bf16_t* __restrict__ x,
                                                          uint8_t* __restrict__ xq,
                                                          uint8_t* __restrict__ xs,
                                                          int64_t nblk) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  uint32_t codes[8];
  const uint32_t sc = mx_block(x + b * 32, codes);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(xq + b * 32);
  dst[0] = u32x4_t{codes[0], codes[1], codes[2], codes[3]};
  dst[1] = u32x4_t{codes[4], codes[5], codes[6], codes[7]};
  xs[b] = (uint8_t)sc;
}

// Weights [groups][rows][K] bf16 -> packed FP8 blocks: SwiGLU (wu set): W_gate
// and W_up with rows = I hidden units, K = d; otherwise W_down with rows = d,
// K = I.  One workgroup per (group, panel, stage) block; 1024 (row, 32-k
// block) pairs per block, the k block in the low bits so that four
// consecutive threads read one row's 256 bytes.
__global__ __launch_bounds__(256) void pack_fp8_kernel(const bf16_t* __restrict__ wg,
                                                       const bf16_t* __restrict__ wu,
                                                       uint8_t* __restrict__ out, int rows, int d,
                                                       int n_panels) {
  const int I = rows;  // rows of one group (SwiGLU: hidden units)
  const int nk = d / F8_BKS;
  const int64_t b = blockIdx.x;
  const int64_t per_group = (int64_t)n_panels * nk;
  const int64_t g = b / per_group;
  const int rem = (int)(b - g * per_group);
  const int nt = rem / nk, kt = rem - nt * nk;
  uint8_t* blk = out + b * F8_BLOCK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pidx = threadIdx.x + 256 * i;
    const int kb = pidx & 3, rp = pidx >> 2;
    const int w = rp >> 6, j = (rp >> 5) & 1, cc = rp & 31;
    // SwiGLU: gate (j = 0) or up (j = 1) row of hidden unit u; plain: row u
    const int64_t u = wu ? (int64_t)nt * 128 + 32 * w + cc
                         : (int64_t)nt * 256 + 64 * w + 32 * j + cc;
    uint32_t codes[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t sc = 0u;  // rows past the end: zero codes, smallest scale
    if (u < I) {
      const bf16_t* src = ((wu && j) ? wu : wg) + (g * I + u) * (int64_t)d +
                          (int64_t)kt * F8_BKS + kb * 32;
      sc = mx_block(src, codes);
    }
    // block kb = 2 ks + half: codes 0-15 to lane cc, 16-31 to lane cc + 32, both
    // in piece 4 ks + 2 j + half; its scale to lane cc + 32 half
    const int ks = kb >> 1, half = kb & 1, q = 4 * ks + 2 * j + half;
    *reinterpret_cast<u32x4_t*>(blk + w * F8_QUARTER + q * 1024 + cc * 16) =
        u32x4_t{codes[0], codes[1], codes[2], codes[3]};
    *reinterpret_cast<u32x4_t*>(blk + w * F8_QUARTER + q * 1024 + (cc + 32) * 16) =
        u32x4_t{codes[4], codes[5], codes[6], codes[7]};
    blk[F8_DATA + w * 256 + (cc + 32 * half) * 4 + 2 * ks + j] = (uint8_t)sc;
  }
}

// NA = live 32-row blocks of the tile.  Workgroup of four wavefronts, one per
// SIMD; wavefront w owns hidden units [32 w, 32 w + 32) of the panel (gate
// and up columns), for every row.  A stage is two MFMA substeps of 64 k.
// Epilogue of the gate/up tile when the down projection runs in FP8: h =
// silu(gate) * up in fp32, staged through LDS one 32-row block at a time; the
// 32 hidden units a wavefront holds for a row are one quantization block
// (they start at a multiple of 32), so lanes r and r + 32 take columns
// 0..15 and 16..31 of row r, share the block's amax through one shuffle, and
// store 16 codes each (16 bytes) and, lane r, the scale byte.
template <int NA>
__device__ __forceinline__ void store_fp8_h_tile(const f32x16_t (&acc)[NA][2], char* smem,
                                                 int wave, int lane, const TileCoord& c,
                                                 const GemmProblem& p) {
  constexpr int OS = 33;                      // padded LDS row (floats): conflict-free
  float* ot = reinterpret_cast<float*>(smem) + wave * (32 * OS);
  const int lrow4 = 4 * (lane >> 5), lcol = lane & 31;
  const int r = lane & 31, hf = lane >> 5;
  const int gcol0 = c.n0 + wave * 32;         // first hidden unit of this wavefront
  uint8_t* __restrict__ codes = static_cast<uint8_t*>(p.C);
#pragma unroll
  for (int i = 0; i < NA; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      ot[(8 * (v >> 2) + lrow4 + (v & 3)) * OS + lcol] = swiglu_fast(acc[i][0][v], acc[i][1][v]);
    __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0): the LDS writes landed
    __builtin_amdgcn_wave_barrier();
    float vals[16];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      vals[e] = ot[r * OS + 16 * hf + e];
      amax = fmaxf(amax, fabsf(vals[e]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int s = mx_scale_exp(amax);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = e4m3_quad(ldexpf(vals[4 * q], -s), ldexpf(vals[4 * q + 1], -s),
                       ldexpf(vals[4 * q + 2], -s), ldexpf(vals[4 * q + 3], -s));
    const int grow = c.m0 + i * 32 + r;
    if (grow < c.m_end) {
      *reinterpret_cast<u32x4_t*>(codes + (int64_t)grow * p.ldc + gcol0 + 16 * hf) =
          u32x4_t{w[0], w[1], w[2], w[3]};
      if (hf == 0) p.c_scales[(int64_t)grow * p.c_scale_ld + gcol0 / 32] = (uint8_t)(s + 127);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);       // reads done before the next block overwrites
    __builtin_amdgcn_wave_barrier();
  }
}

// Pre-activations of the gate/up tile (a | u, bf16) to p.C2: the saving part
// of store_bf16_tile alone.
template <int NA>
__device__ __forceinline__ void store_act_tile(const f32x16_t (&acc)[NA][2], char* smem, int wave,
                                               int lane, const TileCoord& c,
                                               const GemmProblem& p) {
  constexpr int OS = 40;
  bf16_t* ot = reinterpret_cast<bf16_t*>(smem) + wave * (32 * OS);
  const int lrow4 = 4 * (lane >> 5), lcol = lane & 31;
  const int gcol0 = c.n0 + wave * 32;
  bf16_t* __restrict__ C2 = static_cast<bf16_t*>(p.C2);
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        ot[(8 * (v >> 2) + lrow4 + (v & 3)) * OS + lcol] = f32_to_bf16(acc[i][part][v]);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = lane; q < 32 * 4; q += 64) {
        const int rr = q / 4, ch = q - rr * 4;
        const int grow = c.m0 + i * 32 + rr;
        if (grow < c.m_end)
          *reinterpret_cast<u32x4_t*>(&C2[(int64_t)grow * p.ldc2 + part * p.Nout + gcol0 + ch * 8]) =
              *reinterpret_cast<const u32x4_t*>(&ot[rr * OS + ch * 8]);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
}

// MODE: kSwiGLU_BF16 (h bf16), kSwiGLU_FP8 (h quantized) or kStoreBF16 (down)
template <int NA, bool SAVE, int MODE>
__device__ __forceinline__ void run_fp8(const GemmProblem& p, const TileCoord& c, int n_tiles,
                                        char* __restrict__ smem) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int nk = p.K / F8_BKS;
  const int rows = c.m_end - c.m0;
  const int32_t* __restrict__ a_rows = p.a_rows;

  // ---- activation code rows: direct loads into LDS rows of 128 bytes,
  // chunk c of row r at position c ^ ((r >> 1) & 7); instruction t of
  // wavefront w fills rows 8 (w + 4 t) .. + 7; rows past the tile repeat its
  // last row (their products reach accumulator rows that are never stored)
  const char* A_tile = static_cast<const char*>(p.A) + (a_rows ? (int64_t)0 : (int64_t)c.m0 * p.lda);
  uint32_t a_src[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    const int r = 8 * (wave + F8_WAVES * t) + (lane >> 3);
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    const int rs = min(r, rows - 1);
    const uint32_t arow = a_rows ? (uint32_t)a_rows[c.m0 + rs] : (uint32_t)rs;
    a_src[t] = arow * (uint32_t)p.lda + (uint32_t)(lc * 16);
  }
  char* const a_dst = smem + wave * 1024;
  // ---- activation scales: each stage's 4 scale bytes of every tile row go to
  // an LDS area beside the code slot by one 4-byte direct load per wavefront
  // (lane l of wavefront w: tile row 64 w + l, clamped); lane l then reads
  // the dword of row 32 i + l % 32 for row block i and shifts it right by
  // 8 (l / 32): byte 0 is then the scale of block l / 32 of substep 0, and
  // byte 2 that of block 2 + l / 32 (substep 1), as the MFMA takes them
  const uint8_t* __restrict__ xs = p.a_scales;
  uint32_t s_off;
  {
    const int rr = min(64 * wave + lane, rows - 1);
    const uint32_t srow = a_rows ? (uint32_t)a_rows[c.m0 + rr] : (uint32_t)(c.m0 + rr);
    s_off = srow * (uint32_t)p.a_scale_ld;
  }
  char* const s_dst = smem + F8_DEPTH * F8_SLOT + wave * 256;  // + slot * 1024
  const int s_rd = F8_DEPTH * F8_SLOT + (lane & 31) * 4;        // + slot * 1024 + 128 i
  const uint32_t s_sh = 8u * (uint32_t)(lane >> 5);

  // ---- this wavefront's quarter of each weight block, and its scale dword
  const char* B_pan = static_cast<const char*>(p.B0) +
                      ((int64_t)c.g * n_tiles + c.nt) * (int64_t)nk * F8_BLOCK;
  const uint32_t b_off = (uint32_t)(wave * F8_QUARTER + lane * 16);
  const uint32_t bs_off = (uint32_t)(F8_DATA + wave * 256 + lane * 4);

  // ---- fragment reads: lane l, substep ks: row l % 32, 16-byte chunks
  // 4 ks + l / 32 (scale block 2 ks) and 4 ks + 2 + l / 32 (block 2 ks + 1)
  const int swz = ((lane & 31) >> 1) & 7;
  int fr[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      fr[ks][hf] = (lane & 31) * F8_BKS + (((4 * ks + 2 * hf + (lane >> 5)) ^ swz) * 16);

  f32x16_t acc[NA][2];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  i32x8_t fa[NA];
  i32x8_t fb[F8_DEPTH][4];  // [set][2 ks + j]: the two 1 KB pieces of (ks, j)
  uint32_t bsc[F8_DEPTH];
  // this stage's activation scale dwords as read (one per row block); the
  // lane's byte shift is applied at the MFMA, so that no wait for the read
  // lands right behind it
  uint32_t asc[NA];

#define F8_FRAG(dst, slot, ks, i)                                                     \
  {                                                                                   \
    (dst).lo = *reinterpret_cast<const i32x4_t*>(smem + (slot) * F8_SLOT + fr[ks][0] + (i) * 4096); \
    (dst).hi = *reinterpret_cast<const i32x4_t*>(smem + (slot) * F8_SLOT + fr[ks][1] + (i) * 4096); \
  }
  // code piece q (1 KB) of stage kt into set u
#define F8_PIECE(kt, u, q)                                                            \
  {                                                                                   \
    const i32x4_t v_ = *reinterpret_cast<const i32x4_t*>(                             \
        B_pan + (int64_t)(kt) * F8_BLOCK + b_off + (q) * 1024);                       \
    if ((q) & 1) fb[u][(q) >> 1].hi = v_; else fb[u][(q) >> 1].lo = v_;               \
  }
#define F8_SDMA(kt, u)                                                                \
  {                                                                                   \
    const __amdgpu_buffer_rsrc_t r_ = __builtin_amdgcn_make_buffer_rsrc(              \
        (void*)(xs + 4 * (int64_t)(kt)), 0, 0x7fffffff, 0x00020000);                  \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, (lds_void_t*)(s_dst + (u) * 1024), 4, \
                                             s_off, 0, 0, 0);                         \
  }
#define F8_SCALE(slot, i) (*reinterpret_cast<const uint32_t*>(smem + s_rd + (slot) * 1024 + (i) * 128))
#define F8_DMA(kt, u, t)                                                              \
  {                                                                                   \
    const __amdgpu_buffer_rsrc_t r_ = __builtin_amdgcn_make_buffer_rsrc(              \
        (void*)(A_tile + (int64_t)(kt) * F8_BKS), 0, 0x7fffffff, 0x00020000);         \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(                                         \
        r_, (lds_void_t*)(a_dst + (u) * F8_SLOT + (t) * 4096), 16, a_src[t], 0, 0, 0); \
  }
  // every load of stage kt into set / slot u: 8 code pieces, the weight scale
  // dword (F8_WLOADS register loads), NA activation rows, the activation scales
#define F8_LOAD_STAGE(kt, u)                                                          \
  {                                                                                   \
    const char* b_ = B_pan + (int64_t)(kt) * F8_BLOCK;                                \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) F8_PIECE(kt, u, q);                 \
    bsc[u] = *reinterpret_cast<const uint32_t*>(b_ + bs_off);                         \
    _Pragma("unroll") for (int t = 0; t < NA; ++t) F8_DMA(kt, u, t);                  \
    F8_SDMA(kt, u);                                                                   \
  }
  // One substep ks of set u.  For each row block g: its two MFMAs (gate and
  // up column blocks), then, when NEXT, the LDS read of block g's fragment
  // for substep nks of slot nu (the register is free once both MFMAs have
  // read it) and, when nks is 0 (a new stage), of block g's scale dword, then
  // block g's share of the loads of stage KN into set NU: REFILL 1 the weight
  // code pieces and scale dword, REFILL 2 the activation rows and scales.  A
  // scheduling fence after each group keeps this order.
#define F8_SUB(ks, u, NEXT, nu, nks, REFILL, KN, NU)                                  \
  _Pragma("unroll") for (int g_ = 0; g_ < NA; ++g_) {                                 \
    const uint32_t sa_ = asc[g_] >> s_sh;                                             \
    acc[g_][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                     \
        fa[g_], fb[u][2 * (ks)], acc[g_][0], 0, 0, 2 * (ks),                          \
        (int)sa_, 2 * (ks), (int)bsc[u]);                                             \
    acc[g_][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                     \
        fa[g_], fb[u][2 * (ks) + 1], acc[g_][1], 0, 0,                                \
        2 * (ks), (int)sa_, 2 * (ks) + 1, (int)bsc[u]);                               \
    if (NEXT) F8_FRAG(fa[g_], nu, nks, g_);                                           \
    if ((NEXT) && (nks) == 0) asc[g_] = F8_SCALE(nu, g_);                             \
    if ((REFILL) == 1) {                                                              \
      const char* b_ = B_pan + (int64_t)(KN) * F8_BLOCK;                              \
      _Pragma("unroll") for (int q = (g_ * 8) / NA; q < ((g_ + 1) * 8) / NA; ++q)     \
          F8_PIECE(KN, NU, q);                                                        \
      if (g_ == 0) bsc[NU] = *reinterpret_cast<const uint32_t*>(b_ + bs_off);         \
    } else if ((REFILL) == 2) {                                                       \
      F8_DMA(KN, NU, g_);                                                             \
      if (g_ == NA - 1) F8_SDMA(KN, NU);                                              \
    }                                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                \
  }
  // Stage kt uses set / slot u = kt % F8_DEPTH and refills the set and slot of
  // stage kt-1 (every wavefront finished reading that slot before the last
  // barrier) with stage kt+F8_DIST: the weights in substep 0, which also reads
  // the substep-1 fragments, the activations in substep 1, so that each
  // substep's MFMAs have loads between them (the down GEMM runs 4-7% faster
  // than with all loads in substep 0).  Between the two the wavefront waits
  // for its loads of stage kt+1 (they complete in issue order; only the
  // F8_WLOADS weight loads of this stage's refill are newer) and meets the
  // others; substep 1 reads the first fragments of stage kt+1.  In the steady
  // loop a refill past the last stage repeats the last stage's addresses
  // (never read), so every stage keeps the same count of loads in flight.
  // The stages after the loop issue no loads and wait for all of them (a
  // dummy register load there would be dropped by the compiler as dead and
  // leave a count-based wait short).
#define F8_STAGE(kt, u, REFILL)                                                       \
  {                                                                                   \
    const int kn_ = min((kt) + F8_DIST, nk - 1);                                      \
    const int un_ = ((u) + F8_DIST) % F8_DEPTH;                                       \
    F8_SUB(0, u, true, u, 1, (REFILL) ? 1 : 0, kn_, un_);                             \
    ring_barrier<(REFILL) ? F8_WLOADS : 0>();                                         \
    __builtin_amdgcn_sched_barrier(0);                                                \
    F8_SUB(1, u, true, ((u) + 1) % F8_DEPTH, 0, (REFILL) ? 2 : 0, kn_, un_);          \
  }

  // prologue: stages 0 .. F8_DIST-1 (repeating the last stage where nk is
  // smaller); wait for stage 0 only
  // (fenced, so that the loads are issued stage by stage, as the wait counts
  // assume)
#pragma unroll
  for (int u = 0; u < F8_DIST; ++u) {
    F8_LOAD_STAGE(min(u, nk - 1), u);
    __builtin_amdgcn_sched_barrier(0);
  }
  ring_barrier<(F8_DIST - 1) * (10 + NA)>();
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    F8_FRAG(fa[i], 0, 0, i);
    asc[i] = F8_SCALE(0, i);
  }
  int kt = 0;
  for (; kt + F8_DEPTH <= nk; kt += F8_DEPTH) {
#pragma unroll
    for (int u = 0; u < F8_DEPTH; ++u) F8_STAGE(kt + u, u, true);
  }
#pragma unroll
  for (int u = 0; u + 1 < F8_DEPTH; ++u)
    if (kt + u < nk) F8_STAGE(kt + u, u, false);
#undef F8_FRAG
#undef F8_PIECE
#undef F8_DMA
#undef F8_SDMA
#undef F8_SCALE
#undef F8_LOAD_STAGE
#undef F8_SUB
#undef F8_STAGE
  ring_barrier<0>();  // every wavefront is done reading the ring before it is reused
  if constexpr (MODE == kSwiGLU_FP8) {
    store_fp8_h_tile<NA>(acc, smem, wave, lane, c, p);
    if constexpr (SAVE) store_act_tile<NA>(acc, smem, wave, lane, c, p);
  } else {
    store_bf16_tile<NA, MODE != kStoreBF16, SAVE>(acc, smem, wave, lane, c, p);
  }
}

// SAVE: also store the pre-activations to p.C2 (a separate instantiation);
// MODE: the epilogue (gate/up with h in bf16 or FP8, or the plain down
// projection)
template <bool SAVE, int MODE>
__global__ __launch_bounds__(64 * F8_WAVES, 1) void fp8_gemm_kernel(GemmProblem p, int n_tiles,
                                                                    int total_bound,
                                                                    int tile_rows) {
  constexpr bool SWIGLU = MODE != kStoreBF16;
  __shared__ __attribute__((aligned(16))) char smem[F8_DEPTH * (F8_SLOT + 1024)];
  const int logical =
      xcd_logical_tile(p.tile_prefix ? p.tile_prefix[p.G] * n_tiles : total_bound);
  if (logical < 0) return;
  TileCoord c;
  if (!map_tile<kPackedPanel, SWIGLU>(p, n_tiles, logical, tile_rows, c)) return;
  const int nb = (c.m_end - c.m0 + 31) / 32;  // at most F8_MAXRB: checked on the host
  if (nb <= 0) return;
  switch (nb) {
    case 1: run_fp8<1, SAVE, MODE>(p, c, n_tiles, smem); break;
    case 2: run_fp8<2, SAVE, MODE>(p, c, n_tiles, smem); break;
    case 3: run_fp8<3, SAVE, MODE>(p, c, n_tiles, smem); break;
    case 4: run_fp8<4, SAVE, MODE>(p, c, n_tiles, smem); break;
    case 5: run_fp8<5, SAVE, MODE>(p, c, n_tiles, smem); break;
    case 6: run_fp8<6, SAVE, MODE>(p, c, n_tiles, smem); break;
    case 7: run_fp8<7, SAVE, MODE>(p, c, n_tiles, smem); break;
    default: run_fp8<F8_MAXRB, SAVE, MODE>(p, c, n_tiles, smem); break;
  }
}

}  // namespace

int64_t fp8_packed_bytes(int64_t I, int64_t d) {
  return (I / (kPackedPanel / 2)) * (d / F8_BKS) * (int64_t)F8_BLOCK;
}

int64_t fp8_packed_down_bytes(int64_t d, int64_t I) {
  return ((d + kPackedPanel - 1) / kPackedPanel) * (I / F8_BKS) * (int64_t)F8_BLOCK;
}

hipError_t launch_quantize_mx(const bf16_t* x, uint8_t* xq, uint8_t* xs, int64_t rows, int64_t d,
                              hipStream_t s) {
  if (d % 32 != 0) return hipErrorInvalidValue;
  const int64_t nblk = rows * (d / 32);
  if (nblk == 0) return hipSuccess;
  const int64_t grid = (nblk + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, xq, xs, nblk);
  return hipGetLastError();
}

hipError_t launch_pack_weights_fp8(const bf16_t* wg, const bf16_t* wu, uint8_t* out, int groups,
                                   int I, int d, hipStream_t s) {
  if (d % F8_BKS != 0 || I % (kPackedPanel / 2) != 0) return hipErrorInvalidValue;
  const int n_panels = I / (kPackedPanel / 2);
  const int64_t blocks = (int64_t)groups * n_panels * (d / F8_BKS);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, wg, wu, out, I, d,
                     n_panels);
  return hipGetLastError();
}

hipError_t launch_pack_down_fp8(const bf16_t* wd, uint8_t* out, int groups, int d, int I,
                                hipStream_t s) {
  if (I % F8_BKS != 0) return hipErrorInvalidValue;
  const int n_panels = (d + kPackedPanel - 1) / kPackedPanel;
  const int64_t blocks = (int64_t)groups * n_panels * (I / F8_BKS);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, wd, nullptr, out,
                     d, I, n_panels);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const GemmProblem& p, int epilogue, int tile_rows, int64_t max_rows,
                           hipStream_t s) {
  if (p.K < F8_BKS || p.K % F8_BKS != 0 || !p.a_scales || p.a_scale_ld * 32 != p.K)
    return hipErrorInvalidValue;
  if (tile_rows < 32 || tile_rows > 32 * F8_MAXRB || tile_rows % 32 != 0)
    return hipErrorInvalidValue;
  if (epilogue != kSwiGLU_BF16 && epilogue != kSwiGLU_BF16_ACT && epilogue != kStoreBF16 &&
      epilogue != kSwiGLU_FP8)
    return hipErrorInvalidValue;
  const bool swiglu = epilogue != kStoreBF16;
  if (epilogue != kSwiGLU_FP8 && (epilogue == kSwiGLU_BF16_ACT) != (p.C2 != nullptr))
    return hipErrorInvalidValue;
  if (epilogue == kSwiGLU_FP8 && (!p.c_scales || p.c_scale_ld * 32 != p.Nout))
    return hipErrorInvalidValue;
  if (swiglu ? p.Nout % (kPackedPanel / 2) != 0 : p.Nout % 64 != 0) return hipErrorInvalidValue;
  const int n_tiles = swiglu ? p.Nout / (kPackedPanel / 2)
                             : (p.Nout + kPackedPanel - 1) / kPackedPanel;
  int64_t mt_bound;
  if (p.tile_prefix) {
    mt_bound = (max_rows + (int64_t)p.G * (tile_rows - 1)) / tile_rows;
    if (mt_bound > max_rows) mt_bound = max_rows;
  } else {
    mt_bound = (p.M + tile_rows - 1) / tile_rows;
  }
  int64_t blocks = mt_bound * n_tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0) return hipErrorInvalidValue;
  blocks = (blocks + 7) / 8 * 8;
  const dim3 grid((unsigned)blocks), block(64 * F8_WAVES);
  const int total = (int)(mt_bound * n_tiles);
  if (!swiglu)
    hipLaunchKernelGGL((fp8_gemm_kernel<false, kStoreBF16>), grid, block, 0, s, p, n_tiles,
                       total, tile_rows);
  else if (epilogue == kSwiGLU_FP8 && p.C2)
    hipLaunchKernelGGL((fp8_gemm_kernel<true, kSwiGLU_FP8>), grid, block, 0, s, p, n_tiles,
                       total, tile_rows);
  else if (epilogue == kSwiGLU_FP8)
    hipLaunchKernelGGL((fp8_gemm_kernel<false, kSwiGLU_FP8>), grid, block, 0, s, p, n_tiles,
                       total, tile_rows);
  else if (p.C2)
    hipLaunchKernelGGL((fp8_gemm_kernel<true, kSwiGLU_BF16>), grid, block, 0, s, p, n_tiles,
                       total, tile_rows);
  else
    hipLaunchKernelGGL((fp8_gemm_kernel<false, kSwiGLU_BF16>), grid, block, 0, s, p, n_tiles,
                       total, tile_rows);
  return hipGetLastError();
}

}  // namespace moezc
