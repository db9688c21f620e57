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
// each weight panel is streamed from HBM once while it is used 256 times.
// Eight wavefronts in a 2 x 4 grid each own up to four 32-row blocks by two
// 32-column MFMA blocks (128 fp32 accumulators).  An expert with more rows
// than the tile is split into equal parts whose workgroups run side by side
// on one XCD and so share the weight panel in L2.  Row blocks of 32 that hold
// no rows are skipped by the wavefront that owns them (the K loop is
// instantiated per count of live row blocks).  Decode shape (a few rows per
// expert): 32-row tiles, one row block per wavefront.
//
// Tile order: expert, then weight panel, then row part.  Consecutive
// workgroups land on different XCDs (round robin), so each XCD is handed a
// contiguous range of this order: the workgroups of one expert run together
// on one XCD and share its L2 for the expert's activation rows.
//
// Pipeline: stages of 64 k move from global memory straight into LDS rings
// (direct loads, no register staging): two activation slots and up to three
// weight slots, so up to two weight stages stream from HBM while the MFMAs
// of the current stage run.
#include "gemm_tile.hpp"

namespace moezc {

namespace {

// Stage geometry of the LDS ring: BKS = 64 k per stage, rows of 128 bytes
// (eight 16-byte chunks, one full cache line per row) with no padding; chunk c
// of row r is stored at position c ^ ((r >> 1) & 7), which makes the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks.  Global data
// reaches LDS by direct loads (global_load_lds_dwordx4: lane l's 16 bytes
// land at base + 16 l), so no registers stage it.  Whole-line row pieces
// matter: half-line (64-byte) pieces stream several times slower from L2.
constexpr int BKS = 64;
constexpr int ROWB = BKS * 2;  // bytes per LDS row
constexpr int CPR = ROWB / 16; // 16-byte chunks per row
constexpr int RPI = 64 / CPR;  // rows filled by one direct load instruction
constexpr int LDS_MAX = 160 * 1024;

// Two ring slots hold activation (A) stages; the weight (B) ring is as deep
// as the LDS allows (at most three slots), so weights streamed from HBM get
// two stages in flight where the tile leaves room.
template <int BM, int BN>
constexpr int b_slots() {
  return (2 * BM + 3 * BN) * ROWB <= LDS_MAX ? 3 : 2;
}

// LDS bytes of one workgroup: the rings, or the bf16 output staging of the
// epilogue (one padded 32-row block per wavefront), whichever is larger.
template <int BM, int BN, int WAVES_M, int WAVES_N>
constexpr int smem_bytes() {
  constexpr int ring = (2 * BM + b_slots<BM, BN>() * BN) * ROWB;
  constexpr int epi = WAVES_M * WAVES_N * 32 * (BN / WAVES_N + 8) * 2;
  return ring > epi ? ring : epi;
}

template <int EPI, int BM, int BN, int WAVES_M, int WAVES_N, int NA>
__device__ __forceinline__ void run_tile(const GemmProblem& p, const TileCoord& c,
                                         char* __restrict__ smem) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WTN = BN / WAVES_N;
  constexpr int CB = WTN / 32;
  constexpr bool SWIGLU = is_swiglu_bf16(EPI);
  constexpr int HB = CB / 2;
  constexpr int NAc = NA > 0 ? NA : 1;
  constexpr int SLOT_A = BM * ROWB, SLOT_B = BN * ROWB;  // bytes per stage
  constexpr int NSA = 2, NSB = b_slots<BM, BN>();         // ring slots
  char* const ringA = smem;
  char* const ringB = smem + NSA * SLOT_A;
  constexpr int IA = BM / RPI, IB = BN / RPI;  // direct loads per stage
  constexpr int DA = (IA + NW - 1) / NW;      // per wavefront (a few may repeat: same bytes)
  constexpr int DB = (IB + NW - 1) / NW;
  constexpr int DPS = DA + DB;                // direct loads per wavefront per stage
  constexpr int KS = BKS / 16;                // MFMA substeps per stage

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  const bf16_t* __restrict__ B0 =
      static_cast<const bf16_t*>(p.B0) + (int64_t)c.g * p.b_group_stride;
  const bf16_t* __restrict__ B1 =
      SWIGLU ? static_cast<const bf16_t*>(p.B1) + (int64_t)c.g * p.b_group_stride : nullptr;
  // gathered A (a_rows): offsets are taken from the start of A
  const char* A_tile = reinterpret_cast<const char*>(A + (p.a_rows ? 0 : (int64_t)c.m0 * p.lda));
  const char* B_gate = reinterpret_cast<const char*>(B0 + (int64_t)c.n0 * p.ldb);
  const char* B_up = SWIGLU ? reinterpret_cast<const char*>(B1 + (int64_t)c.n0 * p.ldb) : nullptr;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---- direct-load sources: instruction t of this wavefront covers tile rows
  // [RPI j, RPI j + RPI) with j = (wave + NW t) mod IA; lane l fills chunk
  // position l % CPR of row RPI j + l / CPR, i.e. logical chunk
  // (l % CPR) ^ swizzle(row).  Rows past the end are clamped to a valid row
  // (their products only reach accumulator rows that are never stored).
  uint32_t a_src[DA], b_src[DB];
  int a_dst[DA], b_dst[DB];
  bool b_up[DB];
#pragma unroll
  for (int t = 0; t < DA; ++t) {
    const int j = (wave + NW * t) % IA;
    const int r = RPI * j + lane / CPR;
    const int lc = (lane % CPR) ^ ((r >> 1) & 7);
    const int rr = min(r, c.m_end - 1 - c.m0);
    const uint32_t arow = p.a_rows ? (uint32_t)p.a_rows[c.m0 + rr] : (uint32_t)rr;
    a_src[t] = arow * (uint32_t)(p.lda * 2) + (uint32_t)(lc * 16);
    a_dst[t] = RPI * j * ROWB;
  }
#pragma unroll
  for (int t = 0; t < DB; ++t) {
    const int j = (wave + NW * t) % IB;
    const int r = RPI * j + lane / CPR;
    const int lc = (lane % CPR) ^ ((r >> 1) & 7);
    int n;
    if (SWIGLU) {
      b_up[t] = r >= BN / 2;
      n = b_up[t] ? r - BN / 2 : r;
    } else {
      b_up[t] = false;
      n = min(c.n0 + r, p.Nout - 1) - c.n0;
    }
    b_src[t] = (uint32_t)(n * (int)p.ldb * 2 + lc * 16);
    b_dst[t] = RPI * j * ROWB;
  }

  // ---- fragment addresses (bytes within a slot) -------------------------
  // lane l reads row (base + l % 32), logical chunk 2 ks + l / 32; bases are
  // multiples of 32 rows, so the swizzle depends on the lane only
  const int swz = ((lane & 31) >> 1) & 7;
  int fr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) fr[ks] = (lane & 31) * ROWB + ((2 * ks + (lane >> 5)) ^ swz) * 16;
  int a_row[NAc], b_row[CB];
#pragma unroll
  for (int i = 0; i < NAc; ++i) a_row[i] = (i * WAVES_M + wm) * 32 * ROWB;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int br = SWIGLU ? ((j < HB) ? wn * HB * 32 + j * 32 : BN / 2 + wn * HB * 32 + (j - HB) * 32)
                          : wn * WTN + j * 32;
    b_row[j] = br * ROWB;
  }

  f32x16_t acc[NAc][CB];
#pragma unroll
  for (int i = 0; i < NAc; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  bf16x8_t fa[2][NAc], fb[2][CB];

  // issue the direct loads of stage kt: activations into A slot sa, weights
  // into B slot sb
#define MOEZC_DMA_A(kt, sa)                                                          \
  {                                                                                  \
    const char* a_k = A_tile + (((kt) * BKS) % p.a_kwrap) * 2;                       \
    char* sl_ = ringA + (sa) * SLOT_A;                                               \
    _Pragma("unroll") for (int t = 0; t < DA; ++t) __builtin_amdgcn_global_load_lds( \
        (glb_void_t*)(a_k + a_src[t]), (lds_void_t*)(sl_ + a_dst[t]), 16, 0, 0);     \
  }
#define MOEZC_DMA_B(kt, sb)                                                          \
  {                                                                                  \
    const char* bg_k = B_gate + (kt) * BKS * 2;                                      \
    const char* bu_k = SWIGLU ? B_up + (kt) * BKS * 2 : bg_k;                        \
    char* sl_ = ringB + (sb) * SLOT_B;                                               \
    _Pragma("unroll") for (int t = 0; t < DB; ++t) __builtin_amdgcn_global_load_lds( \
        (glb_void_t*)((b_up[t] ? bu_k : bg_k) + b_src[t]),                           \
        (lds_void_t*)(sl_ + b_dst[t]), 16, 0, 0);                                    \
  }
  // fragments of substep ks of the stage in A slot sa / B slot sb
#define MOEZC_LOADF(fs, sa, sb, ks)                                                  \
  {                                                                                  \
    const char* la_ = ringA + (sa) * SLOT_A;                                         \
    const char* lb_ = ringB + (sb) * SLOT_B;                                         \
    const int fo_ = fr[ks];                                                          \
    _Pragma("unroll") for (int i = 0; i < NAc; ++i) fa[fs][i] =                      \
        *reinterpret_cast<const bf16x8_t*>(la_ + a_row[i] + fo_);                    \
    _Pragma("unroll") for (int j = 0; j < CB; ++j) fb[fs][j] =                       \
        *reinterpret_cast<const bf16x8_t*>(lb_ + b_row[j] + fo_);                    \
  }
#define MOEZC_MMA(fs)                                                                \
  {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < NAc; ++i)                                  \
        _Pragma("unroll") for (int j = 0; j < CB; ++j) acc[i][j] =                   \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fs][i], fb[fs][j], acc[i][j], 0, 0, 0); \
  }
  // Stage kt lives in A slot kt % NSA and B slot kt % NSB.  Its first-substep
  // fragments were read at the end of the previous stage.  Substep ks reads
  // the fragments of ks+1, then runs its MFMAs.  Before the last substep the
  // wavefront waits until its own loads of stage kt+1 have landed and meets
  // the others at the barrier: stage kt+1 is then complete in LDS and every
  // wavefront is done with stage kt's slots, which are refilled (A with stage
  // kt+NSA, then B with stage kt+NSB; loads of a stage are issued in that
  // order, so with a three-slot B ring the weights of stage kt+2 - issued
  // after the activations of kt+1 - may stay in flight across the wait).  The
  // last substep's MFMAs then cover the first fragment reads of kt+1.
#define MOEZC_STAGE(kt, sa, sb)                                                      \
  {                                                                                  \
    _Pragma("unroll") for (int ks = 0; ks + 1 < KS; ++ks) {                          \
      if (NA > 0) {                                                                  \
        MOEZC_LOADF((ks + 1) & 1, sa, sb, ks + 1);                                   \
        __builtin_amdgcn_sched_barrier(0);                                           \
        MOEZC_MMA(ks & 1);                                                           \
        __builtin_amdgcn_sched_barrier(0);                                           \
      }                                                                              \
    }                                                                                \
    if (NSB > NSA && (kt) + 2 < nk) ring_barrier<(NSB > NSA ? DB : 0)>();            \
    else ring_barrier<0>();                                                          \
    if ((kt) + NSA < nk) MOEZC_DMA_A((kt) + NSA, sa);                                \
    if ((kt) + NSB < nk) MOEZC_DMA_B((kt) + NSB, sb);                                \
    if (NA > 0) {                                                                    \
      if ((kt) + 1 < nk) MOEZC_LOADF(0, ((sa) + 1) % NSA, ((sb) + 1) % NSB, 0);      \
      __builtin_amdgcn_sched_barrier(0);                                             \
      MOEZC_MMA((KS - 1) & 1);                                                       \
      __builtin_amdgcn_sched_barrier(0);                                             \
    }                                                                                \
  }

  static_assert(KS % 2 == 0, "fragment slots alternate");
  static_assert(NSA == 2 && (NSB == 2 || NSB == 3), "ring waits are written for these depths");
  const int nk = p.K / BKS;
  // prologue, in issue order A(0) B(0) A(1) B(1) [B(2)]
  MOEZC_DMA_A(0, 0);
  MOEZC_DMA_B(0, 0);
  if (nk > 1) {
    MOEZC_DMA_A(1, 1);
    MOEZC_DMA_B(1, 1);
  }
  if (NSB == 3 && nk > 2) MOEZC_DMA_B(2, 2);
  // stage 0 landed; everything issued after it may stay in flight
  if (NSB == 3 && nk > 2) ring_barrier<DA + 2 * DB>();
  else if (nk > 1) ring_barrier<DA + DB>();
  else ring_barrier<0>();
  if (NA > 0) MOEZC_LOADF(0, 0, 0, 0);
  // unrolled over lcm(NSA, NSB) stages so every slot index is a constant
  constexpr int UNR = (NSB == 3) ? 6 : 2;
  for (int kt = 0; kt < nk; kt += UNR) {
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (kt + u < nk) MOEZC_STAGE(kt + u, u % NSA, u % NSB);
  }
#undef MOEZC_DMA_A
#undef MOEZC_DMA_B
#undef MOEZC_LOADF
#undef MOEZC_MMA
#undef MOEZC_STAGE
  if (NA == 0) return;
  ring_barrier<0>();  // every wavefront is done reading the ring before it is reused

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
  // bf16 outputs go through a wavefront-private LDS tile, one 32-row block at
  // a time, so that global stores are whole 16-byte row pieces (every
  // wavefront passed the barrier above, so the ring is free)
  constexpr int OC = SWIGLU ? HB * 32 : CB * 32;  // output columns of this wavefront
  constexpr int OS = OC + 8;                      // padded LDS row (elements)
  bf16_t* ot = reinterpret_cast<bf16_t*>(smem) + wave * (32 * OS);
  const int gcol0 = c.n0 + (SWIGLU ? wn * HB * 32 : wn * WTN);
  bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.C);
  constexpr int CH = OC / 8;  // 16-byte pieces per row
#pragma unroll
  for (int i = 0; i < NAc; ++i) {
#pragma unroll
    for (int j = 0; j < OC / 32; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + lrow4 + (v & 3);
        float val;
        if (SWIGLU) {
          val = swiglu_fast(acc[i][j][v], acc[i][j + HB][v]);
        } else {
          val = acc[i][j][v];
        }
        ot[r * OS + j * 32 + lcol] = f32_to_bf16(val);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes landed
    __builtin_amdgcn_wave_barrier();
    const int grow0 = c.m0 + (i * WAVES_M + wm) * 32;
#pragma unroll
    for (int q = lane; q < 32 * CH; q += 64) {
      const int r = q / CH, ch = q - r * CH;
      const int grow = grow0 + r;
      const int gcol = gcol0 + ch * 8;
      if (grow < c.m_end && gcol < p.Nout)
        *reinterpret_cast<u32x4_t*>(&Cout[(int64_t)grow * p.ldc + gcol]) =
            *reinterpret_cast<const u32x4_t*>(&ot[r * OS + ch * 8]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block overwrites
    __builtin_amdgcn_wave_barrier();
    if constexpr (EPI == kSwiGLU_BF16_ACT) {  // pre-activations: gate to C2[:, n], up to C2[:, Nout + n]
      bf16_t* __restrict__ C2 = static_cast<bf16_t*>(p.C2);
#pragma unroll
      for (int part = 0; part < 2; ++part) {
#pragma unroll
        for (int j = 0; j < OC / 32; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            ot[(8 * (v >> 2) + lrow4 + (v & 3)) * OS + j * 32 + lcol] =
                f32_to_bf16(acc[i][j + part * (SWIGLU ? HB : 0)][v]);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = lane; q < 32 * CH; q += 64) {
          const int r = q / CH, ch = q - r * CH;
          const int grow = grow0 + r;
          const int gcol = gcol0 + ch * 8;
          if (grow < c.m_end && gcol < p.Nout)
            *reinterpret_cast<u32x4_t*>(&C2[(int64_t)grow * p.ldc2 + part * p.Nout + gcol]) =
                *reinterpret_cast<const u32x4_t*>(&ot[r * OS + ch * 8]);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
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
  constexpr bool SWIGLU = is_swiglu_bf16(EPI);
  static_assert((BM / WAVES_M) % 32 == 0 && (BN / WAVES_N) % 32 == 0, "wave tile");
  static_assert(!SWIGLU || ((BN / WAVES_N) / 32) % 2 == 0, "SwiGLU needs gate and up blocks");
  // one LDS block: the ring of stages, reused by the epilogue
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<BM, BN, WAVES_M, WAVES_N>()];

  const int logical = xcd_logical_tile(p.tile_prefix ? p.tile_prefix[p.G] * n_tiles : total_bound);
  if (logical < 0) return;
  TileCoord c;
  if (!map_tile<BN, SWIGLU>(p, n_tiles, logical, BM, c)) return;

  // live 32-row blocks of the tile, and how many of them this wavefront owns
  // (row block i of wavefront row wm is tile block i * WAVES_M + wm)
  const int wm = (threadIdx.x >> 6) / WAVES_N;
  const int nb = (c.m_end - c.m0 + 31) / 32;
  int na = (nb - wm + WAVES_M - 1) / WAVES_M;
  na = na < 0 ? 0 : (na > RB ? RB : na);
  switch (na) {
    case 0: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, 0>(p, c, smem); break;
    case 1: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 1 ? 1 : 0)>(p, c, smem); break;
    case 2: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 2 ? 2 : 0)>(p, c, smem); break;
    case 3: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 3 ? 3 : 0)>(p, c, smem); break;
    default: run_tile<EPI, BM, BN, WAVES_M, WAVES_N, (RB >= 4 ? 4 : 0)>(p, c, smem); break;
  }
}

template <int EPI, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmProblem& p, int64_t max_rows, hipStream_t s) {
  static_assert(BM / WM / 32 <= 4, "at most four row blocks per wavefront");
  const int n_tiles = is_swiglu_bf16(EPI) ? p.Nout / (BN / 2) : (p.Nout + BN - 1) / BN;
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
    case kSwiGLU_BF16_ACT:
      if (!p.C2) return hipErrorInvalidValue;
      return launch_cfg<kSwiGLU_BF16_ACT, BM, BN, WM, WN>(p, max_rows, s);
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
  if (p.K % BKS != 0 || p.a_kwrap % BKS != 0) return hipErrorInvalidValue;
  if (is_swiglu_bf16(epilogue) && tile_rows != 32 && p.Nout % 128 != 0) return hipErrorInvalidValue;
  if (tile_rows == 256) return launch_epi<256, 256, 2, 4>(p, epilogue, max_rows, s);
  if (tile_rows == 128) return launch_epi<128, 256, 2, 4>(p, epilogue, max_rows, s);
  if (tile_rows == 32) return launch_epi<32, 256, 1, 4>(p, epilogue, max_rows, s);
  return hipErrorInvalidValue;
}

}  // namespace moezc
