// Matrix-core GEMM with K-major operands for the backward pass of the MoE layer (declarations
// and the layout contract in gemm_kt.hpp).
//
// Tile 128 x 192 on 4 waves (2 x 2, 64 x 96 per wave, v_mfma_f32_32x32x16_bf16), two workgroups
// per CU, two LDS stages of 64 k. Both operand layouts are staged by buffer_load ... lds (global
// to LDS, 1 KB per instruction, lane l landing at byte 16 l):
//   K-contiguous rows (A[m][k]): 128 bytes of k per row and stage, 16-byte chunks XOR-swizzled by
//     (row / 2) % 8, fragments read with ds_read_b128 (as in the forward GEMM);
//   K-major rows (A[k][m], B[k][n]): 64 rows of k per stage, each holding the tile's 128 or 192
//     contiguous columns, chunks XOR-swizzled by row (swz_km) so that a transposing read meets
//     every LDS bank at most as often as its size requires. A fragment lane needs 8 consecutive k of
//     one column; gfx950's transposing read ds_read_b64_tr_b16 provides them. Within each group
//     of 16 lanes, lane j of the group reads 8 bytes at row k0 + j / 4, column c0 + 4 (j % 4),
//     and receives column c0 + j at rows k0 .. k0 + 3 (the lane layout was checked on the chip);
//     two such reads give the 8 k values.
// Rows of k beyond a K window (the last step of a group) are skipped by the loads and zeroed in
// LDS; columns beyond M or N read a valid column instead (their outputs are never stored).
#include <algorithm>

#include "common.hpp"
#include "gemm_kt.hpp"

namespace moe {
namespace {

constexpr int BM = 128, BN = 192, NW = 4, WGN = 2, WM = 64, WN = 96, MB = 2, NB = 3;
constexpr int EPW = WN + 4;             // epilogue strip row (floats)
constexpr int kBand = 4;                // N-tiles per band of a K-grouped launch's tile order
constexpr int KS = 64;                  // k per stage
constexpr int SA = BM * KS * 2, SB = BN * KS * 2;
constexpr int STAGE = SA + SB;          // 40 KB; two stages

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(uint32_t)n, 0x00020000);
}

__device__ __forceinline__ int swz_mk(int row) { return (row >> 1) & 7; }
// K-major stages: one transposing read of a 32-lane half-wave takes 32 contiguous bytes of each
// of 4 consecutive k rows (k0 .. k0 + 3, k0 a multiple of 4) for two 16-lane groups, 4 chunks
// of 16 bytes per row. The swizzle puts those 4 rows on disjoint banks: rows of 256 bytes (A,
// 128 columns) all start on bank 0, so row k moves its chunks by (k % 4) groups of four; rows of
// 384 bytes (B, 192 columns) alternate between banks 0 and 32, so rows 2 and 3 of each four
// move by one group (chunk ^ 4 stays inside a row of 24 chunks). An XOR keeps it a bijection on
// each row's chunks.
template <int PITCH>
__device__ __forceinline__ int swz_km(int k) {
  static_assert(PITCH == 256 || PITCH == 384, "K-major rows are 128 or 192 bf16 columns");
  return PITCH == 256 ? (k & 3) << 2 : ((k >> 1) & 1) << 2;
}

__device__ __forceinline__ void unpack8(const uint4 q, float* v) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFF);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

// Byte offset of element (k, col) of a K-major stage with PITCH bytes per row of k.
template <int PITCH>
__device__ __forceinline__ int km_addr(int k, int col) {
  return k * PITCH + (((col >> 3) ^ swz_km<PITCH>(k)) << 4) + ((col & 7) << 1);
}

// The 8 consecutive k (k0 .. k0 + 7 of this lane's 16-lane group) of one fragment column from a
// K-major stage: `col0` is the group's first column (a multiple of 16), `j` the lane in its group.
template <int PITCH>
__device__ __forceinline__ bf16x8_t km_frag(const uint8_t* st, int col0, int k0, int j) {
  typedef __attribute__((address_space(3))) v4i16_t lds_v4;
  const int col = col0 + 4 * (j & 3);
  const uint8_t* p0 = st + km_addr<PITCH>(k0 + (j >> 2), col);
  const uint8_t* p1 = st + km_addr<PITCH>(k0 + 4 + (j >> 2), col);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(const void*)p0);
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(const void*)p1);
  const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Tile of block b of a K-grouped launch; false when it has none. The group's K rows are
// [k0, k0 + kc).
//   Every die takes an equal, compact share of each group's tiles, the groups in launch order
// (heaviest first: their tiles cost most). Blocks d, d + 8, d + 16, ... run on die d; its share
// of a group is a contiguous run of the group's tiles numbered in bands of kBand N-tiles, N
// fastest, so the die's tiles have few A and B slabs between them and share them through its L2.
__device__ __forceinline__ bool kgrp_tile(const KtParams& p, int b, int& g, int& row0, int& rows,
                                          int& n0, int& k0, int& kc) {
  const int nN = cdiv(p.N, BN), nM = cdiv(p.M, BM);
  const int per = nM * nN, cs = cdiv(per, kXcds);
  const int d = b % kXcds, j = b / kXcds;
  const int slot = j / cs, q = d * cs + j % cs;
  if (slot >= p.G || q >= per) return false;
  g = p.korder ? p.korder[slot] : slot;
  const int band = q / (kBand * nM), within = q - band * kBand * nM;
  const int nb = min(kBand, nN - band * kBand);
  n0 = (band * kBand + within % nb) * BN;
  row0 = (within / nb) * BM;
  rows = min(BM, p.M - row0);
  k0 = p.kgrp[g];
  kc = p.kgrp[g + 1] - k0;
  return rows > 0;
}

// Blocks of a K-grouped launch: each die gets ceil(tiles per group / 8) per group.
inline int kgrp_blocks(const KtParams& p) {
  return p.G * kXcds * cdiv(cdiv(p.M, BM) * cdiv(p.N, BN), kXcds);
}

// Tile of this workgroup; false when it has none. kwin: the group's K rows [k0, k0 + kc).
__device__ __forceinline__ bool kt_tile(const KtParams& p, int& g, int& row0, int& rows, int& n0,
                                        int& k0, int& kc) {
  const int nN = cdiv(p.N, BN), nM = cdiv(p.M, BM);
  k0 = 0;
  kc = p.K;
  if (p.kgrp) return kgrp_tile(p, blockIdx.x, g, row0, rows, n0, k0, kc);
  const int L = xcd_logical_block(blockIdx.x, gridDim.x);
  if (p.mt_start) {
    const int total = p.mt_start[p.G] * nN;
    if (L >= total) return false;
    const int key = L / nN;
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.mt_start[mid] <= key) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int mt_g = p.mt_start[g + 1] - p.mt_start[g];
    const int local = L - p.mt_start[g] * nN;
    n0 = (local / mt_g) * BN;
    row0 = p.offs[g] + (local % mt_g) * BM;
    rows = min(BM, p.offs[g + 1] - row0);
    return rows > 0;
  }
  if (L >= nM * nN) return false;
  constexpr int GM = 8;
  const int first = (L / (GM * nN)) * GM;
  const int gm = min(GM, nM - first);
  const int within = L - first * nN;
  g = 0;
  row0 = (first + within % gm) * BM;
  n0 = (within / gm) * BN;
  rows = min(BM, p.M - row0);
  return rows > 0;
}

// One K-step of the 128 x 192 tile from the stage at As (A rows, then B rows at As + SA).
template <int TA>
__device__ __forceinline__ void kt_mma(const uint8_t* As, f32x16_t (&acc)[MB][NB], int lane,
                                       int wm, int wn) {
  const uint8_t* Bs = As + SA;
  const int lg = lane >> 4, lj = lane & 15;   // 16-lane group and lane in it (K-major reads)
  bf16x8_t a[2][MB], b[2][NB];
  auto rd = [&](int s, int buf) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if constexpr (TA) {
        a[buf][i] = km_frag<BM * 2>(As, wm * WM + i * 32 + 16 * (lg & 1), 16 * s + 8 * (lg >> 1), lj);
      } else {
        const int r = wm * WM + i * 32 + (lane & 31);
        const int ch = 2 * s + (lane >> 5);
        a[buf][i] = *(const bf16x8_t*)(As + r * 128 + ((ch ^ swz_mk(r)) << 4));
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      b[buf][j] = km_frag<BN * 2>(Bs, wn * WN + j * 32 + 16 * (lg & 1), 16 * s + 8 * (lg >> 1), lj);
  };
  rd(0, 0);
#pragma unroll
  for (int s = 0; s < KS / 16; ++s) {
    if (s < KS / 16 - 1) rd(s + 1, (s + 1) & 1);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][i], b[s & 1][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue (as in the forward GEMM): acc[i][j][r] is C[wm*WM + i*32 + (r/4)*8 + (lane/32)*4 +
// r%4][wn*WN + j*32 + lane%32]; 16-row strips go through this wave's LDS strip `ep` so each lane
// finishes CW consecutive columns of a row: 8 for bf16 outputs, 4 for fp32 (16 bytes either way,
// so that consecutive lanes store consecutive 16-byte chunks of a row). Cg: the group's output.
// NT: the output is a weight gradient (fp32, or bf16 on request), written once and not read
// again by this pass.
template <Elt OUT, Epi EPI, bool NT>
__device__ __forceinline__ void kt_store(const KtParams& p, const f32x16_t (&acc)[MB][NB],
                                         uint8_t* Cg, float* ep, int row0, int rows, int n0,
                                         int lane, int wm, int wn) {
  constexpr int CW = OUT == Elt::F32 ? 4 : 8;
  constexpr int CG = WN / CW, ITEMS = 16 * CG / 64;
  static_assert((16 * CG) % 64 == 0, "strip must split evenly over the wave");
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int srow = (rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3);
          ep[srow * EPW + j * 32 + (lane & 31)] = acc[i][j][8 * h + rr];
        }
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int item = it * 64 + lane;
        const int srow = item / CG, cg = item % CG;
        const int rl = wm * WM + i * 32 + h * 16 + srow;
        const int col = n0 + wn * WN + cg * CW;
        if (rl < rows && col < p.N) {  // N % 8 == 0: a group inside N ends inside it
          const int row = row0 + rl;
          const float4 lo = *(const float4*)(ep + srow * EPW + cg * CW);
          if constexpr (OUT == Elt::F32) {
            float* o = (float*)Cg + (int64_t)row * p.ldc + col;
            if constexpr (NT) {
              const f32x4_t v = {lo.x, lo.y, lo.z, lo.w};
              __builtin_nontemporal_store(v, (f32x4_t*)o);
            } else {
              *(float4*)o = lo;
            }
          } else {
            const float4 hi = *(const float4*)(ep + srow * EPW + cg * CW + 4);
            float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            if constexpr (EPI == Epi::DSqRelu) {  // d/da relu(a)^2 = 2 relu(a), relu(a) in C2
              float r[8];
              unpack8(*(const uint4*)((const uint16_t*)p.C2 + (int64_t)row * p.ldc + col), r);
#pragma unroll
              for (int q = 0; q < 8; ++q) v[q] *= 2.f * r[q];
            }
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
            uint16_t* o = (uint16_t*)Cg + (int64_t)row * p.ldc + col;
            if constexpr (NT) {
              typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
              const u32x4_t wv = {w[0], w[1], w[2], w[3]};
              __builtin_nontemporal_store(wv, (u32x4_t*)o);
            } else {
              *(uint4*)o = make_uint4(w[0], w[1], w[2], w[3]);
            }
          }
        }
      }
    }
  }
}

template <int TA, int TB, Elt OUT, Epi EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_kt_kernel(KtParams p) {
  static_assert(TB == 1, "B is K-major in every backward product");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  int g, row0, rows, n0, k0, kc;
  if (!kt_tile(p, g, row0, rows, n0, k0, kc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  constexpr int A_GRP = TA ? BM * KS * 2 / 1024 / NW : BM / (8 * NW);  // 1-KB loads per wave
  constexpr int B_GRP = BN * KS * 2 / 1024 / NW;
  constexpr int PA = BM * 2, PB = BN * 2;                             // K-major pitches

  // Operand resources. K-major operands start at the group's first k row and end after its
  // last, so a load of a row beyond the window reads nothing.
  const uint8_t* Bg = (const uint8_t*)p.B + (int64_t)g * p.b_gstride * 2;
  const bool gath = p.b_gather != nullptr;  // B rows gathered (K-grouped launches)
  const __amdgpu_buffer_rsrc_t rb =
      gath ? rsrc(p.B, (int64_t)p.b_rows * p.ldb * 2)
           : rsrc(Bg + (int64_t)k0 * p.ldb * 2, (int64_t)kc * p.ldb * 2);
  const __amdgpu_buffer_rsrc_t ra =
      TA ? rsrc((const uint8_t*)p.A + (int64_t)k0 * p.lda * 2, (int64_t)kc * p.lda * 2)
         : rsrc(p.A, (int64_t)p.a_rows * p.lda * 2);

  // Per-lane byte offsets (fixed over the K loop) and, for K-major loads, the lane's k row.
  uint32_t oa[A_GRP], ob[B_GRP];
  int ka[A_GRP], kb[B_GRP];
  const int lrow = lane >> 3, lpos = lane & 7;                        // K-contiguous mapping
  const int cofs = (lpos ^ swz_mk(wave * 8 + lrow)) << 4;
#pragma unroll
  for (int i = 0; i < A_GRP; ++i) {
    if constexpr (TA) {
      const int byte = (wave + NW * i) * 1024 + lane * 16;
      const int kr = byte / PA, slot = (byte % PA) >> 4;
      int col = row0 + ((slot ^ swz_km<PA>(kr)) << 3);
      col = min(col, p.M - 8);
      ka[i] = kr;
      oa[i] = (uint32_t)(kr * p.lda * 2 + col * 2);
    } else {  // padding rows of a partial tile take no access (their products are discarded)
      const int r = (wave + NW * i) * 8 + lrow;
      ka[i] = 0;
      oa[i] = r < rows ? (uint32_t)((int64_t)(row0 + r) * p.lda * 2) + cofs : 0xFFFFFFF0u;
    }
  }
#pragma unroll
  for (int i = 0; i < B_GRP; ++i) {
    const int byte = (wave + NW * i) * 1024 + lane * 16;
    const int kr = byte / PB, slot = (byte % PB) >> 4;
    int col = n0 + ((slot ^ swz_km<PB>(kr)) << 3);
    col = min(col, p.N - 8);
    kb[i] = kr;
    ob[i] = gath ? (uint32_t)(col * 2) : (uint32_t)(kr * p.ldb * 2 + col * 2);
  }
  // gathered B: the source rows of this lane's B loads for the step issued next (loaded one
  // step ahead; -1 past the window)
  int grow[B_GRP];
  auto fetch_rows = [&](int ks) {
    const int left = kc - ks * KS;
#pragma unroll
    for (int i = 0; i < B_GRP; ++i)
      grow[i] = kb[i] < left ? p.b_gather[k0 + ks * KS + kb[i]] : -1;
  };

  const int nk = cdiv(kc, KS);
  // Issue K-step ks into stage st. Dead lanes (k rows beyond the window; for a K-contiguous A,
  // chunks beyond K) take an offset outside the buffer and are zeroed by fix_tail.
  auto issue = [&](int ks, uint8_t* st) {
    const int left = kc - ks * KS;                 // k rows of this step inside the window
    const int sa = TA ? ks * KS * (int)p.lda * 2 : ks * KS * 2;
    const int sb = ks * KS * (int)p.ldb * 2;
#pragma unroll
    for (int i = 0; i < A_GRP; ++i) {
      const bool live = TA ? ka[i] < left : cofs < left * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(st + (wave + NW * i) * 1024), 16,
          (int)(live ? oa[i] : 0xFFFFFFF0u), sa, 0, 0);
    }
    if (gath) {
#pragma unroll
      for (int i = 0; i < B_GRP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(st + SA + (wave + NW * i) * 1024), 16,
            (int)(grow[i] >= 0 ? (uint32_t)grow[i] * (uint32_t)(p.ldb * 2) + ob[i] : 0xFFFFFFF0u),
            0, 0, 0);
      if (ks + 1 < nk) fetch_rows(ks + 1);
    } else {
#pragma unroll
      for (int i = 0; i < B_GRP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(st + SA + (wave + NW * i) * 1024), 16,
            (int)(kb[i] < left ? ob[i] : 0xFFFFFFF0u), sb, 0, 0);
    }
  };
  auto fix_tail = [&](int ks, uint8_t* st) {
    const int left = kc - ks * KS;
    if (left >= KS) return;  // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < A_GRP; ++i)
      if (TA ? ka[i] >= left : cofs >= left * 2)
        *(uint4*)(st + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < B_GRP; ++i)
      if (kb[i] >= left) *(uint4*)(st + SA + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
    __syncthreads();
  };

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](const uint8_t* As) { kt_mma<TA>(As, acc, lane, wm, wn); };

  // Two stages: K-step ks + 1 is loaded while K-step ks is multiplied.
  if (gath && nk > 0) fetch_rows(0);
  if (nk > 0) issue(0, smem);
  for (int ks = 0; ks < nk; ++ks) {
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
    uint8_t* cur = smem + (ks & 1) * STAGE;
    fix_tail(ks, cur);
    if (ks + 1 < nk) issue(ks + 1, smem + ((ks + 1) & 1) * STAGE);
    compute(cur);
  }
  __syncthreads();  // the epilogue reuses the stages

  uint8_t* Cg = (uint8_t*)p.C + (p.kgrp ? (int64_t)g * p.c_gstride * (OUT == Elt::F32 ? 4 : 2) : 0);
  if (p.kgrp)
    kt_store<OUT, EPI, true>(p, acc, Cg, (float*)smem + wave * 16 * EPW, row0, rows, n0, lane, wm, wn);
  else
    kt_store<OUT, EPI, false>(p, acc, Cg, (float*)smem + wave * 16 * EPW, row0, rows, n0, lane, wm, wn);
}

// Data gradients of a row-grouped launch (A K-contiguous over the pair rows, B each group's
// K-major weights), persistent like the forward's grouped GEMMs: two workgroups per CU walk the
// tiles of each die's contiguous range, and a tile's last K-step loads the next tile's first
// K-step into the stage it frees, so those loads overlap the last products and the epilogue.
template <Elt OUT, Epi EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_kt_rows_persist(KtParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  constexpr int A_GRP = BM / (8 * NW), B_GRP = BN * KS * 2 / 1024 / NW;
  constexpr int PB = BN * 2;  // K-major pitch of B
  const int nN = cdiv(p.N, BN);
  const int total = p.mt_start[p.G] * nN;
  const int d = blockIdx.x % kXcds, Qd = gridDim.x / kXcds;
  const int lo_t = d * cdiv(total, kXcds);
  const int hi_t = min(total, lo_t + cdiv(total, kXcds));
  int L = lo_t + (int)blockIdx.x / kXcds;
  if (L >= hi_t) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int lrow = lane >> 3, lpos = lane & 7;
  const int cofs = (lpos ^ swz_mk(wave * 8 + lrow)) << 4;
  const int K = p.K, nk = cdiv(K, KS);
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.A, (int64_t)p.a_rows * p.lda * 2);
  int kb[B_GRP];  // this lane's k row in each of its B loads (the same in every tile)
#pragma unroll
  for (int i = 0; i < B_GRP; ++i) kb[i] = ((wave + NW * i) * 1024 + lane * 16) / PB;

  // A tile: its group, rows and columns; its B resource (the group's weights) and this lane's
  // offsets (padding rows of a partial M-tile point out of range and take no access).
  __amdgpu_buffer_rsrc_t rb_c, rb_n;
  uint32_t oa_c[A_GRP], ob_c[B_GRP], oa_n[A_GRP], ob_n[B_GRP];
  int row0_c, rows_c, n0_c, row0_n = 0, rows_n = 0, n0_n = 0;
  auto setup = [&](int Lt, __amdgpu_buffer_rsrc_t& rbx, uint32_t* oax, uint32_t* obx, int& row0x,
                   int& rowsx, int& n0x) {
    const int key = Lt / nN;
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.mt_start[mid] <= key) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int mt_g = p.mt_start[g + 1] - p.mt_start[g];
    const int local = Lt - p.mt_start[g] * nN;
    n0x = (local / mt_g) * BN;
    row0x = p.offs[g] + (local % mt_g) * BM;
    rowsx = min(BM, p.offs[g + 1] - row0x);
    rbx = rsrc((const uint8_t*)p.B + (int64_t)g * p.b_gstride * 2, (int64_t)K * p.ldb * 2);
#pragma unroll
    for (int i = 0; i < A_GRP; ++i) {
      const int r = (wave + NW * i) * 8 + lrow;
      oax[i] = r < rowsx ? (uint32_t)((int64_t)(row0x + r) * p.lda * 2) + cofs : 0xFFFFFFF0u;
    }
#pragma unroll
    for (int i = 0; i < B_GRP; ++i) {
      const int slot = (((wave + NW * i) * 1024 + lane * 16) % PB) >> 4;
      const int col = min(n0x + ((slot ^ swz_km<PB>(kb[i])) << 3), p.N - 8);
      obx[i] = (uint32_t)(kb[i] * p.ldb * 2 + col * 2);
    }
  };
  // K-step ks of a tile into stage st; chunks beyond K (a partial last step) take an offset
  // outside the buffers and are zeroed after landing
  auto issue = [&](__amdgpu_buffer_rsrc_t rbx, const uint32_t* oax, const uint32_t* obx, int ks,
                   uint8_t* st) {
    const int left = K - ks * KS;
#pragma unroll
    for (int i = 0; i < A_GRP; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(st + (wave + NW * i) * 1024), 16,
          (int)(cofs < left * 2 ? oax[i] : 0xFFFFFFF0u), ks * KS * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < B_GRP; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rbx, (__attribute__((address_space(3))) void*)(st + SA + (wave + NW * i) * 1024), 16,
          (int)(kb[i] < left ? obx[i] : 0xFFFFFFF0u), ks * KS * (int)p.ldb * 2, 0, 0);
  };
  // A workgroup barrier without a memory fence (a fence would also wait for the loads in flight
  // into the other stage); stage_barrier first waits for this wave's own loads of the stage it
  // is about to read, the only vector memory operations outstanding besides epilogue stores.
  auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  auto stage_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0)
    barrier();
  };

  setup(L, rb_c, oa_c, ob_c, row0_c, rows_c, n0_c);
  issue(rb_c, oa_c, ob_c, 0, smem);
  f32x16_t acc[MB][NB];
  int par = 0;  // stage holding K-step 0 of the current tile
  while (true) {
    const int Ln = L + Qd;
    const bool has_next = Ln < hi_t;
    if (has_next) setup(Ln, rb_n, oa_n, ob_n, row0_n, rows_n, n0_n);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int ks = 0; ks < nk; ++ks) {
      stage_barrier();
      uint8_t* st = smem + ((par + ks) & 1) * STAGE;
      const int left = K - ks * KS;
      if (left < KS) {  // uniform: zero the chunks beyond K
#pragma unroll
        for (int i = 0; i < A_GRP; ++i)
          if (cofs >= left * 2)
            *(uint4*)(st + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_GRP; ++i)
          if (kb[i] >= left)
            *(uint4*)(st + SA + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
        barrier();
      }
      uint8_t* other = smem + ((par + ks + 1) & 1) * STAGE;
      if (ks + 1 < nk)
        issue(rb_c, oa_c, ob_c, ks + 1, other);
      else if (has_next)
        issue(rb_n, oa_n, ob_n, 0, other);
      kt_mma<0>(st, acc, lane, wm, wn);
    }
    barrier();  // every wave is done with the last stage: the epilogue reuses it
    int el = lane;
    asm volatile("" : "+v"(el));  // recomputed per tile: its addresses are not kept across tiles
    kt_store<OUT, EPI, false>(p, acc, (uint8_t*)p.C,
                              (float*)(smem + ((par + nk - 1) & 1) * STAGE) + wave * 16 * EPW,
                              row0_c, rows_c, n0_c, el, wm, wn);
    if (!has_next) break;
    rb_c = rb_n;
#pragma unroll
    for (int i = 0; i < A_GRP; ++i) oa_c[i] = oa_n[i];
#pragma unroll
    for (int i = 0; i < B_GRP; ++i) ob_c[i] = ob_n[i];
    row0_c = row0_n;
    rows_c = rows_n;
    n0_c = n0_n;
    par = (par + nk) & 1;
    L = Ln;
  }
}

template <int TA, int TB, Elt OUT, Epi EPI>
hipError_t run_kt(const KtParams& p, int mtiles, hipStream_t s) {
  const int nN = cdiv(p.N, BN), tiles = mtiles * nN;
  if (tiles <= 0) return hipSuccess;
  const int grid = p.kgrp ? kgrp_blocks(p) : cdiv(tiles, kXcds) * kXcds;
  hipLaunchKernelGGL((gemm_kt_kernel<TA, TB, OUT, EPI>), dim3(grid), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_kt(int ta, int tb, Elt out, Epi epi, const KtParams& p, int max_mtiles,
                          hipStream_t s) {
  if (tb != 1 || p.M <= 0 || p.N <= 0 || p.N % 8 || p.ldc % 8 || p.ldb % 8 ||
      (ta && (p.M % 8 || p.lda % 8)) || (!ta && p.K % 8))
    return hipErrorInvalidValue;
  if (epi == Epi::DSqRelu && (!p.C2 || out != Elt::BF16)) return hipErrorInvalidValue;
  // Operand offsets are 32-bit (buffer resources and the per-K-step scalar offset): a K-major
  // operand's K rows, and a K-contiguous A's rows, must span less than 2 GiB.
  constexpr int64_t kLim = ((int64_t)1 << 31) - 1;
  const int64_t krows = p.kgrp ? p.a_rows : p.K;  // K-grouped: the stored rows of both operands
  const int64_t brows = p.b_gather ? p.b_rows : krows;
  if (p.b_gather && (!p.kgrp || p.b_rows < 1)) return hipErrorInvalidValue;
  if ((int64_t)brows * p.ldb * 2 > kLim || (ta && (int64_t)krows * p.lda * 2 > kLim) ||
      (!ta && (int64_t)p.a_rows * p.lda * 2 > kLim))
    return hipErrorInvalidValue;
  const int mt = p.kgrp ? p.G * cdiv(p.M, BM) : (p.mt_start ? max_mtiles : cdiv(p.M, BM));
  if (ta == 0 && p.mt_start && !p.kgrp && p.K > 0 &&
      ((out == Elt::BF16 && epi == Epi::DSqRelu) || (out == Elt::F32 && epi == Epi::Store))) {
    // row-grouped data gradients: persistent
    const int grid = std::min(cdiv(mt * cdiv(p.N, BN), kXcds) * kXcds, persist_grid());
    if (grid <= 0) return hipSuccess;
    if (out == Elt::BF16)
      hipLaunchKernelGGL((gemm_kt_rows_persist<Elt::BF16, Epi::DSqRelu>), dim3(grid), dim3(64 * NW),
                         0, s, p);
    else
      hipLaunchKernelGGL((gemm_kt_rows_persist<Elt::F32, Epi::Store>), dim3(grid), dim3(64 * NW), 0,
                         s, p);
    return hipGetLastError();
  }
  if (ta == 0 && out == Elt::BF16 && epi == Epi::DSqRelu && !p.kgrp)
    return run_kt<0, 1, Elt::BF16, Epi::DSqRelu>(p, mt, s);
  if (ta == 0 && out == Elt::F32 && epi == Epi::Store && !p.kgrp)
    return run_kt<0, 1, Elt::F32, Epi::Store>(p, mt, s);
  if (ta == 0 && out == Elt::BF16 && epi == Epi::Store && !p.kgrp)
    return run_kt<0, 1, Elt::BF16, Epi::Store>(p, mt, s);
  if (ta == 1 && out == Elt::F32 && epi == Epi::Store && !p.mt_start)
    return run_kt<1, 1, Elt::F32, Epi::Store>(p, mt, s);
  if (ta == 1 && out == Elt::BF16 && epi == Epi::Store && !p.mt_start)
    return run_kt<1, 1, Elt::BF16, Epi::Store>(p, mt, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
