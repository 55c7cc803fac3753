// Tiled GEMMs on gfx950 for the MoE layer: the router logits, the routed experts' up / down
// projections (grouped, A rows gathered through the dispatch permutation), the shared expert,
// and the LatentMoE projections.
//
// bf16 / e4m3 tiles run on the matrix cores (v_mfma_f32_32x32x16_bf16,
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales). A workgroup of WGM x WGN waves owns a
// BM x BN output tile. Each K-step stages an SL-byte slab of every A and B row in LDS (SL = 128:
// 64 bf16 or 128 e4m3 values). Slabs are filled by buffer_load_dwordx4 ... lds (global memory
// straight to LDS, no register staging): one instruction fills 1 KB (8 rows x 128 bytes), lane l
// landing at byte 16*l. Operands are addressed through buffer resources that span exactly their
// extent: a per-lane 32-bit row offset plus the K-step offset as a scalar. The 16-byte chunk
// order inside a row is XOR-swizzled by choosing which global chunk each lane fetches, so the
// fragment reads of 16 consecutive rows touch 16 distinct 16-byte bank groups. In a final
// partial K-step, lanes whose chunk lies beyond K skip the access and their slots are zeroed
// once the stage has landed; the padding rows of a partial M-tile skip every access (their
// products are never stored). NS stages are in flight: K-step ks + NS - 1 is loaded while K-step
// ks is multiplied.
// The epilogue stages each wave's accumulators through LDS in 16-row strips so that every lane
// finishes 8 consecutive columns of a row with 16-byte loads and stores.
// Grouped launches (the routed experts) run persistently: two workgroups per CU walk the tiles of
// their die's range, and the last K-step of a tile already loads the first K-step of the
// workgroup's next tile into the stage that step frees, so a tile's first loads overlap the
// previous tile's last products and epilogue.
// fp32 layers use a vector-ALU kernel with the same parameters.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "gemm.hpp"

namespace moe {
namespace {

// A K-step stages SL bytes of every operand row (SL = 128 or 64). The 16-byte chunks of a row
// are XOR-swizzled so that the fragment reads of 16 consecutive rows at one chunk index hit 16
// distinct 16-byte bank groups: rows of 128 bytes swizzle by (row / 2) % 8, rows of 64 bytes by
// (row / 4) % 4.
template <int SL> __device__ __forceinline__ int swz(int row) {
  return SL == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}
template <int SL> __device__ __forceinline__ int slot(int row, int chunk) {
  return row * SL + ((chunk ^ swz<SL>(row)) << 4);
}

// A raw buffer resource over [base, base + bytes): loads at per-lane offsets beyond it return
// zeros without touching memory. bytes is clamped to the 32-bit range of the descriptor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(uint32_t)n, 0x00020000);
}

template <Elt E> struct EltBytes { static constexpr int v = E == Elt::F32 ? 4 : (E == Elt::BF16 ? 2 : 1); };

// Logical tile L -> its group g, first output row, rows (<= BM) and first column. Grouped
// launches walk a device-built prefix of per-group M-tiles (mt_start); inside a group, and for
// dense launches, tiles go in bands of 8 M-tiles, N-major inside a band with M fastest.
template <int BM, int BN>
__device__ __forceinline__ void decode_tile(const GemmParams& p, int nN, int L, int& g, int& row0,
                                            int& rows, int& n0) {
  if (p.mt_start) {
    const int key = L / nN;  // global M-tile index; group g owns [mt_start[g], mt_start[g+1])
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.mt_start[mid] <= key) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int mt_g = p.mt_start[g + 1] - p.mt_start[g];
    const int local = L - p.mt_start[g] * nN;
    constexpr int GB = 8;
    const int first = (local / (GB * nN)) * GB;
    const int gm = min(GB, mt_g - first);
    const int within = local - first * nN;
    n0 = (within / gm) * BN;
    const int mt = first + within % gm;
    row0 = p.offs[g] + mt * BM;
    rows = min(BM, p.offs[g + 1] - row0);
  } else {
    const int nM = cdiv(p.M, BM);
    constexpr int GM = 8;
    const int first = (L / (GM * nN)) * GM;
    const int gm = min(GM, nM - first);
    const int within = L - first * nN;
    const int m = first + within % gm;
    n0 = (within / gm) * BN;
    g = 0;
    row0 = m * BM;
    rows = min(BM, p.M - row0);
  }
}

// Number of logical tiles of a launch (device-side for grouped launches).
template <int BM, int BN>
__device__ __forceinline__ int tile_count(const GemmParams& p, int nN) {
  return p.mt_start ? p.mt_start[p.G] * nN : cdiv(p.M, BM) * nN;
}

// Resolves the tile this workgroup owns (one tile per workgroup). Returns false when the
// workgroup has none.
template <int BM, int BN>
__device__ __forceinline__ bool tile_of(const GemmParams& p, int& g, int& row0, int& rows,
                                        int& n0) {
  const int nN = cdiv(p.N, BN);
  const int L = xcd_logical_block(blockIdx.x, gridDim.x);
  if (L >= tile_count<BM, BN>(p, nN)) return false;
  decode_tile<BM, BN>(p, nN, L, g, row0, rows, n0);
  return rows > 0;
}

// One K-step of a BM x BN tile on the matrix cores, from the stage at As (A rows, then B rows).
// Fragments of k-sub s+1 are read from LDS while the MFMAs of k-sub s issue; scheduling fences
// keep the compiler from hoisting further reads (which would only add registers).
template <int BM, int BN, int WGM, int WGN, Elt AB, int SL>
__device__ __forceinline__ void mma_stage(const uint8_t* As,
                                          f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32],
                                          int lane, int wm, int wn) {
  constexpr int WM = BM / WGM, WN = BN / WGN, MB = WM / 32, NB = WN / 32;
  const uint8_t* Bs = As + BM * SL;
  if constexpr (AB == Elt::BF16) {
    bf16x8_t a[2][MB], b[2][NB];
    auto rd = [&](int s, int buf) {
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < MB; ++i) a[buf][i] = *(const bf16x8_t*)(As + slot<SL>(wm * WM + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < NB; ++j) b[buf][j] = *(const bf16x8_t*)(Bs + slot<SL>(wn * WN + j * 32 + (lane & 31), ch));
    };
    rd(0, 0);
    constexpr int NSUB = SL / 32;  // 16-element k-subs per K-step
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (s < NSUB - 1) rd(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][i], b[s & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    i32x8_t a[2][MB], b[2][NB];
    auto rd = [&](int s, int buf) {
      const int ch = 4 * s + 2 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int r = wm * WM + i * 32 + (lane & 31);
        const i32x4_t lo = *(const i32x4_t*)(As + slot<SL>(r, ch));
        const i32x4_t hi = *(const i32x4_t*)(As + slot<SL>(r, ch + 1));
        a[buf][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int r = wn * WN + j * 32 + (lane & 31);
        const i32x4_t lo = *(const i32x4_t*)(Bs + slot<SL>(r, ch));
        const i32x4_t hi = *(const i32x4_t*)(Bs + slot<SL>(r, ch + 1));
        b[buf][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    rd(0, 0);
    constexpr int NSUB = SL / 64;  // 64-element k-subs per K-step
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (s < NSUB - 1) rd(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[s & 1][i], b[s & 1][j], acc[i][j],
                                                                       0, 0, 0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Epilogue of a tile: acc[i][j][r] is C[wm*WM + i*32 + (r/4)*8 + (lane/32)*4 + r%4]
// [wn*WN + j*32 + lane%32]. Strip h of m-block i (rows 16h .. 16h+15, registers 8h .. 8h+7) goes
// through this wave's LDS strip `ep` (16 x (WN+4) floats); then lane l finishes items l, l + 64,
// ... where item = (row in strip) * (WN/8) + column group.
template <int BM, int BN, int WGM, int WGN, Elt AB, Elt OUT, Epi EPI>
__device__ __forceinline__ void store_tile(const GemmParams& p,
                                           const f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32],
                                           float* ep, int g, int row0, int rows, int n0, int lane,
                                           int wm, int wn) {
  constexpr int WM = BM / WGM, WN = BN / WGN, MB = WM / 32, NB = WN / 32;
  constexpr int EPW = WN + 4;            // epilogue strip row (floats)
  constexpr int CG = WN / 8;             // 8-column groups per strip row
  constexpr int ITEMS = 16 * CG / 64;    // items per lane per strip
  static_assert((16 * CG) % 64 == 0, "strip must split evenly over the wave");
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int r = 8 * h + rr;
          const int srow = (rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3);
          ep[srow * EPW + j * 32 + (lane & 31)] = acc[i][j][r];
        }
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int item = it * 64 + lane;
        const int srow = item / CG, cg = item % CG;
        const int rl = wm * WM + i * 32 + h * 16 + srow;
        const int col = n0 + wn * WN + cg * 8;
        const bool ok = rl < rows && col < p.N;
        const int row = row0 + (rl < rows ? rl : 0);
        float v[8];
        const float4 lo = *(const float4*)(ep + srow * EPW + cg * 8);
        const float4 hi = *(const float4*)(ep + srow * EPW + cg * 8 + 4);
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        if (ok) {
          if constexpr (AB == Elt::FP8) {
            const int64_t src = p.a_gather ? p.a_gather[row] : (int64_t)row;
            const float rs = p.a_scale[src];
            const float* bs = p.b_scale + (int64_t)g * p.N + col;
            const float4 s0 = *(const float4*)bs, s1 = *(const float4*)(bs + 4);
            const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] *= rs * sc[q];
          }
          if constexpr (EPI == Epi::SqRelu) {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = sqrelu(v[q]);
          }
          if constexpr (EPI == Epi::SqReluSave) {  // relu(a) kept for the backward pass
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              w[q] = pack_bf16x2(fmaxf(v[2 * q], 0.f), fmaxf(v[2 * q + 1], 0.f));
            *(uint4*)((uint16_t*)p.C2 + (int64_t)row * p.ldc + col) = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = sqrelu(v[q]);
          }
          // 16-byte stores when the 8 columns lie inside N on an aligned row; else (N or ldc
          // not a multiple of 8, e.g. router logits of E experts) element by element
          const bool whole = col + 8 <= p.N && p.ldc % 8 == 0;
          if constexpr (OUT == Elt::BF16) {
            uint16_t* o = (uint16_t*)p.C + (int64_t)row * p.ldc + col;
            if (whole) {
              uint32_t w[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
              *(uint4*)o = make_uint4(w[0], w[1], w[2], w[3]);
            } else {
              for (int q = 0; q < 8 && col + q < p.N; ++q) o[q] = (uint16_t)f32_to_bf16_bits(v[q]);
            }
          } else {
            float* o = (float*)p.C + (int64_t)row * p.ldc + col;
            if (whole) {
              *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
              *(float4*)(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
            } else {
              for (int q = 0; q < 8 && col + q < p.N; ++q) o[q] = v[q];
            }
          }
        }
      }
    }
  }
}

// -------------------------------------------------------------------------------------------
// Matrix-core kernel (bf16 or e4m3 operands, fp32 accumulation).
// -------------------------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int NS, Elt AB, Elt OUT, Epi EPI, int SL = 128>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mfma(GemmParams p) {
  static_assert(AB == Elt::BF16 || AB == Elt::FP8, "matrix-core path");
  static_assert(NS >= 2, "at least double buffering");
  static_assert(SL == 128 || SL == 64, "64- or 128-byte K-steps");
  int64_t kshift = 0;  // bytes the operand bases moved by for a K slice
  if (p.ksplit > 1) {  // this workgroup's K slice (dense Store launches)
    const int k0 = blockIdx.y * p.kchunk;
    p.K = min(p.kchunk, p.K - k0);
    kshift = (int64_t)k0 * EltBytes<AB>::v;
    p.A = (const uint8_t*)p.A + kshift;
    p.B = (const uint8_t*)p.B + kshift;
    p.C = (uint8_t*)p.C + (int64_t)blockIdx.y * p.M * p.ldc * EltBytes<OUT>::v;
  }
  constexpr int NW = WGM * WGN;
  constexpr int EB = EltBytes<AB>::v;
  constexpr int WM = BM / WGM, WN = BN / WGN, MB = WM / 32, NB = WN / 32;
  constexpr int RPI = 1024 / SL, LPR = SL / 16;  // rows per 1-KB load, lanes per row
  constexpr int A_GRP = BM / (RPI * NW), B_GRP = BN / (RPI * NW);  // 1-KB loads per wave
  constexpr int STAGE = (BM + BN) * SL;
  constexpr int EPW = WN + 4;                                   // epilogue strip row (floats)
  static_assert(A_GRP >= 1 && B_GRP >= 1 && MB >= 1 && NB >= 1, "tile too small");
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0,
                "every tile row must be covered by the waves' 1-KB loads");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tiles are whole 32 x 32 blocks");
  static_assert(NW * 16 * EPW * 4 <= NS * STAGE, "epilogue strips must fit in the stages");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  int g, row0, rows, n0;
  if (!tile_of<BM, BN>(p, g, row0, rows, n0)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int lrow = lane / LPR, lpos = lane % LPR;

  // Operands are read through buffer resources that span exactly their extent in memory, so a
  // read past the end returns zeros instead of touching other memory. Per lane a 32-bit byte
  // offset (row start + this lane's chunk); the K-step offset is a scalar added by the load.
  // Lane (lrow, lpos) of 1-KB group q fills LDS row q*RPI + lrow, slot lpos, which holds global
  // chunk lpos ^ swz(row).
  __amdgpu_buffer_rsrc_t ra = rsrc(p.A, (int64_t)p.a_rows * p.lda * EB - kshift);
  __amdgpu_buffer_rsrc_t rb = rsrc((const uint8_t*)p.B + (int64_t)g * p.b_gstride * EB,
                                   (int64_t)p.N * p.ldb * EB - kshift);
  uint32_t oa[A_GRP], ob[B_GRP];
  // This lane's chunk byte offset. 128-byte rows: the lane's rows (wave + NW*i)*8 + lrow differ
  // by multiples of 16 across groups (NW is even) and swz has period 16. 64-byte rows: swz of
  // row q*16 + lrow depends on lrow only. Either way one offset serves every group.
  static_assert(SL == 64 || NW % 2 == 0, "an even wave count keeps the swizzle constant");
  const int cofs = (lpos ^ swz<SL>(wave * RPI + lrow)) << 4;
  auto set_sources = [&](bool seg2) {
    if (seg2) {
      ra = rsrc(p.A2, (int64_t)p.a2_rows * p.lda2 * EB);
      rb = rsrc(p.B2, (int64_t)p.N * p.ldb2 * EB);
    }
#pragma unroll
    for (int i = 0; i < A_GRP; ++i) {
      const int r = (wave + NW * i) * RPI + lrow;
      if (r >= rows) {  // padding row of a partial tile: no access (its products are discarded)
        oa[i] = 0xFFFFFFF0u;
        continue;
      }
      int64_t src = row0 + r;
      if (!seg2 && p.a_gather) src = p.a_gather[row0 + r];
      oa[i] = (uint32_t)(src * (seg2 ? p.lda2 : p.lda) * EB) + cofs;
    }
#pragma unroll
    for (int i = 0; i < B_GRP; ++i) {
      const int r = (wave + NW * i) * RPI + lrow;
      const int n = n0 + r < p.N ? n0 + r : p.N - 1;
      ob[i] = (uint32_t)((int64_t)n * (seg2 ? p.ldb2 : p.ldb) * EB) + cofs;
    }
  };

  const int kb1 = p.K * EB, kb2 = p.K2 * EB;   // K bytes per segment
  const int nk1 = cdiv(kb1, SL);
  const int nk = nk1 + cdiv(kb2, SL);
  // Bytes of K-step ks that lie inside K when the step is partial, else 0.
  auto tail_of = [&](int ks) {
    const bool seg2 = ks >= nk1;
    const int kb = (seg2 ? ks - nk1 : ks) * SL;
    const int klim = seg2 ? kb2 : kb1;
    return kb + SL <= klim ? 0 : klim - kb;
  };

  // Issue the loads of K-step ks into stage `st`, straight to LDS. In a partial K-step, lanes
  // whose chunk lies beyond K take a per-lane offset outside the buffer (the hardware range
  // check then skips the access); fix_tail() zeroes their slots once the stage has landed.
  auto issue = [&](int ks, uint8_t* st) {
    const bool seg2 = ks >= nk1;
    if (ks == nk1 && nk1 > 0 && kb2 > 0) set_sources(true);
    const int kb = (seg2 ? ks - nk1 : ks) * SL;
    const int tl = tail_of(ks);
    uint8_t* sb = st + BM * SL;
    if (tl == 0) {  // every K-step but a partial last one (uniform branch)
#pragma unroll
      for (int i = 0; i < A_GRP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(st + (wave + NW * i) * 1024), 16,
            (int)oa[i], kb, 0, 0);
#pragma unroll
      for (int i = 0; i < B_GRP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(sb + (wave + NW * i) * 1024), 16,
            (int)ob[i], kb, 0, 0);
    } else {
      const bool live = cofs < tl;
#pragma unroll
      for (int i = 0; i < A_GRP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(st + (wave + NW * i) * 1024), 16,
            (int)(live ? oa[i] : 0xFFFFFFF0u), kb, 0, 0);
#pragma unroll
      for (int i = 0; i < B_GRP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(sb + (wave + NW * i) * 1024), 16,
            (int)(live ? ob[i] : 0xFFFFFFF0u), kb, 0, 0);
    }
  };

  // Zero the slots of a partial K-step that lie beyond K (after the stage has landed).
  auto fix_tail = [&](int ks, uint8_t* st) {
    const int tl = tail_of(ks);
    if (tl == 0) return;  // uniform across the workgroup
    if (cofs >= tl) {
#pragma unroll
      for (int i = 0; i < A_GRP; ++i)
        *(uint4*)(st + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < B_GRP; ++i)
        *(uint4*)(st + BM * SL + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
  };

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](const uint8_t* As) {
    mma_stage<BM, BN, WGM, WGN, AB, SL>(As, acc, lane, wm, wn);
  };

  // Pipeline: K-step ks + NS - 1 is issued while K-step ks is computed. Before computing ks a
  // wave waits until at most (stages issued after ks) x (loads per stage) of its own loads are
  // still in flight, then the barrier makes every wave's slab visible and frees stage ks - 1.
  constexpr int PER = A_GRP + B_GRP;
  auto wait_ahead = [&](int ahead) {
    // s_waitcnt vmcnt(ahead * PER), other counters untouched
#define MOE_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))
    if constexpr (NS >= 4) { if (ahead >= 2) { MOE_VMCNT(2 * PER); return; } }
    if constexpr (NS >= 3) { if (ahead >= 1) { MOE_VMCNT(PER); return; } }
    MOE_VMCNT(0);
#undef MOE_VMCNT
  };
  static_assert((NS - 2) * PER < 64, "vmcnt range");

  set_sources(false);
#pragma unroll
  for (int q = 0; q < NS - 1; ++q)
    if (q < nk) issue(q, smem + q * STAGE);
  for (int ks = 0; ks < nk; ++ks) {
    wait_ahead(min(NS - 2, nk - 1 - ks));
    __syncthreads();
    uint8_t* cur = smem + (ks % NS) * STAGE;
    fix_tail(ks, cur);
    if (ks + NS - 1 < nk) issue(ks + NS - 1, smem + ((ks + NS - 1) % NS) * STAGE);
    compute(cur);
  }
  __syncthreads();  // every wave is done with the stages: the epilogue reuses them

  store_tile<BM, BN, WGM, WGN, AB, OUT, EPI>(p, acc, (float*)smem + wave * 16 * EPW, g, row0, rows,
                                            n0, lane, wm, wn);
}

// -------------------------------------------------------------------------------------------
// Persistent matrix-core kernel for grouped launches (two stages of 128-byte K-steps, one K
// segment). Workgroup b runs on die d = b % 8 as the q-th of that die's Qd workgroups; it walks
// the logical tiles lo + q, lo + q + Qd, ... of its die's contiguous range [lo, hi), so the tiles
// in flight on a die are neighbours (they share weight and activation panels in that die's L2).
// During the last K-step of a tile the workgroup loads the first K-step of its next tile into the
// stage that step frees, and the epilogue stages its strips through the other one.
// -------------------------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, Elt AB, Elt OUT, Epi EPI>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_mfma_persist(GemmParams p) {  // two workgroups per CU: at most 256 registers per lane
  static_assert(AB == Elt::BF16 || AB == Elt::FP8, "matrix-core path");
  constexpr int SL = 128;
  constexpr int NW = WGM * WGN;
  constexpr int EB = EltBytes<AB>::v;
  constexpr int WM = BM / WGM, WN = BN / WGN, MB = WM / 32, NB = WN / 32;
  constexpr int RPI = 1024 / SL, LPR = SL / 16;
  constexpr int A_GRP = BM / (RPI * NW), B_GRP = BN / (RPI * NW);
  constexpr int STAGE = (BM + BN) * SL;
  constexpr int EPW = WN + 4;
  static_assert(A_GRP >= 1 && B_GRP >= 1 && MB >= 1 && NB >= 1, "tile too small");
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0,
                "every tile row must be covered by the waves' 1-KB loads");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tiles are whole 32 x 32 blocks");
  static_assert(NW * 16 * EPW * 4 <= STAGE, "epilogue strips must fit in one stage");
  static_assert(NW % 2 == 0, "an even wave count keeps the swizzle constant");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int nN = cdiv(p.N, BN);
  const int total = tile_count<BM, BN>(p, nN);
  const int d = blockIdx.x % kXcds, Qd = gridDim.x / kXcds;
  const int lo_t = d * cdiv(total, kXcds);
  const int hi_t = min(total, lo_t + cdiv(total, kXcds));
  int L = lo_t + (int)blockIdx.x / kXcds;
  if (L >= hi_t) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int lrow = lane / LPR, lpos = lane % LPR;
  const int cofs = (lpos ^ swz<SL>(wave * RPI + lrow)) << 4;
  const int kb = p.K * EB;
  const int nk = cdiv(kb, SL);
  const int tail = kb % SL;  // bytes of a partial last K-step, 0 when K-steps are whole
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.A, (int64_t)p.a_rows * p.lda * EB);

  // Operand sources of a tile: the buffer resource of its group's weight panel and this lane's
  // row offsets (gathered A rows; padding rows of a partial M-tile are pointed out of range).
  __amdgpu_buffer_rsrc_t rb_c, rb_n;
  uint32_t oa_c[A_GRP], ob_c[B_GRP], oa_n[A_GRP], ob_n[B_GRP];
  int g_c, row0_c, rows_c, n0_c, g_n = 0, row0_n = 0, rows_n = 0, n0_n = 0;
  auto setup = [&](int Lt, __amdgpu_buffer_rsrc_t& rbx, uint32_t* oax, uint32_t* obx, int& gx,
                   int& row0x, int& rowsx, int& n0x) {
    decode_tile<BM, BN>(p, nN, Lt, gx, row0x, rowsx, n0x);
    rbx = rsrc((const uint8_t*)p.B + (int64_t)gx * p.b_gstride * EB, (int64_t)p.N * p.ldb * EB);
#pragma unroll
    for (int i = 0; i < A_GRP; ++i) {
      const int r = (wave + NW * i) * RPI + lrow;
      if (r >= rowsx) {
        oax[i] = 0xFFFFFFF0u;
        continue;
      }
      const int64_t src = p.a_gather ? p.a_gather[row0x + r] : (int64_t)(row0x + r);
      oax[i] = (uint32_t)(src * p.lda * EB) + cofs;
    }
#pragma unroll
    for (int i = 0; i < B_GRP; ++i) {
      const int r = (wave + NW * i) * RPI + lrow;
      const int n = n0x + r < p.N ? n0x + r : p.N - 1;
      obx[i] = (uint32_t)((int64_t)n * p.ldb * EB) + cofs;
    }
  };
  // The loads of K-step ks into stage `st`; in a partial last K-step, lanes whose chunk lies
  // beyond K skip the access (out-of-range offset) and their slots are zeroed after landing.
  auto issue = [&](__amdgpu_buffer_rsrc_t rbx, const uint32_t* oax, const uint32_t* obx, int ks,
                   uint8_t* st) {
    const bool live = !(tail && ks == nk - 1) || cofs < tail;
    uint8_t* sb = st + BM * SL;
#pragma unroll
    for (int i = 0; i < A_GRP; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(st + (wave + NW * i) * 1024), 16,
          (int)(live ? oax[i] : 0xFFFFFFF0u), ks * SL, 0, 0);
#pragma unroll
    for (int i = 0; i < B_GRP; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rbx, (__attribute__((address_space(3))) void*)(sb + (wave + NW * i) * 1024), 16,
          (int)(live ? obx[i] : 0xFFFFFFF0u), ks * SL, 0, 0);
  };
  // A workgroup barrier without a memory fence: the fence would also wait for the loads still in
  // flight into the other stage. Each wave first waits for its own loads of the stage it is about
  // to read (vmcnt(0): those are the only ones outstanding) and its own LDS operations.
  auto stage_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));  // vmcnt(0)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  f32x16_t acc[MB][NB];
  setup(L, rb_c, oa_c, ob_c, g_c, row0_c, rows_c, n0_c);
  issue(rb_c, oa_c, ob_c, 0, smem);
  int par = 0;  // stage that holds K-step 0 of the current tile
  while (true) {
    const int Ln = L + Qd;
    const bool has_next = Ln < hi_t;
    if (has_next) setup(Ln, rb_n, oa_n, ob_n, g_n, row0_n, rows_n, n0_n);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int ks = 0; ks < nk; ++ks) {
      stage_barrier();
      uint8_t* st = smem + ((par + ks) & 1) * STAGE;
      if (tail && ks == nk - 1) {
        if (cofs >= tail) {
#pragma unroll
          for (int i = 0; i < A_GRP; ++i)
            *(uint4*)(st + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < B_GRP; ++i)
            *(uint4*)(st + BM * SL + (wave + NW * i) * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
        }
        barrier();
      }
      uint8_t* other = smem + ((par + ks + 1) & 1) * STAGE;
      if (ks + 1 < nk)
        issue(rb_c, oa_c, ob_c, ks + 1, other);
      else if (has_next)
        issue(rb_n, oa_n, ob_n, 0, other);
      mma_stage<BM, BN, WGM, WGN, AB, SL>(st, acc, lane, wm, wn);
    }
    barrier();  // every wave is done with the last stage: the epilogue reuses it
    store_tile<BM, BN, WGM, WGN, AB, OUT, EPI>(
        p, acc, (float*)(smem + ((par + nk - 1) & 1) * STAGE) + wave * 16 * EPW, g_c, row0_c,
        rows_c, n0_c, lane, wm, wn);
    if (!has_next) break;
    rb_c = rb_n;
#pragma unroll
    for (int i = 0; i < A_GRP; ++i) oa_c[i] = oa_n[i];
#pragma unroll
    for (int i = 0; i < B_GRP; ++i) ob_c[i] = ob_n[i];
    g_c = g_n;
    row0_c = row0_n;
    rows_c = rows_n;
    n0_c = n0_n;
    par = (par + nk) & 1;
    L = Ln;
  }
}

// -------------------------------------------------------------------------------------------
// Vector-ALU kernel for fp32 layers: BM x 64 tiles (BM = 64, or 16 for grouped launches whose
// experts hold few rows), each thread a (BM / 16) x 4 block, K-steps of 16.
// These layers are small, so a K-step's load latency, not its arithmetic, sets the time: the
// loads of the next kF32Ahead steps are in flight (a ring of registers, refilled as each step
// is staged) while a step is multiplied, and the LDS stages alternate so that one barrier per
// step suffices. VEC: every row of A, B (and A2, B2) starts 16-byte aligned and K, K2 are
// multiples of 4, so a thread's 4 k of a row are one 16-byte load. Loads are branch-free
// (steps past the end reload the last one, chunks past K are replaced by zeros after landing),
// so the compiler waits for exactly the step it stages.
// -------------------------------------------------------------------------------------------
constexpr int kF32Ahead = 8;

template <Epi EPI, bool VEC, int BM>
__global__ __launch_bounds__(256) void gemm_f32(GemmParams p) {
  constexpr int BN = 64, BK = 16, PF = kF32Ahead, RM = BM / 16;
  static_assert(BM == 64 || BM == 16, "tile heights provided");
  static_assert(PF % 2 == 0, "the ring slot's parity is the LDS stage's");
  __shared__ float As[2][BK][BM + 4];
  __shared__ float Bs[2][BK][BN + 4];
  int g, row0, rows, n0;
  if (!tile_of<BM, BN>(p, g, row0, rows, n0)) return;
  if (p.ksplit > 1) {  // this workgroup's K slice (dense Store launches, no second segment)
    const int k0 = blockIdx.y * p.kchunk;
    p.K = min(p.kchunk, p.K - k0);
    p.A = (const float*)p.A + k0;
    p.B = (const float*)p.B + k0;
    p.C = (float*)p.C + (int64_t)blockIdx.y * p.M * p.ldc;
  }
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;  // thread's block: rows tr*RM.., cols tc*4..
  // loaders: B row lr, A row lr % BM (with BM = 16 all four waves load A's 16 rows, so every
  // thread issues the same loads; the first wave stages them), k lk .. lk+3
  const int lr = tid >> 2, la = lr % BM, lk = (tid & 3) * 4;
  const bool stage_a = tid < BM * 4;
  const int rr = la < rows ? la : 0;
  const int64_t asrc = p.a_gather ? p.a_gather[row0 + rr] : (int64_t)(row0 + rr);
  const int nn = n0 + lr < p.N ? n0 + lr : p.N - 1;
  const int nk1 = cdiv(p.K, BK), nk = nk1 + cdiv(p.K2, BK);
  const float* a1 = (const float*)p.A + asrc * p.lda;
  const float* b1 = (const float*)p.B + (int64_t)g * p.b_gstride + (int64_t)nn * p.ldb;
  const float* a2 = p.K2 > 0 ? (const float*)p.A2 + (int64_t)(row0 + rr) * p.lda2 : a1;
  const float* b2 = p.K2 > 0 ? (const float*)p.B2 + (int64_t)nn * p.ldb2 : b1;
  // K-step ks (clamped to the last) of this thread's A and B rows: 4 k each, zero past K
  auto load = [&](int ks, float4& va, float4& vb) {
    ks = min(ks, nk - 1);
    const bool seg2 = ks >= nk1;
    const int k0 = (seg2 ? ks - nk1 : ks) * BK + lk;
    const int klim = seg2 ? p.K2 : p.K;
    const float* ap = seg2 ? a2 : a1;
    const float* bp = seg2 ? b2 : b1;
    if constexpr (VEC) {
      const int kc = min(k0, klim - 4);  // K % 4 == 0: the chunk is wholly inside or outside
      const float4 x = *(const float4*)(ap + kc), y = *(const float4*)(bp + kc);
      const bool in = k0 < klim;
      va = in ? x : make_float4(0.f, 0.f, 0.f, 0.f);
      vb = in ? y : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      float x[4], y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kq = min(k0 + q, klim - 1);
        x[q] = ap[kq];
        y[q] = bp[kq];
      }
      va = make_float4(k0 < klim ? x[0] : 0.f, k0 + 1 < klim ? x[1] : 0.f,
                       k0 + 2 < klim ? x[2] : 0.f, k0 + 3 < klim ? x[3] : 0.f);
      vb = make_float4(k0 < klim ? y[0] : 0.f, k0 + 1 < klim ? y[1] : 0.f,
                       k0 + 2 < klim ? y[2] : 0.f, k0 + 3 < klim ? y[3] : 0.f);
    }
  };
  float acc[RM][4] = {};
  if (nk > 0) {
    float4 ra[PF], rb[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) load(u, ra[u], rb[u]);
    for (int ks0 = 0; ks0 < nk; ks0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (ks0 + u >= nk) break;  // uniform
        const int st = u & 1;      // ks0 is even, so this is the step's parity
        if (stage_a) {             // uniform per wave
          As[st][lk + 0][la] = ra[u].x;
          As[st][lk + 1][la] = ra[u].y;
          As[st][lk + 2][la] = ra[u].z;
          As[st][lk + 3][la] = ra[u].w;
        }
        Bs[st][lk + 0][lr] = rb[u].x;
        Bs[st][lk + 1][lr] = rb[u].y;
        Bs[st][lk + 2][lr] = rb[u].z;
        Bs[st][lk + 3][lr] = rb[u].w;
        load(ks0 + u + PF, ra[u], rb[u]);
        // every thread has staged this step, and has finished the step before, which read the
        // stage the next step writes
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
          float a[RM], b[4];
#pragma unroll
          for (int q = 0; q < RM; ++q) a[q] = As[st][kk][tr * RM + q];
#pragma unroll
          for (int q = 0; q < 4; ++q) b[q] = Bs[st][kk][tc * 4 + q];
#pragma unroll
          for (int x = 0; x < RM; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
        }
      }
    }
  }
#pragma unroll
  for (int x = 0; x < RM; ++x) {
    const int rl = tr * RM + x;
    if (rl >= rows) continue;
    const int row = row0 + rl;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int n = n0 + tc * 4 + y;
      if (n >= p.N) continue;
      float v = acc[x][y];
      if constexpr (EPI == Epi::SqRelu) v = sqrelu(v);
      ((float*)p.C)[(int64_t)row * p.ldc + n] = v;
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int NS, Elt AB, Elt OUT, Epi EPI, int SL = 128>
hipError_t run_mfma(const GemmParams& p, int mtiles, hipStream_t s) {
  const int tiles = mtiles * cdiv(p.N, BN);
  if (tiles <= 0) return hipSuccess;
  const int grid = cdiv(tiles, kXcds) * kXcds;
  hipLaunchKernelGGL((gemm_mfma<BM, BN, WGM, WGN, NS, AB, OUT, EPI, SL>), dim3(grid, p.ksplit),
                     dim3(64 * WGM * WGN), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Workgroups of a persistent launch: two per CU (the LDS of two 80 KB stage pairs), rounded down
// to whole groups of 8 (one per die).
int persist_grid() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return std::max(kXcds, (2 * cus[dev]) / kXcds * kXcds);
}

namespace {

template <int BM, int BN, int WGM, int WGN, Elt AB, Elt OUT, Epi EPI>
hipError_t run_persist(const GemmParams& p, int mtiles, hipStream_t s) {
  if (p.K2 > 0 || p.ksplit > 1) return hipErrorInvalidValue;
  const int tiles = mtiles * cdiv(p.N, BN);
  if (tiles <= 0) return hipSuccess;
  const int grid = std::min(cdiv(tiles, kXcds) * kXcds, persist_grid());
  hipLaunchKernelGGL((gemm_mfma_persist<BM, BN, WGM, WGN, AB, OUT, EPI>), dim3(grid),
                     dim3(64 * WGM * WGN), 0, s, p);
  return hipGetLastError();
}

template <Epi EPI, int BM>
hipError_t run_f32_bm(const GemmParams& p, int mtiles, hipStream_t s) {
  const int tiles = mtiles * cdiv(p.N, 64);
  if (tiles <= 0) return hipSuccess;
  const int grid = cdiv(tiles, kXcds) * kXcds;
  const int ks = p.ksplit > 1 ? p.ksplit : 1;
  if (ks > 1 && (EPI != Epi::Store || p.mt_start || p.K2 > 0 || p.kchunk <= 0 ||
                 (int64_t)(ks - 1) * p.kchunk >= p.K || (int64_t)ks * p.kchunk < p.K))
    return hipErrorInvalidValue;
  // 16-byte loads when every row of every operand starts 16-byte aligned (and so do K slices)
  const bool aligned = (((uintptr_t)p.A | (uintptr_t)p.B) & 15) == 0 &&
                       ((p.lda | p.ldb | p.b_gstride | p.K | (ks > 1 ? p.kchunk : 0)) & 3) == 0 &&
                       (p.K2 <= 0 || ((((uintptr_t)p.A2 | (uintptr_t)p.B2) & 15) == 0 &&
                                      ((p.lda2 | p.ldb2 | p.K2) & 3) == 0));
  if (aligned)
    hipLaunchKernelGGL((gemm_f32<EPI, true, BM>), dim3(grid, ks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_f32<EPI, false, BM>), dim3(grid, ks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Grouped launches take the tile height their tile list was built with; dense ones 64.
template <Epi EPI>
hipError_t run_f32(const GemmParams& p, int mtiles, hipStream_t s) {
  if (p.mt_start && p.bm == 16) return run_f32_bm<EPI, 16>(p, mtiles, s);
  if (p.mt_start && p.bm != 0 && p.bm != 64) return hipErrorInvalidValue;
  return run_f32_bm<EPI, 64>(p, mtiles, s);
}

// Dense bf16 launch. Candidate tiles (rates measured on the chip with random bf16 data):
// 256 x 256 on 4 waves (one workgroup per CU), 128 x 192 and 128 x 128 on 4 waves (two
// workgroups per CU). The estimate charges each CU for the whole tiles it receives, so it picks
// the tile that balances best over the 256 CUs.
template <Elt OUT, Epi EPI>
hipError_t run_dense_bf16(const GemmParams& p, hipStream_t s) {
  if (p.ksplit > 1) return run_mfma<128, 128, 2, 2, 2, Elt::BF16, OUT, EPI>(p, cdiv(p.M, 128), s);
  struct Cand { int bm, bn; double rate; };   // rate: relative throughput per CU
  constexpr Cand cands[3] = {{256, 256, 1.03}, {128, 192, 1.0}, {128, 128, 0.94}};
  int best = 0;
  double best_t = 1e300;
  for (int i = 0; i < 3; ++i) {
    const Cand& c = cands[i];
    const double tiles = (double)cdiv(p.M, c.bm) * cdiv(p.N, c.bn);
    const double t = std::ceil(tiles / 256.0) * c.bm * c.bn / c.rate;
    if (t < best_t) { best_t = t; best = i; }
  }
  if (best == 0) return run_mfma<256, 256, 2, 2, 2, Elt::BF16, OUT, EPI>(p, cdiv(p.M, 256), s);
  if (best == 1) return run_mfma<128, 192, 2, 2, 2, Elt::BF16, OUT, EPI>(p, cdiv(p.M, 128), s);
  return run_mfma<128, 128, 2, 2, 2, Elt::BF16, OUT, EPI>(p, cdiv(p.M, 128), s);
}

}  // namespace

hipError_t launch_gemm(const GemmKind& k, const GemmParams& p, int max_mtiles, hipStream_t s) {
  // Grouped launches (mt_start set) walk M-tiles of kGroupBM rows (64 for fp32 layers): the
  // dispatch step built mt_start with that height.
  const bool grouped = p.mt_start != nullptr;
  if (k.ab == Elt::F32) {
    const int mt = grouped ? max_mtiles : cdiv(p.M, 64);
    switch (k.epi) {
      case Epi::Store: return run_f32<Epi::Store>(p, mt, s);
      case Epi::SqRelu: return run_f32<Epi::SqRelu>(p, mt, s);
      default: return hipErrorInvalidValue;
    }
  }
  constexpr int GB = kGroupBM;
  // Operand offsets are 32-bit (buffer resources, per-lane row offsets and the per-K-step
  // scalar offset): A's rows and one group's B panel must each span less than 2 GiB.
  constexpr int64_t kLim = ((int64_t)1 << 31) - 1;
  const int64_t eb = k.ab == Elt::FP8 ? 1 : 2;
  if ((int64_t)p.a_rows * p.lda * eb > kLim || (int64_t)p.N * p.ldb * eb > kLim ||
      (p.K2 > 0 && ((int64_t)p.a2_rows * p.lda2 * eb > kLim || (int64_t)p.N * p.ldb2 * eb > kLim)))
    return hipErrorInvalidValue;
  if (k.ab == Elt::BF16) {
    if (k.epi == Epi::SqReluSave && (!p.C2 || k.out != Elt::BF16 || p.N % 8 || p.ldc % 8))
      return hipErrorInvalidValue;
    if (grouped) {
      // 128 x 192 tiles on 4 waves, two workgroups per CU: the fastest routed shape measured,
      // persistent so that each tile's first loads overlap the previous tile's end
      if (k.out == Elt::BF16 && k.epi == Epi::SqRelu)
        return run_persist<GB, 192, 2, 2, Elt::BF16, Elt::BF16, Epi::SqRelu>(p, max_mtiles, s);
      if (k.out == Elt::BF16 && k.epi == Epi::Store)
        return run_persist<GB, 192, 2, 2, Elt::BF16, Elt::BF16, Epi::Store>(p, max_mtiles, s);
      if (k.out == Elt::BF16 && k.epi == Epi::SqReluSave)
        return run_persist<GB, 192, 2, 2, Elt::BF16, Elt::BF16, Epi::SqReluSave>(p, max_mtiles, s);
      return hipErrorInvalidValue;
    }
    if (k.out == Elt::F32 && k.epi == Epi::Store) return run_dense_bf16<Elt::F32, Epi::Store>(p, s);
    if (k.out == Elt::BF16 && k.epi == Epi::Store) return run_dense_bf16<Elt::BF16, Epi::Store>(p, s);
    if (k.out == Elt::BF16 && k.epi == Epi::SqRelu) return run_dense_bf16<Elt::BF16, Epi::SqRelu>(p, s);
    if (p.ksplit > 1) return hipErrorInvalidValue;
    if (k.out == Elt::BF16 && k.epi == Epi::SqReluSave)
      return run_dense_bf16<Elt::BF16, Epi::SqReluSave>(p, s);
    return hipErrorInvalidValue;
  }
  if (k.ab == Elt::FP8 && grouped && k.out == Elt::BF16) {
    // the same 128 x 192 / 4-wave shape measured fastest for e4m3 as for bf16
    if (k.epi == Epi::SqRelu)
      return run_persist<GB, 192, 2, 2, Elt::FP8, Elt::BF16, Epi::SqRelu>(p, max_mtiles, s);
    if (k.epi == Epi::Store)
      return run_persist<GB, 192, 2, 2, Elt::FP8, Elt::BF16, Epi::Store>(p, max_mtiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
