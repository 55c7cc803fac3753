// Tiled GEMMs on gfx950 for the MoE layer: the router logits, the routed experts' up / down
// projections (grouped, A rows gathered through the dispatch permutation), the shared expert,
// and the LatentMoE projections.
//
// bf16 / fp8 tiles run on the matrix cores: v_mfma_f32_32x32x16_bf16 and
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit scales). A workgroup of 4 waves owns a BM x BN
// output tile, each wave a (BM/2) x (BN/2) quarter. Every K-step stages a 128-byte slab of each
// A and B row in LDS (64 bf16 or 128 e4m3 values), double buffered, with the 16-byte chunk index
// XOR-swizzled by (row / 2) % 8 so that fragment reads of 16 consecutive rows hit 16 distinct
// 16-byte bank groups. fp32 layers use a vector-ALU variant with the same parameters.
#include "common.hpp"
#include "gemm.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSlab = 128;  // bytes of one row per K-step

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kSlab + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <Elt E> struct EltBytes { static constexpr int v = E == Elt::F32 ? 4 : (E == Elt::BF16 ? 2 : 1); };

// Resolves the tile this workgroup owns. Returns false when the workgroup has no tile.
template <int BM, int BN>
__device__ __forceinline__ bool tile_of(const GemmParams& p, int& g, int& row0, int& rows,
                                        int& n0) {
  const int nN = cdiv(p.N, BN);
  const int L = xcd_logical_block(blockIdx.x, gridDim.x);
  if (p.mt_start) {
    const int total = p.mt_start[p.G] * nN;
    if (L >= total) return false;
    const int key = L / nN;  // global M-tile index; group g owns [mt_start[g], mt_start[g+1])
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.mt_start[mid] <= key) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int mt_g = p.mt_start[g + 1] - p.mt_start[g];
    const int local = L - p.mt_start[g] * nN;
    n0 = (local / mt_g) * BN;          // a group's tiles: N-major, M fastest (weight panel reuse)
    const int mt = local % mt_g;
    const int gr0 = p.offs[g];
    row0 = gr0 + mt * BM;
    rows = min(BM, p.offs[g + 1] - row0);
  } else {
    const int nM = cdiv(p.M, BM);
    if (L >= nM * nN) return false;
    constexpr int GM = 8;              // bands of 8 M-tiles, N-major inside a band
    const int first = (L / (GM * nN)) * GM;
    const int gm = min(GM, nM - first);
    const int within = L - first * nN;
    const int m = first + within % gm;
    n0 = (within / gm) * BN;
    g = 0;
    row0 = m * BM;
    rows = min(BM, p.M - row0);
  }
  return rows > 0;
}

// -------------------------------------------------------------------------------------------
// Matrix-core kernel (bf16 or e4m3 operands, fp32 accumulation).
// -------------------------------------------------------------------------------------------
template <int BM, int BN, Elt AB, Elt OUT, Epi EPI, bool AQ, Elt YT>
__global__ __launch_bounds__(kThreads) void gemm_mfma(GemmParams p) {
  static_assert(AB == Elt::BF16 || AB == Elt::FP8, "matrix-core path");
  static_assert(!AQ || AB == Elt::FP8, "quantise-on-load feeds e4m3 tiles");
  constexpr int EB = EltBytes<AB>::v;
  constexpr int WM = BM / 2, WN = BN / 2, MB = WM / 32, NB = WN / 32;
  constexpr int A_CH = BM * 8 / kThreads;      // 16-byte chunks per thread per K-step (A)
  constexpr int AQ_CH = BM * 16 / kThreads;    // bf16 source chunks per thread (quantised A)
  constexpr int B_CH = BN * 8 / kThreads;
  static_assert(A_CH >= 1 && B_CH >= 1 && MB >= 1 && NB >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * kSlab];

  int g, row0, rows, n0;
  if (!tile_of<BM, BN>(p, g, row0, rows, n0)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Source rows of this thread's A chunks (clamped into the tile; extra rows are never stored).
  const uint8_t* a_row[AQ ? AQ_CH : A_CH];
  float a_sc[AQ ? AQ_CH : 1];
  if constexpr (!AQ) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int r = (tid >> 3) + i * (kThreads / 8);
      const int rr = r < rows ? r : 0;
      const int64_t src = p.a_gather ? p.a_gather[row0 + rr] : (int64_t)(row0 + rr);
      a_row[i] = (const uint8_t*)p.A + src * p.lda * EB;
    }
  } else {
#pragma unroll
    for (int i = 0; i < AQ_CH; ++i) {
      const int r = (tid >> 4) + i * (kThreads / 16);
      const int rr = r < rows ? r : 0;
      a_row[i] = (const uint8_t*)p.A + (int64_t)(row0 + rr) * p.lda * 2;
      const float amax = p.row_amax[row0 + rr];
      a_sc[i] = amax > 0.f ? amax / 448.f : 1.f;   // the per-row scale; codes = h / scale
    }
  }
  const uint8_t* b_row[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int n = n0 + (tid >> 3) + i * (kThreads / 8);
    const int nn = n < p.N ? n : p.N - 1;
    b_row[i] = (const uint8_t*)p.B + ((int64_t)g * p.b_gstride + (int64_t)nn * p.ldb) * EB;
  }

  const int kb1 = p.K * EB;                         // bytes of K in segment 1
  const int nk1 = cdiv(kb1, kSlab);
  const int kb2 = p.K2 * EB;
  const int nk = nk1 + cdiv(kb2, kSlab);

  uint4 ra[AQ ? AQ_CH : A_CH], rb[B_CH];

  auto load = [&](int ks) {
    const bool seg2 = ks >= nk1;
    const int kb = (seg2 ? ks - nk1 : ks) * kSlab;
    const int klim = seg2 ? kb2 : kb1;
    if constexpr (!AQ) {
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const int off = kb + ((tid & 7) << 4);
        const uint8_t* base = a_row[i];
        if (seg2) {
          const int r = (tid >> 3) + i * (kThreads / 8);
          const int rr = r < rows ? r : 0;
          base = (const uint8_t*)p.A2 + (int64_t)(row0 + rr) * p.lda2 * EB;
        }
        ra[i] = off < klim ? *(const uint4*)(base + off) : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < AQ_CH; ++i) {
        const int off = 2 * kb + ((tid & 15) << 4);  // bf16 source bytes
        ra[i] = off < 2 * klim ? *(const uint4*)(a_row[i] + off) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int off = kb + ((tid & 7) << 4);
      const uint8_t* base = b_row[i];
      if (seg2) {
        const int n = n0 + (tid >> 3) + i * (kThreads / 8);
        const int nn = n < p.N ? n : p.N - 1;
        base = (const uint8_t*)p.B2 + (int64_t)nn * p.ldb2 * EB;
      }
      rb[i] = off < klim ? *(const uint4*)(base + off) : make_uint4(0, 0, 0, 0);
    }
  };

  auto store = [&](int buf) {
    uint8_t* As = smem + buf * (BM + BN) * kSlab;
    uint8_t* Bs = As + BM * kSlab;
    if constexpr (!AQ) {
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const int r = (tid >> 3) + i * (kThreads / 8);
        *(uint4*)(As + swz(r, tid & 7)) = ra[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < AQ_CH; ++i) {
        const int r = (tid >> 4) + i * (kThreads / 16);
        const int q = tid & 15;  // bf16 chunk: elements 8q .. 8q+7 -> fp8 bytes 8q .. 8q+7
        const float s = a_sc[i];
        const uint4 v = ra[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t c[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float f0 = bf16_bits_to_f32(w[2 * h] & 0xFFFF) / s;
          const float f1 = bf16_bits_to_f32(w[2 * h] >> 16) / s;
          const float f2 = bf16_bits_to_f32(w[2 * h + 1] & 0xFFFF) / s;
          const float f3 = bf16_bits_to_f32(w[2 * h + 1] >> 16) / s;
          c[h] = cvt_fp8x2(f0, f1) | (cvt_fp8x2(f2, f3) << 16);
        }
        *(uint2*)(As + swz(r, q >> 1) + ((q & 1) << 3)) = make_uint2(c[0], c[1]);
      }
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int r = (tid >> 3) + i * (kThreads / 8);
      *(uint4*)(Bs + swz(r, tid & 7)) = rb[i];
    }
  };

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int buf) {
    const uint8_t* As = smem + buf * (BM + BN) * kSlab;
    const uint8_t* Bs = As + BM * kSlab;
    if constexpr (AB == Elt::BF16) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = 2 * s + (lane >> 5);
        bf16x8_t a[MB], b[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) a[i] = *(const bf16x8_t*)(As + swz(wm * WM + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int j = 0; j < NB; ++j) b[j] = *(const bf16x8_t*)(Bs + swz(wn * WN + j * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int ch = 4 * s + 2 * (lane >> 5);
        i32x8_t a[MB], b[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int r = wm * WM + i * 32 + (lane & 31);
          const i32x4_t lo = *(const i32x4_t*)(As + swz(r, ch));
          const i32x4_t hi = *(const i32x4_t*)(As + swz(r, ch + 1));
          a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int r = wn * WN + j * 32 + (lane & 31);
          const i32x4_t lo = *(const i32x4_t*)(Bs + swz(r, ch));
          const i32x4_t hi = *(const i32x4_t*)(Bs + swz(r, ch + 1));
          b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j],
                                                                         0, 0, 0, 127, 0, 127);
      }
    }
  };

  if (nk > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < nk) load(ks + 1);
      compute(cur);
      if (ks + 1 < nk) store(cur ^ 1);
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][r] is C[wm*WM + i*32 + (r/4)*8 + (lane/32)*4 + r%4][wn*WN + j*32 + lane%32]
  const int colL = lane & 31;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const bool rok = rl < rows;
      const int row = row0 + (rok ? rl : 0);
      float rs = 1.f;
      if constexpr (AB == Elt::FP8) {
        if constexpr (AQ) {
          const float amax = p.row_amax[row];
          rs = amax > 0.f ? amax / 448.f : 1.f;
        } else {
          const int64_t src = p.a_gather ? p.a_gather[row] : (int64_t)row;
          rs = p.a_scale[src];
        }
      }
      float rmax = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + wn * WN + j * 32 + colL;
        const bool ok = rok && n < p.N;
        float v = acc[i][j][r];
        if constexpr (AB == Elt::FP8) v *= rs * p.b_scale[(int64_t)g * p.N + (n < p.N ? n : 0)];
        if constexpr (EPI == Epi::SqRelu || EPI == Epi::SqReluAmax) v = sqrelu(v);
        if constexpr (EPI == Epi::Combine) {
          if (ok) {
            for (int jj = 0; jj < p.topk; ++jj) {
              const int64_t q = (int64_t)row * p.topk + jj;
              const float gte = p.gates[q];
              const int64_t yr = p.pos[q];
              if (yr < 0) continue;  // dropped pair
              float yv;
              if constexpr (YT == Elt::BF16)
                yv = bf16_bits_to_f32(((const uint16_t*)p.Y)[yr * p.ldy + n]);
              else
                yv = ((const float*)p.Y)[yr * p.ldy + n];
              v += gte * yv;
            }
          }
        }
        if (ok) {
          if constexpr (OUT == Elt::BF16) {
            const uint32_t hb = f32_to_bf16_bits(v);
            ((uint16_t*)p.C)[(int64_t)row * p.ldc + n] = (uint16_t)hb;
            if constexpr (EPI == Epi::SqReluAmax) rmax = fmaxf(rmax, bf16_bits_to_f32(hb));
          } else {
            ((float*)p.C)[(int64_t)row * p.ldc + n] = v;
          }
        }
      }
      if constexpr (EPI == Epi::SqReluAmax) {
#pragma unroll
        for (int m = 1; m < 32; m <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, m, 32));
        if (colL == 0 && rok) atomicMax((unsigned int*)&p.row_amax[row], __float_as_uint(rmax));
      }
    }
  }
}

// -------------------------------------------------------------------------------------------
// Vector-ALU kernel for fp32 layers: 64 x 64 tile, each thread a 4 x 4 block, K-steps of 16.
// -------------------------------------------------------------------------------------------
template <Epi EPI>
__global__ __launch_bounds__(kThreads) void gemm_f32(GemmParams p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  int g, row0, rows, n0;
  if (!tile_of<BM, BN>(p, g, row0, rows, n0)) return;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;  // thread's 4 x 4 block: rows tr*4.., cols tc*4..
  // loader: 64 rows x 16 k = 1024 values = 4 per thread; thread loads row lr, k lk..lk+3
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int rr = lr < rows ? lr : 0;
  const int64_t asrc = p.a_gather ? p.a_gather[row0 + rr] : (int64_t)(row0 + rr);
  const int nn = n0 + lr < p.N ? n0 + lr : p.N - 1;
  const int nk1 = cdiv(p.K, BK), nk = nk1 + cdiv(p.K2, BK);
  float acc[4][4] = {};
  for (int ks = 0; ks < nk; ++ks) {
    const bool seg2 = ks >= nk1;
    const int k0 = (seg2 ? ks - nk1 : ks) * BK + lk;
    const int klim = seg2 ? p.K2 : p.K;
    const float* ap = seg2 ? (const float*)p.A2 + (int64_t)(row0 + rr) * p.lda2
                           : (const float*)p.A + asrc * p.lda;
    const float* bp = seg2 ? (const float*)p.B2 + (int64_t)nn * p.ldb2
                           : (const float*)p.B + (int64_t)g * p.b_gstride + (int64_t)nn * p.ldb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      As[lk + q][lr] = k0 + q < klim ? ap[k0 + q] : 0.f;
      Bs[lk + q][lr] = k0 + q < klim ? bp[k0 + q] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { a[q] = As[kk][tr * 4 + q]; b[q] = Bs[kk][tc * 4 + q]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int rl = tr * 4 + x;
    if (rl >= rows) continue;
    const int row = row0 + rl;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int n = n0 + tc * 4 + y;
      if (n >= p.N) continue;
      float v = acc[x][y];
      if constexpr (EPI == Epi::SqRelu) v = sqrelu(v);
      if constexpr (EPI == Epi::Combine) {
        for (int jj = 0; jj < p.topk; ++jj) {
          const int64_t q = (int64_t)row * p.topk + jj;
          const int64_t yr = p.pos[q];
          if (yr < 0) continue;  // dropped pair
          v += p.gates[q] * ((const float*)p.Y)[yr * p.ldy + n];
        }
      }
      ((float*)p.C)[(int64_t)row * p.ldc + n] = v;
    }
  }
}

template <int BM, int BN, Elt AB, Elt OUT, Epi EPI, bool AQ, Elt YT>
hipError_t run_mfma(const GemmParams& p, int max_mtiles, hipStream_t s) {
  const int tiles = max_mtiles * cdiv(p.N, BN);
  const int grid = cdiv(tiles, kXcds) * kXcds;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_mfma<BM, BN, AB, OUT, EPI, AQ, YT>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <Epi EPI>
hipError_t run_f32(const GemmParams& p, int max_mtiles, hipStream_t s) {
  const int tiles = max_mtiles * cdiv(p.N, 64);
  const int grid = cdiv(tiles, kXcds) * kXcds;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32<EPI>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmKind& k, const GemmParams& p, int max_mtiles, hipStream_t s) {
  constexpr int BM = kGroupBM;
  // Dense launches (no group list) size their own M-tile count from M. Grouped fp32 launches
  // use 64-row tiles, so their group list must have been built with bm = 64.
  if (k.ab == Elt::F32) {
    const int mt = p.mt_start ? max_mtiles : cdiv(p.M, 64);
    switch (k.epi) {
      case Epi::Store: return run_f32<Epi::Store>(p, mt, s);
      case Epi::SqRelu: return run_f32<Epi::SqRelu>(p, mt, s);
      case Epi::Combine: return run_f32<Epi::Combine>(p, mt, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int mt = p.mt_start ? max_mtiles : cdiv(p.M, BM);
  if (k.ab == Elt::BF16) {
    if (k.out == Elt::F32 && k.epi == Epi::Store)
      return run_mfma<BM, 128, Elt::BF16, Elt::F32, Epi::Store, false, Elt::BF16>(p, mt, s);
    if (k.out == Elt::BF16 && k.epi == Epi::Store)
      return run_mfma<BM, 128, Elt::BF16, Elt::BF16, Epi::Store, false, Elt::BF16>(p, mt, s);
    if (k.out == Elt::BF16 && k.epi == Epi::SqRelu)
      return run_mfma<BM, 128, Elt::BF16, Elt::BF16, Epi::SqRelu, false, Elt::BF16>(p, mt, s);
    if (k.out == Elt::BF16 && k.epi == Epi::Combine && k.y == Elt::BF16)
      return run_mfma<BM, 128, Elt::BF16, Elt::BF16, Epi::Combine, false, Elt::BF16>(p, mt, s);
    if (k.out == Elt::BF16 && k.epi == Epi::Combine && k.y == Elt::F32)
      return run_mfma<BM, 128, Elt::BF16, Elt::BF16, Epi::Combine, false, Elt::F32>(p, mt, s);
    return hipErrorInvalidValue;
  }
  if (k.ab == Elt::FP8) {
    if (k.out == Elt::BF16 && k.epi == Epi::SqReluAmax && !p.a_quant)
      return run_mfma<BM, 128, Elt::FP8, Elt::BF16, Epi::SqReluAmax, false, Elt::BF16>(p, mt, s);
    if (k.out == Elt::BF16 && k.epi == Epi::Store && p.a_quant)
      return run_mfma<BM, 128, Elt::FP8, Elt::BF16, Epi::Store, true, Elt::BF16>(p, mt, s);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
