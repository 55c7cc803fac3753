// Decode path of the MoE layer on gfx950. With tens of tokens, reading the touched experts'
// weights dominates and the layer is HBM-bound ("NVIDIA Nemotron 3: Efficient and Open
// Intelligence", section 2.2, latency-oriented deployment), so each touched expert's weight
// matrix is read from HBM exactly once.
//
// Work comes in units of 16 weight rows. A persistent grid of 1024 waves (one per SIMD) claims
// units from device counters that the dispatch step cleared, in two phases:
//   1. "wide" units: the shared expert's blocks and the blocks of experts with more than 16
//      tokens, up to 64 tokens per pass (four 16-token slices);
//   2. "narrow" units: the blocks of experts with at most 16 tokens. This is the bulk of the
//      bytes, so loads are double buffered in registers with a one-unit lookahead: while the
//      last k batch of a unit is multiplied, the first batch of the next claimed unit is in
//      flight.
// Inside a unit the weights are the matrix-core "A" operand and the tokens the "B" operand of
// v_mfma_f32_16x16x32_bf16: lane l loads 16 bytes of weight row (l % 16) at k offset
// 8 * (l / 16) of each 32-wide k step straight from HBM into registers (no LDS).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kUnitRows = 16;
constexpr int kStreamWaves = 1024;  // 4 per CU, one per SIMD
constexpr int UN = 16;              // narrow units: 32-wide k steps per load batch
constexpr int UW = 4;               // wide units: k steps per batch
constexpr int NSW = 4;              // wide units: 16-token slices per pass

__device__ __forceinline__ bf16x8_t ld16(const uint16_t* p) { return *(const bf16x8_t*)p; }

__device__ __forceinline__ int claim(int32_t* counter, int lane) {
  int u = 0;
  if (lane == 0) u = atomicAdd(counter, 1);
  return __shfl(u, 0);
}

// One lane's part of a 16 x 16 output block: 4 consecutive columns n .. n+3 of row orow.
__device__ __forceinline__ void store_block(const f32x4_t v, void* out, int64_t ldo,
                                            int64_t orow, int n, bool sq) {
  if (sq) {
    const uint2 q = make_uint2(pack_bf16x2(sqrelu(v[0]), sqrelu(v[1])),
                               pack_bf16x2(sqrelu(v[2]), sqrelu(v[3])));
    *(uint2*)((uint16_t*)out + orow * ldo + n) = q;
  } else {
    *(float4*)((float*)out + orow * ldo + n) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Wide unit: rows n0 .. n0+15 of W ([N][K]) against rows [row_begin, row_begin + nrows) of the
// activations, 64 tokens per pass.
__device__ void wide_unit(const uint16_t* __restrict__ A, int64_t lda,
                          const int32_t* __restrict__ gather, int row_begin, int nrows,
                          const uint16_t* __restrict__ W, int N, int K, int n0, void* out,
                          int64_t ldo, bool sq, int lane) {
  const uint16_t* wrow = W + (int64_t)min(n0 + (lane & 15), N - 1) * K;
  const int kq = (lane >> 4) * 8;
  for (int t0 = 0; t0 < nrows; t0 += 16 * NSW) {
    const int ns = min(NSW, cdiv(nrows - t0, 16));
    const uint16_t* arow[NSW];
#pragma unroll
    for (int s = 0; s < NSW; ++s) {
      const int tr = min(t0 + s * 16 + (lane & 15), nrows - 1);
      const int64_t src = gather ? gather[row_begin + tr] : (int64_t)(row_begin + tr);
      arow[s] = A + src * lda;
    }
    f32x4_t acc[NSW];
#pragma unroll
    for (int s = 0; s < NSW; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += 32 * UW) {
      bf16x8_t wf[UW], xf[UW][NSW];
#pragma unroll
      for (int u = 0; u < UW; ++u) {
        const int kk = k0 + u * 32 + kq;
        const bool ok = kk < K;
        wf[u] = ok ? ld16(wrow + kk) : bf16x8_t{};
#pragma unroll
        for (int s = 0; s < NSW; ++s)
          if (s < ns) xf[u][s] = ok ? ld16(arow[s] + kk) : bf16x8_t{};
      }
#pragma unroll
      for (int u = 0; u < UW; ++u)
#pragma unroll
        for (int s = 0; s < NSW; ++s)
          if (s < ns) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], xf[u][s], acc[s], 0, 0, 0);
    }
    // acc[s][r] = out[token t0 + s*16 + lane%16][n0 + (lane/16)*4 + r]
    const int n = n0 + (lane >> 4) * 4;
#pragma unroll
    for (int s = 0; s < NSW; ++s) {
      const int tr = t0 + s * 16 + (lane & 15);
      if (s < ns && tr < nrows && n < N) store_block(acc[s], out, ldo, row_begin + tr, n, sq);
    }
  }
}

// A narrow unit resolved to this lane's pointers: 16 weight rows, up to 16 token rows.
struct Narrow {
  const uint16_t* w;   // this lane's weight row
  const uint16_t* a;   // this lane's token row
  int64_t orow;        // output row of this lane's token
  int n;               // first of this lane's 4 output columns
  int nrows, tr;       // tokens of the unit, this lane's token index
  int nbat;            // load batches over K
};

__global__ __launch_bounds__(256, 1) void stream_kernel(StreamParams p) {
  const int lane = threadIdx.x & 63;
  const bool sq = p.sqrelu_bf16;
  const int nbr = cdiv(p.N, kUnitRows);

  // ---- phase 1: wide units (shared expert blocks, then blocks of experts with > 16 tokens)
  {
    const int nbs = p.Ws ? cdiv(p.Ns, kUnitRows) : 0;
    const int total = nbs + *p.n_wide * nbr;
    for (;;) {
      const int u = claim(p.counter, lane);
      if (u >= total) break;  // every wave leaves once the list is exhausted
      if (u < nbs) {
        wide_unit(p.As, p.lda_s, nullptr, 0, p.Ts, p.Ws, p.Ns, p.Ks, u * kUnitRows, p.out_s,
                  p.ldo_s, sq, lane);
      } else {
        const int v = u - nbs;
        const int g = p.wide[v / nbr];
        const int rb0 = p.offs[g];
        wide_unit(p.A, p.lda, p.gather, rb0, p.offs[g + 1] - rb0, p.W + (int64_t)g * p.N * p.K,
                  p.N, p.K, (v % nbr) * kUnitRows, p.out, p.ldo, sq, lane);
      }
    }
  }

  // ---- phase 2: narrow units, double-buffered loads with a one-unit lookahead
  const int total = *p.n_narrow * nbr;
  const int kq = (lane >> 4) * 8;
  auto resolve = [&](int u, Narrow& s) {
    const int g = p.narrow[u / nbr];
    const int n0 = (u % nbr) * kUnitRows;
    const int rb0 = p.offs[g];
    s.nrows = p.offs[g + 1] - rb0;
    s.tr = lane & 15;
    const int tr = min(s.tr, s.nrows - 1);
    s.a = p.A + (int64_t)(p.gather ? p.gather[rb0 + tr] : rb0 + tr) * p.lda;
    s.w = p.W + (int64_t)g * p.N * p.K + (int64_t)min(n0 + (lane & 15), p.N - 1) * p.K;
    s.orow = rb0 + s.tr;
    s.n = n0 + (lane >> 4) * 4;
    s.nbat = cdiv(p.K, 32 * UN);
  };
  auto issue = [&](const Narrow& s, int b, bf16x8_t* wf, bf16x8_t* xf) {
#pragma unroll
    for (int q = 0; q < UN; ++q) {
      const int kk = b * 32 * UN + q * 32 + kq;
      const bool ok = kk < p.K;
      wf[q] = ok ? ld16(s.w + kk) : bf16x8_t{};
      xf[q] = ok ? ld16(s.a + kk) : bf16x8_t{};
    }
  };

  Narrow cur, nxt;
  bf16x8_t wc[UN], xc[UN], wn[UN], xn[UN];
  int u = claim(p.counter + 1, lane);
  if (u >= total) return;
  resolve(u, cur);
  issue(cur, 0, wc, xc);
  int b = 0;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (;;) {
    bool more = true, fresh = false;
    if (b + 1 < cur.nbat) {
      issue(cur, b + 1, wn, xn);
    } else {
      const int un = claim(p.counter + 1, lane);
      if (un < total) {
        resolve(un, nxt);
        issue(nxt, 0, wn, xn);
        fresh = true;
      } else {
        more = false;  // the list is exhausted: this is the wave's last batch
      }
    }
#pragma unroll
    for (int q = 0; q < UN; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wc[q], xc[q], acc, 0, 0, 0);
    if (b + 1 == cur.nbat) {  // unit done: lanes holding a real token store their 4 columns
      if (cur.tr < cur.nrows && cur.n < p.N) store_block(acc, p.out, p.ldo, cur.orow, cur.n, sq);
      acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (!more) break;
#pragma unroll
    for (int q = 0; q < UN; ++q) {
      wc[q] = wn[q];
      xc[q] = xn[q];
    }
    if (fresh) {
      cur = nxt;
      b = 0;
    } else {
      ++b;
    }
  }
}

}  // namespace

hipError_t launch_stream(const StreamParams& p, hipStream_t s) {
  hipLaunchKernelGGL(stream_kernel, dim3(kStreamWaves / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
