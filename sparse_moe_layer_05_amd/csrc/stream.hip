// Decode path of the MoE layer on gfx950: with tens of tokens, reading the touched experts'
// weights dominates and the layer is HBM-bound ("NVIDIA Nemotron 3: Efficient and Open
// Intelligence", section 2.2, latency-oriented deployment). Each touched expert's weight matrix
// is therefore read from HBM once, by waves that each own a 64-row panel of it.
//
// Inside a wave the weights are the matrix-core "A" operand and the expert's tokens the "B"
// operand of v_mfma_f32_16x16x32_bf16: lane l loads 16 bytes of weight row (l % 16) at k offset
// 8 * (l / 16) of each 32-wide k step, so one load instruction covers 16 rows x 64 contiguous
// bytes, and the weights never pass through LDS. Up to 64 tokens (4 slices of 16) share each
// weight fragment; groups with more rows loop over 64-token chunks.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int RB = 4;  // 16-row weight blocks per wave: 64 rows
constexpr int U = 4;   // 32-wide k steps per load batch: 128 k
constexpr int NS = 4;  // 16-token slices per pass: 64 tokens
constexpr int kRowsPerWave = 16 * RB;

__device__ __forceinline__ bf16x8_t ld16(const uint16_t* p) { return *(const bf16x8_t*)p; }

__global__ __launch_bounds__(256, 2) void stream_kernel(StreamParams p, int items_routed,
                                                        int items_shared) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int routed = p.E * items_routed;

  const uint16_t* A;
  const uint16_t* W;
  const int32_t* gather;
  void* out;
  int64_t lda, ldo;
  int N, K, row_begin, nrows, nb;
  if (wave < routed) {
    const int g = wave / items_routed;
    nb = wave - g * items_routed;
    row_begin = p.offs[g];
    nrows = p.offs[g + 1] - row_begin;
    A = p.A; lda = p.lda; gather = p.gather; N = p.N; K = p.K;
    W = p.W + (int64_t)g * N * K;
    out = p.out; ldo = p.ldo;
  } else if (wave < routed + items_shared) {
    nb = wave - routed;
    row_begin = 0;
    nrows = p.Ts;
    A = p.As; lda = p.lda_s; gather = nullptr; N = p.Ns; K = p.Ks;
    W = p.Ws;
    out = p.out_s; ldo = p.ldo_s;
  } else {
    return;
  }
  const int n0 = nb * kRowsPerWave;
  if (nrows <= 0 || n0 >= N) return;

  const uint16_t* wrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int n = min(n0 + rb * 16 + (lane & 15), N - 1);
    wrow[rb] = W + (int64_t)n * K;
  }
  const int kq = (lane >> 4) * 8;

  for (int t0 = 0; t0 < nrows; t0 += 16 * NS) {
    const int ns = min(NS, cdiv(nrows - t0, 16));
    const uint16_t* arow[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int tr = min(t0 + s * 16 + (lane & 15), nrows - 1);
      const int64_t src = gather ? gather[row_begin + tr] : (int64_t)(row_begin + tr);
      arow[s] = A + src * lda;
    }
    f32x4_t acc[NS][RB];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[s][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += 32 * U) {
      bf16x8_t wf[U][RB], xf[U][NS];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u * 32 + kq;
        const bool ok = kk < K;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) wf[u][rb] = ok ? ld16(wrow[rb] + kk) : bf16x8_t{};
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (s < ns) xf[u][s] = ok ? ld16(arow[s] + kk) : bf16x8_t{};
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (s < ns)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc[s][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][rb], xf[u][s],
                                                                   acc[s][rb], 0, 0, 0);
    }
    // acc[s][rb][r] = out[token t0 + s*16 + lane%16][n0 + rb*16 + (lane/16)*4 + r]
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int tr = t0 + s * 16 + (lane & 15);
      if (s >= ns || tr >= nrows) continue;
      const int64_t orow = row_begin + tr;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int n = n0 + rb * 16 + (lane >> 4) * 4;
        if (n >= N) continue;
        const f32x4_t v = acc[s][rb];
        if (p.sqrelu_bf16) {
          const uint2 q = make_uint2(pack_bf16x2(sqrelu(v[0]), sqrelu(v[1])),
                                     pack_bf16x2(sqrelu(v[2]), sqrelu(v[3])));
          *(uint2*)((uint16_t*)out + orow * ldo + n) = q;
        } else {
          *(float4*)((float*)out + orow * ldo + n) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_stream(const StreamParams& p, hipStream_t s) {
  const int items_routed = cdiv(p.N, kRowsPerWave);
  const int items_shared = p.Ws ? cdiv(p.Ns, kRowsPerWave) : 0;
  const int waves = p.E * items_routed + items_shared;
  if (waves <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_kernel, dim3(cdiv(waves, 4)), dim3(256), 0, s, p, items_routed,
                     items_shared);
  return hipGetLastError();
}

}  // namespace moe
