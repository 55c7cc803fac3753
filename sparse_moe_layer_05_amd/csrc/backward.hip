// Non-GEMM kernels of the MoE layer's backward pass (bf16 layers): the padded per-expert offsets
// and launch order, the gradient through the routing gates, the router weight gradient, the sum
// that forms dx, and the per-token sum of the LatentMoE experts' input gradient.
//
// The gradient is that of the forward of the Nemotron 3 MoE layer ("NVIDIA Nemotron 3: Efficient
// and Open Intelligence", section 2.2; "Nemotron 3 Nano: Open, Efficient Mixture-of-Experts
// Hybrid Mamba-Transformer Model for Agentic Reasoning", section "技术框架") with the top-k
// selection held fixed: it is piecewise constant, so the gradient reaches the router only
// through the gate weights g_j = s_j / sum_m s_m, s = sigmoid(logits). The per-expert bias of
// aux-loss-free balancing ("Nemotron 3 Nano：開放高效的 MoE 混合 Mamba-Transformer 智能體推理模型",
// section 2.2) only steers the selection and has no gradient.
#include <cmath>

#include "backward.hpp"
#include "common.hpp"

#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kTile = 64;  // pair rows per chunk of the router weight gradient

// Chunk numbering of the router weight gradient: koffs[g + 1] = koffs[g] + roundup(counts[g],
// 64), so expert g owns chunks koffs[g] / 64 .. koffs[g + 1] / 64 - 1; and the experts by
// descending count (ties: lower index first), the launch order of the weight-gradient products.
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* counts, int G,
                                                           int32_t* koffs, int32_t* order) {
  // one thread per expert (G <= kMaxE = blockDim.x); counts staged in LDS
  __shared__ int32_t cnt[kMaxE];
  __shared__ int32_t scan[kMaxE];
  const int g = threadIdx.x;
  const int c = g < G ? counts[g] : 0;
  if (g < G) cnt[g] = c;
  __syncthreads();
  if (g < G) {
    int rank = 0;
    for (int q = 0; q < G; ++q) rank += cnt[q] > c || (cnt[q] == c && q < g);
    order[rank] = g;
  }
  // inclusive scan of the padded counts (integer sums: exact in any order)
  scan[g] = g < G ? (c + kTile - 1) / kTile * kTile : 0;
  __syncthreads();
  for (int o = 1; o < kMaxE; o <<= 1) {
    const int add = g >= o ? scan[g - o] : 0;
    __syncthreads();
    scan[g] += add;
    __syncthreads();
  }
  if (g == 0) koffs[0] = 0;
  if (g < G) koffs[g + 1] = scan[g];
}

// One workgroup per token t. With Y_j the forward's expert output row of pair (t, j):
//   dg_j = <dy_t, Y_j>,  s_j = sigmoid(logit of e_j),  Z = sum_j s_j,
//   dz_j = (dg_j - sum_m g_m dg_m) / Z * s_j (1 - s_j),
//   dYp[pos(t, j)] = bf16(g_j dy_t),  dzp[pos(t, j)] = dz_j.
// The rows Y_j are read kPairBatch at a time with all their loads in flight, and those dot
// products are reduced together; each is still summed in a fixed order (per thread along the
// row, then a butterfly within each wave, then the waves in order).
constexpr int kPairBatch = 8;
__global__ __launch_bounds__(256) void bwd_route_kernel(const uint16_t* __restrict__ dy,
                                                        const uint16_t* __restrict__ Yp,
                                                        const float* __restrict__ logits,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ gates,
                                                        const int32_t* __restrict__ pos,
                                                        int H, int E, int k,
                                                        uint16_t* __restrict__ dYp,
                                                        float* __restrict__ dzp) {
  constexpr int KB = kPairBatch;
  __shared__ float red[4][KB];
  __shared__ float dg[kMaxK];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* dyt = dy + (int64_t)t * H;
  const int nch = H / 8;
  for (int j0 = 0; j0 < k; j0 += KB) {
    int r[KB];
    float part[KB];
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      r[q] = j0 + q < k ? pos[(int64_t)t * k + j0 + q] : -1;
      part[q] = 0.f;
    }
    for (int c = tid; c < nch; c += 256) {
      const uint4 a = *(const uint4*)(dyt + c * 8);
      uint4 b[KB];
#pragma unroll
      for (int q = 0; q < KB; ++q)
        if (r[q] >= 0) b[q] = *(const uint4*)(Yp + (int64_t)r[q] * H + c * 8);
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        if (r[q] < 0) continue;
        const uint32_t wb[4] = {b[q].x, b[q].y, b[q].z, b[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part[q] += bf16_bits_to_f32(wa[e] & 0xFFFF) * bf16_bits_to_f32(wb[e] & 0xFFFF);
          part[q] += bf16_bits_to_f32(wa[e] >> 16) * bf16_bits_to_f32(wb[e] >> 16);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      float v = part[q];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) red[wave][q] = v;
    }
    __syncthreads();
    if (tid < KB && j0 + tid < k) {
      float sum = 0.f;
      for (int w = 0; w < 4; ++w) sum += red[w][tid];  // fixed order
      dg[j0 + tid] = sum;
    }
    __syncthreads();  // red is reused by the next batch; dg is read below
  }
  if (tid == 0) {
    float Z = 0.f, gdg = 0.f;
    float sj[kMaxK];
    for (int j = 0; j < k; ++j) {
      const int e = idx[(int64_t)t * k + j];
      sj[j] = (float)(1.0 / (1.0 + exp(-(double)logits[(int64_t)t * E + e])));
      Z += sj[j];
      gdg += gates[(int64_t)t * k + j] * dg[j];
    }
    for (int j = 0; j < k; ++j) {
      const int r = pos[(int64_t)t * k + j];
      if (r >= 0) dzp[r] = (dg[j] - gdg) / Z * sj[j] * (1.f - sj[j]);
    }
  }
  // rows g_j dy_t: each chunk of dy is loaded once and stored scaled to the token's k rows
  for (int c = tid; c < nch; c += 256) {
    const uint4 a = *(const uint4*)(dyt + c * 8);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
    for (int j = 0; j < k; ++j) {
      const int r = pos[(int64_t)t * k + j];
      if (r < 0) continue;
      const float g = gates[(int64_t)t * k + j];
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_bf16x2(g * bf16_bits_to_f32(wa[e] & 0xFFFF), g * bf16_bits_to_f32(wa[e] >> 16));
      *(uint4*)(dYp + (int64_t)r * H + c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// dW_r[e][h] = sum over expert e's pair rows p (ascending) of dzp[p] * x[perm[p]][h], in two
// passes with a fixed chunking, so that the popular experts' rows are spread over many
// workgroups and the sum stays deterministic. Expert e's rows are cut into chunks of 64 in
// order; its chunks are numbered koffs[e] / 64 .. koffs[e + 1] / 64 - 1 (koffs: per-expert
// offsets padded to multiples of 64). Pass 1: one workgroup per (chunk, 256 columns) writes the
// chunk's sum; wave w adds rows w, w + 4, ... of the chunk, the four partial sums are added in
// wave order. Pass 2: dW_r[e] = sum of e's chunk sums in chunk order.
__global__ __launch_bounds__(256) void router_weight_chunks_kernel(
    const float* dzp, const uint16_t* x, const int32_t* perm, const int32_t* offs,
    const int32_t* koffs, int E, int H, float* part) {
  __shared__ float4 acc_w[4][64];
  const int q = blockIdx.y;  // chunk
  if (q * kTile >= koffs[E]) return;
  int lo = 0, hi = E - 1;    // expert holding chunk q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (koffs[mid] <= q * kTile) lo = mid; else hi = mid - 1;
  }
  const int p0 = offs[lo] + (q * kTile - koffs[lo]);
  const int p1 = min(p0 + kTile, offs[lo + 1]);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = blockIdx.x * 256 + lane * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < H) {
    // this wave's rows p0 + wave, p0 + wave + 4, ...: every load in flight, then added in order
    constexpr int RW = kTile / 4;
    int src[RW];
    float z[RW];
    uint2 v[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int p = p0 + wave + 4 * i;
      src[i] = p < p1 ? perm[p] : -1;
      z[i] = p < p1 ? dzp[p] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (src[i] >= 0) v[i] = *(const uint2*)(x + (int64_t)src[i] * H + c);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (src[i] < 0) continue;
      acc.x += z[i] * bf16_bits_to_f32(v[i].x & 0xFFFF);
      acc.y += z[i] * bf16_bits_to_f32(v[i].x >> 16);
      acc.z += z[i] * bf16_bits_to_f32(v[i].y & 0xFFFF);
      acc.w += z[i] * bf16_bits_to_f32(v[i].y >> 16);
    }
  }
  acc_w[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && c < H) {
    float4 t = acc_w[0][lane];
    for (int w = 1; w < 4; ++w) {
      const float4 u = acc_w[w][lane];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    *(float4*)(part + (int64_t)q * H + c) = t;
  }
}

__global__ __launch_bounds__(256) void router_weight_sum_kernel(const float* part,
                                                                const int32_t* koffs, int H,
                                                                float* dWr) {
  const int e = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  const int q1 = koffs[e + 1] / kTile;
  for (int q0 = koffs[e] / kTile; q0 < q1; q0 += 8) {  // 8 chunk sums in flight, added in order
    float4 u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (q0 + i < q1) u[i] = *(const float4*)(part + (int64_t)(q0 + i) * H + c);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (q0 + i < q1) { s.x += u[i].x; s.y += u[i].y; s.z += u[i].z; s.w += u[i].w; }
  }
  *(float4*)(dWr + (int64_t)e * H + c) = s;
}

// dx[t] = dxa[t] + dxb[t] (each optional) + sum_j du[pos(t, j)] (du optional)
//         + sum_j dzp[pos(t, j)] W_r[e_j], added in that fixed order, fp32. The rows of du are
// read kPairBatch at a time with all their loads in flight; the pointers do not alias, so two
// column chunks' loads can be in flight together.
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float* __restrict__ dxa,
                                                     const float* __restrict__ dxb,
                                                     const float* __restrict__ du,
                                                     const float* __restrict__ dzp,
                                                     const uint16_t* __restrict__ Wr,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ pos, int H, int k,
                                                     float* __restrict__ dx) {
  constexpr int KB = kPairBatch;
  const int t = blockIdx.x;
  const int32_t* post = pos + (int64_t)t * k;
  const int32_t* idxt = idx + (int64_t)t * k;
#pragma unroll 2
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    float4 a = dxa ? *(const float4*)(dxa + (int64_t)t * H + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (dxb) {
      const float4 q = *(const float4*)(dxb + (int64_t)t * H + c);
      a.x += q.x; a.y += q.y; a.z += q.z; a.w += q.w;
    }
    if (du) {
      for (int j0 = 0; j0 < k; j0 += KB) {
        int r[KB];
        float4 u[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q) {
          r[q] = j0 + q < k ? post[j0 + q] : -1;
          if (r[q] >= 0) u[q] = *(const float4*)(du + (int64_t)r[q] * H + c);
        }
#pragma unroll
        for (int q = 0; q < KB; ++q)
          if (r[q] >= 0) { a.x += u[q].x; a.y += u[q].y; a.z += u[q].z; a.w += u[q].w; }
      }
    }
    for (int j = 0; j < k; ++j) {  // W_r rows are few and stay in cache: one at a time
      const int r = post[j];
      if (r < 0) continue;
      const float z = dzp[r];
      const uint2 w = *(const uint2*)(Wr + (int64_t)idxt[j] * H + c);
      a.x += z * bf16_bits_to_f32(w.x & 0xFFFF);
      a.y += z * bf16_bits_to_f32(w.x >> 16);
      a.z += z * bf16_bits_to_f32(w.y & 0xFFFF);
      a.w += z * bf16_bits_to_f32(w.y >> 16);
    }
    *(float4*)(dx + (int64_t)t * H + c) = a;
  }
}

// out[t] = bf16(sum_j du[pos(t, j)]) in j order: the gradient of a token's expert input (the
// LatentMoE projection u), rows of D. Pair rows are read kPairBatch at a time.
__global__ __launch_bounds__(256) void pairs_to_tokens_kernel(const float* __restrict__ du,
                                                              const int32_t* __restrict__ pos,
                                                              int D, int k,
                                                              uint16_t* __restrict__ out) {
  constexpr int KB = kPairBatch;
  const int t = blockIdx.x;
  const int32_t* post = pos + (int64_t)t * k;
#pragma unroll 2
  for (int c = threadIdx.x * 4; c < D; c += 1024) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += KB) {
      int r[KB];
      float4 u[KB];
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        r[q] = j0 + q < k ? post[j0 + q] : -1;
        if (r[q] >= 0) u[q] = *(const float4*)(du + (int64_t)r[q] * D + c);
      }
#pragma unroll
      for (int q = 0; q < KB; ++q)
        if (r[q] >= 0) { a.x += u[q].x; a.y += u[q].y; a.z += u[q].z; a.w += u[q].w; }
    }
    *(uint2*)(out + (int64_t)t * D + c) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
  }
}

}  // namespace

hipError_t launch_pad_offsets(const int32_t* counts, int G, int32_t* koffs, int32_t* order,
                              hipStream_t s) {
  if (G < 1 || G > kMaxE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(kMaxE), 0, s, counts, G, koffs, order);
  return hipGetLastError();
}

hipError_t launch_bwd_route(const uint16_t* dy, const uint16_t* Yp, const float* logits,
                            const int32_t* idx, const float* gates, const int32_t* pos, int T,
                            int H, int E, int k, uint16_t* dYp, float* dzp, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (H % 8 || k > kMaxK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_route_kernel, dim3(T), dim3(256), 0, s, dy, Yp, logits, idx, gates,
                     pos, H, E, k, dYp, dzp);
  return hipGetLastError();
}

hipError_t launch_bwd_router_weight(const float* dzp, const uint16_t* x, const int32_t* perm,
                                    const int32_t* offs, const int32_t* koffs, int E, int H,
                                    int max_chunks, float* part, float* dWr, hipStream_t s) {
  if (H % 4) return hipErrorInvalidValue;
  if (max_chunks > 0)
    hipLaunchKernelGGL(router_weight_chunks_kernel, dim3(cdiv(H, 256), max_chunks), dim3(256), 0,
                       s, dzp, x, perm, offs, koffs, E, H, part);
  hipLaunchKernelGGL(router_weight_sum_kernel, dim3(cdiv(H, 1024), E), dim3(256), 0, s, part,
                     koffs, H, dWr);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const float* dxa, const float* dxb, const float* du, const float* dzp,
                         const uint16_t* Wr, const int32_t* idx, const int32_t* pos, int T, int H,
                         int k, float* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (H % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dx_kernel, dim3(T), dim3(256), 0, s, dxa, dxb, du, dzp, Wr, idx, pos, H,
                     k, dx);
  return hipGetLastError();
}

hipError_t launch_pairs_to_tokens(const float* du, const int32_t* pos, int T, int D, int k,
                                  uint16_t* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (D % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pairs_to_tokens_kernel, dim3(T), dim3(256), 0, s, du, pos, D, k, out);
  return hipGetLastError();
}

}  // namespace moe
