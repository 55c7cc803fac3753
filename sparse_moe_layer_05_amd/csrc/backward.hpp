// Launchers of the non-GEMM kernels of the MoE layer's backward pass (bf16 layers). The GEMMs
// of the pass are in gemm_kt.hpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// koffs[g + 1] = koffs[g] + roundup(counts[g], 64), koffs[0] = 0; order = the groups by
// descending count, ties by index.
hipError_t launch_pad_offsets(const int32_t* counts, int G, int32_t* koffs, int32_t* order,
                              hipStream_t s);

// Gradient through the routing gates, per token: dg_j = <dy_t, Yp[pos(t,j)]>,
// dz_j = (dg_j - sum_m g_m dg_m) / Z * s_j (1 - s_j) with s = sigmoid(logits), Z = sum_j s_j;
// writes dYp[pos(t,j)] = bf16(g_j dy_t) and dzp[pos(t,j)] = dz_j.
hipError_t launch_bwd_route(const uint16_t* dy, const uint16_t* Yp, const float* logits,
                            const int32_t* idx, const float* gates, const int32_t* pos, int T,
                            int H, int E, int k, uint16_t* dYp, float* dzp, hipStream_t s);

// dW_r[e] = sum over expert e's pair rows p (ascending) of dzp[p] x[perm[p]], fp32: sums of
// 64-row chunks (numbered by koffs / 64, at most max_chunks of them) into part
// [max_chunks][H], then each expert's chunk sums in order.
hipError_t launch_bwd_router_weight(const float* dzp, const uint16_t* x, const int32_t* perm,
                                    const int32_t* offs, const int32_t* koffs, int E, int H,
                                    int max_chunks, float* part, float* dWr, hipStream_t s);

// dx[t] = dxa[t] + dxb[t] (each optional) + sum_j du[pos(t,j)] (du optional)
//         + sum_j dzp[pos(t,j)] W_r[idx(t,j)], fp32, in that order.
hipError_t launch_bwd_dx(const float* dxa, const float* dxb, const float* du, const float* dzp,
                         const uint16_t* Wr, const int32_t* idx, const int32_t* pos, int T, int H,
                         int k, float* dx, hipStream_t s);

// out[t] = bf16(sum_j du[pos(t,j)]) for rows of D (fp32 pair rows in, bf16 token rows out).
hipError_t launch_pairs_to_tokens(const float* du, const int32_t* pos, int T, int D, int k,
                                  uint16_t* out, hipStream_t s);

}  // namespace moe
