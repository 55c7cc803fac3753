// Launchers of the non-GEMM kernels of the MoE layer (routing, dispatch, combine, fp8
// activation quantisation, decode-path expert streaming).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"

namespace moe {

// Dispatch of more than kDispatchSmallT tokens runs over chunks of 256, 128 or 64 tokens, one
// workgroup each. A chunk is halved while it holds more than 2048 (token, slot) pairs and the
// call keeps at most 128 chunks: many slots per token (LatentMoE's 24) then spread over more
// workgroups, while the one-workgroup scan still adds few chunk counts per expert.
constexpr int kDispatchSmallT = 256;   // up to this many tokens: one workgroup does it all
inline int dispatch_chunk(int T, int k) {
  int ch = 256;
  while (ch > 64 && ch * k > 2048 && ((int64_t)T + ch / 2 - 1) / (ch / 2) <= 128) ch /= 2;
  return ch;
}
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

// logits [T, E] fp32 -> idx [T, k] (descending key, lower index on ties), gates [T, k].
// With nsplit > 1, `logits` holds nsplit partial sums [nsplit][T][E] that are added in slice
// order first (and written to logits_out when it is not null).
hipError_t launch_topk(const float* logits, int nsplit, const float* b, int T, int E, int k,
                       int32_t* idx, float* gates, float* logits_out, hipStream_t s);

// Router K-split for small T: number of K slices (and the slice width) that give the dense
// router GEMM about one workgroup per CU.
void router_split(int T, int E, int H, int* nsplit, int* kchunk);
// The same for the fp32 router (vector-ALU GEMM).
void router_split_f32(int T, int E, int H, int* nsplit, int* kchunk);

// Dispatch scratch: chunk_counts and chunk_base, each [ceil(T / dispatch_chunk(T, k)), E] int32.
inline size_t dispatch_scratch_ints(int T, int E, int k) {
  const int ch = dispatch_chunk(T, k);
  return 2 * (size_t)(((int64_t)T + ch - 1) / ch) * (size_t)E;
}

// Extra dispatch product for the decode path: the touched experts cut into slices of at most
// kSliceRows consecutive pair rows, ascending by expert then row. Slice i covers pair rows
// slice_r[i] .. min(slice_r[i] + kSliceRows, offsets[slice_e[i] + 1]) - 1 of expert slice_e[i].
// Each array holds at most E + T*k / kSliceRows entries.
constexpr int kSliceRows = 16;
struct DispatchExtras {
  int32_t* slice_e = nullptr;   // expert of each slice
  int32_t* slice_r = nullptr;   // first pair row of each slice
  int32_t* n_slices = nullptr;  // [1]: number of slices
};
inline int max_slices(int P, int E) { return E + P / kSliceRows; }

// idx [T, k] -> counts [E], offsets [E + 1], perm [T*k], pos [T, k]; optionally the prefix of
// ceil(counts / bm) M-tiles (mt_start [E + 1], for grouped GEMMs) and the decode extras.
// Pairs with an out-of-range or repeated expert are dropped (pos = -1).
hipError_t launch_dispatch(const int32_t* idx, int T, int E, int k, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* scratch,
                           int bm, int32_t* mt_start, const DispatchExtras& ex, hipStream_t s);

// out[t] = S[t] (optional, fp32) + sum_j gates[t, j] * Y[pos[t, j]], in fixed j order, rounded
// once to out_elt. S may come as ns fp32 slabs s_slab elements apart (partial sums over ranges
// of its K), added in slab order first.
hipError_t launch_combine(const void* Y, Elt y_elt, int64_t ldy, const float* S, int64_t lds,
                          const int32_t* pos, const float* gates, int T, int D, int k, void* out,
                          Elt out_elt, int64_t ldo, hipStream_t s, int ns = 1,
                          int64_t s_slab = 0);

// Per-row e4m3 quantisation of bf16 rows: scale[t] = amax / 448 (1 for a zero row),
// q[t, :] = e4m3(x * fp32(448 / amax)).
hipError_t launch_quant_rows(const uint16_t* x, int64_t ldx, int T, int H, uint8_t* q,
                             float* scale, hipStream_t s);

// Aux-loss-free bias step: b[e] += gamma * sign(target[e] - counts[e]) in fp32; target NULL means
// the mean load, compared exactly as sign(sum(counts) - E * counts[e]).
hipError_t launch_bias_update(const int32_t* counts, const float* target, int E, float gamma,
                              float* b, hipStream_t s);

enum StreamStore : int { kStoreF32 = 0, kStoreSqRelu = 1, kStoreBF16 = 2 };

// Decode path: every routed group g (expert) with rows offs[g] .. offs[g+1] and, optionally, the
// shared expert (rows 0 .. Ts-1 of As) stream their weight matrix [N][K] from HBM exactly once:
//   out[r, n] = act( sum_k A[src(r), k] * W[g][n, k] )
// act = bf16(relu(acc)^2) for the up projection, fp32 acc for the down projection.
struct StreamParams {
  // routed weight format: BF16 (bf16 tokens), or FP8 / MXFP4 / MXFP8 (e4m3 token codes with a
  // scale per source row; no shared slot)
  Elt wt = Elt::BF16;
  // routed experts
  const void* A = nullptr;            // activation rows (bf16 or e4m3), lda elements apart
  int64_t lda = 0;
  const float* a_scale = nullptr;     // e4m3 tokens: dequantisation scale per source row
  const int32_t* gather = nullptr;    // source row of pair row r = gather[r] (nullptr: r)
  const int32_t* offs = nullptr;      // [E + 1]
  int E = 0;
  const void* W = nullptr;            // [E][N][K] (MXFP4: [E][N][K / 2] bytes)
  const float* w_scale = nullptr;     // FP8: per output channel [E][N]
  const uint8_t* w_mx = nullptr;      // MXFP4 / MXFP8: E8M0 block scales [E][N][K / 32]
  int N = 0, K = 0;
  void* out = nullptr;                // pair rows, ldo elements apart
  int64_t ldo = 0;
  // shared expert (Ws == nullptr: none)
  const void* As = nullptr;           // bf16
  int64_t lda_s = 0;
  const void* Ws = nullptr;           // [Ns][Ks] bf16
  int Ns = 0, Ks = 0, Ts = 0;
  void* out_s = nullptr;              // ksplit_s > 1: ksplit_s fp32 slabs [Ts][ldo_s]
  int64_t ldo_s = 0;
  int ksplit_s = 1;                   // K ranges of the shared slot (kStoreF32 only)
  int store = 0;                      // kStoreF32: fp32 acc; kStoreSqRelu: bf16(relu(acc)^2);
                                      // kStoreBF16: bf16(acc)
  // slices of the routed experts from the dispatch step (see DispatchExtras); n_slices NULL:
  // no routed units (a dense weight-streaming product through the shared slot alone)
  const int32_t* slice_e = nullptr;
  const int32_t* slice_r = nullptr;
  const int32_t* n_slices = nullptr;
};
hipError_t launch_stream(const StreamParams& p, hipStream_t s);

// out[t, n] = store(sum over s of part[s][t][n]) for the S fp32 slabs [T][ld] of a split
// weight-streaming product (slab order), store as in StreamStore.
hipError_t launch_reduce_slabs(const float* part, int S, int T, int N, int64_t ld, void* out,
                               int64_t ldo, int mode, hipStream_t s);

// Size of the per-device library-owned workspace of moe_layer_forward_static
// (MOE_STATIC_WORKSPACE_BYTES in the C header).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;

// Device address and size of that workspace on the current device. The address is looked up
// once per device (hipGetSymbolAddress) and kept; nothing is allocated.
hipError_t static_scratch(void** ptr, size_t* bytes);

}  // namespace moe
