// Router top-k, dispatch, combine and fp8 activation quantisation for the MoE layer (gfx950).
//
// Routing follows the Nemotron 3 MoE layer: the router picks k of E experts per token
// ("NVIDIA AI发布了Nemotron 3：一款混合Mamba Transformer MoE堆栈", section
// "混合Mamba Transformer MoE架构") with an aux-loss-free per-expert bias that only steers the
// selection ("Nemotron 3 Nano：開放高效的 MoE 混合 Mamba-Transformer 智能體推理模型", section
// 2.2); sigmoid scores renormalised over the selected experts are the gate weights.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

#include <algorithm>

namespace moe {
namespace {

// ------------------------------------------------------------------------------------ top-k
// Order-preserving map of a float's bits to an unsigned integer (larger float, larger integer).
__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Wave-wide maximum of a 64-bit value by DPP row shifts and row broadcasts (lane 63 ends with
// the result over all 64 lanes), then read back from lane 63 as a wave-uniform value. A lane
// whose DPP source is outside its row (or whose row is masked off) combines with 0, the
// identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_max_step_u64(uint64_t v) {
  const uint32_t lo =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xf, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xf, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step_u64<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step_u64<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step_u64<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step_u64<0x118, 0xf>(v);  // row_shr:8: lane 15 of each row holds the row's max
  v = dpp_max_step_u64<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step_u64<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// k rounds of selection over the keys of one token; lane l holds experts l, l + 64, ... Each
// expert carries one 64-bit value, its key's order-preserving bits above its inverted index, so
// that one wave-wide maximum per round yields the largest key and, among equal keys, the lowest
// expert (a float maximum followed by an index minimum took two reductions a round). The values
// are distinct, so round j retires the largest value below round j-1's: nothing is cleared and
// no score is read inside a round, whose cost is one dependent chain. Lane j keeps round j's
// winner; the scores are fetched afterwards and summed in round order on every lane.
// TREE: each lane's largest value below the last winner as a tree over its slots (shorter chain;
// faster with one token per workgroup, slower with four waves of tokens per workgroup).
// Writes the k experts (descending key) and their gates (scores renormalised over the
// selection).
template <int NPER, bool TREE>
__device__ __forceinline__ void select_topk(const float* key, const float* sc, int lane, int E,
                                            int k, int32_t* __restrict__ idx_t,
                                            float* __restrict__ gates_t) {
  uint64_t c[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    c[i] = e < E ? ((uint64_t)okey(key[i]) << 32) | (uint32_t)~e : 0;
  }
  uint64_t prev = ~0ull, mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t m = 0;
    if constexpr (TREE) {
      uint64_t a[NPER];
#pragma unroll
      for (int i = 0; i < NPER; ++i) a[i] = c[i] < prev ? c[i] : 0;
#pragma unroll
      for (int w = 1; w < NPER; w *= 2)
#pragma unroll
        for (int i = 0; i + w < NPER; i += 2 * w) a[i] = a[i + w] > a[i] ? a[i + w] : a[i];
      m = a[0];
    } else {
#pragma unroll
      for (int i = 0; i < NPER; ++i) m = c[i] < prev && c[i] > m ? c[i] : m;
    }
    prev = wave_max_u64(m);
    if (lane == j) mine = prev;
  }
  const int be = (int)~(uint32_t)mine;
  const int slot = lane < k ? be >> 6 : 0, owner = lane < k ? be & 63 : 0;
  float bs = 0.f;  // the score lane `owner` holds in slot `slot`
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const float t = __int_as_float(__builtin_amdgcn_ds_bpermute(owner << 2, __float_as_int(sc[i])));
    bs = slot == i ? t : bs;
  }
  float sum = 0.f;  // the same order j = 0..k-1 on every lane: deterministic
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bs), j));
  if (lane < k) {
    idx_t[lane] = be;
    gates_t[lane] = bs / sum;
  }
}

// One wave per token, four tokens per workgroup (many tokens): lane l holds experts l, l + 64, ...
// and adds the K-slice partials of a split router in slice order; scores, keys and selection as
// in topk_kernel.
template <int NPER>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ logits,
                                                        int nsplit, const float* __restrict__ bias,
                                                        int T, int E, int k,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ gates,
                                                        float* __restrict__ logits_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float zs[NPER], key[NPER], sc[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    zs[i] = e < E ? logits[(int64_t)t * E + e] : 0.f;
  }
#pragma unroll 4
  for (int q = 1; q < nsplit; ++q) {
    float v[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? logits[((int64_t)q * T + t) * E + e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i) zs[i] += v[i];
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      if (logits_out) logits_out[(int64_t)t * E + e] = zs[i];
      const float s = (float)(1.0 / (1.0 + exp(-(double)zs[i])));
      sc[i] = s;
      key[i] = s + bias[e];
    } else {
      sc[i] = 0.f;
      key[i] = -INFINITY;
    }
  }
  select_topk<NPER, false>(key, sc, lane, E, k, idx + (int64_t)t * k, gates + (int64_t)t * k);
}

// One workgroup of 256 threads per token. Phase 1: thread i owns experts i, i + 256, ... (EPT of
// them): it adds the nsplit K-slice partials of the split-K router in slice order (the loads of
// up to 16 slices of all its experts are issued together), then forms the score and the key.
// s = fp32(1 / (1 + exp(-z))) is evaluated in double so that the rounded score does not depend
// on a particular single-precision exp; key = s + b is one binary32 addition. Phase 2: wave 0
// selects; lane l holds experts l, l + 64, ... and k rounds of a wave-wide arg-max over
// (key desc, expert asc) by DPP retire one winner each.
template <int NPER>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int nsplit,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ gates,
                                                   float* __restrict__ logits_out) {
  constexpr int EPT = NPER >= 4 ? NPER / 4 : 1;  // experts per thread in phase 1
  constexpr int SLAB = 16;                        // K slices whose loads are in flight together
  __shared__ float key_l[64 * NPER], sc_l[64 * NPER];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  float z[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + 256 * i;
    z[i] = e < E ? logits[(int64_t)t * E + e] : 0.f;
  }
  for (int q0 = 1; q0 < nsplit; q0 += SLAB) {
    float v[EPT][SLAB];
#pragma unroll
    for (int i = 0; i < EPT; ++i)
#pragma unroll
      for (int q = 0; q < SLAB; ++q) {
        const int e = tid + 256 * i;
        v[i][q] = e < E && q0 + q < nsplit ? logits[((int64_t)(q0 + q) * T + t) * E + e] : 0.f;
      }
#pragma unroll
    for (int i = 0; i < EPT; ++i)
#pragma unroll
      for (int q = 0; q < SLAB; ++q)
        if (q0 + q < nsplit) z[i] += v[i][q];
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + 256 * i;
    if (e < 64 * NPER) {
      if (e < E) {
        if (logits_out) logits_out[(int64_t)t * E + e] = z[i];
        const float sg = (float)(1.0 / (1.0 + exp(-(double)z[i])));
        sc_l[e] = sg;
        key_l[e] = sg + bias[e];
      } else {
        sc_l[e] = 0.f;
        key_l[e] = -INFINITY;
      }
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  float key[NPER], sc[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    key[i] = key_l[lane + 64 * i];
    sc[i] = sc_l[lane + 64 * i];
  }
  select_topk<NPER, true>(key, sc, lane, E, k, idx + (int64_t)t * k, gates + (int64_t)t * k);
}

// --------------------------------------------------------------------------------- dispatch
// Tokens are cut into chunks of CH = 256, 128 or 64 (one workgroup each, thread i = token i of
// the chunk; dispatch_chunk picks CH). Inside a chunk, an LDS bitmask per expert (CH / 32 words) records which of the
// chunk's tokens chose it; the popcount of the bits below a token is its stable rank inside the
// chunk, and chunk bases from a prefix over chunks make the global order "experts ascending,
// tokens ascending" without any order-deciding atomics. The masks are stored word-major, word w
// of expert e at w * E + e, so that the lanes of a wave, which set bits for unrelated experts,
// and a sweep over experts spread over the LDS banks (expert-major rows of 8 words put every
// expert on one of 8 banks). Smaller chunks give more workgroups: LatentMoE prefill (4096
// tokens, 24 slots each) had 16 workgroups of 256 tokens, now 64 of 64.
template <int CH>
__device__ __forceinline__ uint64_t build_masks(const int32_t* __restrict__ idx, int T, int E,
                                                int k, uint32_t* mask, int t, int tid) {
  constexpr int W = CH / 32;  // mask words per expert
  for (int i = tid; i < E * W; i += CH) mask[i] = 0;
  __syncthreads();
  uint64_t valid = 0;  // bit j: pair (t, j) is kept (k <= 64)
  if (t < T) {
    const uint32_t bit = 1u << (tid & 31);
    for (int j0 = 0; j0 < k; j0 += 8) {  // a token's slots, 8 loads in flight, in slot order
      int ev[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ev[i] = j0 + i < k ? idx[(int64_t)t * k + j0 + i] : -1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((unsigned)ev[i] >= (unsigned)E) continue;
        const uint32_t old = atomicOr(&mask[(tid >> 5) * E + ev[i]], bit);
        if (!(old & bit)) valid |= 1ull << (j0 + i);  // a repeated expert in one token is dropped
      }
    }
  }
  __syncthreads();
  return valid;
}

template <int CH>
__global__ __launch_bounds__(CH) void dispatch_count(const int32_t* __restrict__ idx, int T, int E,
                                                     int k, int32_t* __restrict__ ccount) {
  extern __shared__ uint32_t mask[];
  const int tid = threadIdx.x, c = blockIdx.x;
  build_masks<CH>(idx, T, E, k, mask, c * CH + tid, tid);
  for (int e = tid; e < E; e += CH) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < CH / 32; ++w) n += __popc(mask[w * E + e]);
    ccount[(int64_t)c * E + e] = n;
  }
}

// Block-wide inclusive scans of four per-thread values over 1024 threads (16 waves): wave scans
// by shuffles, wave 0 scans the 16 wave totals, and each wave adds the totals before it.
__device__ __forceinline__ void scan4(int32_t (*s)[1024], int e) {
  __shared__ int32_t wt[16][4];
  const int lane = e & 63, w = e >> 6;
  int v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = s[q][e];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = __shfl_up(v[q], d);
      if (lane >= d) v[q] += o;
    }
  if (lane == 63)
#pragma unroll
    for (int q = 0; q < 4; ++q) wt[w][q] = v[q];
  __syncthreads();
  // wave 0: inclusive scan of the wave totals (lanes 16 g + i all hold total i; each group of
  // 16 lanes scans its own copy)
  int u[4] = {0, 0, 0, 0}, own[4] = {0, 0, 0, 0};
  if (w == 0) {
    const int i = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) own[q] = u[q] = wt[i][q];
#pragma unroll
    for (int d = 1; d < 16; d <<= 1)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int o = __shfl_up(u[q], d);
        if (i >= d) u[q] += o;
      }
  }
  __syncthreads();
  if (w == 0 && lane < 16)
#pragma unroll
    for (int q = 0; q < 4; ++q) wt[lane][q] = u[q] - own[q];  // totals of the waves before
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) s[q][e] = v[q] + wt[w][q];
  __syncthreads();
}

// Per-expert totals -> counts, offsets, M-tile prefix, decode slices; thread e = expert e.
// s[0..2] end as the inclusive scans of counts, M-tiles and slices (s[3] is unused).
__device__ __forceinline__ void dispatch_totals(int e, int E, int tot, int bm,
                                                int32_t (*s)[1024], int32_t* counts,
                                                int32_t* offsets, int32_t* mt_start,
                                                const DispatchExtras& ex) {
  const int mt = bm > 0 ? (tot + bm - 1) / bm : 0;
  const bool in = e < E;
  const int ns = in ? (tot + kSliceRows - 1) / kSliceRows : 0;
  s[0][e] = in ? tot : 0;
  s[1][e] = in ? mt : 0;
  s[2][e] = ns;
  s[3][e] = 0;
  __syncthreads();
  scan4(s, e);
  if (in) {
    const int base = s[0][e] - tot;
    counts[e] = tot;
    offsets[e] = base;
    if (e == E - 1) offsets[E] = s[0][e];
    if (mt_start) {
      mt_start[e] = s[1][e] - mt;
      if (e == E - 1) mt_start[E] = s[1][e];
    }
    if (ex.slice_e) {
      const int first = s[2][e] - ns;
      for (int j = 0; j < ns; ++j) {
        ex.slice_e[first + j] = e;
        ex.slice_r[first + j] = base + j * kSliceRows;
      }
      if (e == E - 1) ex.n_slices[0] = s[2][e];
    }
  }
}

// One workgroup of 1024 threads, thread e = expert e.
__global__ __launch_bounds__(1024) void dispatch_scan(const int32_t* __restrict__ ccount,
                                                      int nchunks, int E, int bm,
                                                      int32_t* __restrict__ cbase,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ mt_start,
                                                      DispatchExtras ex) {
  __shared__ int32_t s[4][1024];
  const int e = threadIdx.x;
  // chunk counts read 8 at a time with their loads in flight
  int tot = 0;
  if (e < E)
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c0 + i < nchunks ? ccount[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) tot += v[i];
    }
  dispatch_totals(e, E, tot, bm, s, counts, offsets, mt_start, ex);
  if (e < E) {
    int run = s[0][e] - tot;
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c0 + i < nchunks ? ccount[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (c0 + i >= nchunks) break;
        cbase[(int64_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
  }
}

// All of dispatch in one workgroup when T fits one chunk (T <= 256): masks, totals, scatter.
// Work is spread over the T*k (token, slot) pairs, thread i taking pairs i, i + 1024, ... (at
// most 16). A pair is kept when its expert is in range and no earlier slot of the same token
// chose that expert (the first occurrence wins, decided without atomics).
constexpr int kSmallPairs = 16;   // pairs per thread: T*k <= 256*64
constexpr int kSmallStage = 8;    // slots per token above which the selections go to LDS
template <bool STAGED>
__global__ __launch_bounds__(1024) void dispatch_small(const int32_t* __restrict__ idx, int T,
                                                       int E, int k, int bm,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ pos,
                                                       int32_t* __restrict__ mt_start,
                                                       DispatchExtras ex) {
  __shared__ uint32_t mask[kMaxE * 8];
  __shared__ int32_t s[4][1024];
  extern __shared__ int16_t sel[];  // STAGED: the T * k selections, -1 where out of range
  const int tid = threadIdx.x;
  const int P = T * k;
  // STAGED (many slots per token): the earlier slots of a pair's token are read from LDS
  // rather than L2; with few slots the loads from L2 measured faster
  constexpr bool staged = STAGED;
  for (int i = tid; i < E * 8; i += 1024) mask[i] = 0;
  int ex_of[kSmallPairs];
  uint32_t keep = 0;
#pragma unroll
  for (int c = 0; c < kSmallPairs; ++c) {
    const int pr = tid + 1024 * c;
    ex_of[c] = pr < P ? idx[pr] : -1;
    if (staged && pr < P) sel[pr] = (int16_t)((unsigned)ex_of[c] < (unsigned)E ? ex_of[c] : -1);
  }
  __syncthreads();  // mask cleared, selections staged
#pragma unroll
  for (int c = 0; c < kSmallPairs; ++c) {
    const int pr = tid + 1024 * c;
    const int e = ex_of[c];
    if (pr < P && (unsigned)e < (unsigned)E) {
      const int t = pr / k, j = pr - t * k;
      bool dup = false;  // independent loads, no early exit
      if constexpr (staged)
        for (int jj = 0; jj < j; ++jj) dup |= sel[t * k + jj] == e;
      else
        for (int jj = 0; jj < j; ++jj) dup |= idx[(int64_t)t * k + jj] == e;
      if (!dup) keep |= 1u << c;
    }
  }
#pragma unroll
  for (int c = 0; c < kSmallPairs; ++c)
    if ((keep >> c) & 1u) {
      const int t = (tid + 1024 * c) / k;
      atomicOr(&mask[(t >> 5) * E + ex_of[c]], 1u << (t & 31));
    }
  __syncthreads();
  int tot = 0;
  if (tid < E)
#pragma unroll
    for (int w = 0; w < 8; ++w) tot += __popc(mask[w * E + tid]);
  dispatch_totals(tid, E, tot, bm, s, counts, offsets, mt_start, ex);
  // s[0][e] - count[e] is the base of expert e; counts are re-derived from the masks below.
#pragma unroll
  for (int c = 0; c < kSmallPairs; ++c) {
    const int pr = tid + 1024 * c;
    if (pr >= P) continue;
    if (!((keep >> c) & 1u)) {
      pos[pr] = -1;
      continue;
    }
    const int e = ex_of[c];
    const int t = pr / k, w = t >> 5;
    const uint32_t below = (1u << (t & 31)) - 1u;
    int cnt = 0, rank = __popc(mask[w * E + e] & below);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      cnt += __popc(mask[q * E + e]);
      if (q < w) rank += __popc(mask[q * E + e]);
    }
    const int r = s[0][e] - cnt + rank;
    perm[r] = t;
    pos[pr] = r;
  }
}

template <int CH>
__global__ __launch_bounds__(CH) void dispatch_scatter(const int32_t* __restrict__ idx, int T,
                                                       int E, int k,
                                                       const int32_t* __restrict__ cbase,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ pos) {
  extern __shared__ uint32_t mask[];
  const int tid = threadIdx.x, c = blockIdx.x, t = c * CH + tid;
  const uint64_t valid = build_masks<CH>(idx, T, E, k, mask, t, tid);
  if (t >= T) return;
  const int w = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
  for (int j0 = 0; j0 < k; j0 += 8) {  // 8 slots at a time: their loads in flight together
    int ev[8], base[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + i;
      ev[i] = j < k && ((valid >> j) & 1ull) ? idx[(int64_t)t * k + j] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) base[i] = ev[i] >= 0 ? cbase[(int64_t)c * E + ev[i]] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + i;
      if (j >= k) continue;
      if (ev[i] < 0) {
        pos[(int64_t)t * k + j] = -1;
        continue;
      }
      const int e = ev[i];
      int rank = __popc(mask[w * E + e] & below);
      for (int q = 0; q < w; ++q) rank += __popc(mask[q * E + e]);
      const int r = base[i] + rank;
      perm[r] = t;
      pos[(int64_t)t * k + j] = r;
    }
  }
}

// ---------------------------------------------------------------------------------- combine
// One workgroup per token; each thread owns 8 consecutive columns (one 16-byte bf16 load or two
// fp32 loads per source row). Sum order: S (fp32; its ns slabs in order) first, then j = 0..k-1.
template <Elt YT, Elt OT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ Y, int64_t ldy,
                                                      const float* __restrict__ S, int64_t lds,
                                                      int ns, int64_t s_slab,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ gates, int T,
                                                      int D, int k, void* __restrict__ out,
                                                      int64_t ldo) {
  // workgroup (t, y) covers columns [y * cpb, (y + 1) * cpb) of token t, cpb = D / gridDim.y
  // rounded up to whole 8-column groups of the block
  const int t = blockIdx.x;
  const int cpb = cdiv(cdiv(D, gridDim.y), 8) * 8;
  const int cend = min(D, (int)(blockIdx.y + 1) * cpb);
  for (int c = blockIdx.y * cpb + threadIdx.x * 8; c < cend; c += blockDim.x * 8) {
    float acc[8];
    auto load8 = [&](const void* base, int64_t row, int64_t ld, float* v) {
      if constexpr (YT == Elt::BF16) {
        const uint4 q = *(const uint4*)((const uint16_t*)base + row * ld + c);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFF);
          v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        }
      } else {
        const float4 a = *(const float4*)((const float*)base + row * ld + c);
        const float4 b = *(const float4*)((const float*)base + row * ld + c + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
    };
    if (S) {
      const float4 a = *(const float4*)(S + t * lds + c);
      const float4 b = *(const float4*)(S + t * lds + c + 4);
      acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
      acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
      for (int q = 1; q < ns; ++q) {
        const float* Sq = S + q * s_slab + t * lds + c;
        const float4 e = *(const float4*)Sq, f = *(const float4*)(Sq + 4);
        acc[0] += e.x; acc[1] += e.y; acc[2] += e.z; acc[3] += e.w;
        acc[4] += f.x; acc[5] += f.y; acc[6] += f.z; acc[7] += f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    // rows j0 .. j0+7 are loaded together, then added in j order
    constexpr int JB = 8;
    for (int j0 = 0; j0 < k; j0 += JB) {
      float v[JB][8], g[JB];
      bool ok[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj;
        const int r = j < k ? pos[(int64_t)t * k + j] : -1;
        ok[jj] = r >= 0;
        g[jj] = ok[jj] ? gates[(int64_t)t * k + j] : 0.f;
        if (ok[jj]) load8(Y, r, ldy, v[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj)
        if (ok[jj])
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[jj], v[jj][i], acc[i]);
    }
    if constexpr (OT == Elt::BF16) {
      uint4 q;
      q.x = pack_bf16x2(acc[0], acc[1]);
      q.y = pack_bf16x2(acc[2], acc[3]);
      q.z = pack_bf16x2(acc[4], acc[5]);
      q.w = pack_bf16x2(acc[6], acc[7]);
      *(uint4*)((uint16_t*)out + (int64_t)t * ldo + c) = q;
    } else {
      float* o = (float*)out + (int64_t)t * ldo + c;
      *(float4*)o = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *(float4*)(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// -------------------------------------------------------------------------------- quantise
// One wave per row, four rows per workgroup: amax by a wave reduction (no barrier), then e4m3
// codes of x * (448 / amax). A row of up to 64 * 8 * kQuantRegs elements is read once and kept
// in registers; longer rows are read a second time for the codes. (A workgroup per row spent
// most of its time on the block reduction's barrier for rows of a few KB.)
constexpr int kQuantRegs = 8;
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x,
                                                         int64_t ldx, int T, int H,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* row = x + (int64_t)t * ldx;
  uint4 keep[kQuantRegs];
  float m = 0.f;
  auto amax8 = [&](const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] & 0xFFFF)));
      m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] >> 16)));
    }
  };
#pragma unroll
  for (int r = 0; r < kQuantRegs; ++r) {
    const int c = (r * 64 + lane) * 8;
    keep[r] = c < H ? *(const uint4*)(row + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < kQuantRegs; ++r) amax8(keep[r]);
  for (int c = (kQuantRegs * 64 + lane) * 8; c < H; c += 64 * 8) amax8(*(const uint4*)(row + c));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float amax = m;
  const float inv = amax > 0.f ? 448.f / amax : 1.f;   // codes = e4m3(x * inv)
  if (lane == 0) scale[t] = amax > 0.f ? amax / 448.f : 1.f;
  auto codes8 = [&](const uint4 v, int c) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float f0 = bf16_bits_to_f32(w[2 * h] & 0xFFFF) * inv;
      const float f1 = bf16_bits_to_f32(w[2 * h] >> 16) * inv;
      const float f2 = bf16_bits_to_f32(w[2 * h + 1] & 0xFFFF) * inv;
      const float f3 = bf16_bits_to_f32(w[2 * h + 1] >> 16) * inv;
      o[h] = cvt_fp8x2(f0, f1) | (cvt_fp8x2(f2, f3) << 16);
    }
    *(uint2*)(q + (int64_t)t * H + c) = make_uint2(o[0], o[1]);
  };
#pragma unroll
  for (int r = 0; r < kQuantRegs; ++r) {
    const int c = (r * 64 + lane) * 8;
    if (c < H) codes8(keep[r], c);
  }
  for (int c = (kQuantRegs * 64 + lane) * 8; c < H; c += 64 * 8) codes8(*(const uint4*)(row + c), c);
}

// One workgroup; thread e handles expert e (loops for E > 1024). The mean-load comparison is done
// in integers: sign(sum/E - c) = sign(sum - E*c).
__global__ __launch_bounds__(1024) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                           const float* __restrict__ target,
                                                           int E, float gamma,
                                                           float* __restrict__ b) {
  __shared__ long long total;
  if (!target) {
    long long part = 0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) part += counts[e];
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    atomicAdd((unsigned long long*)&total, (unsigned long long)part);  // exact: integer sum
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int sgn;
    if (target) {
      const float d = target[e] - (float)counts[e];
      sgn = (d > 0.f) - (d < 0.f);
    } else {
      const long long d = total - (long long)E * counts[e];
      sgn = (d > 0) - (d < 0);
    }
    if (sgn) b[e] = b[e] + (sgn > 0 ? gamma : -gamma);
  }
}

}  // namespace

hipError_t launch_topk(const float* logits, int nsplit, const float* b, int T, int E, int k,
                       int32_t* idx, float* gates, float* logits_out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // few tokens with a split router: a workgroup per token adds the partials; else a wave per
  // token
  const bool wg = nsplit > 1 && T < 1024;
  const dim3 grid(wg ? T : (T + 3) / 4), block(256);
#define MOE_TOPK(NPER)                                                                         \
  do {                                                                                         \
    if (wg)                                                                                    \
      hipLaunchKernelGGL(topk_kernel<NPER>, grid, block, 0, s, logits, nsplit, b, T, E, k, idx, \
                         gates, logits_out);                                                   \
    else                                                                                       \
      hipLaunchKernelGGL(topk_wave_kernel<NPER>, grid, block, 0, s, logits, nsplit, b, T, E, k, \
                         idx, gates, logits_out);                                              \
  } while (0)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

void router_split(int T, int E, int H, int* nsplit, int* kchunk) {
  // Few output tiles leave most CUs idle: split K so that the launch reaches about 256 tiles
  // (slices of at least 128 columns) below 128 tiles, about 512 (slices of at least 256 columns)
  // below 512. The top-k kernel adds the slices' partial logits in slice order.
  const int tiles = cdiv(T, 128) * cdiv(E, 128);
  int n = 1;
  if (tiles > 0 && tiles < 128) n = std::max(1, std::min(256 / tiles, H / 128));
  else if (tiles >= 128 && tiles < 512) n = std::max(1, std::min(512 / tiles, H / 256));
  const int chunk = cdiv(cdiv(H, n), 64) * 64;   // whole 64-wide K-steps per slice
  *kchunk = chunk;
  *nsplit = cdiv(H, chunk);
}

void router_split_f32(int T, int E, int H, int* nsplit, int* kchunk) {
  // The fp32 router's 64 x 64 tiles take one K-step of 16 at a time: with few tiles, split K
  // toward about 256 workgroups, in slices of at least 32 columns (a multiple of 16).
  const int tiles = cdiv(T, 64) * cdiv(E, 64);
  int n = 1;
  if (tiles > 0 && tiles < 256) n = std::max(1, std::min(256 / tiles, H / 32));
  const int chunk = cdiv(cdiv(H, n), 16) * 16;
  *kchunk = chunk;
  *nsplit = cdiv(H, chunk);
}

hipError_t launch_dispatch(const int32_t* idx, int T, int E, int k, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* scratch,
                           int bm, int32_t* mt_start, const DispatchExtras& ex, hipStream_t s) {
  if (T <= kDispatchSmallT) {
    if (k > kSmallStage)
      hipLaunchKernelGGL(dispatch_small<true>, dim3(1), dim3(1024),
                         (size_t)T * k * sizeof(int16_t), s, idx, T, E, k, bm, counts, offsets,
                         perm, pos, mt_start, ex);
    else
      hipLaunchKernelGGL(dispatch_small<false>, dim3(1), dim3(1024), 0, s, idx, T, E, k, bm,
                         counts, offsets, perm, pos, mt_start, ex);
    return hipGetLastError();
  }
  const int ch = dispatch_chunk(T, k), nch = (int)(((int64_t)T + ch - 1) / ch);
  int32_t* ccount = scratch;
  int32_t* cbase = scratch + (size_t)nch * E;
  const size_t lds = (size_t)E * (ch / 32) * sizeof(uint32_t);
  auto run = [&](auto count, auto scatter) {
    hipLaunchKernelGGL(count, dim3(nch), dim3(ch), lds, s, idx, T, E, k, ccount);
    hipLaunchKernelGGL(dispatch_scan, dim3(1), dim3(1024), 0, s, ccount, nch, E, bm, cbase,
                       counts, offsets, mt_start, ex);
    hipLaunchKernelGGL(scatter, dim3(nch), dim3(ch), lds, s, idx, T, E, k, cbase, perm, pos);
  };
  if (ch == 64)
    run(dispatch_count<64>, dispatch_scatter<64>);
  else if (ch == 128)
    run(dispatch_count<128>, dispatch_scatter<128>);
  else
    run(dispatch_count<256>, dispatch_scatter<256>);
  return hipGetLastError();
}

hipError_t launch_combine(const void* Y, Elt y_elt, int64_t ldy, const float* S, int64_t lds,
                          const int32_t* pos, const float* gates, int T, int D, int k, void* out,
                          Elt out_elt, int64_t ldo, hipStream_t s, int ns, int64_t s_slab) {
  if (T <= 0) return hipSuccess;
  if (ns < 1 || (ns > 1 && !S)) return hipErrorInvalidValue;
  // Many tokens: one workgroup per token. Few tokens (decode): a token's columns are split over
  // workgroups of one wave, 512 columns each, so that enough of them run at once.
  const bool few = T < 1024;
  const int threads = few ? 64 : (D / 8 >= 256 ? 256 : ((D / 8 + 63) / 64) * 64);
  const dim3 grid(T, few ? cdiv(D, 512) : 1), block(threads);
  if (y_elt == Elt::BF16 && out_elt == Elt::BF16)
    hipLaunchKernelGGL((combine_kernel<Elt::BF16, Elt::BF16>), grid, block, 0, s, Y, ldy, S, lds, ns, s_slab, pos, gates, T, D, k, out, ldo);
  else if (y_elt == Elt::F32 && out_elt == Elt::BF16)
    hipLaunchKernelGGL((combine_kernel<Elt::F32, Elt::BF16>), grid, block, 0, s, Y, ldy, S, lds, ns, s_slab, pos, gates, T, D, k, out, ldo);
  else if (y_elt == Elt::F32 && out_elt == Elt::F32)
    hipLaunchKernelGGL((combine_kernel<Elt::F32, Elt::F32>), grid, block, 0, s, Y, ldy, S, lds, ns, s_slab, pos, gates, T, D, k, out, ldo);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t ldx, int T, int H, uint8_t* q,
                             float* scale, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(cdiv(T, 4)), dim3(256), 0, s, x, ldx, T, H, q,
                     scale);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, const float* target, int E, float gamma,
                              float* b, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(1024), 0, s, counts, target, E, gamma, b);
  return hipGetLastError();
}

}  // namespace moe

