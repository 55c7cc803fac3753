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
// One wave per token. Lane l holds experts l, l + 64, ...; k rounds of a wave-wide arg-max
// over (key desc, expert asc) by butterfly shuffles, the winner's owner lane retiring it.
// s = fp32(1 / (1 + exp(-z))) is evaluated in double so that the rounded score does not depend
// on a particular single-precision exp; key = s + b is one binary32 addition.
template <int NPER>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int nsplit,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ gates,
                                                   float* __restrict__ logits_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float key[NPER], sc[NPER], zs[NPER];
  // K-slice partials (split-K router), summed in slice order; the loads of one slice for all of
  // this lane's experts are independent, so they are issued together
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
      const float z = zs[i];
      if (logits_out) logits_out[(int64_t)t * E + e] = z;
      const float s = (float)(1.0 / (1.0 + exp(-(double)z)));
      sc[i] = s;
      key[i] = s + bias[e];
    } else {
      sc[i] = 0.f;
      key[i] = -INFINITY;
    }
  }
  uint32_t taken = 0;
  float sum = 0.f, mine = 0.f;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY, bs = 0.f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = lane + 64 * i;
      const bool free = !((taken >> i) & 1u) && e < E;
      if (free && (key[i] > bk || (key[i] == bk && e < be))) {
        bk = key[i];
        be = e;
        bs = sc[i];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ok = __shfl_xor(bk, m);
      const int oe = __shfl_xor(be, m);
      const float os = __shfl_xor(bs, m);
      if (ok > bk || (ok == bk && oe < be)) {
        bk = ok;
        be = oe;
        bs = os;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    sum += bs;                       // same order j = 0..k-1 on every lane: deterministic
    if (lane == j) mine = bs;
    if (lane == 0) idx[(int64_t)t * k + j] = be;
  }
  if (lane < k) gates[(int64_t)t * k + lane] = mine / sum;
}

// --------------------------------------------------------------------------------- dispatch
// Tokens are cut into chunks of 256 (one workgroup each). Inside a chunk, an LDS bitmask per
// expert records which of the 256 tokens chose it; the popcount of the bits below a token is
// its stable rank inside the chunk, and chunk bases from a prefix over chunks make the global
// order "experts ascending, tokens ascending" without any order-deciding atomics.
__device__ __forceinline__ uint64_t build_masks(const int32_t* __restrict__ idx, int T, int E,
                                                int k, uint32_t* mask, int t, int tid) {
  for (int i = tid; i < E * 8; i += kDispatchChunk) mask[i] = 0;
  __syncthreads();
  uint64_t valid = 0;  // bit j: pair (t, j) is kept (k <= 64)
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(int64_t)t * k + j];
      if ((unsigned)e < (unsigned)E) {
        const uint32_t bit = 1u << (tid & 31);
        const uint32_t old = atomicOr(&mask[e * 8 + (tid >> 5)], bit);
        if (!(old & bit)) valid |= 1ull << j;  // a repeated expert in one token is dropped
      }
    }
  }
  __syncthreads();
  return valid;
}

__global__ __launch_bounds__(kDispatchChunk) void dispatch_count(const int32_t* __restrict__ idx,
                                                                 int T, int E, int k,
                                                                 int32_t* __restrict__ ccount) {
  extern __shared__ uint32_t mask[];
  const int tid = threadIdx.x, c = blockIdx.x;
  build_masks(idx, T, E, k, mask, c * kDispatchChunk + tid, tid);
  for (int e = tid; e < E; e += kDispatchChunk) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) n += __popc(mask[e * 8 + w]);
    ccount[(int64_t)c * E + e] = n;
  }
}

// Block-wide inclusive scans (Hillis-Steele) of four per-thread values over 1024 threads.
__device__ __forceinline__ void scan4(int32_t (*s)[1024], int e) {
  for (int d = 1; d < 1024; d <<= 1) {
    int v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = e >= d ? s[q][e - d] : 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q][e] += v[q];
    __syncthreads();
  }
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
  int tot = 0;
  if (e < E)
    for (int c = 0; c < nchunks; ++c) tot += ccount[(int64_t)c * E + e];
  dispatch_totals(e, E, tot, bm, s, counts, offsets, mt_start, ex);
  if (e < E) {
    int run = s[0][e] - tot;
    for (int c = 0; c < nchunks; ++c) {
      cbase[(int64_t)c * E + e] = run;
      run += ccount[(int64_t)c * E + e];
    }
  }
}

// All of dispatch in one workgroup when T fits one chunk (T <= 256): masks, totals, scatter.
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
  const int tid = threadIdx.x;
  for (int i = tid; i < E * 8; i += 1024) mask[i] = 0;
  __syncthreads();
  uint64_t valid = 0;
  if (tid < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(int64_t)tid * k + j];
      if ((unsigned)e < (unsigned)E) {
        const uint32_t bit = 1u << (tid & 31);
        const uint32_t old = atomicOr(&mask[e * 8 + (tid >> 5)], bit);
        if (!(old & bit)) valid |= 1ull << j;
      }
    }
  }
  __syncthreads();
  int tot = 0;
  if (tid < E)
#pragma unroll
    for (int w = 0; w < 8; ++w) tot += __popc(mask[tid * 8 + w]);
  dispatch_totals(tid, E, tot, bm, s, counts, offsets, mt_start, ex);
  // s[0][e] - count[e] is the base of expert e; counts are re-derived from the masks below.
  if (tid < T) {
    const int w = tid >> 5;
    const uint32_t below = (1u << (tid & 31)) - 1u;
    for (int j = 0; j < k; ++j) {
      if (!((valid >> j) & 1ull)) {
        pos[(int64_t)tid * k + j] = -1;
        continue;
      }
      const int e = idx[(int64_t)tid * k + j];
      int cnt = 0, rank = __popc(mask[e * 8 + w] & below);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        cnt += __popc(mask[e * 8 + q]);
        if (q < w) rank += __popc(mask[e * 8 + q]);
      }
      const int r = s[0][e] - cnt + rank;
      perm[r] = tid;
      pos[(int64_t)tid * k + j] = r;
    }
  }
}

__global__ __launch_bounds__(kDispatchChunk) void dispatch_scatter(
    const int32_t* __restrict__ idx, int T, int E, int k, const int32_t* __restrict__ cbase,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  extern __shared__ uint32_t mask[];
  const int tid = threadIdx.x, c = blockIdx.x, t = c * kDispatchChunk + tid;
  const uint64_t valid = build_masks(idx, T, E, k, mask, t, tid);
  if (t >= T) return;
  const int w = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
  for (int j = 0; j < k; ++j) {
    if (!((valid >> j) & 1ull)) {
      pos[(int64_t)t * k + j] = -1;
      continue;
    }
    const int e = idx[(int64_t)t * k + j];
    int rank = __popc(mask[e * 8 + w] & below);
    for (int q = 0; q < w; ++q) rank += __popc(mask[e * 8 + q]);
    const int r = cbase[(int64_t)c * E + e] + rank;
    perm[r] = t;
    pos[(int64_t)t * k + j] = r;
  }
}

// ---------------------------------------------------------------------------------- combine
// One workgroup per token; each thread owns 8 consecutive columns (one 16-byte bf16 load or two
// fp32 loads per source row). Sum order: S (fp32) first, then j = 0..k-1.
template <Elt YT, Elt OT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ Y, int64_t ldy,
                                                      const float* __restrict__ S, int64_t lds,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ gates, int T,
                                                      int D, int k, void* __restrict__ out,
                                                      int64_t ldo) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < D; c += blockDim.x * 8) {
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
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int j = 0; j < k; ++j) {
      const int r = pos[(int64_t)t * k + j];
      if (r < 0) continue;
      const float g = gates[(int64_t)t * k + j];
      float v[8];
      load8(Y, r, ldy, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
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
// One workgroup per row: amax by wave shuffles + LDS, then e4m3 codes of x * (448 / amax).
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x,
                                                         int64_t ldx, int H,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  __shared__ float s_max[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint16_t* row = x + (int64_t)t * ldx;
  float m = 0.f;
  for (int c = tid * 8; c < H; c += 256 * 8) {
    const uint4 v = *(const uint4*)(row + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] & 0xFFFF)));
      m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] >> 16)));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) s_max[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float inv = amax > 0.f ? 448.f / amax : 1.f;   // codes = e4m3(x * inv)
  if (tid == 0) scale[t] = amax > 0.f ? amax / 448.f : 1.f;
  for (int c = tid * 8; c < H; c += 256 * 8) {
    const uint4 v = *(const uint4*)(row + c);
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
  }
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
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_TOPK(NPER) hipLaunchKernelGGL(topk_kernel<NPER>, grid, block, 0, s, logits, nsplit, b, \
                                          T, E, k, idx, gates, logits_out)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

void router_split(int T, int E, int H, int* nsplit, int* kchunk) {
  const int tiles = cdiv(T, 128) * cdiv(E, 128);
  const int n = (tiles == 0 || tiles >= 128) ? 1 : std::max(1, std::min(256 / tiles, H / 128));
  const int chunk = cdiv(cdiv(H, n), 64) * 64;   // whole 64-wide K-steps per slice
  *kchunk = chunk;
  *nsplit = cdiv(H, chunk);
}

hipError_t launch_dispatch(const int32_t* idx, int T, int E, int k, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* scratch,
                           int bm, int32_t* mt_start, const DispatchExtras& ex, hipStream_t s) {
  const int nch = (T + kDispatchChunk - 1) / kDispatchChunk;
  if (nch <= 1) {
    hipLaunchKernelGGL(dispatch_small, dim3(1), dim3(1024), 0, s, idx, T, E, k, bm, counts,
                       offsets, perm, pos, mt_start, ex);
    return hipGetLastError();
  }
  int32_t* ccount = scratch;
  int32_t* cbase = scratch + (size_t)nch * E;
  const size_t lds = (size_t)E * 8 * sizeof(uint32_t);
  hipLaunchKernelGGL(dispatch_count, dim3(nch), dim3(kDispatchChunk), lds, s, idx, T, E, k,
                     ccount);
  hipLaunchKernelGGL(dispatch_scan, dim3(1), dim3(1024), 0, s, ccount, nch, E, bm, cbase, counts,
                     offsets, mt_start, ex);
  hipLaunchKernelGGL(dispatch_scatter, dim3(nch), dim3(kDispatchChunk), lds, s, idx, T, E, k,
                     cbase, perm, pos);
  return hipGetLastError();
}

hipError_t launch_combine(const void* Y, Elt y_elt, int64_t ldy, const float* S, int64_t lds,
                          const int32_t* pos, const float* gates, int T, int D, int k, void* out,
                          Elt out_elt, int64_t ldo, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int threads = D / 8 >= 256 ? 256 : ((D / 8 + 63) / 64) * 64;
  const dim3 grid(T), block(threads);
  if (y_elt == Elt::BF16 && out_elt == Elt::BF16)
    hipLaunchKernelGGL((combine_kernel<Elt::BF16, Elt::BF16>), grid, block, 0, s, Y, ldy, S, lds, pos, gates, T, D, k, out, ldo);
  else if (y_elt == Elt::F32 && out_elt == Elt::BF16)
    hipLaunchKernelGGL((combine_kernel<Elt::F32, Elt::BF16>), grid, block, 0, s, Y, ldy, S, lds, pos, gates, T, D, k, out, ldo);
  else if (y_elt == Elt::F32 && out_elt == Elt::F32)
    hipLaunchKernelGGL((combine_kernel<Elt::F32, Elt::F32>), grid, block, 0, s, Y, ldy, S, lds, pos, gates, T, D, k, out, ldo);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t ldx, int T, int H, uint8_t* q,
                             float* scale, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(T), dim3(256), 0, s, x, ldx, H, q, scale);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, const float* target, int E, float gamma,
                              float* b, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(1024), 0, s, counts, target, E, gamma, b);
  return hipGetLastError();
}

}  // namespace moe

