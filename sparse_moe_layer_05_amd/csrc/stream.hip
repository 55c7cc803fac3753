// Decode path of the MoE layer on gfx950. With tens of tokens, reading the touched experts'
// weights dominates and the layer is HBM-bound ("NVIDIA Nemotron 3: Efficient and Open
// Intelligence", section 2.2, latency-oriented deployment), so each touched expert's weight
// matrix is read from HBM once.
//
// Work comes in units of 16 weight rows against one slice of at most 16 tokens of one expert
// (the shared expert's tokens are cut into slices the same way). All units cost about the same,
// so a persistent grid of 1024 waves (one per SIMD) deals them out round robin: unit j goes to
// wave j mod 1024, and no wave holds more than one unit more than any other. Waves are numbered
// die by die, so units with neighbouring numbers run at the same time on one die: the slices of
// one expert that share weight rows take the rows from HBM once and from that die's L2 after.
//
// Loads are double buffered in registers with a one-unit lookahead: while a unit streams, the
// next one is resolved, and its first k batch is in flight while the current unit's last batch
// is multiplied. Inside a unit the weights are the matrix-core "A" operand and the tokens the
// "B" operand, loaded straight from HBM into registers (no LDS): bf16 through
// v_mfma_f32_16x16x32_bf16, or e4m3 expert weights with e4m3 token rows through
// v_mfma_scale_f32_16x16x128_f8f6f4 (per-channel and per-token scales applied to the result,
// as in "Nemotron 3 Nano：開放高效的 MoE 混合 Mamba-Transformer 智能體推理模型", section 4,
// FP8 expert weights).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kUnitRows = 16;
constexpr int kStreamWaves = 1024;  // 4 per CU, one per SIMD

// Unit lookups are wave-uniform: reading them through the constant address space makes them
// scalar loads, which are counted apart from the vector loads, so a lookup never waits for the
// weight loads in flight (vector loads complete in issue order).
typedef const __attribute__((address_space(4))) int32_t* scalar_ptr;
__device__ __forceinline__ int sload(const int32_t* p, int i) { return ((scalar_ptr)p)[i]; }

// One lane's part of a 16 x 16 output block: 4 consecutive columns n .. n+3 of row orow.
__device__ __forceinline__ void store_block(const f32x4_t v, void* out, int64_t ldo,
                                            int64_t orow, int n, int mode) {
  if (mode == kStoreF32) {
    *(float4*)((float*)out + orow * ldo + n) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    const bool sq = mode == kStoreSqRelu;
    const uint2 q = make_uint2(pack_bf16x2(sq ? sqrelu(v[0]) : v[0], sq ? sqrelu(v[1]) : v[1]),
                               pack_bf16x2(sq ? sqrelu(v[2]) : v[2], sq ? sqrelu(v[3]) : v[3]));
    *(uint2*)((uint16_t*)out + orow * ldo + n) = q;
  }
}

// Operand element types: bf16 (v_mfma_f32_16x16x32_bf16, 32 elements = 64 bytes per k step)
// and OCP e4m3 (v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales, 128 elements = 128
// bytes per k step). Lane l holds 16 (bf16) or 32 (e4m3) consecutive bytes of row l % 16 at byte
// (l / 16) * LB of each step, for weights and tokens alike; the result register r of lane l is
// out[weight row (l / 16) * 4 + r][token l % 16].
template <Elt T> struct Fmt;
template <> struct Fmt<Elt::BF16> {
  static constexpr int SB = 64, LB = 16, U = 6;  // step bytes, lane bytes, steps per batch
};
template <> struct Fmt<Elt::FP8> {
  static constexpr int SB = 128, LB = 32, U = 3;
};

// A unit resolved to this lane's pointers. Pointers include the lane's byte offset within a k
// step.
struct Unit {
  const uint8_t* w;   // this lane's weight row
  const uint8_t* a;   // this lane's token row
  void* out;
  int64_t ldo;
  int64_t orow;       // output row of this lane's token
  int n;              // first of this lane's 4 output columns
  int N, KB;          // weight rows of the expert, bytes of a row (K * element size)
  int nrows;          // tokens of the slice
  float asc;          // e4m3: this lane's token scale
  const float* wsc;   // e4m3: scales of this lane's 4 output channels
};

// Streams the units this wave is dealt: first, first + nwaves, ... below total;
// resolve(u, unit) fills a unit.
//
// Each k batch covers U steps; the loads of the following batch (of this unit or, after its last
// batch, of the next unit) are in flight while a batch is multiplied. The two register sets swap
// roles between consecutive batches and are never copied (a copy would wait for the loads in
// flight). kFull (every row spans at least one batch): the last batch of a unit is moved back to
// end exactly at K and the weight chunks it shares with the batch before are zeroed, so every
// load of a batch is one base address plus an immediate offset and every batch issues the same
// number of loads, which lets the compiler wait for exactly the batch it multiplies. !kFull:
// loads of the last batch past K are clamped into the row and zeroed.
template <Elt T, bool kFull, class Resolve>
__device__ void stream_units(int first, int total, int nwaves, int lane, int mode,
                             Resolve resolve) {
  constexpr int SB = Fmt<T>::SB, LB = Fmt<T>::LB, U = Fmt<T>::U, C = LB / 16, BB = U * SB;
  const int lb = (lane >> 4) * LB;  // this lane's byte offset within a step
  const int tr = lane & 15;
  if (first >= total) return;
  Unit cur, nxt;
  int u = first;
  resolve(u, cur);
  int un = u + nwaves < total ? u + nwaves : -1;
  if (un >= 0) resolve(un, nxt);

  auto nbat_of = [&](int KB) { return cdiv(KB, BB); };
  auto kbase = [&](int KB, int b) { return kFull ? min(b * BB, KB - BB) : b * BB; };
  // loads of batch b of unit s, or of batch 0 of unit o when other is set (chosen field by
  // field: choosing a whole unit would put both in memory)
  auto issue = [&](const Unit& s, const Unit& o, bool other, int b, uint4* wf, uint4* xf) {
    const int KB = other ? o.KB : s.KB;
    const uint8_t* w = other ? o.w : s.w;
    const uint8_t* a = other ? o.a : s.a;
    const int kb = kbase(KB, b);
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int off = kFull ? kb + q * SB + c * 16 : min(kb + q * SB + c * 16, KB - 16 - lb);
        wf[q * C + c] = *(const uint4*)(w + off);
        xf[q * C + c] = *(const uint4*)(a + off);
      }
  };
  // last batch b: zero the weight chunks that an earlier batch already covered, or that lie
  // past K
  auto mask = [&](int KB, int b, uint4* wf) {
    const int kb = kbase(KB, b);
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int at = kb + q * SB + lb + c * 16;
        const bool drop = kFull ? at < b * BB : at >= KB;
        if (drop) wf[q * C + c] = make_uint4(0, 0, 0, 0);
      }
  };
  auto mfma = [&](const uint4* wf, const uint4* xf, int q, f32x4_t acc) {
    if constexpr (T == Elt::BF16) {
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wf[q]),
                                                    __builtin_bit_cast(bf16x8_t, xf[q]), acc,
                                                    0, 0, 0);
    } else {
      const uint4 w0 = wf[2 * q], w1 = wf[2 * q + 1], x0 = xf[2 * q], x1 = xf[2 * q + 1];
      const i32x8_t wa = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                          (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
      const i32x8_t xa = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xa, acc, 0, 0, 0, 127, 0, 127);
    }
  };

  uint4 w0[U * C], w1[U * C], x0[U * C], x1[U * C];
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int b = 0, nbat = nbat_of(cur.KB);
  // One k batch: put the following batch in flight into (wnxt, xnxt), multiply (wcur, xcur).
  // After a wave's last unit the following batch re-reads the unit's first one (unused) so that
  // the load count stays the same. Returns false once the wave is done.
  auto step = [&](uint4* wcur, uint4* xcur, uint4* wnxt, uint4* xnxt) {
    const bool last = b + 1 == nbat;
    issue(cur, nxt, last && un >= 0, last ? 0 : b + 1, wnxt, xnxt);
    if (last) mask(cur.KB, b, wcur);
#pragma unroll
    for (int q = 0; q < U; ++q) acc = mfma(wcur, xcur, q, acc);
    if (!last) {
      ++b;
      return true;
    }
    // unit done: acc[r] = out[token tr][n + r]; lanes holding a real token store
    if (tr < cur.nrows && cur.n < cur.N) {
      if constexpr (T == Elt::FP8) {
        const float4 sc = *(const float4*)cur.wsc;
        acc[0] *= cur.asc * sc.x;
        acc[1] *= cur.asc * sc.y;
        acc[2] *= cur.asc * sc.z;
        acc[3] *= cur.asc * sc.w;
      }
      store_block(acc, cur.out, cur.ldo, cur.orow, cur.n, mode);
    }
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (un < 0) return false;
    cur = nxt;
    u = un;
    b = 0;
    nbat = nbat_of(cur.KB);
    un = u + nwaves < total ? u + nwaves : -1;
    if (un >= 0) resolve(un, nxt);
    return true;
  };
  issue(cur, cur, false, 0, w0, x0);
  for (;;) {
    if (!step(w0, x0, w1, x1)) break;
    if (!step(w1, x1, w0, x0)) break;
  }
}

// The units of one launch that this wave streams with operands of type T: the shared expert's
// (shared_part, bf16 only) and the routed experts' (routed_part).
template <Elt T>
__device__ void run_units(const StreamParams& p, int wave, int nwaves, bool shared_part,
                          bool routed_part) {
  constexpr int EB = T == Elt::FP8 ? 1 : 2;
  constexpr int LB = Fmt<T>::LB;
  const int lane = threadIdx.x & 63;
  const int tr = lane & 15;
  const int lb = (lane >> 4) * LB;

  // units [0, nsh): the shared expert, row block major, its token slices minor (slices that
  // share weight rows run side by side and share them through L2);
  // units [nsh, nsh + nrt): the routed slices, slice major, row block minor (neighbouring waves
  // stream neighbouring rows of one expert's matrix)
  const int nss = p.Ws && shared_part ? cdiv(p.Ts, kSliceRows) : 0;
  const int nsh = nss ? cdiv(p.Ns, kUnitRows) * nss : 0;
  const int nsl = p.n_slices && routed_part ? sload(p.n_slices, 0) : 0;
  const int nbr = cdiv(p.N, kUnitRows);
  const int nrt = nbr * nsl;
  const uint8_t* As = (const uint8_t*)p.As;
  const uint8_t* Ws = (const uint8_t*)p.Ws;
  const uint8_t* A = (const uint8_t*)p.A;
  const uint8_t* W = (const uint8_t*)p.W;
  auto resolve = [&](int u, Unit& s) {
    int n0, src;
    if (u < nsh) {
      n0 = (u / nss) * kUnitRows;
      const int r0 = (u % nss) * kSliceRows;
      s.nrows = min(p.Ts - r0, kSliceRows);
      s.orow = r0 + tr;
      src = r0 + min(tr, s.nrows - 1);
      s.a = As + (int64_t)src * p.lda_s * EB + lb;
      s.w = Ws + (int64_t)min(n0 + tr, p.Ns - 1) * p.Ks * EB + lb;
      s.out = p.out_s;
      s.ldo = p.ldo_s;
      s.N = p.Ns;
      s.KB = p.Ks * EB;
      s.asc = 1.f;
      s.wsc = nullptr;
    } else {
      const int v = u - nsh;
      const int i = v / nbr;
      n0 = (v % nbr) * kUnitRows;
      const int g = sload(p.slice_e, i);
      const int r0 = sload(p.slice_r, i);
      s.nrows = min(sload(p.offs, g + 1) - r0, kSliceRows);
      s.orow = r0 + tr;
      src = r0 + min(tr, s.nrows - 1);
      if (p.gather) {
        // the slice's token rows as scalar loads; each lane keeps its own
        int row = 0;
#pragma unroll
        for (int j = 0; j < kSliceRows; ++j) {
          const int r = sload(p.gather, r0 + min(j, s.nrows - 1));
          if (tr == j) row = r;
        }
        src = row;
      }
      s.a = A + (int64_t)src * p.lda * EB + lb;
      s.w = W + ((int64_t)g * p.N + min(n0 + tr, p.N - 1)) * p.K * EB + lb;
      s.out = p.out;
      s.ldo = p.ldo;
      s.N = p.N;
      s.KB = p.K * EB;
      s.asc = p.a_scale ? p.a_scale[src] : 1.f;
      s.wsc = p.w_scale ? p.w_scale + (int64_t)g * p.N + min(n0 + (lane >> 4) * 4, p.N - 4)
                        : nullptr;
    }
    s.n = n0 + (lane >> 4) * 4;
  };
  // the shifted-last-batch path needs every unit's row to span at least one batch
  constexpr int BB = Fmt<T>::U * Fmt<T>::SB;
  const bool full = (nrt == 0 || p.K * EB >= BB) && (nsh == 0 || p.Ks * EB >= BB);
  if (full)
    stream_units<T, true>(wave, nsh + nrt, nwaves, lane, p.store, resolve);
  else
    stream_units<T, false>(wave, nsh + nrt, nwaves, lane, p.store, resolve);
}

// One launch: every wave streams its share of the units (the shared expert's first, bf16 only,
// then the routed experts').
template <Elt T>
__global__ __launch_bounds__(256, 1) void stream_kernel(StreamParams p) {
  // waves numbered die by die: consecutive numbers share a CU, then a die
  const int wave = xcd_logical_block(blockIdx.x, gridDim.x) * 4 +
                   __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  run_units<T>(p, wave, gridDim.x * 4, T == Elt::BF16, true);
}

}  // namespace

hipError_t launch_stream(const StreamParams& p, hipStream_t s) {
  static_assert(kStreamWaves / 4 % kXcds == 0, "the wave numbering needs whole dies");
  if (p.fp8) {
    // e4m3 launches carry routed units only, with both scale sets
    if (p.Ws || !p.a_scale || !p.w_scale) return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_kernel<Elt::FP8>, dim3(kStreamWaves / 4), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(stream_kernel<Elt::BF16>, dim3(kStreamWaves / 4), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace moe
