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
// "B" operand of v_mfma_f32_16x16x32_bf16: lane l loads 16 bytes of weight row (l % 16) at k
// offset 8 * (l / 16) of each 32-wide k step straight from HBM into registers (no LDS).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kUnitRows = 16;
constexpr int kStreamWaves = 1024;  // 4 per CU, one per SIMD
constexpr int UN = 6;               // 32-wide k steps per load batch

// Unit lookups are wave-uniform: reading them through the constant address space makes them
// scalar loads, which are counted apart from the vector loads, so a lookup never waits for the
// weight loads in flight (vector loads complete in issue order).
typedef const __attribute__((address_space(4))) int32_t* scalar_ptr;
__device__ __forceinline__ int sload(const int32_t* p, int i) { return ((scalar_ptr)p)[i]; }

__device__ __forceinline__ bf16x8_t ld16(const uint16_t* p) { return *(const bf16x8_t*)p; }

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

// A unit resolved to this lane's pointers. Pointers include the lane's k offset within a
// 32-wide step.
struct Unit {
  const uint16_t* w;  // this lane's weight row
  const uint16_t* a;  // this lane's token row
  void* out;
  int64_t ldo;
  int64_t orow;       // output row of this lane's token
  int n;              // first of this lane's 4 output columns
  int N, K;           // weight rows and columns of the expert
  int nrows;          // tokens of the slice
};

// Streams the units this wave is dealt: first, first + nwaves, ... below total;
// resolve(u, unit) fills a unit.
//
// Each k batch covers U steps of 32 columns; the loads of the following batch (of this unit or,
// after its last batch, of the next unit) are in flight while a batch is multiplied. The two
// register sets swap roles between consecutive batches and are never copied (a copy would wait
// for the loads in flight). kFull (every K >= 32*U): the last batch of a unit is moved back to
// end exactly at K and the weight chunks it shares with the batch before are zeroed, so every
// load of a batch is one base address plus an immediate offset and every batch issues the same
// number of loads, which lets the compiler wait for exactly the batch it multiplies. !kFull:
// loads of the last batch past K are clamped into the row and zeroed.
template <int U, bool kFull, class Resolve>
__device__ void stream_units(int first, int total, int nwaves, int lane, int mode,
                             Resolve resolve) {
  const int kq = (lane >> 4) * 8;
  const int tr = lane & 15;
  if (first >= total) return;
  Unit cur, nxt;
  int u = first;
  resolve(u, cur);
  int un = u + nwaves < total ? u + nwaves : -1;
  if (un >= 0) resolve(un, nxt);

  auto nbat_of = [&](int K) { return cdiv(K, 32 * U); };
  auto kbase = [&](int K, int b) { return kFull ? min(b * 32 * U, K - 32 * U) : b * 32 * U; };
  // loads of batch b of unit s, or of batch 0 of unit o when other is set (chosen field by
  // field: choosing a whole unit would put both in memory)
  auto issue = [&](const Unit& s, const Unit& o, bool other, int b, bf16x8_t* wf,
                   bf16x8_t* xf) {
    const int K = other ? o.K : s.K;
    const uint16_t* w = other ? o.w : s.w;
    const uint16_t* a = other ? o.a : s.a;
    const int kb = kbase(K, b);
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int kk = kFull ? kb + q * 32 : min(kb + q * 32, K - 8 - kq);
      wf[q] = ld16(w + kk);
      xf[q] = ld16(a + kk);
    }
  };
  // last batch b: zero the weight chunks that an earlier batch already covered, or that lie
  // past K
  auto mask = [&](int K, int b, bf16x8_t* wf) {
    const int kb = kbase(K, b);
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const bool drop = kFull ? kb + q * 32 + kq < b * 32 * U : kb + q * 32 + kq >= K;
      if (drop) wf[q] = bf16x8_t{};
    }
  };

  bf16x8_t w0[U], w1[U], x0[U], x1[U];
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int b = 0, nbat = nbat_of(cur.K);
  // One k batch: put the following batch in flight into (wnxt, xnxt), multiply (wcur, xcur).
  // After a wave's last unit the following batch re-reads the unit's first one (unused) so that
  // the load count stays the same. Returns false once the wave is done.
  auto step = [&](bf16x8_t* wcur, bf16x8_t* xcur, bf16x8_t* wnxt, bf16x8_t* xnxt) {
    const bool last = b + 1 == nbat;
    issue(cur, nxt, last && un >= 0, last ? 0 : b + 1, wnxt, xnxt);
    if (last) mask(cur.K, b, wcur);
#pragma unroll
    for (int q = 0; q < U; ++q)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wcur[q], xcur[q], acc, 0, 0, 0);
    if (!last) {
      ++b;
      return true;
    }
    // unit done: acc[r] = out[token tr][n + r]; lanes holding a real token store
    if (tr < cur.nrows && cur.n < cur.N) store_block(acc, cur.out, cur.ldo, cur.orow, cur.n, mode);
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (un < 0) return false;
    cur = nxt;
    u = un;
    b = 0;
    nbat = nbat_of(cur.K);
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

__global__ __launch_bounds__(256, 1) void stream_kernel(StreamParams p) {
  const int lane = threadIdx.x & 63;
  const int tr = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int nwaves = gridDim.x * 4;
  // waves numbered die by die: consecutive numbers share a CU, then a die
  const int wave = xcd_logical_block(blockIdx.x, gridDim.x) * 4 +
                   __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // units [0, nsh): the shared expert, row block major, its token slices minor (slices that
  // share weight rows run side by side and share them through L2);
  // units [nsh, nsh + nrt): the routed slices, slice major, row block minor (neighbouring waves
  // stream neighbouring rows of one expert's matrix)
  const int nss = p.Ws ? cdiv(p.Ts, kSliceRows) : 0;
  const int nsh = nss ? cdiv(p.Ns, kUnitRows) * nss : 0;
  const int nsl = p.n_slices ? sload(p.n_slices, 0) : 0;
  const int nbr = cdiv(p.N, kUnitRows);
  const int nrt = nbr * nsl;
  auto resolve = [&](int u, Unit& s) {
    int n0, src;
    if (u < nsh) {
      n0 = (u / nss) * kUnitRows;
      const int r0 = (u % nss) * kSliceRows;
      s.nrows = min(p.Ts - r0, kSliceRows);
      s.orow = r0 + tr;
      src = r0 + min(tr, s.nrows - 1);
      s.a = p.As + (int64_t)src * p.lda_s + kq;
      s.w = p.Ws + (int64_t)min(n0 + tr, p.Ns - 1) * p.Ks + kq;
      s.out = p.out_s;
      s.ldo = p.ldo_s;
      s.N = p.Ns;
      s.K = p.Ks;
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
      s.a = p.A + (int64_t)src * p.lda + kq;
      s.w = p.W + (int64_t)g * p.N * p.K + (int64_t)min(n0 + tr, p.N - 1) * p.K + kq;
      s.out = p.out;
      s.ldo = p.ldo;
      s.N = p.N;
      s.K = p.K;
    }
    s.n = n0 + (lane >> 4) * 4;
  };
  // the shifted-last-batch path needs every unit's K to span at least one batch
  const bool full = (nrt == 0 || p.K >= 32 * UN) && (nsh == 0 || p.Ks >= 32 * UN);
  if (full)
    stream_units<UN, true>(wave, nsh + nrt, nwaves, lane, p.store, resolve);
  else
    stream_units<UN, false>(wave, nsh + nrt, nwaves, lane, p.store, resolve);
}

}  // namespace

hipError_t launch_stream(const StreamParams& p, hipStream_t s) {
  static_assert(kStreamWaves / 4 % kXcds == 0, "the wave numbering needs whole dies");
  hipLaunchKernelGGL(stream_kernel, dim3(kStreamWaves / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
