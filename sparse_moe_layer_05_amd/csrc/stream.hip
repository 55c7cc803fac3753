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
// v_mfma_f32_16x16x32_bf16, or 8-bit / 4-bit expert weights with e4m3 token rows through
// v_mfma_scale_f32_16x16x128_f8f6f4: e4m3 weights with per-channel scales applied to the result
// ("Nemotron 3 Nano：開放高效的 MoE 混合 Mamba-Transformer 智能體推理模型", section 4, FP8 expert
// weights), or OCP microscaling MXFP4 (E2M1) / MXFP8 (E4M3) weights whose E8M0 block scales the
// matrix core applies itself (the native gfx950 counterpart of the micro-block scaled FP4 in
// "NVIDIA Nemotron 3: Efficient and Open Intelligence", section 2.4). Token scales are applied
// to the result.
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

// Operand layouts. A k step is KS elements, one matrix-core instruction. In every step lane l
// holds weight row l % 16 and token row l % 16; the result register r of lane l is
// out[weight row (l / 16) * 4 + r][token l % 16]. With g = l / 16, the bytes a lane loads in a
// step are CW (weights) or CA (tokens) 16-byte chunks at byte LW * g + c * CWS, or
// LA * g + c * CAS, from the step's start:
//  - bf16 (16x16x32 bf16): 8 elements 8g .. 8g + 7 of the step, one chunk;
//  - e4m3 x e4m3 with unit block scales (16x16x128): the lane's 32 bytes 32g .. 32g + 31; any
//    order of k serves as long as both operands use it;
//  - with real block scales the matrix core's own order of k matters. It takes an e4m3
//    operand's k as 16g .. 16g + 15 and 64 + 16g .. 64 + 16g + 15 (two chunks 64 bytes apart),
//    an E2M1 operand's k as 32g .. 32g + 31 (one chunk of 16 bytes, element 2i in the low
//    nibble of byte i), and the E8M0 scale a lane passes as covering k 32g .. 32g + 31 of its
//    row. So MXFP4 / MXFP8 weights and the e4m3 tokens they meet are loaded in that order.
template <Elt T> struct Fmt;
// R: blocks of 16 weight rows per unit, sharing the unit's token loads; U(R): steps per batch.
// bf16 routed launches take two blocks: a unit's token bytes otherwise equal its weight bytes,
// and two blocks measured 2% faster on the Nano decode step (four slower, from the longer tail
// of fewer units); three where every unit is whole (the launch picks them). Dense launches of the shared slot alone have few units and keep one block;
// their batches of 5 steps keep the kernel at 136 registers, so that one of its waves fits on a
// SIMD beside one of any routed kernel (at most 368 of 512) and the two launches overlap.
template <> struct Fmt<Elt::BF16> {
  static constexpr int KS = 32, R = 2;            // elements per step, routed row blocks
  static constexpr int U(int r) { return r == 1 ? 5 : 4; }
  static constexpr int WH = 4, AB = 2;           // weight half-bytes / token bytes per element
  static constexpr int CW = 1, LW = 16, CWS = 0;
  static constexpr int CA = 1, LA = 16, CAS = 0;
};
// 8-bit weights: two row blocks per unit as well (measured 2-11% faster per decode step than one).
template <> struct Fmt<Elt::FP8> {
  static constexpr int KS = 128, R = 2;
  static constexpr int U(int) { return 3; }
  static constexpr int WH = 2, AB = 1;
  static constexpr int CW = 2, LW = 32, CWS = 16;
  static constexpr int CA = 2, LA = 32, CAS = 16;
};
// 4-bit weights: a 16-row unit would carry half the bytes of an 8-bit one for the same fixed
// cost per unit and twice as many token bytes per weight byte; two row blocks restore both.
// Rows of at most kMx4ShortK elements take four row blocks in batches of 4 steps instead of two
// in batches of 8: a batch then does not overrun a 512-element row, and half as many units carry
// the per-unit costs (LatentMoE decode, K of 1024 and 512: 176 -> 150 us per step; Nano decode,
// K of 2688 and 1856, measured slower with four).
constexpr int kMx4ShortK = 1024;
template <> struct Fmt<Elt::MXFP4> {
  static constexpr int KS = 128, R = 2;
  static constexpr int U(int r) { return r == 4 ? 4 : 8; }
  static constexpr int WH = 1, AB = 1;
  static constexpr int CW = 1, LW = 16, CWS = 0;
  static constexpr int CA = 2, LA = 16, CAS = 64;
};
template <> struct Fmt<Elt::MXFP8> {
  static constexpr int KS = 128, R = 2;
  static constexpr int U(int) { return 4; }
  static constexpr int WH = 2, AB = 1;
  static constexpr int CW = 2, LW = 16, CWS = 64;
  static constexpr int CA = 2, LA = 16, CAS = 64;
};
template <Elt T> constexpr bool kBlockScaled = T == Elt::MXFP4 || T == Elt::MXFP8;
static_assert(Fmt<Elt::MXFP4>::U(2) % 4 == 0 && Fmt<Elt::MXFP4>::U(4) % 4 == 0 &&
                  Fmt<Elt::MXFP4>::KS == 128,
              "wide scale loads take a batch's scales 4 steps (16 blocks of 32) at a time");
constexpr int kMxBlock = 32;  // elements per E8M0 scale

// A unit resolved to this lane's pointers. Pointers include the lane's byte offset within a k
// step.
struct Unit {
  const uint8_t* w;   // this lane's weight row (row block 0)
  const uint8_t* a;   // this lane's token row
  const uint8_t* wx;  // MXFP4 / MXFP8: E8M0 scales of this lane's weight row, from block g
  int64_t w1;         // bytes from this lane's weight row to its row in block 1, clamped to the
                      // last row (bf16 and e4m3; block-scaled matrices use a fixed stride)
  void* out;
  int64_t ldo;
  int64_t orow;       // output row of this lane's token
  int n;              // first of this lane's 4 output columns (row block r: n + 16 r)
  int N, K;           // weight rows of the expert, elements of a row
  int nrows;          // tokens of the slice
  float asc;          // e4m3 tokens: this lane's token scale
  const float* wsc;   // FP8: the expert's output-channel scales
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
template <Elt T, int R, bool kFull, bool kWideScale, class Resolve>
__device__ void stream_units(int first, int total, int nwaves, int lane, int mode,
                             Resolve resolve) {
  using F = Fmt<T>;
  constexpr int KS = F::KS, U = F::U(R), CW = F::CW, CA = F::CA, BK = U * KS;
  constexpr int SW = KS * F::WH / 2, SA = KS * F::AB;  // bytes of a step
  constexpr bool kMx = kBlockScaled<T>;
  const int g = lane >> 4;
  const int lbw = g * F::LW, lba = g * F::LA;  // this lane's byte offsets within a step
  const int tr = lane & 15;
  if (first >= total) return;
  Unit cur, nxt;
  int u = first;
  resolve(u, cur);
  int un = u + nwaves < total ? u + nwaves : -1;
  if (un >= 0) resolve(un, nxt);

  auto nbat_of = [&](int K) { return cdiv(K, BK); };
  auto kbase = [&](int K, int b) { return kFull ? min(b * BK, K - BK) : b * BK; };
  // loads of batch b of unit s, or of batch 0 of unit o when other is set (chosen field by
  // field: choosing a whole unit would put both in memory)
  auto issue = [&](const Unit& s, const Unit& o, bool other, int b, uint4* wf, uint4* xf,
                   int* sf) {
    const int K = other ? o.K : s.K;
    const uint8_t* w = other ? o.w : s.w;
    const uint8_t* a = other ? o.a : s.a;
    const int kb = kbase(K, b);
    const int kbw = kb * F::WH / 2, kba = kb * F::AB;
    const int KBw = K * F::WH / 2, KBa = K * F::AB;
    // block-scaled matrices have whole row blocks: their further blocks are a fixed stride away
    // (no per-unit offsets, which keeps the MXFP4 kernel's registers within what lets it share
    // a SIMD with the dense bf16 launches of the side stream)
    const int64_t w1 = R == 1 || kMx ? 0 : (other ? o.w1 : s.w1);
#pragma unroll
    for (int q = 0; q < U; ++q) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CW; ++c) {
          const int off = kbw + q * SW + c * F::CWS;
          wf[(q * R + r) * CW + c] = *(const uint4*)(w + (kMx ? (int64_t)r * kUnitRows * KBw
                                                                : r * w1) +
                                                     (kFull ? off : min(off, KBw - 16 - lbw)));
        }
#pragma unroll
      for (int c = 0; c < CA; ++c) {
        const int off = kba + q * SA + c * F::CAS;
        xf[q * CA + c] = *(const uint4*)(a + (kFull ? off : min(off, KBa - 16 - lba)));
      }
      if constexpr (kMx && !kWideScale) {
        const uint8_t* wx = other ? o.wx : s.wx;
        const int blk = kb / kMxBlock + q * (KS / kMxBlock);
#pragma unroll
        for (int r = 0; r < R; ++r)
          sf[q * R + r] = wx[r * kUnitRows * (K / kMxBlock) +
                             (kFull ? blk : min(blk, K / kMxBlock - 1 - g))];
      }
    }
    if constexpr (kMx && kWideScale) {
      // The batch's 4U scales of a row are 4U contiguous bytes at a 4-byte-aligned offset: one
      // 16-byte load per 4 steps holds this lane's blocks g, g + 4, g + 8, g + 12 (byte g of
      // each dword; the matrix-core call extracts it), where a byte load per step and row block
      // took a vector memory instruction each.
      typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
      const uint8_t* rb = (other ? o.wx : s.wx) - g + kb / kMxBlock;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int h = 0; h < U / 4; ++h) {
          const u32x4a4 v = *(const u32x4a4*)(rb + r * kUnitRows * (K / kMxBlock) + 16 * h);
          sf[(4 * h + 0) * R + r] = (int)v.x;
          sf[(4 * h + 1) * R + r] = (int)v.y;
          sf[(4 * h + 2) * R + r] = (int)v.z;
          sf[(4 * h + 3) * R + r] = (int)v.w;
        }
    }
  };
  // last batch b: zero the weight chunks that an earlier batch already covered, or that lie
  // past K
  auto mask = [&](int K, int b, uint4* wf) {
    const int kb = kbase(K, b);
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const int at = kb + q * KS + (lbw + c * F::CWS) * 2 / F::WH;  // first element
        const bool drop = kFull ? at < b * BK : at >= K;
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (drop) wf[(q * R + r) * CW + c] = make_uint4(0, 0, 0, 0);
      }
  };
  auto cat8 = [](uint4 p, uint4 q) {
    return i32x8_t{(int)p.x, (int)p.y, (int)p.z, (int)p.w, (int)q.x, (int)q.y, (int)q.z,
                   (int)q.w};
  };
  // step q of row block r
  auto mfma = [&](const uint4* wf, const uint4* xf, const int* sf, int q, int r, f32x4_t acc) {
    const int i = q * R + r;
    if constexpr (T == Elt::BF16) {
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wf[i]),
                                                    __builtin_bit_cast(bf16x8_t, xf[q]), acc,
                                                    0, 0, 0);
    } else if constexpr (T == Elt::FP8) {
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          cat8(wf[2 * i], wf[2 * i + 1]), cat8(xf[2 * q], xf[2 * q + 1]), acc, 0, 0, 0, 127, 0,
          127);
    } else if constexpr (T == Elt::MXFP8) {
      const int sc = kWideScale ? (sf[i] >> (8 * g)) & 0xFF : sf[i];
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          cat8(wf[2 * i], wf[2 * i + 1]), cat8(xf[2 * q], xf[2 * q + 1]), acc, 0, 0, 0, sc, 0,
          127);
    } else {
      // E2M1 weights (format 4) fill the operand's first four registers
      const int sc = kWideScale ? (sf[i] >> (8 * g)) & 0xFF : sf[i];
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          cat8(wf[i], make_uint4(0, 0, 0, 0)), cat8(xf[2 * q], xf[2 * q + 1]), acc, 4, 0, 0, sc,
          0, 127);
    }
  };

  uint4 w0[U * R * CW], w1[U * R * CW], x0[U * CA], x1[U * CA];
  int s0[U * R], s1[U * R];
  f32x4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int b = 0, nbat = nbat_of(cur.K);
  // One k batch: put the following batch in flight into (wnxt, xnxt, snxt), multiply the
  // current one. After a wave's last unit the following batch re-reads the unit's first one
  // (unused) so that the load count stays the same. Returns false once the wave is done.
  auto step = [&](uint4* wcur, uint4* xcur, int* scur, uint4* wnxt, uint4* xnxt, int* snxt) {
    const bool last = b + 1 == nbat;
    issue(cur, nxt, last && un >= 0, last ? 0 : b + 1, wnxt, xnxt, snxt);
    if (last) mask(cur.K, b, wcur);
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mfma(wcur, xcur, scur, q, r, acc[r]);
    if (!last) {
      ++b;
      return true;
    }
    // unit done: acc[r][i] = out[token tr][n + 16 r + i]; lanes holding a real token store
#pragma unroll
    for (int r = 0; r < R; ++r) {
      f32x4_t v = acc[r];
      if (tr < cur.nrows && cur.n + kUnitRows * r < cur.N) {
        if constexpr (T == Elt::FP8) {
          const float4 sc = *(const float4*)(cur.wsc + cur.n + kUnitRows * r);
          v[0] *= cur.asc * sc.x;
          v[1] *= cur.asc * sc.y;
          v[2] *= cur.asc * sc.z;
          v[3] *= cur.asc * sc.w;
        } else if constexpr (kMx) {
          v[0] *= cur.asc;
          v[1] *= cur.asc;
          v[2] *= cur.asc;
          v[3] *= cur.asc;
        }
        store_block(v, cur.out, cur.ldo, cur.orow, cur.n + kUnitRows * r, mode);
      }
      acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (un < 0) return false;
    cur = nxt;
    u = un;
    b = 0;
    nbat = nbat_of(cur.K);
    un = u + nwaves < total ? u + nwaves : -1;
    if (un >= 0) resolve(un, nxt);
    return true;
  };
  issue(cur, cur, false, 0, w0, x0, s0);
  for (;;) {
    if (!step(w0, x0, s0, w1, x1, s1)) break;
    if (!step(w1, x1, s1, w0, x0, s0)) break;
  }
}

// The units of one launch that this wave streams with weights of type T: the shared expert's
// (shared_part, bf16 only) and the routed experts' (routed_part).
template <Elt T, int R>
__device__ void run_units(const StreamParams& p, int wave, int nwaves, bool shared_part,
                          bool routed_part) {
  using F = Fmt<T>;
  const int lane = threadIdx.x & 63;
  const int tr = lane & 15;
  const int g = lane >> 4;
  const int lbw = g * F::LW, lba = g * F::LA;

  // units [0, nsh): the shared expert, row block major, its token slices minor (slices that
  // share weight rows run side by side and share them through L2);
  // units [nsh, nsh + nrt): the routed slices, slice major, row block minor (neighbouring waves
  // stream neighbouring rows of one expert's matrix)
  // the shared slot's K may be split in ksplit_s ranges of Kc elements, each written to its own
  // fp32 slab of the output (summed by a separate reduction)
  const int nks = p.ksplit_s > 1 ? p.ksplit_s : 1;
  const int Kc = p.Ks / nks;
  const int nss = p.Ws && shared_part ? cdiv(p.Ts, kSliceRows) * nks : 0;
  const int nsh = nss ? cdiv(p.Ns, kUnitRows * R) * nss : 0;
  const int nsl = p.n_slices && routed_part ? sload(p.n_slices, 0) : 0;
  const int nbr = cdiv(p.N, kUnitRows * R);
  const int nrt = nbr * nsl;
  const uint8_t* As = (const uint8_t*)p.As;
  const uint8_t* Ws = (const uint8_t*)p.Ws;
  const uint8_t* A = (const uint8_t*)p.A;
  const uint8_t* W = (const uint8_t*)p.W;
  auto resolve = [&](int u, Unit& s) {
    int n0, src;
    if (u < nsh) {  // bf16 shared expert (only with T == BF16)
      n0 = (u / nss) * kUnitRows * R;
      const int ks = (u % nss) % nks;  // K range, fastest
      const int r0 = (u % nss) / nks * kSliceRows;
      s.nrows = min(p.Ts - r0, kSliceRows);
      s.orow = r0 + tr;
      src = r0 + min(tr, s.nrows - 1);
      s.a = As + ((int64_t)src * p.lda_s + (int64_t)ks * Kc) * F::AB + lba;
      s.w = Ws + ((int64_t)min(n0 + tr, p.Ns - 1) * p.Ks + (int64_t)ks * Kc) * F::WH / 2 + lbw;
      // full rows of Ks elements apart, also when this unit covers one K range of them
      if constexpr (R > 1)
        s.w1 = (int64_t)(min(n0 + kUnitRows + tr, p.Ns - 1) - min(n0 + tr, p.Ns - 1)) * p.Ks *
               F::WH / 2;
      else
        s.w1 = 0;
      s.wx = nullptr;
      s.out = nks > 1 ? (void*)((float*)p.out_s + (int64_t)ks * p.Ts * p.ldo_s) : p.out_s;
      s.ldo = p.ldo_s;
      s.N = p.Ns;
      s.K = Kc;
      s.asc = 1.f;
      s.wsc = nullptr;
    } else {
      const int v = u - nsh;
      const int i = v / nbr;
      n0 = (v % nbr) * kUnitRows * R;
      const int e = sload(p.slice_e, i);
      const int r0 = sload(p.slice_r, i);
      s.nrows = min(sload(p.offs, e + 1) - r0, kSliceRows);
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
      const int64_t wrow = (int64_t)e * p.N + min(n0 + tr, p.N - 1);
      if constexpr (R > 1 && !kBlockScaled<T>)
        s.w1 = (int64_t)(min(n0 + kUnitRows + tr, p.N - 1) - min(n0 + tr, p.N - 1)) * p.K *
               F::WH / 2;
      else
        s.w1 = 0;
      s.a = A + (int64_t)src * p.lda * F::AB + lba;
      s.w = W + wrow * p.K * F::WH / 2 + lbw;
      s.wx = kBlockScaled<T> ? p.w_mx + wrow * (p.K / kMxBlock) + g : nullptr;
      s.out = p.out;
      s.ldo = p.ldo;
      s.N = p.N;
      s.K = p.K;
      s.asc = p.a_scale ? p.a_scale[src] : 1.f;
      s.wsc = p.w_scale ? p.w_scale + (int64_t)e * p.N : nullptr;  // the expert's scales
    }
    s.n = n0 + g * 4;
  };
  // the shifted-last-batch path needs every unit's row to span at least one batch
  constexpr int BK = F::U(R) * F::KS;
  const bool full = (nrt == 0 || p.K >= BK) && (nsh == 0 || Kc >= BK);
  // MXFP4 kernels load a batch's scales 16 bytes at a time (kWideScale) when a row's scale
  // count is a multiple of 4: a byte load per step and row block becomes one 16-byte load per 4
  // steps (LatentMoE decode 153.5 -> 135.5 us per step with four row blocks, Nano 198.5 -> 193.1
  // with two). Not MXFP8 (two row blocks, 8 byte loads per batch): measured 1.3% slower.
  if constexpr (T == Elt::MXFP4) {
    if (full && (p.K / kMxBlock) % 4 == 0) {
      stream_units<T, R, true, true>(wave, nsh + nrt, nwaves, lane, p.store, resolve);
      return;
    }
  }
  if (full)
    stream_units<T, R, true, false>(wave, nsh + nrt, nwaves, lane, p.store, resolve);
  else
    stream_units<T, R, false, false>(wave, nsh + nrt, nwaves, lane, p.store, resolve);
}

// One launch: every wave streams its share of the units (the shared expert's first, bf16 only,
// then the routed experts').
template <Elt T, int R>
__global__ __launch_bounds__(256, 1) void stream_kernel(StreamParams p) {
  // waves numbered die by die: consecutive numbers share a CU, then a die
  const int wave = xcd_logical_block(blockIdx.x, gridDim.x) * 4 +
                   __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  run_units<T, R>(p, wave, gridDim.x * 4, T == Elt::BF16, true);
}

// out[t, n] = store(sum_s part[s][t][n]) over the S fp32 slabs of a split shared slot, added in
// slab order; 8 columns per thread.
__global__ __launch_bounds__(256) void reduce_slabs_kernel(const float* __restrict__ part, int S,
                                                           int T, int N, int64_t ld,
                                                           void* __restrict__ out, int64_t ldo,
                                                           int mode) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cg = N / 8;
  if (i >= (int64_t)T * cg) return;
  const int t = (int)(i / cg), n = (int)(i % cg) * 8;
  float4 a = *(const float4*)(part + (int64_t)t * ld + n);
  float4 b = *(const float4*)(part + (int64_t)t * ld + n + 4);
  for (int s = 1; s < S; ++s) {
    const float* q = part + ((int64_t)s * T + t) * ld + n;
    const float4 c = *(const float4*)q, d = *(const float4*)(q + 4);
    a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
    b.x += d.x; b.y += d.y; b.z += d.z; b.w += d.w;
  }
  store_block(f32x4_t{a.x, a.y, a.z, a.w}, out, ldo, t, n, mode);
  store_block(f32x4_t{b.x, b.y, b.z, b.w}, out, ldo, t, n + 4, mode);
}

// A dense product through the shared slot alone (bf16, one row block per unit). A wave of it must
// fit on a SIMD beside a wave of the MXFP4 kernel (152 + 360 of the 512 registers): the bf16
// shared expert of a layer with narrow experts streams on a side stream next to those launches.
__global__ __launch_bounds__(256, 1) void stream_dense_kernel(StreamParams p) {
  const int wave = xcd_logical_block(blockIdx.x, gridDim.x) * 4 +
                   __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  run_units<Elt::BF16, 1>(p, wave, gridDim.x * 4, true, false);
}

}  // namespace

hipError_t launch_reduce_slabs(const float* part, int S, int T, int N, int64_t ld, void* out,
                               int64_t ldo, int mode, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (N % 8) return hipErrorInvalidValue;
  const int64_t items = (int64_t)T * (N / 8);
  hipLaunchKernelGGL(reduce_slabs_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s,
                     part, S, T, N, ld, out, ldo, mode);
  return hipGetLastError();
}

hipError_t launch_stream(const StreamParams& p, hipStream_t s) {
  static_assert(kStreamWaves / 4 % kXcds == 0, "the wave numbering needs whole dies");
  const dim3 grid(kStreamWaves / 4), block(256);
  // 8-bit and 4-bit launches carry routed units only, with their scales
  const bool narrow = p.wt != Elt::BF16;
  if (narrow && (p.Ws || !p.a_scale)) return hipErrorInvalidValue;
  // a split shared slot writes fp32 slabs of whole 16-byte chunks of K
  if (p.ksplit_s > 1 && (p.store != kStoreF32 || p.Ks % (p.ksplit_s * 8))) return hipErrorInvalidValue;
  switch (p.wt) {
    case Elt::BF16:
      // routed units (and maybe the shared slot's); three row blocks when every unit is whole
      // (Nano's down projection: 387.0 -> 384.4 us per decode step; the e4m3 and MXFP8
      // kernels measured 3% slower with three)
      if (p.n_slices && p.N % (kUnitRows * 3) == 0 && (!p.Ws || p.Ns % (kUnitRows * 3) == 0))
        hipLaunchKernelGGL((stream_kernel<Elt::BF16, 3>), grid, block, 0, s, p);
      else if (p.n_slices)
        hipLaunchKernelGGL((stream_kernel<Elt::BF16, Fmt<Elt::BF16>::R>), grid, block, 0, s, p);
      else             // a dense product through the shared slot alone
        hipLaunchKernelGGL(stream_dense_kernel, grid, block, 0, s, p);
      break;
    case Elt::FP8:
      if (!p.w_scale) return hipErrorInvalidValue;
      hipLaunchKernelGGL((stream_kernel<Elt::FP8, Fmt<Elt::FP8>::R>), grid, block, 0, s, p);
      break;
    case Elt::MXFP4:
    case Elt::MXFP8:
      // block scales cover 32 elements; a unit's row blocks must lie inside the matrix
      if (!p.w_mx || p.K % kMxBlock) return hipErrorInvalidValue;
      if (p.wt == Elt::MXFP4) {
        if (p.K <= kMx4ShortK && p.N % (kUnitRows * 4) == 0) {
          hipLaunchKernelGGL((stream_kernel<Elt::MXFP4, 4>), grid, block, 0, s, p);
        } else {
          if (p.N % (kUnitRows * Fmt<Elt::MXFP4>::R)) return hipErrorInvalidValue;
          hipLaunchKernelGGL((stream_kernel<Elt::MXFP4, Fmt<Elt::MXFP4>::R>), grid, block, 0, s, p);
        }
      } else {
        if (p.N % (kUnitRows * Fmt<Elt::MXFP8>::R)) return hipErrorInvalidValue;
        hipLaunchKernelGGL((stream_kernel<Elt::MXFP8, Fmt<Elt::MXFP8>::R>), grid, block, 0, s, p);
      }
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
