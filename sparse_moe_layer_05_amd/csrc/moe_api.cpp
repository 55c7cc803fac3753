// C ABI of the gfx950 MoE layer library: argument validation, workspace layout, path choice and
// the launch sequence of one layer call. Everything is enqueued on the caller's stream; nothing
// here allocates, frees or waits.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe.h"
#include "backward.hpp"
#include "gemm_kt.hpp"
#include "kernels.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

struct Plan {
  int path = 0;                 // MOE_PATH_GROUPED or MOE_PATH_STREAM
  Elt act = Elt::BF16, ex = Elt::BF16;
  int T = 0, H = 0, E = 0, k = 0, I = 0, Is = 0, L = 0, D = 0, P = 0, bm = 0;
  size_t logits = 0, idx = 0, gates = 0, counts = 0, offsets = 0, perm = 0, pos = 0;
  size_t zpart = 0, slices = 0;  // router K-slices, decode slices of the touched experts
  size_t S = 0;                               // shared-expert output [T, H] fp32 (grouped path)
  int nsplit = 1, kchunk = 0;
  size_t dscratch = 0, mt_start = 0, xq = 0, sx = 0, hq = 0, sh = 0, xl = 0, z = 0, h = 0, hs = 0;
  size_t Y = 0, total = 0;
  int lsplit = 1;    // K ranges of the streamed projection into the latent width (decode)
  size_t xpart = 0;  // its fp32 slabs [lsplit][T][L]
  int ssplit = 1;    // K ranges of the shared expert's down projection on the decode path (plain
                     // layer): fp32 slabs [ssplit][T][H] after the pair rows of Y
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kNarrowSharedSplit = 4;

int32_t make_plan(const moe_desc_t* d, bool latent_call, Plan* pl) {
  if (!d) return MOE_ERR_INVALID_ARG;
  const int64_t T = d->T, H = d->H, E = d->E, k = d->k, I = d->I, Is = d->I_shared, L = d->latent;
  if (T < 0 || H < 16 || H % 16 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK || I < 16 ||
      I % 16 || Is < 0 || Is % 16 || L < 0 || L % 16)
    return MOE_ERR_INVALID_ARG;
  if (latent_call != (L > 0)) return MOE_ERR_INVALID_ARG;
  if (T * k > INT32_MAX / 2 || T * (H > L ? H : L) > ((int64_t)1 << 40)) return MOE_ERR_INVALID_ARG;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const bool fp8 = d->expert_dtype == MOE_FP8_E4M3;
  const bool mx = d->expert_dtype == MOE_MXFP4 || d->expert_dtype == MOE_MXFP8;
  if (!fp8 && !mx && d->expert_dtype != d->act_dtype) return MOE_ERR_UNSUPPORTED;
  if ((fp8 || mx) && d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  // block-scaled rows are whole 32-element blocks, in both projections
  const int64_t Dw = L ? L : H;
  if (mx && (Dw % 32 || I % 32)) return MOE_ERR_INVALID_ARG;
  if (d->flags & ~(MOE_PATH_MASK | MOE_ROUTING_GIVEN)) return MOE_ERR_INVALID_ARG;
  Plan p;
  p.act = d->act_dtype == MOE_F32 ? Elt::F32 : Elt::BF16;
  p.ex = fp8 ? Elt::FP8
             : d->expert_dtype == MOE_MXFP4 ? Elt::MXFP4
             : d->expert_dtype == MOE_MXFP8 ? Elt::MXFP8 : p.act;
  p.T = (int)T; p.H = (int)H; p.E = (int)E; p.k = (int)k; p.I = (int)I; p.Is = (int)Is;
  p.L = (int)L; p.D = L ? (int)L : (int)H; p.P = (int)(T * k);
  const uint32_t path = d->flags & MOE_PATH_MASK;
  // the decode path streams bf16, e4m3 and block-scaled experts (the last have no other path)
  const bool stream_ok = p.act == Elt::BF16 && (p.ex == Elt::BF16 || fp8 || mx);
  if (path == MOE_PATH_AUTO)
    p.path = (stream_ok && ((int64_t)p.P <= 8 * E || mx)) ? MOE_PATH_STREAM : MOE_PATH_GROUPED;
  else if (path == MOE_PATH_STREAM)
    p.path = stream_ok ? MOE_PATH_STREAM : -1;
  else if (path == MOE_PATH_GROUPED)
    p.path = mx ? -1 : MOE_PATH_GROUPED;
  else
    return MOE_ERR_INVALID_ARG;
  if (p.path < 0) return MOE_ERR_UNSUPPORTED;
  // The matrix-core GEMMs address each operand through 32-bit buffer offsets: x, the experts'
  // intermediate rows h, the shared expert's, the latent rows and every weight matrix (of one
  // expert) must each span less than 2 GiB. (fp32 layers use 64-bit addressing.)
  if (p.act == Elt::BF16) {
    constexpr int64_t kOp = ((int64_t)1 << 31) - 1;
    const int64_t eh = fp8 || mx ? 1 : 2;
    if (T * H * 2 > kOp || T * k * I * eh > kOp || T * Is * 2 > kOp || T * L * 2 > kOp ||
        E * H * 2 > kOp || I * Dw * 2 > kOp || Is * H * 2 > kOp || L * H * 2 > kOp)
      return MOE_ERR_INVALID_ARG;
  }
  // fp32 grouped launches: 16-row tiles when experts average at most 16 rows, else 64
  p.bm = p.act == Elt::F32 ? ((int64_t)p.T * p.k <= 16LL * p.E ? 16 : 64) : kGroupBM;

  const size_t ea = p.act == Elt::F32 ? 4 : 2;  // activation / intermediate element bytes
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return at;
  };
  const size_t P = (size_t)p.P, Tz = (size_t)p.T, Ez = (size_t)p.E;
  if (p.act == Elt::BF16) router_split(p.T, p.E, p.H, &p.nsplit, &p.kchunk);
  else router_split_f32(p.T, p.E, p.H, &p.nsplit, &p.kchunk);
  p.logits = take(Tz * Ez * 4);
  if (p.nsplit > 1) p.zpart = take((size_t)p.nsplit * Tz * Ez * 4);
  p.slices = take((2 * (size_t)max_slices(p.P, p.E) + 1) * 4);  // decode slices, their count
  p.idx = take(P * 4);
  p.gates = take(P * 4);
  p.counts = take(Ez * 4);
  p.offsets = take((Ez + 1) * 4);
  p.perm = take(P * 4);
  p.pos = take(P * 4);
  p.dscratch = take(dispatch_scratch_ints(p.T, p.E, p.k) * 4);
  p.mt_start = take((Ez + 1) * 4);
  if (fp8 || mx) {  // per-row e4m3 copies of the expert inputs and of h
    p.xq = take(Tz * (size_t)p.D);
    p.sx = take(Tz * 4);
    p.hq = take(P * (size_t)p.I);
    p.sh = take(P * 4);
  }
  if (p.L) {
    p.xl = take(Tz * (size_t)p.L * ea);
    p.z = take(Tz * (size_t)p.L * ea);
    if (p.path == MOE_PATH_STREAM) {
      // x W_in^T streams W_in once; with few units (L/16 row blocks x T/16 token slices) each
      // wave would walk all of H alone, so K is split until about one unit per wave
      const int64_t units = (int64_t)((p.L + 15) / 16) * ((p.T + 15) / 16);
      while (units * p.lsplit * 2 <= 1024 && H % (p.lsplit * 2 * 8) == 0 &&
             H / (p.lsplit * 2) >= 256)
        p.lsplit *= 2;
      if (p.lsplit > 1) p.xpart = take((size_t)p.lsplit * Tz * (size_t)p.L * 4);
    }
  }
  p.h = take(P * (size_t)p.I * ea);
  if (p.Is) p.hs = take(Tz * (size_t)p.Is * ea);
  if (p.Is && !p.L && p.path == MOE_PATH_GROUPED) p.S = take(Tz * (size_t)p.H * 4);
  if (p.path == MOE_PATH_STREAM) {
    // The shared expert's down projection (K = I_s) is dealt out with the routed one (K = I) in
    // units of 32 rows: cut its K into about I_s / I ranges so that all units are about the same
    // size and the round-robin deal stays balanced (Nano: 3712 = 2 x 1856).
    // With 8-bit or 4-bit experts the shared expert streams in launches of its own on the side
    // stream; there four K ranges shorten each wave's chain of dependent batches (I_s / 4 of
    // K instead of all of it), so that it leaves the routed launches' bandwidth sooner.
    if (p.Is && !p.L) {
      int ns = p.ex == Elt::BF16 ? (p.Is + p.I / 2) / p.I : kNarrowSharedSplit;
      ns = ns < 1 ? 1 : (ns > 4 ? 4 : ns);
      while (ns > 1 && p.Is % (ns * 8)) --ns;
      p.ssplit = ns;
    }
    const size_t rows = P + ((p.Is && !p.L) ? (size_t)p.ssplit * Tz : 0);
    p.Y = take(rows * (size_t)p.D * 4);
  } else {
    p.Y = take(P * (size_t)p.D * ea);
  }
  p.total = off;
  *pl = p;
  return MOE_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Per device: a second stream (default priority) and two events, made on first use and kept for
// the life of the process. The decode path forks the shared expert onto it: that work does not
// depend on routing, so it overlaps the router, top-k, dispatch and the routed experts, and is
// joined back before the combine (a fork / join that stream capture also records).
// The events are re-recorded by every call, so a call holds the device's `mu` from its fork
// record to its last wait on `ready` / `join`: another thread's call cannot re-record them in
// between.
struct Side {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, ready = nullptr;  // ready: expert inputs quantised
  std::mutex mu;
};
constexpr int kMaxDevices = 64;
Side g_side[kMaxDevices];
std::mutex g_side_mu;

hipError_t side_of(Side** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_side_mu);
  Side& sd = g_side[dev];
  if (!sd.s) {
    hipStream_t st = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, ready = nullptr;
    if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&join, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&ready, hipEventDisableTiming)) != hipSuccess) {
      if (fork) (void)hipEventDestroy(fork);
      if (join) (void)hipEventDestroy(join);
      (void)hipStreamDestroy(st);
      return e;
    }
    sd.fork = fork; sd.join = join; sd.ready = ready;
    sd.s = st;
  }
  *out = &sd;
  return hipSuccess;
}

// Joins the side stream back into `s` on every exit once work was forked onto it, so that an
// error return never leaves the caller's stream unordered with work that still writes into the
// caller's buffers. The success path joins explicitly and sets `done`.
struct SideJoin {
  Side* side = nullptr;
  hipStream_t s = nullptr;
  bool done = false;
  ~SideJoin() {
    if (side && !done) {
      (void)hipEventRecord(side->join, side->s);
      (void)hipStreamWaitEvent(s, side->join, 0);
    }
  }
};

// ---------------------------------------------------------------- launch trace (diagnostics)
struct Trace {
  int cap = 0, n = 0;
  hipEvent_t* ev = nullptr;
  const char** names = nullptr;
  char filter[64] = {0};
};
Trace g_trace;

// Brackets the launches made during its lifetime with two events on `s`.
struct TraceSpan {
  int slot = -1;
  hipStream_t s;
  TraceSpan(const char* name, hipStream_t st) : s(st) {
    if (g_trace.n >= g_trace.cap) return;
    if (strncmp(name, g_trace.filter, strlen(g_trace.filter)) != 0) return;
    slot = g_trace.n++;
    g_trace.names[slot] = name;
    (void)hipEventRecord(g_trace.ev[2 * slot], s);
  }
  ~TraceSpan() {
    if (slot >= 0) (void)hipEventRecord(g_trace.ev[2 * slot + 1], s);
  }
};

#define MOE_SPAN(name) TraceSpan span_##__LINE__(name, s)
#define MOE_SPAN_ON(name, st) TraceSpan span_##__LINE__(name, st)

#define MOE_TRY(expr)                                   \
  do {                                                  \
    const hipError_t e_ = (expr);                       \
    if (e_ != hipSuccess) return MOE_ERR_HIP;           \
  } while (0)

// Dense GEMM helper: C[M, N] = epi(A[M, K] . B[N, K]^T) (+ A2 . B2^T when K2 > 0).
hipError_t dense(Elt ab, Elt out, Epi epi, const void* A, int64_t lda, const void* B, int64_t ldb,
                 void* C, int64_t ldc, int M, int N, int K, hipStream_t s,
                 const void* A2 = nullptr, int64_t lda2 = 0, const void* B2 = nullptr,
                 int64_t ldb2 = 0, int K2 = 0) {
  GemmParams g;
  g.A = A; g.lda = lda; g.a_rows = M; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K;
  g.A2 = A2; g.lda2 = lda2; g.a2_rows = M; g.B2 = B2; g.ldb2 = ldb2; g.K2 = K2;
  return launch_gemm(GemmKind{ab, out, epi}, g, 0, s);
}

// Dense bf16 product with few rows, out[t, n] = A[t, :] . W[n, :] for t < T, through the
// weight-streaming kernel (its shared-expert slot alone): W is read from HBM once, spread over
// every SIMD, where a tiled GEMM would leave most CUs idle at this M.
hipError_t stream_dense(const void* A, int64_t lda, const void* W, int N, int K, int T, void* out,
                        int64_t ldo, int store, hipStream_t s, int ksplit = 1) {
  StreamParams p;
  p.As = (const uint16_t*)A; p.lda_s = lda; p.Ws = (const uint16_t*)W; p.Ns = N; p.Ks = K;
  p.Ts = T; p.out_s = out; p.ldo_s = ldo; p.store = store; p.ksplit_s = ksplit;
  return launch_stream(p, s);
}

int32_t forward(const moe_desc_t* d, const moe_weights_t* w, void* y, void* ws, size_t ws_bytes,
                moe_routing_t* r, void* stream, bool latent_call) {
  Plan pl;
  int32_t rc = make_plan(d, latent_call, &pl);
  if (rc) return rc;
  if (pl.T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if (!w || !y) return MOE_ERR_INVALID_ARG;
  const bool given = d->flags & MOE_ROUTING_GIVEN;
  // 8-bit or 4-bit expert weights: e4m3 with per-channel scales, or MXFP4 / MXFP8 blocks
  const bool narrow = pl.ex == Elt::FP8 || pl.ex == Elt::MXFP4 || pl.ex == Elt::MXFP8;
  if (!w->x || !w->b || !w->W_up || !w->W_down || (!given && !w->W_r)) return MOE_ERR_INVALID_ARG;
  if (narrow && (!w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
  if (pl.Is && (!w->Ws_up || !w->Ws_down)) return MOE_ERR_INVALID_ARG;
  if (pl.L && (!w->W_in || !w->W_out)) return MOE_ERR_INVALID_ARG;
  if (given && (!r || !r->idx || !r->gates)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {w->x, w->W_r, w->W_up, w->W_down, w->Ws_up, w->Ws_down, w->W_in,
                        w->W_out, y};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < pl.total || !aligned16(ws)) return MOE_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  auto pick = [&](auto* user, size_t off) {
    using Ptr = decltype(user);
    return user ? user : (Ptr)(base + off);
  };
  const int T = pl.T, H = pl.H, E = pl.E, k = pl.k, I = pl.I, Is = pl.Is, L = pl.L, D = pl.D,
            P = pl.P;
  float* logits = pick(r ? r->logits : (float*)nullptr, pl.logits);
  int32_t* idx = pick(r ? r->idx : (int32_t*)nullptr, pl.idx);
  float* gates = pick(r ? r->gates : (float*)nullptr, pl.gates);
  int32_t* counts = pick(r ? r->counts : (int32_t*)nullptr, pl.counts);
  int32_t* offsets = pick(r ? r->offsets : (int32_t*)nullptr, pl.offsets);
  int32_t* perm = pick(r ? r->perm : (int32_t*)nullptr, pl.perm);
  int32_t* pos = pick(r ? r->pos : (int32_t*)nullptr, pl.pos);
  int32_t* dscr = (int32_t*)(base + pl.dscratch);
  int32_t* mt_start = (int32_t*)(base + pl.mt_start);
  void* h = base + pl.h;
  void* hs = pl.Is ? base + pl.hs : nullptr;
  void* Y = base + pl.Y;
  const Elt act = pl.act;
  const bool stream_path = pl.path == MOE_PATH_STREAM;

  // (0) decode path of a plain layer with 8-bit or 4-bit experts: the bf16 shared expert
  // (weight 1, every token, independent of routing) cannot share the narrow launches, so it
  // streams on the side stream while the routed work proceeds on `s`. (A bf16 layer deals its
  // shared-expert units out in the routed launches instead, which measured faster there.) The
  // per-row e4m3 copy of x does not depend on routing either: it runs first on the side stream.
  Side* side = nullptr;
  std::unique_lock<std::mutex> side_lock;  // released after `join` below has run
  SideJoin join;
  if (stream_path && narrow && Is && !L) {
    MOE_TRY(side_of(&side));
    side_lock = std::unique_lock<std::mutex>(side->mu);
    MOE_TRY(hipEventRecord(side->fork, s));
    join.side = side;
    join.s = s;
    MOE_TRY(hipStreamWaitEvent(side->s, side->fork, 0));
    {
      MOE_SPAN_ON("quant_rows:x", side->s);
      MOE_TRY(launch_quant_rows((const uint16_t*)w->x, H, T, H, base + pl.xq,
                                (float*)(base + pl.sx), side->s));
    }
    MOE_TRY(hipEventRecord(side->ready, side->s));
    {
      MOE_SPAN_ON("stream:shared_up", side->s);
      MOE_TRY(stream_dense(w->x, H, w->Ws_up, Is, H, T, hs, Is, kStoreSqRelu, side->s));
    }
    {
      MOE_SPAN_ON("stream:shared_down", side->s);
      MOE_TRY(stream_dense(hs, Is, w->Ws_down, H, Is, T, (float*)Y + (size_t)P * D, D, kStoreF32,
                           side->s, pl.ssplit));
    }
    MOE_TRY(hipEventRecord(side->join, side->s));
  }

  // (1) router: logits = x W_r^T, then top-k and gates
  if (!given) {
    float* zsrc = pl.nsplit > 1 ? (float*)(base + pl.zpart) : logits;
    {
      MOE_SPAN(act == Elt::F32 ? "gemm_f32_store:router" : "gemm_bf16_f32out:router");
      GemmParams g;
      g.A = w->x; g.lda = H; g.a_rows = T; g.B = w->W_r; g.ldb = H; g.C = zsrc; g.ldc = E;
      g.M = T; g.N = E; g.K = H; g.ksplit = pl.nsplit; g.kchunk = pl.kchunk;
      MOE_TRY(launch_gemm(GemmKind{act, Elt::F32, Epi::Store}, g, 0, s));
    }
    {
      MOE_SPAN("topk:router");
      MOE_TRY(launch_topk(zsrc, pl.nsplit, w->b, T, E, k, idx, gates,
                          pl.nsplit > 1 ? logits : nullptr, s));
    }
  }
  // (2) dispatch: counts, offsets, stable permutation, inverse positions, M-tile prefix
  int32_t* slices = (int32_t*)(base + pl.slices);
  const int max_sl = max_slices(P, E);
  {
    MOE_SPAN("dispatch:all");
    DispatchExtras ex;
    if (stream_path) {
      ex.slice_e = slices;
      ex.slice_r = slices + max_sl;
      ex.n_slices = slices + 2 * max_sl;
    }
    MOE_TRY(launch_dispatch(idx, T, E, k, counts, offsets, perm, pos, dscr,
                            stream_path ? 0 : pl.bm, stream_path ? nullptr : mt_start, ex, s));
  }
  // (3) routed experts read x, or its projection into the latent width
  const void* xin = w->x;
  if (L) {
    void* xl = base + pl.xl;
    if (stream_path && pl.lsplit > 1) {
      float* part = (float*)(base + pl.xpart);
      {
        MOE_SPAN("stream:latent_in");
        MOE_TRY(stream_dense(w->x, H, w->W_in, L, H, T, part, L, kStoreF32, s, pl.lsplit));
      }
      MOE_SPAN("reduce:latent_in");
      MOE_TRY(launch_reduce_slabs(part, pl.lsplit, T, L, L, xl, L, kStoreBF16, s));
    } else if (stream_path) {
      MOE_SPAN("stream:latent_in");
      MOE_TRY(stream_dense(w->x, H, w->W_in, L, H, T, xl, L, kStoreBF16, s));
    } else {
      MOE_SPAN(act == Elt::F32 ? "gemm_f32_store:latent_in" : "gemm_bf16_store:latent_in");
      MOE_TRY(dense(act, act, Epi::Store, w->x, H, w->W_in, H, xl, L, T, L, H, s));
    }
    xin = xl;
  }
  // (4) routed experts (+ the shared expert on the stream path of a plain layer)
  Elt y_elt = act;
  if (stream_path && narrow) {
    // 8-bit / 4-bit experts: expert inputs and the h rows quantised per row to e4m3, routed
    // units on the narrow streaming kernel; the bf16 shared expert streams in launches of its
    // own
    y_elt = Elt::F32;
    uint8_t* xq = base + pl.xq;
    float* sx = (float*)(base + pl.sx);
    uint8_t* hq = base + pl.hq;
    float* sh = (float*)(base + pl.sh);
    const bool mx = pl.ex != Elt::FP8;
    const char* up_name = pl.ex == Elt::FP8     ? "stream_e4m3:up"
                          : pl.ex == Elt::MXFP4 ? "stream_mxfp4:up"
                                                : "stream_mxfp8:up";
    const char* dn_name = pl.ex == Elt::FP8     ? "stream_e4m3:down"
                          : pl.ex == Elt::MXFP4 ? "stream_mxfp4:down"
                                                : "stream_mxfp8:down";
    if (side) {
      MOE_TRY(hipStreamWaitEvent(s, side->ready, 0));  // quantised on the side stream
    } else {
      MOE_SPAN("quant_rows:x");
      MOE_TRY(launch_quant_rows((const uint16_t*)xin, D, T, D, xq, sx, s));
    }
    StreamParams up;
    up.wt = pl.ex;
    up.A = xq; up.lda = D; up.a_scale = sx; up.gather = perm; up.offs = offsets; up.E = E;
    up.W = w->W_up; up.N = I; up.K = D; up.out = h; up.ldo = I;
    if (mx)
      up.w_mx = (const uint8_t*)w->s_up;
    else
      up.w_scale = (const float*)w->s_up;
    up.store = kStoreSqRelu;
    up.slice_e = slices; up.slice_r = slices + max_sl; up.n_slices = slices + 2 * max_sl;
    {
      MOE_SPAN(up_name);
      MOE_TRY(launch_stream(up, s));
    }
    {
      MOE_SPAN("quant_rows:h");
      MOE_TRY(launch_quant_rows((const uint16_t*)h, I, P, I, hq, sh, s));
    }
    StreamParams dn;
    dn.wt = pl.ex;
    dn.A = hq; dn.lda = I; dn.a_scale = sh; dn.offs = offsets; dn.E = E;
    dn.W = w->W_down; dn.N = D; dn.K = I; dn.out = Y; dn.ldo = D;
    if (mx)
      dn.w_mx = (const uint8_t*)w->s_down;
    else
      dn.w_scale = (const float*)w->s_down;
    dn.store = kStoreF32;
    dn.slice_e = slices; dn.slice_r = slices + max_sl; dn.n_slices = slices + 2 * max_sl;
    {
      MOE_SPAN(dn_name);
      MOE_TRY(launch_stream(dn, s));
    }
  } else if (stream_path) {
    y_elt = Elt::F32;
    const bool sh = Is && !L;
    StreamParams up;
    up.A = xin; up.lda = D; up.gather = perm; up.offs = offsets; up.E = E;
    up.W = w->W_up; up.N = I; up.K = D; up.out = h; up.ldo = I;
    if (sh) {  // the shared expert's units share the launch with the routed ones
      up.As = w->x; up.lda_s = H; up.Ws = w->Ws_up;
      up.Ns = Is; up.Ks = H; up.Ts = T; up.out_s = hs; up.ldo_s = Is;
    }
    up.store = kStoreSqRelu;
    up.slice_e = slices; up.slice_r = slices + max_sl; up.n_slices = slices + 2 * max_sl;
    {
      MOE_SPAN("stream:up");
      MOE_TRY(launch_stream(up, s));
    }
    StreamParams dn;
    dn.A = h; dn.lda = I; dn.offs = offsets; dn.E = E;
    dn.W = w->W_down; dn.N = D; dn.K = I; dn.out = Y; dn.ldo = D;
    if (sh) {
      dn.As = hs; dn.lda_s = Is; dn.Ws = w->Ws_down;
      dn.Ns = H; dn.Ks = Is; dn.Ts = T; dn.out_s = (float*)Y + (size_t)P * D; dn.ldo_s = D;
      dn.ksplit_s = pl.ssplit;
    }
    dn.store = kStoreF32;
    dn.slice_e = slices; dn.slice_r = slices + max_sl; dn.n_slices = slices + 2 * max_sl;
    {
      MOE_SPAN("stream:down");
      MOE_TRY(launch_stream(dn, s));
    }
  } else {
    const int max_mt = max_group_mtiles(P, E, pl.bm);
    GemmParams up;
    up.lda = D; up.a_rows = T; up.a_gather = perm;
    up.B = w->W_up; up.ldb = D; up.b_gstride = (int64_t)I * D;
    up.C = h; up.ldc = I; up.N = I; up.K = D;
    up.offs = offsets; up.mt_start = mt_start; up.G = E; up.bm = pl.bm;
    GemmParams dn;
    dn.A = h; dn.lda = I; dn.a_rows = P;
    dn.B = w->W_down; dn.ldb = I; dn.b_gstride = (int64_t)D * I;
    dn.C = Y; dn.ldc = D; dn.N = D; dn.K = I;
    dn.offs = offsets; dn.mt_start = mt_start; dn.G = E; dn.bm = pl.bm;
    if (pl.ex == Elt::FP8) {
      // e4m3 expert weights: the expert input rows and the h rows are quantised per row to
      // e4m3 (scale = row amax / 448) and both projections run on fp8 matrix cores.
      uint8_t* xq = base + pl.xq;
      float* sx = (float*)(base + pl.sx);
      uint8_t* hq = base + pl.hq;
      float* sh = (float*)(base + pl.sh);
      {
        MOE_SPAN("quant_rows:x");
        MOE_TRY(launch_quant_rows((const uint16_t*)xin, D, T, D, xq, sx, s));
      }
      up.A = xq; up.a_scale = sx; up.b_scale = (const float*)w->s_up;
      {
        MOE_SPAN("gemm_fp8_sqrelu:routed_up");
        MOE_TRY(launch_gemm(GemmKind{Elt::FP8, Elt::BF16, Epi::SqRelu}, up, max_mt, s));
      }
      {
        MOE_SPAN("quant_rows:h");
        MOE_TRY(launch_quant_rows((const uint16_t*)h, I, P, I, hq, sh, s));
      }
      dn.A = hq; dn.a_scale = sh; dn.b_scale = (const float*)w->s_down;
      {
        MOE_SPAN("gemm_fp8_store:routed_down");
        MOE_TRY(launch_gemm(GemmKind{Elt::FP8, Elt::BF16, Epi::Store}, dn, max_mt, s));
      }
    } else {
      up.A = xin;
      {
        MOE_SPAN(act == Elt::F32 ? "gemm_f32_sqrelu:routed_up" : "gemm_bf16_sqrelu:routed_up");
        MOE_TRY(launch_gemm(GemmKind{act, act, Epi::SqRelu}, up, max_mt, s));
      }
      {
        MOE_SPAN(act == Elt::F32 ? "gemm_f32_store:routed_down" : "gemm_bf16_store:routed_down");
        MOE_TRY(launch_gemm(GemmKind{act, act, Epi::Store}, dn, max_mt, s));
      }
    }
  }
  // (5) combine (+ shared expert) and, for LatentMoE, the projection back to H
  if (!L) {
    const float* S = nullptr;
    if (Is && !stream_path) {
      // shared expert in H (always on, weight 1): S = relu(x Ws_up^T)^2 Ws_down^T in fp32
      float* Sw = (float*)(base + pl.S);
      {
        MOE_SPAN(act == Elt::F32 ? "gemm_f32_sqrelu:shared_up" : "gemm_bf16_sqrelu:shared_up");
        MOE_TRY(dense(act, act, Epi::SqRelu, w->x, H, w->Ws_up, H, hs, Is, T, Is, H, s));
      }
      {
        MOE_SPAN(act == Elt::F32 ? "gemm_f32_store:shared_down" : "gemm_bf16_f32out:shared_down");
        MOE_TRY(dense(act, Elt::F32, Epi::Store, hs, Is, w->Ws_down, Is, Sw, H, T, H, Is, s));
      }
      S = Sw;
    } else if (Is && stream_path) {
      S = (const float*)Y + (size_t)P * D;
      if (side) {  // shared rows of Y are written
        MOE_TRY(hipStreamWaitEvent(s, side->join, 0));
        join.done = true;
      }
    }
    MOE_SPAN("combine:y");
    const int ns = stream_path && S ? pl.ssplit : 1;  // the shared output's K-range slabs
    MOE_TRY(launch_combine(Y, y_elt, D, S, H, pos, gates, T, D, k, y, act, H, s, ns,
                           (int64_t)T * H));
  } else {
    void* z = base + pl.z;
    {
      MOE_SPAN("combine:z");
      MOE_TRY(launch_combine(Y, y_elt, D, nullptr, 0, pos, gates, T, L, k, z, act, L, s));
    }
    if (Is) {
      {
        MOE_SPAN(act == Elt::F32 ? "gemm_f32_sqrelu:shared_up" : "gemm_bf16_sqrelu:shared_up");
        MOE_TRY(dense(act, act, Epi::SqRelu, w->x, H, w->Ws_up, H, hs, Is, T, Is, H, s));
      }
      MOE_SPAN(act == Elt::F32 ? "gemm_f32_store:latent_out" : "gemm_bf16_store:latent_out");
      MOE_TRY(dense(act, act, Epi::Store, z, L, w->W_out, L, y, H, T, H, L, s, hs, Is,
                    w->Ws_down, Is, Is));
    } else if (stream_path) {
      MOE_SPAN("stream:latent_out");
      MOE_TRY(stream_dense(z, L, w->W_out, H, L, T, y, H, kStoreBF16, s));
    } else {
      MOE_SPAN(act == Elt::F32 ? "gemm_f32_store:latent_out" : "gemm_bf16_store:latent_out");
      MOE_TRY(dense(act, act, Epi::Store, z, L, w->W_out, L, y, H, T, H, L, s));
    }
  }
  return hip_status(hipGetLastError());
}

// ---------------------------------------------------------------- backward pass (bf16)

struct BwdPlan {
  int T = 0, H = 0, E = 0, k = 0, I = 0, Is = 0, L = 0, D = 0, P = 0, Ppad = 0;
  int nsplit = 1, kchunk = 0;
  size_t logits = 0, zpart = 0, idx = 0, gates = 0, counts = 0, offsets = 0, perm = 0, pos = 0;
  size_t dscratch = 0, mt_start = 0, koffs = 0, korder = 0;
  size_t r = 0, h = 0, Yp = 0, hs = 0, rs = 0;                 // saved: expert activations
  size_t u = 0, z = 0;                                         // saved (LatentMoE): x W_in^T, z
  size_t dYp = 0, dzp = 0, da = 0, du = 0, das = 0, dxs = 0;   // backward intermediates
  size_t wr_part = 0;                                          // dW_r chunk sums
  size_t dacc = 0, dut = 0, dxl = 0;                           // LatentMoE: dz, du per token, dx
  size_t total = 0;
};

int32_t make_bwd_plan(const moe_desc_t* d, BwdPlan* out) {
  Plan fp;
  moe_desc_t dd = *d;
  dd.flags = MOE_PATH_GROUPED;
  int32_t rc = make_plan(&dd, d->latent > 0, &fp);
  if (rc) return rc;
  if (d->flags & ~(MOE_PATH_MASK | MOE_ROUTING_GIVEN | MOE_SAVED_IN_WORKSPACE | MOE_WGRAD_BF16))
    return MOE_ERR_INVALID_ARG;
  if (d->flags & MOE_ROUTING_GIVEN) return MOE_ERR_UNSUPPORTED;
  if (d->act_dtype != MOE_BF16 || d->expert_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  // the pair-ordered rows g dy [P, D] are a GEMM operand too: under 2 GiB
  if ((int64_t)fp.P * fp.D * 2 > ((int64_t)1 << 31) - 1) return MOE_ERR_INVALID_ARG;
  BwdPlan p;
  p.T = fp.T; p.H = fp.H; p.E = fp.E; p.k = fp.k; p.I = fp.I; p.Is = fp.Is; p.P = fp.P;
  p.L = fp.L; p.D = fp.D;
  p.nsplit = fp.nsplit; p.kchunk = fp.kchunk;
  // dW_r chunks: each expert's pair rows in chunks of 64 (at most 63 padding rows each)
  p.Ppad = (p.P + 63) / 64 * 64 + 64 * p.E;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return at;
  };
  const size_t T = p.T, H = p.H, E = p.E, I = p.I, Is = p.Is, P = p.P, D = p.D, L = p.L;
  p.logits = take(T * E * 4);
  if (p.nsplit > 1) p.zpart = take((size_t)p.nsplit * T * E * 4);
  p.idx = take(P * 4);
  p.gates = take(P * 4);
  p.counts = take(E * 4);
  p.offsets = take((E + 1) * 4);
  p.perm = take(P * 4);
  p.pos = take(P * 4);
  p.dscratch = take(dispatch_scratch_ints(p.T, p.E, p.k) * 4);
  p.mt_start = take((E + 1) * 4);
  p.koffs = take((E + 1) * 4);
  p.korder = take(E * 4);
  p.r = take(P * I * 2);
  p.h = take(P * I * 2);
  p.Yp = take(P * D * 2);
  if (L) {
    p.u = take(T * L * 2);
    p.z = take(T * L * 2);
  }
  if (Is) {
    p.hs = take(T * Is * 2);
    p.rs = take(T * Is * 2);
  }
  p.dYp = take(P * D * 2);
  p.dzp = take(P * 4);
  p.wr_part = take((size_t)(p.Ppad / 64) * H * 4);
  p.da = take(P * I * 2);
  p.du = take(P * D * 4);
  if (Is) {
    p.das = take(T * Is * 2);
    p.dxs = take(T * H * 4);
  }
  if (L) {
    p.dacc = take(T * L * 2);
    p.dut = take(T * L * 2);
    p.dxl = take(T * H * 4);
  }
  p.total = off;
  *out = p;
  return MOE_OK;
}

// Routing, dispatch and the expert activations the backward pass reads, into the backward
// workspace: logits, selection and gates, the dispatch arrays, the dW_r chunk numbering and the
// heaviest-first expert order, relu(a) and h = relu(a)^2 per pair row, the expert outputs Y
// (bf16, pair rows), for LatentMoE the projection u = x W_in^T and the gated sum z, and for the
// shared expert relu(a_s) and h_s.
int32_t bwd_activations(const BwdPlan& pl, const moe_weights_t* w, uint8_t* base,
                        hipStream_t s) {
  auto at = [&](size_t off) { return (void*)(base + off); };
  const int T = pl.T, H = pl.H, E = pl.E, k = pl.k, I = pl.I, Is = pl.Is, P = pl.P, L = pl.L,
            D = pl.D;
  float* logits = (float*)at(pl.logits);
  int32_t* idx = (int32_t*)at(pl.idx);
  float* gates = (float*)at(pl.gates);
  int32_t* counts = (int32_t*)at(pl.counts);
  int32_t* offsets = (int32_t*)at(pl.offsets);
  int32_t* perm = (int32_t*)at(pl.perm);
  int32_t* pos = (int32_t*)at(pl.pos);
  int32_t* mt_start = (int32_t*)at(pl.mt_start);
  int32_t* koffs = (int32_t*)at(pl.koffs);
  int32_t* korder = (int32_t*)at(pl.korder);
  const int max_mt = max_group_mtiles(P, E, kGroupBM);
  // routing and dispatch as in the forward call (the router reads x in H)
  {
    float* zsrc = pl.nsplit > 1 ? (float*)at(pl.zpart) : logits;
    {
      MOE_SPAN("gemm_bf16_f32out:router");
      GemmParams g;
      g.A = w->x; g.lda = H; g.a_rows = T; g.B = w->W_r; g.ldb = H; g.C = zsrc; g.ldc = E;
      g.M = T; g.N = E; g.K = H; g.ksplit = pl.nsplit; g.kchunk = pl.kchunk;
      MOE_TRY(launch_gemm(GemmKind{Elt::BF16, Elt::F32, Epi::Store}, g, 0, s));
    }
    {
      MOE_SPAN("topk:router");
      MOE_TRY(launch_topk(zsrc, pl.nsplit, w->b, T, E, k, idx, gates,
                          pl.nsplit > 1 ? logits : nullptr, s));
    }
    MOE_SPAN("dispatch:all");
    MOE_TRY(launch_dispatch(idx, T, E, k, counts, offsets, perm, pos, (int32_t*)at(pl.dscratch),
                            kGroupBM, mt_start, DispatchExtras(), s));
    MOE_TRY(launch_pad_offsets(counts, E, koffs, korder, s));
  }
  // the experts' input: x, or its projection into the latent width
  const void* xin = w->x;
  if (L) {
    MOE_SPAN("gemm_bf16_store:latent_in");
    MOE_TRY(dense(Elt::BF16, Elt::BF16, Epi::Store, w->x, H, w->W_in, H, at(pl.u), L, T, L, H, s));
    xin = at(pl.u);
  }
  // expert activations: relu(a) and h = relu(a)^2 per pair row, then the expert outputs Y
  void* r = at(pl.r);
  void* h = at(pl.h);
  void* Yp = at(pl.Yp);
  {
    GemmParams up;
    up.A = xin; up.lda = D; up.a_rows = T; up.a_gather = perm;
    up.B = w->W_up; up.ldb = D; up.b_gstride = (int64_t)I * D;
    up.C = h; up.C2 = r; up.ldc = I; up.N = I; up.K = D;
    up.offs = offsets; up.mt_start = mt_start; up.G = E;
    MOE_SPAN("gemm_bf16_sqrelu:bwd_routed_up");
    MOE_TRY(launch_gemm(GemmKind{Elt::BF16, Elt::BF16, Epi::SqReluSave}, up, max_mt, s));
  }
  {
    GemmParams dn;
    dn.A = h; dn.lda = I; dn.a_rows = P;
    dn.B = w->W_down; dn.ldb = I; dn.b_gstride = (int64_t)D * I;
    dn.C = Yp; dn.ldc = D; dn.N = D; dn.K = I;
    dn.offs = offsets; dn.mt_start = mt_start; dn.G = E;
    MOE_SPAN("gemm_bf16_store:bwd_routed_down");
    MOE_TRY(launch_gemm(GemmKind{Elt::BF16, Elt::BF16, Epi::Store}, dn, max_mt, s));
  }
  if (L) {  // z = sum_j g_j Y_j in the latent width, as the forward combines it
    MOE_SPAN("combine:z");
    MOE_TRY(launch_combine(Yp, Elt::BF16, L, nullptr, 0, pos, gates, T, L, k, at(pl.z),
                           Elt::BF16, L, s));
  }
  if (Is) {
    GemmParams g;
    g.A = w->x; g.lda = H; g.a_rows = T; g.B = w->Ws_up; g.ldb = H; g.C = at(pl.hs);
    g.C2 = at(pl.rs); g.ldc = Is; g.M = T; g.N = Is; g.K = H;
    MOE_SPAN("gemm_bf16_sqrelu:bwd_shared_up");
    MOE_TRY(launch_gemm(GemmKind{Elt::BF16, Elt::BF16, Epi::SqReluSave}, g, 0, s));
  }
  return MOE_OK;
}

int32_t check_bwd_args(const BwdPlan& pl, const moe_weights_t* w) {
  if (!w || !w->x || !w->W_r || !w->b || !w->W_up || !w->W_down) return MOE_ERR_INVALID_ARG;
  if (pl.Is && (!w->Ws_up || !w->Ws_down)) return MOE_ERR_INVALID_ARG;
  if (pl.L && (!w->W_in || !w->W_out)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {w->x, w->W_r, w->W_up, w->W_down, w->Ws_up, w->Ws_down, w->W_in,
                        w->W_out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int32_t backward(const moe_desc_t* d, const moe_weights_t* w, const void* dy, moe_grads_t* gr,
                 void* ws, size_t ws_bytes, hipStream_t s) {
  if (!d) return MOE_ERR_INVALID_ARG;
  BwdPlan pl;
  int32_t rc = make_bwd_plan(d, &pl);
  if (rc) return rc;
  if (pl.T == 0) return MOE_OK;
  if ((rc = check_bwd_args(pl, w))) return rc;
  if (!dy || !gr || !gr->dx || !gr->dW_r || !gr->dW_up || !gr->dW_down) return MOE_ERR_INVALID_ARG;
  if (pl.Is && (!gr->dWs_up || !gr->dWs_down)) return MOE_ERR_INVALID_ARG;
  if (pl.L && (!gr->dW_in || !gr->dW_out)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {dy, gr->dx, gr->dW_r, gr->dW_up, gr->dW_down, gr->dWs_up, gr->dWs_down,
                        gr->dW_in, gr->dW_out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < pl.total || !aligned16(ws)) return MOE_ERR_WORKSPACE;

  uint8_t* base = (uint8_t*)ws;
  auto at = [&](size_t off) { return (void*)(base + off); };
  const int T = pl.T, H = pl.H, E = pl.E, k = pl.k, I = pl.I, Is = pl.Is, P = pl.P, L = pl.L,
            D = pl.D;
  float* logits = (float*)at(pl.logits);
  int32_t* idx = (int32_t*)at(pl.idx);
  float* gates = (float*)at(pl.gates);
  int32_t* offsets = (int32_t*)at(pl.offsets);
  int32_t* perm = (int32_t*)at(pl.perm);
  int32_t* pos = (int32_t*)at(pl.pos);
  int32_t* mt_start = (int32_t*)at(pl.mt_start);
  int32_t* koffs = (int32_t*)at(pl.koffs);
  int32_t* korder = (int32_t*)at(pl.korder);
  const int max_mt = max_group_mtiles(P, E, kGroupBM);

  if (!(d->flags & MOE_SAVED_IN_WORKSPACE)) {  // else moe_layer_forward_train left them
    rc = bwd_activations(pl, w, base, s);
    if (rc) return rc;
  }
  void* r = at(pl.r);
  void* h = at(pl.h);
  void* Yp = at(pl.Yp);
  void* hs = Is ? at(pl.hs) : nullptr;
  void* rs = Is ? at(pl.rs) : nullptr;

  // (1) LatentMoE: the experts' gated sum z left through y = z W_out^T, so they see
  // dacc = dy W_out (bf16) in place of dy; dW_out = dy^T z
  const void* dye = dy;
  if (L) {
    {
      MOE_SPAN("gemm_kt_bf16out:bwd_latent_out_dgrad");
      KtParams g;
      g.A = dy; g.lda = H; g.a_rows = T; g.B = w->W_out; g.ldb = L;
      g.C = at(pl.dacc); g.ldc = L; g.M = T; g.N = L; g.K = H;
      MOE_TRY(launch_gemm_kt(0, 1, Elt::BF16, Epi::Store, g, 0, s));
    }
    {
      MOE_SPAN("gemm_kt_f32out:bwd_latent_out_wgrad");
      KtParams g;
      g.A = dy; g.lda = H; g.B = at(pl.z); g.ldb = L;
      g.C = gr->dW_out; g.ldc = L; g.M = H; g.N = L; g.K = T;
      MOE_TRY(launch_gemm_kt(1, 1, Elt::F32, Epi::Store, g, 0, s));
    }
    dye = at(pl.dacc);
  }
  // (2) gradient through the gates: dY rows (g_j dy_t) and the logit gradient per pair
  uint16_t* dYp = (uint16_t*)at(pl.dYp);
  float* dzp = (float*)at(pl.dzp);
  {
    MOE_SPAN("bwd_route:gates");
    MOE_TRY(launch_bwd_route((const uint16_t*)dye, (const uint16_t*)Yp, logits, idx, gates, pos,
                             T, D, E, k, dYp, dzp, s));
  }
  // (3) data gradients, reading the weights as stored (K-major for these products):
  // da = (dY W_down[e]) * 2 relu(a), du = da W_up[e]; the shared expert's pair likewise
  void* da = at(pl.da);
  float* du = (float*)at(pl.du);
  {
    KtParams g;
    g.A = dYp; g.lda = D; g.a_rows = P;
    g.B = w->W_down; g.ldb = I; g.b_gstride = (int64_t)D * I;
    g.C = da; g.C2 = r; g.ldc = I; g.M = P; g.N = I; g.K = D;
    g.offs = offsets; g.mt_start = mt_start; g.G = E;
    MOE_SPAN("gemm_kt_dsqrelu:bwd_routed_dgrad_down");
    MOE_TRY(launch_gemm_kt(0, 1, Elt::BF16, Epi::DSqRelu, g, max_mt, s));
  }
  {
    KtParams g;
    g.A = da; g.lda = I; g.a_rows = P;
    g.B = w->W_up; g.ldb = D; g.b_gstride = (int64_t)I * D;
    g.C = du; g.ldc = D; g.M = P; g.N = D; g.K = I;
    g.offs = offsets; g.mt_start = mt_start; g.G = E;
    MOE_SPAN("gemm_kt_f32out:bwd_routed_dgrad_up");
    MOE_TRY(launch_gemm_kt(0, 1, Elt::F32, Epi::Store, g, max_mt, s));
  }
  float* dxs = Is ? (float*)at(pl.dxs) : nullptr;
  void* das = Is ? at(pl.das) : nullptr;
  if (Is) {
    {
      MOE_SPAN("gemm_kt_dsqrelu:bwd_shared_dgrad_down");
      KtParams g;
      g.A = dy; g.lda = H; g.a_rows = T; g.B = w->Ws_down; g.ldb = Is;
      g.C = das; g.C2 = rs; g.ldc = Is; g.M = T; g.N = Is; g.K = H;
      MOE_TRY(launch_gemm_kt(0, 1, Elt::BF16, Epi::DSqRelu, g, 0, s));
    }
    MOE_SPAN("gemm_kt_f32out:bwd_shared_dgrad_up");
    KtParams g;
    g.A = das; g.lda = Is; g.a_rows = T; g.B = w->Ws_up; g.ldb = H;
    g.C = dxs; g.ldc = H; g.M = T; g.N = H; g.K = Is;
    MOE_TRY(launch_gemm_kt(0, 1, Elt::F32, Epi::Store, g, 0, s));
  }
  // (4) dx: the experts' input gradient (through W_in for LatentMoE), the shared expert's,
  // and the router's through the gates
  if (L) {
    uint16_t* dut = (uint16_t*)at(pl.dut);
    {
      MOE_SPAN("pairs_to_tokens:du");
      MOE_TRY(launch_pairs_to_tokens(du, pos, T, L, k, dut, s));
    }
    {
      MOE_SPAN("gemm_kt_f32out:bwd_latent_in_dgrad");
      KtParams g;
      g.A = dut; g.lda = L; g.a_rows = T; g.B = w->W_in; g.ldb = H;
      g.C = at(pl.dxl); g.ldc = H; g.M = T; g.N = H; g.K = L;
      MOE_TRY(launch_gemm_kt(0, 1, Elt::F32, Epi::Store, g, 0, s));
    }
    {
      MOE_SPAN("gemm_kt_f32out:bwd_latent_in_wgrad");
      KtParams g;  // dW_in [L][H] = du^T x
      g.A = dut; g.lda = L; g.B = w->x; g.ldb = H;
      g.C = gr->dW_in; g.ldc = H; g.M = L; g.N = H; g.K = T;
      MOE_TRY(launch_gemm_kt(1, 1, Elt::F32, Epi::Store, g, 0, s));
    }
    MOE_SPAN("bwd_dx:dx");
    MOE_TRY(launch_bwd_dx((const float*)at(pl.dxl), dxs, nullptr, dzp,
                          (const uint16_t*)w->W_r, idx, pos, T, H, k, gr->dx, s));
  } else {
    MOE_SPAN("bwd_dx:dx");
    MOE_TRY(launch_bwd_dx(dxs, nullptr, du, dzp, (const uint16_t*)w->W_r, idx, pos, T, H, k,
                          gr->dx, s));
  }
  {
    MOE_SPAN("bwd_router_weight:dW_r");
    MOE_TRY(launch_bwd_router_weight(dzp, (const uint16_t*)w->x, perm, offsets, koffs, E, H,
                                     pl.Ppad / 64, (float*)at(pl.wr_part), gr->dW_r, s));
  }

  // (5) routed weight gradients, reduced over each expert's own pair rows (the K window
  // [offsets[e], offsets[e+1]) of the pair-ordered operands, read as stored; the experts'
  // inputs are read from the token rows through the dispatch permutation), heaviest first.
  // The expert weight gradients are fp32, or bf16 on request (the same sums, rounded).
  const bool wg16 = d->flags & MOE_WGRAD_BF16;
  const Elt wg = wg16 ? Elt::BF16 : Elt::F32;
  {
    KtParams g;  // dW_down[e] [D][I] = dY_e^T h_e
    g.A = dYp; g.lda = D; g.B = h; g.ldb = I; g.a_rows = P;
    g.C = gr->dW_down; g.ldc = I; g.c_gstride = (int64_t)D * I;
    g.M = D; g.N = I; g.G = E; g.kgrp = offsets; g.korder = korder;
    MOE_SPAN(wg16 ? "gemm_kt_wgrad_bf16:bwd_routed_wgrad_down"
                  : "gemm_kt_f32out:bwd_routed_wgrad_down");
    MOE_TRY(launch_gemm_kt(1, 1, wg, Epi::Store, g, 0, s));
  }
  {
    KtParams g;  // dW_up[e] [I][D] = da_e^T (expert input)_e
    g.A = da; g.lda = I; g.B = L ? at(pl.u) : w->x; g.ldb = D; g.a_rows = P;
    g.b_gather = perm; g.b_rows = T;
    g.C = gr->dW_up; g.ldc = D; g.c_gstride = (int64_t)I * D;
    g.M = I; g.N = D; g.G = E; g.kgrp = offsets; g.korder = korder;
    MOE_SPAN(wg16 ? "gemm_kt_wgrad_bf16:bwd_routed_wgrad_up" : "gemm_kt_f32out:bwd_routed_wgrad_up");
    MOE_TRY(launch_gemm_kt(1, 1, wg, Epi::Store, g, 0, s));
  }
  // (6) the shared expert's weight gradients over all tokens
  if (Is) {
    {
      MOE_SPAN(wg16 ? "gemm_kt_wgrad_bf16:bwd_shared_wgrad_down"
                    : "gemm_kt_f32out:bwd_shared_wgrad_down");
      KtParams g;  // dWs_down [H][I_s] = dy^T h_s
      g.A = dy; g.lda = H; g.B = hs; g.ldb = Is;
      g.C = gr->dWs_down; g.ldc = Is; g.M = H; g.N = Is; g.K = T;
      MOE_TRY(launch_gemm_kt(1, 1, wg, Epi::Store, g, 0, s));
    }
    MOE_SPAN(wg16 ? "gemm_kt_wgrad_bf16:bwd_shared_wgrad_up" : "gemm_kt_f32out:bwd_shared_wgrad_up");
    KtParams g;  // dWs_up [I_s][H] = da_s^T x
    g.A = das; g.lda = Is; g.B = w->x; g.ldb = H;
    g.C = gr->dWs_up; g.ldc = H; g.M = Is; g.N = H; g.K = T;
    MOE_TRY(launch_gemm_kt(1, 1, wg, Epi::Store, g, 0, s));
  }
  return hip_status(hipGetLastError());
}

// Forward pass that keeps what the backward pass reads (in the backward workspace layout):
// routing, dispatch and the expert activations (bwd_activations), then the output exactly as the
// grouped forward path computes it: the shared expert and the combine, or for LatentMoE the
// projection of z back to H with the shared expert as a second K segment.
int32_t forward_train(const moe_desc_t* d, const moe_weights_t* w, void* y, void* ws,
                      size_t ws_bytes, hipStream_t s) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->flags & MOE_SAVED_IN_WORKSPACE) return MOE_ERR_INVALID_ARG;
  BwdPlan pl;
  int32_t rc = make_bwd_plan(d, &pl);
  if (rc) return rc;
  if (pl.T == 0) return MOE_OK;
  if ((rc = check_bwd_args(pl, w))) return rc;
  if (!y || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < pl.total || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  rc = bwd_activations(pl, w, base, s);
  if (rc) return rc;
  const int T = pl.T, H = pl.H, k = pl.k, Is = pl.Is, L = pl.L;
  if (L) {
    MOE_SPAN("gemm_bf16_store:latent_out");
    if (Is)
      MOE_TRY(dense(Elt::BF16, Elt::BF16, Epi::Store, base + pl.z, L, w->W_out, L, y, H, T, H, L,
                    s, base + pl.hs, Is, w->Ws_down, Is, Is));
    else
      MOE_TRY(dense(Elt::BF16, Elt::BF16, Epi::Store, base + pl.z, L, w->W_out, L, y, H, T, H, L,
                    s));
    return hip_status(hipGetLastError());
  }
  float* S = nullptr;
  if (Is) {  // shared expert S = h_s Ws_down^T in fp32 (the dx buffer is free until the backward)
    S = (float*)(base + pl.dxs);
    MOE_SPAN("gemm_bf16_f32out:shared_down");
    MOE_TRY(dense(Elt::BF16, Elt::F32, Epi::Store, base + pl.hs, Is, w->Ws_down, Is, S, H, T, H,
                  Is, s));
  }
  MOE_SPAN("combine:y");
  MOE_TRY(launch_combine(base + pl.Yp, Elt::BF16, H, S, H, (const int32_t*)(base + pl.pos),
                         (const float*)(base + pl.gates), T, H, k, y, Elt::BF16, H, s));
  return hip_status(hipGetLastError());
}

}  // namespace

extern "C" {

int32_t moe_workspace_size(const moe_desc_t* desc, size_t* bytes) {
  if (!desc || !bytes) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const int32_t rc = make_plan(desc, desc->latent > 0, &pl);
  if (rc) return rc;
  *bytes = pl.total;
  return MOE_OK;
}

int32_t moe_layer_forward(const moe_desc_t* desc, const moe_weights_t* w, void* y, void* ws,
                          size_t ws_bytes, moe_routing_t* routing, void* stream) {
  return forward(desc, w, y, ws, ws_bytes, routing, stream, false);
}

int32_t latent_moe_forward(const moe_desc_t* desc, const moe_weights_t* w, void* y, void* ws,
                           size_t ws_bytes, moe_routing_t* routing, void* stream) {
  return forward(desc, w, y, ws, ws_bytes, routing, stream, true);
}

int32_t moe_layer_forward_static(const moe_desc_t* desc, const moe_weights_t* w, void* y,
                                 moe_routing_t* routing, void* stream) {
  if (!desc) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const bool latent = desc->latent > 0;
  int32_t rc = make_plan(desc, latent, &pl);
  if (rc) return rc;
  if (pl.total > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  // set-up on the first call on a device: the array's device address (looked up once and
  // kept) and the side stream the narrow decode path forks onto; later calls only read them
  void* ws = nullptr;
  size_t bytes = 0;
  Side* side = nullptr;
  if (static_scratch(&ws, &bytes) != hipSuccess || side_of(&side) != hipSuccess)
    return MOE_ERR_HIP;
  return forward(desc, w, y, ws, bytes, routing, stream, latent);
}

int32_t moe_route(const float* logits, const void* x, const void* W_r, const float* b, int32_t T,
                  int32_t H, int32_t E, int32_t k, moe_dtype_t dt, int32_t* idx, float* gates,
                  float* logits_out, void* stream) {
  if (!b || !idx || !gates || T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return MOE_ERR_INVALID_ARG;
  if (!logits) {
    if (!x || !W_r || !logits_out || H < 16 || H % 16 || !aligned16(x) || !aligned16(W_r))
      return MOE_ERR_INVALID_ARG;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  }
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (!logits) {
    const Elt e = dt == MOE_F32 ? Elt::F32 : Elt::BF16;
    MOE_TRY(dense(e, Elt::F32, Epi::Store, x, H, W_r, H, logits_out, E, T, E, H, s));
    logits = logits_out;
  }
  MOE_TRY(launch_topk(logits, 1, b, T, E, k, idx, gates, nullptr, s));
  return MOE_OK;
}

int32_t moe_dispatch_workspace_size(int32_t T, int32_t E, int32_t k, size_t* bytes) {
  if (!bytes || T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return MOE_ERR_INVALID_ARG;
  *bytes = dispatch_scratch_ints(T, E, k) * sizeof(int32_t);
  return MOE_OK;
}

int32_t moe_dispatch(const int32_t* idx, int32_t T, int32_t E, int32_t k, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* pos, void* ws, size_t ws_bytes,
                     void* stream) {
  size_t need = 0;
  int32_t rc = moe_dispatch_workspace_size(T, E, k, &need);
  if (rc) return rc;
  if (!idx || !counts || !offsets || !perm || !pos) return MOE_ERR_INVALID_ARG;
  if (need && (!ws || ws_bytes < need || !aligned16(ws))) return MOE_ERR_WORKSPACE;
  MOE_TRY(launch_dispatch(idx, T, E, k, counts, offsets, perm, pos, (int32_t*)ws, 0, nullptr,
                          DispatchExtras(), (hipStream_t)stream));
  return MOE_OK;
}

int32_t moe_bias_update(const int32_t* counts, const float* target, int32_t E, float gamma,
                        float* b, void* stream) {
  if (E < 1 || !counts || !b) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(counts, target, E, gamma, b, (hipStream_t)stream));
}

int32_t moe_trace_enable(int32_t capacity, const char* filter) {
  if (capacity < 0) return MOE_ERR_INVALID_ARG;
  if (filter && strlen(filter) >= sizeof(g_trace.filter)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 2 * g_trace.cap; ++i) (void)hipEventDestroy(g_trace.ev[i]);
  delete[] g_trace.ev;
  delete[] g_trace.names;
  g_trace = Trace();
  if (capacity == 0) return MOE_OK;
  g_trace.ev = new hipEvent_t[2 * (size_t)capacity];
  g_trace.names = new const char*[capacity];
  for (int i = 0; i < 2 * capacity; ++i) {
    // timing-only events: recording one issues no system-scope fence (no L2 write-back and
    // invalidate between the traced launches); the reader synchronises the device first
    if (hipEventCreateWithFlags(&g_trace.ev[i], hipEventDisableSystemFence) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(g_trace.ev[j]);
      delete[] g_trace.ev;
      delete[] g_trace.names;
      g_trace = Trace();
      return MOE_ERR_HIP;
    }
  }
  g_trace.cap = capacity;
  if (filter) strcpy(g_trace.filter, filter);
  return MOE_OK;
}

int32_t moe_trace_count(void) { return g_trace.n; }

int32_t moe_trace_read(int32_t i, const char** name, float* ms) {
  if (i < 0 || i >= g_trace.n || !name || !ms) return MOE_ERR_INVALID_ARG;
  *name = g_trace.names[i];
  return hip_status(hipEventElapsedTime(ms, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]));
}

void moe_trace_reset(void) { g_trace.n = 0; }

int32_t moe_backward_workspace_size(const moe_desc_t* desc, size_t* bytes) {
  if (!desc || !bytes) return MOE_ERR_INVALID_ARG;
  BwdPlan pl;
  const int32_t rc = make_bwd_plan(desc, &pl);
  if (rc) return rc;
  *bytes = pl.total;
  return MOE_OK;
}

int32_t moe_layer_forward_train(const moe_desc_t* desc, const moe_weights_t* w, void* y,
                                void* ws, size_t ws_bytes, void* stream) {
  return forward_train(desc, w, y, ws, ws_bytes, (hipStream_t)stream);
}

int32_t moe_layer_backward(const moe_desc_t* desc, const moe_weights_t* w, const void* dy,
                           moe_grads_t* grads, void* ws, size_t ws_bytes, void* stream) {
  return backward(desc, w, dy, grads, ws, ws_bytes, (hipStream_t)stream);
}

const char* moe_status_str(int32_t code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype, shape or path";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
