// C ABI of the gfx950 MoE layer library: argument validation, workspace layout, path choice and
// the launch sequence of one layer call. Everything is enqueued on the caller's stream; nothing
// here allocates, frees or waits.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "moe.h"
#include "kernels.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

struct Plan {
  int path = 0;                 // MOE_PATH_GROUPED or MOE_PATH_STREAM
  Elt act = Elt::BF16, ex = Elt::BF16;
  int T = 0, H = 0, E = 0, k = 0, I = 0, Is = 0, L = 0, D = 0, P = 0, bm = 0;
  size_t logits = 0, idx = 0, gates = 0, counts = 0, offsets = 0, perm = 0, pos = 0;
  size_t dscratch = 0, mt_start = 0, xq = 0, sx = 0, hmax = 0, xl = 0, z = 0, h = 0, hs = 0;
  size_t Y = 0, total = 0;
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

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
  if (!fp8 && d->expert_dtype != d->act_dtype) return MOE_ERR_UNSUPPORTED;
  if (fp8 && d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->flags & ~(MOE_PATH_MASK | MOE_ROUTING_GIVEN)) return MOE_ERR_INVALID_ARG;
  Plan p;
  p.act = d->act_dtype == MOE_F32 ? Elt::F32 : Elt::BF16;
  p.ex = fp8 ? Elt::FP8 : p.act;
  p.T = (int)T; p.H = (int)H; p.E = (int)E; p.k = (int)k; p.I = (int)I; p.Is = (int)Is;
  p.L = (int)L; p.D = L ? (int)L : (int)H; p.P = (int)(T * k);
  const uint32_t path = d->flags & MOE_PATH_MASK;
  const bool stream_ok = p.act == Elt::BF16 && p.ex == Elt::BF16;
  if (path == MOE_PATH_AUTO)
    p.path = (stream_ok && (int64_t)p.P <= 8 * E) ? MOE_PATH_STREAM : MOE_PATH_GROUPED;
  else if (path == MOE_PATH_STREAM)
    p.path = stream_ok ? MOE_PATH_STREAM : -1;
  else if (path == MOE_PATH_GROUPED)
    p.path = MOE_PATH_GROUPED;
  else
    return MOE_ERR_INVALID_ARG;
  if (p.path < 0) return MOE_ERR_UNSUPPORTED;
  p.bm = p.act == Elt::F32 ? 64 : kGroupBM;

  const size_t ea = p.act == Elt::F32 ? 4 : 2;  // activation / intermediate element bytes
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return at;
  };
  const size_t P = (size_t)p.P, Tz = (size_t)p.T, Ez = (size_t)p.E;
  p.logits = take(Tz * Ez * 4);
  p.idx = take(P * 4);
  p.gates = take(P * 4);
  p.counts = take(Ez * 4);
  p.offsets = take((Ez + 1) * 4);
  p.perm = take(P * 4);
  p.pos = take(P * 4);
  p.dscratch = take(dispatch_scratch_ints(p.T, p.E) * 4);
  p.mt_start = take((Ez + 1) * 4);
  if (fp8) {
    p.xq = take(Tz * (size_t)p.D);
    p.sx = take(Tz * 4);
    p.hmax = take(P * 4);
  }
  if (p.L) {
    p.xl = take(Tz * (size_t)p.L * ea);
    p.z = take(Tz * (size_t)p.L * ea);
  }
  p.h = take(P * (size_t)p.I * ea);
  if (p.Is) p.hs = take(Tz * (size_t)p.Is * ea);
  if (p.path == MOE_PATH_STREAM) {
    const size_t rows = P + ((p.Is && !p.L) ? Tz : 0);
    p.Y = take(rows * (size_t)p.D * 4);
  } else {
    p.Y = take(P * (size_t)p.D * ea);
  }
  p.total = off;
  *pl = p;
  return MOE_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

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
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K;
  g.A2 = A2; g.lda2 = lda2; g.B2 = B2; g.ldb2 = ldb2; g.K2 = K2;
  return launch_gemm(GemmKind{ab, out, epi}, g, 0, s);
}

int32_t forward(const moe_desc_t* d, const moe_weights_t* w, void* y, void* ws, size_t ws_bytes,
                moe_routing_t* r, void* stream, bool latent_call) {
  Plan pl;
  int32_t rc = make_plan(d, latent_call, &pl);
  if (rc) return rc;
  if (pl.T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if (!w || !y) return MOE_ERR_INVALID_ARG;
  const bool given = d->flags & MOE_ROUTING_GIVEN;
  const bool fp8 = pl.ex == Elt::FP8;
  if (!w->x || !w->b || !w->W_up || !w->W_down || (!given && !w->W_r)) return MOE_ERR_INVALID_ARG;
  if (fp8 && (!w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
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
  float* hmax = fp8 ? (float*)(base + pl.hmax) : nullptr;
  void* h = base + pl.h;
  void* hs = pl.Is ? base + pl.hs : nullptr;
  void* Y = base + pl.Y;
  const Elt act = pl.act;
  const bool stream_path = pl.path == MOE_PATH_STREAM;

  // (1) router: logits = x W_r^T, then top-k and gates
  if (!given) {
    MOE_TRY(dense(act, Elt::F32, Epi::Store, w->x, H, w->W_r, H, logits, E, T, E, H, s));
    MOE_TRY(launch_topk(logits, w->b, T, E, k, idx, gates, s));
  }
  // (2) dispatch: counts, offsets, stable permutation, inverse positions, M-tile prefix
  MOE_TRY(launch_dispatch(idx, T, E, k, counts, offsets, perm, pos, dscr,
                          stream_path ? 0 : pl.bm, stream_path ? nullptr : mt_start, hmax, s));
  // (3) routed experts read x, or its projection into the latent width
  const void* xin = w->x;
  if (L) {
    void* xl = base + pl.xl;
    MOE_TRY(dense(act, act, Epi::Store, w->x, H, w->W_in, H, xl, L, T, L, H, s));
    xin = xl;
  }
  // (4) routed experts (+ the shared expert on the stream path of a plain layer)
  Elt y_elt = act;
  if (stream_path) {
    y_elt = Elt::F32;
    const bool sh = Is && !L;
    StreamParams up;
    up.A = (const uint16_t*)xin; up.lda = D; up.gather = perm; up.offs = offsets; up.E = E;
    up.W = (const uint16_t*)w->W_up; up.N = I; up.K = D; up.out = h; up.ldo = I;
    if (sh) {
      up.As = (const uint16_t*)w->x; up.lda_s = H; up.Ws = (const uint16_t*)w->Ws_up;
      up.Ns = Is; up.Ks = H; up.Ts = T; up.out_s = hs; up.ldo_s = Is;
    }
    up.sqrelu_bf16 = 1;
    MOE_TRY(launch_stream(up, s));
    StreamParams dn;
    dn.A = (const uint16_t*)h; dn.lda = I; dn.offs = offsets; dn.E = E;
    dn.W = (const uint16_t*)w->W_down; dn.N = D; dn.K = I; dn.out = Y; dn.ldo = D;
    if (sh) {
      dn.As = (const uint16_t*)hs; dn.lda_s = Is; dn.Ws = (const uint16_t*)w->Ws_down;
      dn.Ns = H; dn.Ks = Is; dn.Ts = T; dn.out_s = (float*)Y + (size_t)P * D; dn.ldo_s = D;
    }
    dn.sqrelu_bf16 = 0;
    MOE_TRY(launch_stream(dn, s));
  } else {
    const int max_mt = max_group_mtiles(P, E, pl.bm);
    GemmParams up;
    up.lda = D; up.a_gather = perm;
    up.B = w->W_up; up.ldb = D; up.b_gstride = (int64_t)I * D;
    up.C = h; up.ldc = I; up.N = I; up.K = D;
    up.offs = offsets; up.mt_start = mt_start; up.G = E;
    GemmParams dn;
    dn.A = h; dn.lda = I;
    dn.B = w->W_down; dn.ldb = I; dn.b_gstride = (int64_t)D * I;
    dn.C = Y; dn.ldc = D; dn.N = D; dn.K = I;
    dn.offs = offsets; dn.mt_start = mt_start; dn.G = E;
    if (fp8) {
      uint8_t* xq = base + pl.xq;
      float* sx = (float*)(base + pl.sx);
      MOE_TRY(launch_quant_rows((const uint16_t*)xin, D, T, D, xq, sx, s));
      up.A = xq; up.a_scale = sx; up.b_scale = w->s_up; up.row_amax = hmax;
      MOE_TRY(launch_gemm(GemmKind{Elt::FP8, Elt::BF16, Epi::SqReluAmax}, up, max_mt, s));
      dn.a_quant = 1; dn.row_amax = hmax; dn.b_scale = w->s_down;
      MOE_TRY(launch_gemm(GemmKind{Elt::FP8, Elt::BF16, Epi::Store}, dn, max_mt, s));
    } else {
      up.A = xin;
      MOE_TRY(launch_gemm(GemmKind{act, act, Epi::SqRelu}, up, max_mt, s));
      MOE_TRY(launch_gemm(GemmKind{act, act, Epi::Store}, dn, max_mt, s));
    }
  }
  // (5) combine (+ shared expert) and, for LatentMoE, the projection back to H
  if (!L) {
    if (Is && !stream_path) {
      MOE_TRY(dense(act, act, Epi::SqRelu, w->x, H, w->Ws_up, H, hs, Is, T, Is, H, s));
      GemmParams g;
      g.A = hs; g.lda = Is; g.B = w->Ws_down; g.ldb = Is; g.C = y; g.ldc = H;
      g.M = T; g.N = H; g.K = Is;
      g.gates = gates; g.pos = pos; g.topk = k; g.Y = Y; g.ldy = D;
      MOE_TRY(launch_gemm(GemmKind{act, act, Epi::Combine, y_elt}, g, 0, s));
    } else {
      const void* S = (Is && stream_path) ? (const void*)((float*)Y + (size_t)P * D) : nullptr;
      MOE_TRY(launch_combine(Y, y_elt, D, S, D, pos, gates, T, D, k, y, act, H, s));
    }
  } else {
    void* z = base + pl.z;
    MOE_TRY(launch_combine(Y, y_elt, D, nullptr, 0, pos, gates, T, L, k, z, act, L, s));
    if (Is) {
      MOE_TRY(dense(act, act, Epi::SqRelu, w->x, H, w->Ws_up, H, hs, Is, T, Is, H, s));
      MOE_TRY(dense(act, act, Epi::Store, z, L, w->W_out, L, y, H, T, H, L, s, hs, Is,
                    w->Ws_down, Is, Is));
    } else {
      MOE_TRY(dense(act, act, Epi::Store, z, L, w->W_out, L, y, H, T, H, L, s));
    }
  }
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
  MOE_TRY(launch_topk(logits, b, T, E, k, idx, gates, s));
  return MOE_OK;
}

int32_t moe_dispatch_workspace_size(int32_t T, int32_t E, int32_t k, size_t* bytes) {
  if (!bytes || T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return MOE_ERR_INVALID_ARG;
  *bytes = dispatch_scratch_ints(T, E) * sizeof(int32_t);
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
                          nullptr, (hipStream_t)stream));
  return MOE_OK;
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
