// Parameters and launchers of the tiled GEMM family used by the MoE layer:
//   C[m, n] = epilogue( sum_k A[m, k] * B[n, k] )      (both operands K-contiguous)
// A holds activations (token rows, optionally gathered through an index list), B holds weights
// stored [G][N][K] (one [N][K] panel per expert). Grouped launches walk a device-built list of
// (expert, M-tile) pairs, so no host round trip is needed to learn the per-expert token counts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// FP8 is OCP e4m3. MXFP4 / MXFP8 are OCP microscaling weight formats (E2M1 or E4M3 elements,
// one E8M0 scale per 32 consecutive K elements); only the decode streaming kernel reads them.
enum class Elt : int { F32 = 0, BF16 = 1, FP8 = 2, MXFP4 = 3, MXFP8 = 4 };

enum class Epi : int {
  Store = 0,        // C = acc
  SqRelu = 1,       // C = relu(acc)^2
  SqReluSave = 2,   // C = relu(acc)^2 and C2 = relu(acc) (the factor the backward pass needs)
  DSqRelu = 3       // C = acc * 2 * C2: the squared ReLU's derivative at the saved relu(a)
                    // (backward products only, gemm_kt.hpp)
};

struct GemmParams {
  // A operand: rows of K elements; row r of group g is a_gather[offs[g] + r] when a_gather is
  // set, else offs[g] + r.
  const void* A = nullptr;
  int64_t lda = 0;  // elements
  int a_rows = 0;   // rows of A that may be read (the extent of the operand in memory)
  const int32_t* a_gather = nullptr;
  const float* a_scale = nullptr;  // e4m3 A: dequantisation scale per *source* row
  // B operand: [G][N][K], b_gstride elements between experts; fp8: per-channel scales [G][N]
  const void* B = nullptr;
  int64_t ldb = 0;
  int64_t b_gstride = 0;
  const float* b_scale = nullptr;
  // Optional second K segment for dense launches: acc += A2[m, :] . B2[n, :]
  const void* A2 = nullptr;
  int64_t lda2 = 0;
  int a2_rows = 0;
  const void* B2 = nullptr;
  int64_t ldb2 = 0;
  int K2 = 0;
  // Output; C2 is the second matrix of the SqReluSave epilogue (same shape, ldc)
  void* C = nullptr;
  int64_t ldc = 0;
  void* C2 = nullptr;
  int M = 0, N = 0, K = 0;
  // Split-K (dense launches only): slice y of ksplit covers K columns [y*kchunk, (y+1)*kchunk)
  // and writes its partial product to C + y * M * ldc (Store epilogue).
  int ksplit = 1;
  int kchunk = 0;
  // Grouping (both null for a dense launch of M rows)
  const int32_t* offs = nullptr;      // [G + 1] row offsets
  const int32_t* mt_start = nullptr;  // [G + 1] prefix of ceil(rows_g / BM)
  int G = 0;
  // fp32 grouped launches: the M-tile height BM that mt_start counts (16 or 64; 0 means 64)
  int bm = 0;
};

struct GemmKind {
  Elt ab;      // element type of A and B as fed to the matrix cores (F32: vector ALU path)
  Elt out;     // C element type
  Epi epi;
};

// Tile height of the grouped launches; the dispatch step builds mt_start with it.
constexpr int kGroupBM = 128;

// Upper bound of M-tiles over all groups for P routed rows in G groups (each group wastes < 1).
inline int max_group_mtiles(int P, int G, int BM) { return (P + G * (BM - 1)) / BM; }

hipError_t launch_gemm(const GemmKind& kind, const GemmParams& p, int max_mtiles,
                       hipStream_t stream);

// Workgroups of a persistent launch on the current device: two per CU, a multiple of 8.
int persist_grid();

}  // namespace moe
