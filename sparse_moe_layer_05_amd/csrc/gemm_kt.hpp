// Matrix-core GEMM whose operands may be stored K-major (the backward pass of the MoE layer):
//   C[m, n] = epilogue( sum_k A(m, k) * B(n, k) )
// with, per operand, either the K-contiguous layout of the forward GEMMs (A[m][k], B[n][k]) or
// the K-major layout A[k][m] / B[k][n] (M or N contiguous). A K-major tile is staged in LDS as
// rows of k and turned into matrix-core fragments by gfx950's transposing LDS read. This lets
// the data gradients read the weights as stored (W_down[e] is [H][I], i.e. K-major for
// dY . W_down[e]) and the weight gradients read the pair-ordered activations as stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"

namespace moe {

struct KtParams {
  const void* A = nullptr;   // bf16
  int64_t lda = 0;           // elements between rows as stored
  const void* B = nullptr;   // bf16; row-grouped launches step b_gstride elements per group
  int64_t ldb = 0;
  int64_t b_gstride = 0;
  void* C = nullptr;         // Store / DSqRelu output; k-grouped launches step c_gstride
  void* C2 = nullptr;        // DSqRelu: relu(a) saved by the forward, same shape as C
  int64_t ldc = 0;
  int64_t c_gstride = 0;
  int M = 0, N = 0, K = 0;
  int a_rows = 0;            // stored rows of A that may be read (K-grouped: rows of A and B)
  // Row-grouped launches (data gradients): group g owns rows [offs[g], offs[g+1]) of A and C
  // (M-tiles from mt_start) and its own B at B + g * b_gstride.
  const int32_t* offs = nullptr;
  const int32_t* mt_start = nullptr;
  int G = 0;
  // K-grouped launches (weight gradients): group g reduces over the stored K rows
  // [kgrp[g], kgrp[g+1]) of both K-major operands; korder (optional) is the launch order.
  const int32_t* kgrp = nullptr;
  const int32_t* korder = nullptr;
  // K-grouped launches, optional: stored K row k of B is row b_gather[k] of B (b_rows rows), so
  // a pair-ordered operand is read straight from the token rows it gathers.
  const int32_t* b_gather = nullptr;
  int b_rows = 0;
};

// ta / tb: 1 when A / B is stored K-major. Provided: (ta, tb, out, epi) in
//   (0, 1, BF16, DSqRelu), (0, 1, F32, Store),
//   (0, 1, BF16, Store)                         data gradients (dense or row-grouped)
//   (1, 1, F32, Store), (1, 1, BF16, Store)     weight gradients (dense or K-grouped)
// N, ldc and the K-major leading dimensions must be multiples of 8, and so must M when A is
// K-major and K when it is not; each operand must span less than 2 GiB (32-bit offsets).
// max_mtiles bounds the M-tiles of a row-grouped launch (its grid).
hipError_t launch_gemm_kt(int ta, int tb, Elt out, Epi epi, const KtParams& p, int max_mtiles,
                          hipStream_t s);

}  // namespace moe
