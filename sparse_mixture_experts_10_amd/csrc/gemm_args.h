// Arguments of one grouped GEMM pass, shared by the GEMM kernels and the C ABI.
#pragma once

#include <stdint.h>

namespace moe {

// One grouped GEMM pass  C[r, n] = epi( sum_k A[r, k] * B[g(r)][n, k] ).
struct GemmArgs {
  const void* A;             // [rows, K], or [*, K] read through a_rows
  const int32_t* a_rows;     // nullptr, or: packed row r reads A row a_rows[r]
  const int32_t* group_offset;  // [G+1] device, or nullptr: one group of dense_M rows
  int G;
  int64_t dense_M;
  int64_t max_rows;          // rows >= max_rows are neither read nor written
  const void* B;             // [G][N][K] (or [S][N][Kseg] when S > 1, one group)
  int N, K;
  int S, Kseg;               // K = S * Kseg; B segment s holds columns [s*Kseg, (s+1)*Kseg)
  const void* bias;          // [G][N], or [S][N] summed over s when S > 1
  void* C;                   // [rows, N]
  int act;                   // activation, or -1 for none
  float* sq_part;            // [max_rows][n_tiles] partial sum of squares, or nullptr
  bool out_f32;              // C is fp32 (no staging; bias and activation still apply)
  bool n_major;              // tile order inside a group: N tiles outer (set by the launcher)
};

}  // namespace moe
