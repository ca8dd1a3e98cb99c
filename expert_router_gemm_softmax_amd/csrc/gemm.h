// Internal interface of the grouped GEMM kernels (gemm.hip).
#pragma once

#include "common.h"

namespace moe {

// Problem shapes (see gemm.hip):
//   ROW  C_e[m_e, N] = A_e[m_e, K] B_e, rows of expert e contiguous in A/C
//   KRAG C_g[M, N]  = A_g^T B_g over the rows of group g (ragged K)
enum { MODE_ROW = 0, MODE_KRAG = 1 };
// Epilogues: store s; A and H = gelu(A); dA = acc * gelu'(Aux); store fp32;
// C = RN_s(acc + Aux) with Aux fp32 laid out like C
enum { EPI_STORE = 0, EPI_GELU = 1, EPI_DGELU = 2, EPI_F32 = 3, EPI_ADDF32 = 4 };

struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  void* C2;              // EPI_GELU: H = gelu(A_out)
  const void* Aux;       // EPI_DGELU: forward pre-activation (s); EPI_ADDF32:
                         // fp32 addend; both laid out like C
  const int32_t* offsets;  // group g = rows [offsets[g], offsets[g+1]); nullptr:
                           // KRAG uniform groups of `chunk` rows, ROW one group
                           // of M rows
  const int32_t* tiles;    // ROW: prefix of M tiles per expert, [E+1]
  int E;                 // number of groups
  int M, N, K;           // ROW: N, K (and M for one group); KRAG: M, N, and
                         // K = total rows (uniform groups)
  int chunk;             // KRAG uniform groups: rows per group
  int lda, ldb, ldc;     // leading dims (elements)
  int64_t b_estride;     // ROW: elements between experts' B
  int64_t c_estride;     // KRAG: elements between groups' C
  int bm, bn;            // ROW one-group problems with K-contiguous B and an
                         // fp32 or fp32-add epilogue: block tile (64 or 128
                         // each for fp32, 128 x 128 for fp32-add); 0 = auto
  float* part;           // ROW, bf16: workspace for the split-K tail (fp32
                         // partial tiles, kGemmPartFloats); nullptr = no split
  const int32_t* kplan;  // KRAG with per-expert offsets, bf16: the split plan
                         // (block_krag_plan); nullptr = no split
  float* kslab;          // its fp32 partial slabs [slab][M][N]
  int ksplit;            // ROW one-group problems, bf16 MFMA kernel: K parts
                         // (0 or 1: none); part p covers K elements
                         // [p K/ksplit, (p+1) K/ksplit) and writes its own
                         // result at C + p c_kstride (epilogue fp32 only)
  int64_t c_kstride;
  int slots;             // filled by the launcher: concurrent blocks per round
  int ntn, ntm;          // filled by the launcher
};

// Launch one grouped GEMM.  bf16 storage: MFMA kernel; fp32: VALU kernel.
// ROW mode needs the tile prefix of the ROW schedule in g.tiles.
int launch_gemm(int kernel_id, int mode, bool b_kcontig, int epi, const moe_cfg& c,
                GemmArgs g, hipStream_t s);
int launch_gemm_schedule(const moe_cfg& c, const int32_t* offsets, int32_t* tiles,
                         hipStream_t s);

}  // namespace moe
