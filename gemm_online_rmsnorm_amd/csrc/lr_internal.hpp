// Internal launch interface between the C ABI (lr_api.cpp) and the kernels
// (lr_kernels.hip). Host-only declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lr {

// GEMM operations (layout + epilogue); see lr_gemm.hpp for the epilogues.
enum GemmOp : int {
  OP_NT_STORE = 0,    // Y = X W^T [/ rowdiv] [+ res]           (grouped)
  OP_NT_ORMS = 1,     // Online RMSNorm down-projection
  OP_NT_SWIGLU = 2,   // two NT pairs, Y = SiLU(acc0) * acc1
  OP_SWIGLU_BWD = 3,  // NT, NT, NN pairs -> m, dg, du
  OP_NN_STORE = 4,    // Y = X W [/ rowdiv] [+ res]             (grouped)
  OP_NN_RMSBWD = 5,   // RMSNorm backward epilogue + column sums
  OP_TN_WGRAD = 6,    // fp32 Y = X^T W [* colscale]            (grouped)
  OP_SWIGLU_BWD2 = 7, // NT, NT pairs (g, u) + dm from res -> m, dg, du (pipelined engine)
  OP_NT_RMSBWD = 8,   // RMSNorm backward epilogue + column sums, NT (pipelined engine)
  OP_COUNT = 9,
};

struct GemmDesc {
  int M = 0, N = 0, K = 0;
  const void* a[3] = {nullptr, nullptr, nullptr};
  int64_t lda[3] = {0, 0, 0};
  const void* b[3] = {nullptr, nullptr, nullptr};
  int64_t ldb[3] = {0, 0, 0};
  void* c[3] = {nullptr, nullptr, nullptr};
  int64_t ldc[3] = {0, 0, 0};
  const void* res = nullptr;
  int64_t ldres = 0;
  const void* hsrc = nullptr;
  int64_t ldh = 0;
  const float* rowdiv = nullptr;
  const float* rowcoef = nullptr;
  const void* colscale = nullptr;
  float* colsum = nullptr;
  float* rms_out = nullptr;
  float* ss_out = nullptr;
  int n_panels = 1;
  int panel_width = 0;  // columns per Online RMSNorm panel
  float inv_D = 0.f;
  float eps = 0.f;
  int emit_partial = 0;
  int ksplit = 1;                // split-K factor (pipelined engine only)
  int64_t c_split_stride = 0;    // output element stride between splits
  // Column sums run as a side job after the outputs (pipelined engine only):
  // cs_out[c] = sum_r cs_part[r * cs_n + c] in a fixed order.
  const float* cs_part = nullptr;
  int cs_rows = 0, cs_n = 0;
  float* cs_out = nullptr;
};

// Tile sizes an operation uses for a dtype (0 = LR_F32, 1 = LR_BF16).
int gemm_tile_m(int op, int dtype);
int gemm_tile_k(int op, int dtype);

// Enqueue one GEMM launch over `groups` operand groups (grid z).
hipError_t run_gemm(int op, int dtype, const GemmDesc& d, int groups, hipStream_t s);

// Whether run_gemm takes the pipelined engine for this call, and the M-tile
// it then uses (the RMSNorm-backward column partials have one row per M-tile).
bool uses_engine2(int op, int dtype, const GemmDesc& d, int groups);
int gemm2_tile_m(int op, const GemmDesc& d, int groups);
// M-tile of the kernel run_gemm dispatches for this call.
int gemm_tile_m_used(int op, int dtype, const GemmDesc& d, int groups);
// Smallest M-tile any GEMM kernel uses (sizes per-M-tile workspaces).
constexpr int kMinTileM = 64;

// Weight-gradient (TN) GEMM with deterministic split-K: when the output grid
// is too small to fill the chip, K is cut into `splits` slices whose fp32
// partials go to `part` (run_wgrad_gemm); run_wgrad_sum then adds them in a
// fixed order, with the column scale applied, into d.c[slot]. With one slice
// the GEMM writes d.c directly and no sum is needed. wgrad_part_bytes gives
// the partial workspace a call needs; wgrad_splits the slice count a call
// with `part_bytes` of workspace at `part` runs with (1 without enough).
size_t wgrad_part_bytes(int dtype, const GemmDesc& d, int groups);
int wgrad_splits(int dtype, const GemmDesc& d, int groups, const void* part, size_t part_bytes);
hipError_t run_wgrad_gemm(int dtype, const GemmDesc& d, int groups, int splits, void* part,
                          hipStream_t s);
hipError_t run_wgrad_sum(const GemmDesc& d, int groups, int splits, const void* part,
                         hipStream_t s);

// Weight gradients of up to three problems of different M, N (same K) in one
// launch, problem i writing p[i].c[0] (column scale p[i].colscale); the
// column-sum side job is taken from p[0]. wgrad_multi_ok: all of them can
// run so; wgrad_multi_split: the K-split for their tiles together (1: none);
// with a split the partials of problem i lie at part +
// wgrad_multi_part_offset(p, i, splits) floats, and run_wgrad_sum then
// adds each problem's slices (as a one-group call on those partials).
bool wgrad_multi_ok(int dtype, const GemmDesc* p, int n);
int wgrad_multi_split(const GemmDesc* p, int n);
size_t wgrad_multi_part_bytes(const GemmDesc* p, int n, int splits);
int64_t wgrad_multi_part_offset(const GemmDesc* p, int i, int splits);
hipError_t run_wgrad_multi_gemm(const GemmDesc* p, int n, int splits, void* part, hipStream_t s);

// Memory-bound helpers.
hipError_t run_fold_gamma(int dtype, const void* A, int64_t lda, const void* gamma, void* out,
                          int rows, int cols, hipStream_t s);
// Two folds of the same width in one launch (job 0's rows, then job 1's).
hipError_t run_fold_gamma2(int dtype, const void* A0, int64_t lda0, const void* g0, void* o0,
                           int rows0, const void* A1, int64_t lda1, const void* g1, void* o1,
                           int rows1, int cols, hipStream_t s);
hipError_t run_rowdot_coef(int dtype, const void* a, int64_t lda, const void* b, int64_t ldb,
                           int width, const float* rms, float inv_D, float* coef, int rows,
                           hipStream_t s);
hipError_t run_colsum(const float* part, int tiles, int n, float* out, hipStream_t s);
hipError_t run_finalize(int dtype, const void* P, int64_t ldp, const float* ss, int rows,
                        int width, float inv_D, float eps, void* z, int64_t ldz, float* rms_out,
                        hipStream_t s);

// bf16 transposes out[c][r] = in[r][c] of up to kMaxTranspose matrices in
// one launch (rows x cols each, leading dimensions ldi and ldo in elements).
// Every row is whole 16-byte chunks (cols % 8 == 0) and every matrix whole
// 64-row tiles (rows % 64 == 0); the caller checks.
struct TransposeJob {
  const void* in = nullptr;
  int64_t ldi = 0;
  int rows = 0, cols = 0;
  void* out = nullptr;
  int64_t ldo = 0;
};
constexpr int kMaxTranspose = 8;
hipError_t run_transpose_bf16(const TransposeJob* jobs, int n, hipStream_t s);

}  // namespace lr
