// Kernels of the low-rank block for gfx950: GEMM instantiations and the
// memory-bound helpers (gamma folding, r-wide row dots, column reductions,
// rank-share finalisation).
#include <mutex>

#include "lr_common.hpp"
#include "lr_gemm.hpp"
#include "lr_internal.hpp"

namespace lr {

// Tile shapes. bf16: 256x128 for the single-pair GEMMs (one 128x64 tile
// per wave, 32 accumulator registers of 4 floats), 128x128 for the
// two- and three-pair GEMMs and the weight gradients (64x64 per wave).
// fp32: 64x64 tiles with k-tiles of 32.
using TBig = Tile<256, 128, 64, 2, 2>;
using TMid = Tile<128, 128, 64, 2, 2>;
using TF32 = Tile<64, 64, 32, 2, 2>;

int gemm_tile_m(int op, int dtype) {
  if (dtype == 0) return TF32::BM;
  switch (op) {
    case OP_NT_SWIGLU:
    case OP_SWIGLU_BWD:
    case OP_TN_WGRAD:
      return TMid::BM;
    default:
      return TBig::BM;
  }
}

int gemm_tile_k(int, int dtype) { return dtype == 0 ? TF32::BK : TBig::BK; }

template <class TL, typename T, int NPAIR, uint32_t MC, int EPI>
static hipError_t launch(const GemmDesc& d, int groups, hipStream_t s) {
  auto kern = gemm_kernel<TL, T, NPAIR, MC, EPI>;
  constexpr int lds = gemm_lds_bytes<TL, T, NPAIR>();
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  if (attr_err != hipSuccess) return attr_err;
  GemmArgs g{};
  g.M = d.M;
  g.N = d.N;
  g.K = d.K;
  g.tiles_m = (d.M + TL::BM - 1) / TL::BM;
  g.tiles_n = (d.N + TL::BN - 1) / TL::BN;
  for (int i = 0; i < 3; ++i) {
    g.a[i] = d.a[i];
    g.lda[i] = d.lda[i];
    g.b[i] = d.b[i];
    g.ldb[i] = d.ldb[i];
    g.c[i] = d.c[i];
    g.ldc[i] = d.ldc[i];
  }
  g.res = d.res;
  g.ldres = d.ldres;
  g.hsrc = d.hsrc;
  g.ldh = d.ldh;
  g.rowdiv = d.rowdiv;
  g.rowcoef = d.rowcoef;
  g.colscale = d.colscale;
  g.colsum = d.colsum;
  g.rms_out = d.rms_out;
  g.ss_out = d.ss_out;
  g.n_panels = d.n_panels;
  const int ktiles_total = (d.K + TL::BK - 1) / TL::BK;
  g.panel_ktiles = (d.n_panels > 1) ? d.panel_width / TL::BK : ktiles_total;
  g.inv_D = d.inv_D;
  g.eps = d.eps;
  g.emit_partial = d.emit_partial;
  if (g.tiles_m == 0 || g.tiles_n == 0 || groups == 0) return hipSuccess;
  dim3 grid(g.tiles_m * g.tiles_n, 1, groups);
  hipLaunchKernelGGL(kern, grid, dim3(TL::NT), lds, s, g);
  return hipGetLastError();
}

template <typename T, class TL1, class TL2, class TLW>
static hipError_t dispatch(int op, const GemmDesc& d, int groups, hipStream_t s) {
  switch (op) {
    case OP_NT_STORE:
      return launch<TL1, T, 1, 0u, EPI_STORE>(d, groups, s);
    case OP_NT_ORMS:
      return launch<TL1, T, 1, 0u, EPI_ORMS>(d, groups, s);
    case OP_NT_SWIGLU:
      return launch<TL2, T, 2, 0u, EPI_SWIGLU>(d, groups, s);
    case OP_SWIGLU_BWD:
      return launch<TL2, T, 3, 32u, EPI_SWIGLU_BWD>(d, groups, s);
    case OP_NN_STORE:
      return launch<TL1, T, 1, 2u, EPI_STORE>(d, groups, s);
    case OP_NN_RMSBWD:
      return launch<TL1, T, 1, 2u, EPI_RMSBWD>(d, groups, s);
    case OP_TN_WGRAD:
      return launch<TLW, T, 1, 3u, EPI_WGRAD>(d, groups, s);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t run_gemm(int op, int dtype, const GemmDesc& d, int groups, hipStream_t s) {
  if (dtype == 0) return dispatch<float, TF32, TF32, TF32>(op, d, groups, s);
  return dispatch<bf16_t, TBig, TMid, TMid>(op, d, groups, s);
}

// ---------------------------------------------------------------------------
// Memory-bound kernels
// ---------------------------------------------------------------------------

// out[n, k] = A[n, k] * gamma[k] (rounded to the storage type).
template <typename T>
__global__ __launch_bounds__(256) void fold_gamma_kernel(const T* __restrict__ A, int64_t lda,
                                                         const T* __restrict__ gamma,
                                                         T* __restrict__ out, int rows,
                                                         int cols) {
  constexpr int VEC = Elem<T>::VEC;
  const int vpr = cols / VEC;
  const int64_t total = (int64_t)rows * vpr;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / vpr), c = (int)(i % vpr) * VEC;
    float a[VEC], gm[VEC];
    unpack16<T>(*reinterpret_cast<const u32x4*>(A + r * lda + c), a);
    unpack16<T>(*reinterpret_cast<const u32x4*>(gamma + c), gm);
#pragma unroll
    for (int e = 0; e < VEC; ++e) a[e] *= gm[e];
    *reinterpret_cast<u32x4*>(out + (int64_t)r * cols + c) = pack16<T>(a);
  }
}

// coef[t] = (sum_j a[t, j] b[t, j]) / rms[t] * inv_D, one wave per row.
template <typename T>
__global__ __launch_bounds__(256) void rowdot_coef_kernel(const T* __restrict__ a, int64_t lda,
                                                          const T* __restrict__ b, int64_t ldb,
                                                          int width, const float* __restrict__ rms,
                                                          float inv_D, float* __restrict__ coef,
                                                          int rows) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  for (int t = wave; t < rows; t += nwaves) {
    const T* pa = a + (int64_t)t * lda;
    const T* pb = b + (int64_t)t * ldb;
    float acc = 0.f;
    for (int c = lane * VEC; c < width; c += 64 * VEC) {
      float x[VEC], y[VEC];
      unpack16<T>(*reinterpret_cast<const u32x4*>(pa + c), x);
      unpack16<T>(*reinterpret_cast<const u32x4*>(pb + c), y);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc = __builtin_fmaf(x[e], y[e], acc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) coef[t] = acc / rms[t] * inv_D;
  }
}

// out[c] = sum_t part[t, c], t in a fixed order.
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ part, int tiles,
                                                     int n, float* __restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  float s = 0.f;
  for (int t = 0; t < tiles; ++t) s += part[(int64_t)t * n + c];
  out[c] = s;
}

// Rank-share finalisation after the (identity) all-reduce:
// rms[t] = sqrt(ss[t] * inv_D + eps); z[t, :] = P[t, :] / rms[t].
template <typename T>
__global__ __launch_bounds__(256) void finalize_kernel(const T* __restrict__ P, int64_t ldp,
                                                       const float* __restrict__ ss, int rows,
                                                       int width, float inv_D, float eps,
                                                       T* __restrict__ z, int64_t ldz,
                                                       float* __restrict__ rms_out) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  for (int t = wave; t < rows; t += nwaves) {
    const float rmsg = sqrtf(ss[t] * inv_D + eps);
    const float s = 1.0f / rmsg;
    if (lane == 0 && rms_out) rms_out[t] = rmsg;
    for (int c = lane * VEC; c < width; c += 64 * VEC) {
      float x[VEC];
      unpack16<T>(*reinterpret_cast<const u32x4*>(P + (int64_t)t * ldp + c), x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] *= s;
      *reinterpret_cast<u32x4*>(z + (int64_t)t * ldz + c) = pack16<T>(x);
    }
  }
}

static int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

hipError_t run_fold_gamma(int dtype, const void* A, int64_t lda, const void* gamma, void* out,
                          int rows, int cols, hipStream_t s) {
  if (dtype == 0) {
    hipLaunchKernelGGL(fold_gamma_kernel<float>, dim3(grid_for((int64_t)rows * cols / 4, 256)),
                       dim3(256), 0, s, static_cast<const float*>(A), lda,
                       static_cast<const float*>(gamma), static_cast<float*>(out), rows, cols);
  } else {
    hipLaunchKernelGGL(fold_gamma_kernel<bf16_t>, dim3(grid_for((int64_t)rows * cols / 8, 256)),
                       dim3(256), 0, s, static_cast<const bf16_t*>(A), lda,
                       static_cast<const bf16_t*>(gamma), static_cast<bf16_t*>(out), rows,
                       cols);
  }
  return hipGetLastError();
}

hipError_t run_rowdot_coef(int dtype, const void* a, int64_t lda, const void* b, int64_t ldb,
                           int width, const float* rms, float inv_D, float* coef, int rows,
                           hipStream_t s) {
  const int grid = grid_for(rows, 4);
  if (dtype == 0) {
    hipLaunchKernelGGL(rowdot_coef_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(a), lda, static_cast<const float*>(b), ldb,
                       width, rms, inv_D, coef, rows);
  } else {
    hipLaunchKernelGGL(rowdot_coef_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const bf16_t*>(a), lda, static_cast<const bf16_t*>(b), ldb,
                       width, rms, inv_D, coef, rows);
  }
  return hipGetLastError();
}

hipError_t run_colsum(const float* part, int tiles, int n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(colsum_kernel, dim3((n + 255) / 256), dim3(256), 0, s, part, tiles, n, out);
  return hipGetLastError();
}

hipError_t run_finalize(int dtype, const void* P, int64_t ldp, const float* ss, int rows,
                        int width, float inv_D, float eps, void* z, int64_t ldz, float* rms_out,
                        hipStream_t s) {
  const int grid = grid_for(rows, 4);
  if (dtype == 0) {
    hipLaunchKernelGGL(finalize_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(P), ldp, ss, rows, width, inv_D, eps,
                       static_cast<float*>(z), ldz, rms_out);
  } else {
    hipLaunchKernelGGL(finalize_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const bf16_t*>(P), ldp, ss, rows, width, inv_D, eps,
                       static_cast<bf16_t*>(z), ldz, rms_out);
  }
  return hipGetLastError();
}

}  // namespace lr
