// Kernels of the low-rank block for gfx950: GEMM instantiations and the
// memory-bound helpers (gamma folding, r-wide row dots, column reductions,
// rank-share finalisation).
#include <algorithm>
#include <atomic>
#include <mutex>

#include "lr_common.hpp"
#include "lr_gemm.hpp"
#include "lr_gemm2.hpp"
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
  g.groups = groups;
  g.ktiles_split = ktiles_total;
  g.c_split_stride = 0;
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

// ---------------------------------------------------------------------------
// Pipelined engine (lr_gemm2.hpp) for bf16 GEMMs with K a multiple of the
// k-tile. The large tile is 256 x 256 with 8 waves (two per SIMD, 128 x 64
// each), so that one wave's barrier and LDS waits are covered by the other
// wave's MFMAs; smaller grids fall back to 256 x 128 or 128 x 128 tiles with
// 4 waves. The gate/up pair GEMMs of small grids use k-tiles of 32 in
// three stages.
// ---------------------------------------------------------------------------
using P256x256 = Tile2<256, 256, 64, 2, 4, 2>;
// The same tile with separate rings: 3 stages of the A tile, 2 of the B
// tile (160 KB), for the one-pair NT products (Online RMSNorm included).
using P256x256a = Tile2<256, 256, 64, 2, 4, 2, 1, 3>;
using P256x128 = Tile2<256, 128, 64, 2, 2, 2>;
using P128x128 = Tile2<128, 128, 64, 2, 2, 2>;
using P2x128x128 = Tile2<128, 128, 32, 2, 2, 3>;
// Gate and up products side by side: 256 x (128 gate + 128 up) B rows,
// 8 waves each running one pair on a 128 x 64 wave tile.
using PS256x128 = Tile2<256, 256, 32, 2, 4, 3, 2>;
// The same pairing on 192 rows with k-tiles of 64 in two stages (all of the
// LDS): every HBM-to-LDS load then covers whole 128-byte rows; loads of
// 64-byte row halves, which k-tiles of 32 give, copy at half the rate and
// bound the 256-row tile.
using PS192x128 = Tile2<192, 256, 64, 2, 4, 2, 2>;
// Block-diagonal gate/up tile: 256 rows x 128 columns of both g and u, the
// K loop running the gate pair and then the up pair; a stage is one pair's
// A and B tiles (48 KB), so three stages fit, and every wave (64 x 64 of
// both) combines g and u in registers without an exchange.
using PBD256x128 = Tile2<256, 128, 64, 4, 2, 3, 1, 0, 1>;
// The block-diagonal tile at 160 x 128 with 4 waves of 80 x 64 and two 36
// KB stages, the gate packed to bf16 once the gate pair is done (which
// frees the registers for 80-row wave tiles at two waves per SIMD): two
// workgroups share a CU and drift apart, so one tile's epilogue runs beside
// the other's main loop. Both SwiGLU products run it; against the 256 x
// 128 tile (forward) and a 128 x 128 tile with fp32 gate accumulators
// (recompute + backward) it moves 10% fewer bytes per FLOP from L2 and
// through LDS (measured at the 7B shape: forward 722 -> 679 us, recompute
// + backward 882 -> 794 us, the step 1% faster).
using PBDP160x128 = Tile2<160, 128, 64, 2, 2, 2, 1, 0, 2>;

// Compute units of the current device (looked up once per device).
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class TL, int NPAIR, uint32_t MC, int EPI>
static hipError_t launch2(const GemmDesc& d, int groups, hipStream_t s) {
  auto kern = gemm2_kernel<TL, NPAIR, MC, EPI>;
  constexpr int lds = gemm2_lds_bytes<TL, NPAIR, EPI>();
  static_assert(lds <= 160 * 1024, "LDS budget exceeded");
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
  g.tiles_n = (d.N + TL::BNO - 1) / TL::BNO;
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
  g.panel_ktiles = (d.n_panels > 1) ? d.panel_width / TL::BK : d.K / TL::BK;
  g.inv_D = d.inv_D;
  g.eps = d.eps;
  g.emit_partial = d.emit_partial;
  g.groups = groups;
  const int split = d.ksplit > 1 ? d.ksplit : 1;
  g.ktiles_split = d.K / TL::BK / split;
  g.c_split_stride = d.c_split_stride;
  g.cs_part = d.cs_part;
  g.cs_rows = d.cs_rows;
  g.cs_n = d.cs_n;
  g.cs_out = d.cs_out;
  if (g.tiles_m == 0 || g.tiles_n == 0 || groups == 0) return hipSuccess;
  if constexpr (gemm2_persist<TL, NPAIR, EPI>()) {
    // One workgroup per CU walks the tiles; a multiple of 8 workgroups
    // whenever one runs several, so that a tile keeps its XCD.
    if (split != 1) return hipErrorInvalidValue;
    const int64_t total = (int64_t)g.tiles_m * g.tiles_n * groups;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    const int64_t ncu = device_cus() / 8 * 8;
    g.vtiles = (int)total;
    const int nwg = (int)(total > ncu && ncu > 0 ? ncu : total);
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(TL::NT), lds, s, g);
    return hipGetLastError();
  } else {
    dim3 grid(g.tiles_m * g.tiles_n, 1, groups * split);
    hipLaunchKernelGGL(kern, grid, dim3(TL::NT), lds, s, g);
    return hipGetLastError();
  }
}

static int64_t ntiles(const GemmDesc& d, int bm, int bn, int groups) {
  return (int64_t)((d.M + bm - 1) / bm) * ((d.N + bn - 1) / bn) * groups;
}

// Whether the pipelined engine can run this GEMM: k-tiles divide K, the
// M/N-contiguous operands have whole 8-element chunks, every per-lane load
// offset fits in 32 bits, and the Online RMSNorm panels are whole k-tiles.
// Elements from an operand's first element to one past its last one.
static int64_t operand_extent(bool mc, int64_t ld, int rows, int K) {
  return mc ? (int64_t)(K - 1) * ld + rows : (int64_t)(rows - 1) * ld + K;
}

static bool eligible2(int op, const GemmDesc& d, int groups, int bk) {
  if (d.K % bk != 0 || d.M < 1 || d.N < 1 || d.N % 8 != 0) return false;
  uint32_t mc = 0;
  int npair = 1;
  switch (op) {
    case OP_NN_STORE:
    case OP_NN_RMSBWD: mc = 2u; break;
    case OP_NT_RMSBWD: break;
    case OP_TN_WGRAD: mc = 3u; break;
    case OP_NT_SWIGLU:
    case OP_SWIGLU_BWD2: npair = 2; break;
    default: break;
  }
  const int nsl = (npair == 1) ? groups : npair;
  for (int p = 0; p < nsl; ++p) {
    const int lp = (npair == 1) ? 0 : p;  // the groups of a grouped GEMM share pair 0's layout
    const bool amc = (mc >> (2 * lp)) & 1u, bmc = (mc >> (2 * lp + 1)) & 1u;
    // M/N-contiguous tiles need whole 16-byte row chunks; every operand's
    // byte extent must fit the 32-bit offsets of a buffer resource.
    if (amc && d.M % 8 != 0) return false;
    if (bmc && d.N % 8 != 0) return false;
    if (operand_extent(amc, d.lda[p], d.M, d.K) >= ((int64_t)1 << 31)) return false;
    if (operand_extent(bmc, d.ldb[p], d.N, d.K) >= ((int64_t)1 << 31)) return false;
  }
  if (op == OP_NT_ORMS && d.n_panels > 1 && d.panel_width % bk != 0) return false;
  // The epilogue addresses a tile's outputs and element inputs with 32-bit
  // byte offsets from the tile origin.
  const int64_t ld_max = (int64_t)1 << 21;
  for (int p = 0; p < 3; ++p)
    if (d.ldc[p] >= ld_max) return false;
  if (d.ldres >= ld_max || d.ldh >= ld_max) return false;
  return true;
}

static constexpr int kCUs = 256;

// Fraction of the CU slots the last partial wave of workgroups leaves busy.
static double wave_eff(int64_t tiles) {
  const int64_t waves = (tiles + kCUs - 1) / kCUs;
  return waves ? (double)tiles / (double)(waves * kCUs) : 0.0;
}

// Tile choice of the single-pair GEMMs: the 256 x 256 tile unless its grid
// leaves most CUs idle, then 256 x 128, then 128 x 128.
static int single_tile(const GemmDesc& d, int groups) {
  const int64_t t256 = ntiles(d, 256, 256, groups), t128 = ntiles(d, 256, 128, groups);
  if (t256 >= kCUs && wave_eff(t256) >= 0.75) return 0;
  if (t128 >= kCUs && wave_eff(t128) >= 0.75) return 1;
  if (t256 >= kCUs) return 0;
  if (t128 >= kCUs) return 1;
  return 2;
}

template <int EPI, uint32_t MC>
static hipError_t launch_single(const GemmDesc& d, int groups, hipStream_t s) {
  switch (single_tile(d, groups)) {
    case 0:
      if constexpr (MC != 0u) return launch2<P256x256, 1, MC, EPI>(d, groups, s);
      else return launch2<P256x256a, 1, MC, EPI>(d, groups, s);
    case 1: return launch2<P256x128, 1, MC, EPI>(d, groups, s);
    default: return launch2<P128x128, 1, MC, EPI>(d, groups, s);
  }
}

// Tile choice of the gate/up pair GEMMs: 4 the packed block-diagonal 160 x
// 128 tile, two per CU, 3 the block-diagonal 256 x 128 tile, 0 the 192-row
// split tile (k-tiles of 64), 1 the 256-row split tile (k-tiles of 32), 2
// the 128 x 128 two-pair tile for grids that would leave CUs idle.
static int split_tile(const GemmDesc& d) {
  if (d.K % 64 == 0 && ntiles(d, 160, 128, 1) >= 2 * kCUs) return 4;
  if (d.K % 64 == 0 && ntiles(d, 256, 128, 1) >= kCUs) return 3;
  if (d.K % 64 == 0 && ntiles(d, 192, 128, 1) >= kCUs) return 0;
  if (ntiles(d, 256, 128, 1) >= kCUs) return 1;
  return 2;
}

// Weight gradients: 256 x 256 tiles when both output sides allow it, and a
// split of K that minimises (waves of workgroups) / (split) plus a small cost
// per extra split for the partial-sum traffic.
static bool wgrad_big_tile(const GemmDesc& d) { return d.M >= 256 && d.N >= 256; }

static int wgrad_split(const GemmDesc& d, int groups) {
  const bool big = wgrad_big_tile(d);
  const int64_t t = ntiles(d, big ? 256 : 128, big ? 256 : 128, groups);
  const int nk = d.K / 64;
  int best = 1;
  double best_cost = 1e30;
  for (int sp : {1, 2, 3, 4, 6, 8}) {
    if (nk % sp != 0 || nk / sp < 4) continue;
    const double waves = (double)((t * sp + kCUs - 1) / kCUs);
    const double cost = waves / sp + 0.03 * (sp - 1);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

static hipError_t run_gemm2(int op, const GemmDesc& d, int groups, hipStream_t s) {
  if (op == OP_TN_WGRAD) {
    // Long K per slice (at most 2 slices): separate rings measured 2-5%
    // faster; with 4 or more slices they were ~3% slower.
    if (wgrad_big_tile(d) && d.ksplit <= 2) return launch2<P256x256a, 1, 3u, EPI_WGRAD>(d, groups, s);
    if (wgrad_big_tile(d)) return launch2<P256x256, 1, 3u, EPI_WGRAD>(d, groups, s);
    return launch2<P128x128, 1, 3u, EPI_WGRAD>(d, groups, s);
  }
  switch (op) {
    case OP_NT_STORE: return launch_single<EPI_STORE, 0u>(d, groups, s);
    case OP_NT_ORMS: return launch_single<EPI_ORMS, 0u>(d, groups, s);
    case OP_NN_STORE: return launch_single<EPI_STORE, 2u>(d, groups, s);
    case OP_NN_RMSBWD: return launch_single<EPI_RMSBWD, 2u>(d, groups, s);
    case OP_NT_RMSBWD: return launch_single<EPI_RMSBWD, 0u>(d, groups, s);
    case OP_NT_SWIGLU:
      switch (split_tile(d)) {
        case 4: return launch2<PBDP160x128, 2, 0u, EPI_SWIGLU>(d, 1, s);
        case 3: return launch2<PBD256x128, 2, 0u, EPI_SWIGLU>(d, 1, s);
        case 0: return launch2<PS192x128, 2, 0u, EPI_SWIGLU>(d, 1, s);
        case 1: return launch2<PS256x128, 2, 0u, EPI_SWIGLU>(d, 1, s);
        default: return launch2<P2x128x128, 2, 0u, EPI_SWIGLU>(d, 1, s);
      }
    case OP_SWIGLU_BWD2:
      switch (split_tile(d)) {
        case 4: return launch2<PBDP160x128, 2, 0u, EPI_SWIGLU_BWD2>(d, 1, s);
        case 3: return launch2<PBD256x128, 2, 0u, EPI_SWIGLU_BWD2>(d, 1, s);
        case 0: return launch2<PS192x128, 2, 0u, EPI_SWIGLU_BWD2>(d, 1, s);
        case 1: return launch2<PS256x128, 2, 0u, EPI_SWIGLU_BWD2>(d, 1, s);
        default: return launch2<P2x128x128, 2, 0u, EPI_SWIGLU_BWD2>(d, 1, s);
      }
    default: return hipErrorInvalidValue;
  }
}

static int engine2_bk(int op) {
  return (op == OP_NT_SWIGLU || op == OP_SWIGLU_BWD2) ? 32 : 64;
}

int gemm2_tile_m(int op, const GemmDesc& d, int groups) {
  if (op == OP_NT_SWIGLU || op == OP_SWIGLU_BWD2) {
    const int t = split_tile(d);
    return t == 4 ? 160 : t == 0 ? 192 : ((t == 1 || t == 3) ? 256 : 128);
  }
  return single_tile(d, groups) == 2 ? 128 : 256;
}

// The three-pair recompute (dm in the same tile) runs on the general engine
// only: on this engine the recompute is a dm product and a two-pair tile,
// which take the same shapes as the forward's gate/up tile.
bool uses_engine2(int op, int dtype, const GemmDesc& d, int groups) {
  return dtype == 1 && op != OP_SWIGLU_BWD && eligible2(op, d, groups, engine2_bk(op));
}

int gemm_tile_m_used(int op, int dtype, const GemmDesc& d, int groups) {
  return uses_engine2(op, dtype, d, groups) ? gemm2_tile_m(op, d, groups)
                                            : gemm_tile_m(op, dtype);
}

// out[slot][i, j] = colscale[j] * sum_s part[s][slot][i, j], s in order.
// The outputs of the groups of one grouped weight gradient.
struct SumOut {
  float* out[3];
  int64_t ldo[3];
};
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t split_stride,
                                                            int64_t count, int groups, int n,
                                                            const bf16_t* __restrict__ colscale,
                                                            SumOut o) {
  // part holds groups x count floats per slice (group g at g * count), the
  // slices split_stride apart; group g's sum goes to o.out[g].
  const int64_t nq = count / 4;
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < nq * groups;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(q / nq);
    const int64_t e = (q - g * nq) * 4;
    const float* pg = part + g * count;
    // Slices in order 0, 1, 2, ...; four loads in flight at a time.
    f32x4 acc = *reinterpret_cast<const f32x4*>(pg + e);
    int sp = 1;
    for (; sp + 3 < splits; sp += 4) {
      f32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const f32x4*>(pg + (sp + k) * split_stride + e);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += v[k];
    }
    for (; sp < splits; ++sp) acc += *reinterpret_cast<const f32x4*>(pg + sp * split_stride + e);
    const int64_t row = e / n;
    const int col = (int)(e % n);
    if (colscale) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] *= Elem<bf16_t>::load(colscale + col + k);
    }
    float* out = g == 0 ? o.out[0] : (g == 1 ? o.out[1] : o.out[2]);
    const int64_t ldo = g == 0 ? o.ldo[0] : (g == 1 ? o.ldo[1] : o.ldo[2]);
    *reinterpret_cast<f32x4*>(out + row * ldo + col) = acc;
  }
}

size_t wgrad_part_bytes(int dtype, const GemmDesc& d, int groups) {
  if (!uses_engine2(OP_TN_WGRAD, dtype, d, groups)) return 0;
  const int sp = wgrad_split(d, groups);
  if (sp <= 1) return 0;
  return (size_t)sp * groups * (size_t)d.M * d.N * sizeof(float);
}

int wgrad_splits(int dtype, const GemmDesc& d, int groups, const void* part, size_t part_bytes) {
  const size_t need = wgrad_part_bytes(dtype, d, groups);
  if (need == 0 || part == nullptr || part_bytes < need || d.N % 4 != 0) return 1;
  return wgrad_split(d, groups);
}

hipError_t run_wgrad_gemm(int dtype, const GemmDesc& d, int groups, int splits, void* part,
                          hipStream_t s) {
  if (splits <= 1) return run_gemm(OP_TN_WGRAD, dtype, d, groups, s);
  GemmDesc q = d;
  q.ksplit = splits;
  const int64_t mn = (int64_t)d.M * d.N;
  q.c_split_stride = groups * mn;
  q.colscale = nullptr;
  float* pbase = static_cast<float*>(part);
  for (int gidx = 0; gidx < groups; ++gidx) {
    q.c[gidx] = pbase + gidx * mn;
    q.ldc[gidx] = d.N;
  }
  return run_gemm2(OP_TN_WGRAD, q, groups, s);
}

hipError_t run_wgrad_sum(const GemmDesc& d, int groups, int splits, const void* part,
                         hipStream_t s) {
  if (groups < 1 || groups > 3) return hipErrorInvalidValue;
  const int64_t mn = (int64_t)d.M * d.N;
  SumOut o{};
  for (int gidx = 0; gidx < groups; ++gidx) {
    o.out[gidx] = static_cast<float*>(d.c[gidx]);
    o.ldo[gidx] = d.ldc[gidx];
  }
  const int64_t nq = mn / 4 * groups;
  const int grid = (int)std::min<int64_t>((nq + 255) / 256, 8192);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<const float*>(part), splits, groups * mn, mn, groups, d.N,
                     static_cast<const bf16_t*>(d.colscale), o);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight gradients of up to three problems with different M, N (same K) in
// one launch: problems whose 256 x 256 grids are each too small for the GPU
// but together fill it run whole-K tiles side by side instead of splitting
// K (no partial sums); with fewer tiles than that K is still split, the
// partials of problem i at part + off_i (slices M_i N_i apart).
// ---------------------------------------------------------------------------
bool wgrad_multi_ok(int dtype, const GemmDesc* p, int n) {
  if (dtype != 1 || n < 1 || n > 3) return false;
  for (int i = 0; i < n; ++i) {
    if (p[i].K != p[0].K || p[i].N % 4 != 0 || !wgrad_big_tile(p[i])) return false;
    if (!uses_engine2(OP_TN_WGRAD, dtype, p[i], 1)) return false;
  }
  return true;
}

int wgrad_multi_split(const GemmDesc* p, int n) {
  int64_t t = 0;
  for (int i = 0; i < n; ++i) t += ntiles(p[i], 256, 256, 1);
  const int nk = p[0].K / 64;
  int best = 1;
  double best_cost = 1e30;
  for (int sp : {1, 2, 3, 4, 6, 8}) {
    if (nk % sp != 0 || nk / sp < 4) continue;
    const double waves = (double)((t * sp + kCUs - 1) / kCUs);
    const double cost = waves / sp + 0.03 * (sp - 1);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

size_t wgrad_multi_part_bytes(const GemmDesc* p, int n, int splits) {
  if (splits <= 1) return 0;
  size_t b = 0;
  for (int i = 0; i < n; ++i) b += (size_t)splits * (size_t)p[i].M * p[i].N * sizeof(float);
  return b;
}

int64_t wgrad_multi_part_offset(const GemmDesc* p, int i, int splits) {
  int64_t off = 0;
  for (int j = 0; j < i; ++j) off += (int64_t)splits * p[j].M * p[j].N;
  return off;
}

template <class TL>
static hipError_t launch2_multi(const GemmDesc* p, int n, int splits, float* part, hipStream_t s) {
  auto kern = gemm2_kernel<TL, 1, 3u, EPI_WGRAD>;
  constexpr int lds = gemm2_lds_bytes<TL, 1, EPI_WGRAD>();
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  if (attr_err != hipSuccess) return attr_err;
  GemmArgs g{};
  g.K = p[0].K;
  g.groups = 1;
  g.ktiles_split = p[0].K / TL::BK / splits;
  g.nprob = n;
  int base = 0;
  for (int i = 0; i < 3; ++i) {
    const GemmDesc& d = p[i < n ? i : n - 1];
    const bool live = i < n;
    g.a[i] = d.a[0];
    g.lda[i] = d.lda[0];
    g.b[i] = d.b[0];
    g.ldb[i] = d.ldb[0];
    g.Mp[i] = d.M;
    g.Np[i] = d.N;
    g.tiles_mp[i] = (d.M + TL::BM - 1) / TL::BM;
    g.tiles_np[i] = (d.N + TL::BNO - 1) / TL::BNO;
    g.prob_base[i] = base;
    if (live) base += g.tiles_mp[i] * g.tiles_np[i];
    if (splits > 1) {
      g.c[i] = part + wgrad_multi_part_offset(p, i < n ? i : n - 1, splits);
      g.ldc[i] = d.N;
      g.colscales[i] = nullptr;
    } else {
      g.c[i] = d.c[0];
      g.ldc[i] = d.ldc[0];
      g.colscales[i] = d.colscale;
    }
    g.csplit[i] = (int64_t)d.M * d.N;
  }
  // Problems past n start past the last workgroup.
  for (int i = n; i < 3; ++i) g.prob_base[i] = base;
  g.prob_base[3] = base;
  g.cs_part = p[0].cs_part;
  g.cs_rows = p[0].cs_rows;
  g.cs_n = p[0].cs_n;
  g.cs_out = p[0].cs_out;
  if (base == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(base, 1, splits), dim3(TL::NT), lds, s, g);
  return hipGetLastError();
}

hipError_t run_wgrad_multi_gemm(const GemmDesc* p, int n, int splits, void* part, hipStream_t s) {
  float* pf = static_cast<float*>(part);
  if (splits <= 2) return launch2_multi<P256x256a>(p, n, splits, pf, s);
  return launch2_multi<P256x256>(p, n, splits, pf, s);
}

hipError_t run_gemm(int op, int dtype, const GemmDesc& d, int groups, hipStream_t s) {
  if (uses_engine2(op, dtype, d, groups)) return run_gemm2(op, d, groups, s);
  if (op == OP_SWIGLU_BWD2) return hipErrorInvalidValue;  // pipelined engine only
  if (dtype == 0) return dispatch<float, TF32, TF32, TF32>(op, d, groups, s);
  return dispatch<bf16_t, TBig, TMid, TMid>(op, d, groups, s);
}

// ---------------------------------------------------------------------------
// Memory-bound kernels
// ---------------------------------------------------------------------------

// out[n, k] = A[n, k] * gamma[k] (rounded to the storage type), for one or
// two (A, gamma, out) jobs of the same width in one launch: rows [0, rows0)
// are job 0's, the next rows1 job 1's.
template <typename T>
struct FoldJob {
  const T* A;
  int64_t lda;
  const T* gamma;
  T* out;
  int rows;
};
template <typename T>
__global__ __launch_bounds__(256) void fold_gamma_kernel(FoldJob<T> j0, FoldJob<T> j1, int cols) {
  constexpr int VEC = Elem<T>::VEC;
  const int vpr = cols / VEC;
  const int64_t total0 = (int64_t)j0.rows * vpr, total = total0 + (int64_t)j1.rows * vpr;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool first = i < total0;
    const int64_t li = first ? i : i - total0;
    const int r = (int)(li / vpr), c = (int)(li % vpr) * VEC;
    const T* A = first ? j0.A : j1.A;
    const T* gmp = first ? j0.gamma : j1.gamma;
    T* out = first ? j0.out : j1.out;
    const int64_t lda = first ? j0.lda : j1.lda;
    float a[VEC], gm[VEC];
    unpack16<T>(*reinterpret_cast<const u32x4*>(A + r * lda + c), a);
    unpack16<T>(*reinterpret_cast<const u32x4*>(gmp + c), gm);
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
    // Up to U chunks of both rows are in flight before the first FMA.
    constexpr int U = 8;
    for (int c0 = lane * VEC; c0 < width; c0 += U * 64 * VEC) {
      u32x4 ra[U], rb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64 * VEC;
        ra[u] = rb[u] = u32x4{0u, 0u, 0u, 0u};
        if (c < width) {
          ra[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pa + c));
          rb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pb + c));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[VEC], y[VEC];
        unpack16<T>(ra[u], x);
        unpack16<T>(rb[u], y);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = __builtin_fmaf(x[e], y[e], acc);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) coef[t] = acc / rms[t] * inv_D;
  }
}

// out[c] = sum_t part[t, c] in a fixed order: four row groups of a block
// each add every fourth partial row, then the four sums are added in order.
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ part, int tiles,
                                                     int n, float* __restrict__ out) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (c < n)
    for (int t = q; t < tiles; t += 4) s += part[(int64_t)t * n + c];
  red[q][lane] = s;
  __syncthreads();
  if (q == 0 && c < n) out[c] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// Rank-share finalisation after the (identity) all-reduce:
// rms[t] = sqrt(ss[t] * inv_D + eps); z[t, :] = P[t, :] / rms[t].
template <typename T>
__global__ __launch_bounds__(256) void finalize_kernel(const T* __restrict__ P, int64_t ldp,
                                                       const float* __restrict__ ss, int rows,
                                                       int width, float inv_D, float eps,
                                                       T* __restrict__ z, int64_t ldz,
                                                       float* __restrict__ rms_out) {
  // One 16-byte chunk per thread: blockIdx.x picks 256 chunks of a row,
  // blockIdx.y (stepping by gridDim.y) the row, so every load is independent.
  constexpr int VEC = Elem<T>::VEC;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * VEC;
  for (int t = blockIdx.y; t < rows; t += gridDim.y) {
    const float rmsg = sqrtf(ss[t] * inv_D + eps);
    if (c == 0 && rms_out) rms_out[t] = rmsg;
    if (c < width) {
      const float s = 1.0f / rmsg;
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

template <typename T>
static hipError_t fold2(const void* A0, int64_t lda0, const void* g0, void* o0, int rows0,
                        const void* A1, int64_t lda1, const void* g1, void* o1, int rows1,
                        int cols, hipStream_t s) {
  const FoldJob<T> j0{static_cast<const T*>(A0), lda0, static_cast<const T*>(g0),
                      static_cast<T*>(o0), rows0};
  const FoldJob<T> j1{static_cast<const T*>(A1 ? A1 : A0), A1 ? lda1 : lda0,
                      static_cast<const T*>(A1 ? g1 : g0), static_cast<T*>(A1 ? o1 : o0),
                      A1 ? rows1 : 0};
  const int64_t chunks = ((int64_t)j0.rows + j1.rows) * cols / Elem<T>::VEC;
  hipLaunchKernelGGL(fold_gamma_kernel<T>, dim3(grid_for(chunks, 256)), dim3(256), 0, s, j0, j1,
                     cols);
  return hipGetLastError();
}

hipError_t run_fold_gamma(int dtype, const void* A, int64_t lda, const void* gamma, void* out,
                          int rows, int cols, hipStream_t s) {
  return dtype == 0 ? fold2<float>(A, lda, gamma, out, rows, nullptr, 0, nullptr, nullptr, 0,
                                   cols, s)
                    : fold2<bf16_t>(A, lda, gamma, out, rows, nullptr, 0, nullptr, nullptr, 0,
                                    cols, s);
}

hipError_t run_fold_gamma2(int dtype, const void* A0, int64_t lda0, const void* g0, void* o0,
                           int rows0, const void* A1, int64_t lda1, const void* g1, void* o1,
                           int rows1, int cols, hipStream_t s) {
  return dtype == 0 ? fold2<float>(A0, lda0, g0, o0, rows0, A1, lda1, g1, o1, rows1, cols, s)
                    : fold2<bf16_t>(A0, lda0, g0, o0, rows0, A1, lda1, g1, o1, rows1, cols, s);
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
  hipLaunchKernelGGL(colsum_kernel, dim3((n + 63) / 64), dim3(256), 0, s, part, tiles, n, out);
  return hipGetLastError();
}

hipError_t run_finalize(int dtype, const void* P, int64_t ldp, const float* ss, int rows,
                        int width, float inv_D, float eps, void* z, int64_t ldz, float* rms_out,
                        hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int vec = dtype == 0 ? 4 : 8;
  const dim3 grid((unsigned)std::max(1, (width / vec + 255) / 256), (unsigned)std::min(rows, 65535));
  if (dtype == 0) {
    hipLaunchKernelGGL(finalize_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(P), ldp, ss, rows, width, inv_D, eps,
                       static_cast<float*>(z), ldz, rms_out);
  } else {
    hipLaunchKernelGGL(finalize_kernel<bf16_t>, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(P), ldp, ss, rows, width, inv_D, eps,
                       static_cast<bf16_t*>(z), ldz, rms_out);
  }
  return hipGetLastError();
}


// bf16 transposes: a workgroup moves one 64 x 64 tile through LDS. A
// thread loads 16-byte chunks of two consecutive rows and writes, per
// column, the two rows' values as one 32-bit word of the LDS tile, stored
// column by column ([64 columns][32 row pairs + 4]); an output chunk (8
// rows of one column) is then one 16-byte LDS read. Jobs come one after
// another in the grid (first_tile[j] their first tile).
struct TransposeJobs {
  TransposeJob j[kMaxTranspose];
  int first_tile[kMaxTranspose + 1];
  int n;
};
__global__ __launch_bounds__(256) void transpose_bf16_kernel(TransposeJobs t) {
  __shared__ __align__(16) uint32_t tile[64][32 + 4];
  const int b = blockIdx.x;
  int ji = 0;
  while (ji + 1 < t.n && b >= t.first_tile[ji + 1]) ++ji;
  const TransposeJob& J = t.j[ji];
  const int tcols = (J.cols + 63) / 64;
  const int lt = b - t.first_tile[ji];
  const int r0 = (lt / tcols) * 64, c0 = (lt % tcols) * 64;
  const uint16_t* in = static_cast<const uint16_t*>(J.in);
  uint16_t* out = static_cast<uint16_t*>(J.out);
  {
    const int p = threadIdx.x >> 3, c = (threadIdx.x & 7) * 8;  // rows 2p, 2p + 1
    if (c0 + c < J.cols) {
      const uint16_t* src = in + (int64_t)(r0 + 2 * p) * J.ldi + c0 + c;
      const u32x4 a = *reinterpret_cast<const u32x4*>(src);
      const u32x4 bb = *reinterpret_cast<const u32x4*>(src + J.ldi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile[c + 2 * e][p] = (a[e] & 0xFFFFu) | (bb[e] << 16);
        tile[c + 2 * e + 1][p] = (a[e] >> 16) | (bb[e] & 0xFFFF0000u);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int oc = (threadIdx.x >> 3) + 32 * k, ch = threadIdx.x & 7;  // rows 8 ch .. + 7
    if (c0 + oc < J.cols) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&tile[oc][4 * ch]);
      *reinterpret_cast<u32x4*>(out + (int64_t)(c0 + oc) * J.ldo + r0 + 8 * ch) = v;
    }
  }
}

hipError_t run_transpose_bf16(const TransposeJob* jobs, int n, hipStream_t s) {
  if (n < 1 || n > kMaxTranspose) return hipErrorInvalidValue;
  TransposeJobs t{};
  t.n = n;
  int tiles = 0;
  for (int i = 0; i < n; ++i) {
    const TransposeJob& J = jobs[i];
    if (J.rows % 64 != 0 || J.cols % 8 != 0 || J.rows < 0 || J.cols < 0 || !J.in || !J.out)
      return hipErrorInvalidValue;
    t.j[i] = J;
    t.first_tile[i] = tiles;
    tiles += (J.rows / 64) * ((J.cols + 63) / 64);
  }
  t.first_tile[n] = tiles;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(tiles), dim3(256), 0, s, t);
  return hipGetLastError();
}

}  // namespace lr
