// MFMA GEMM engine for gfx950 with the block's fused epilogues.
//
// One workgroup computes a BM x BN tile of C[i, j] = sum_k A(i, k) B(j, k)
// for up to three operand pairs at once (each pair has its own accumulator),
// then runs one epilogue over the accumulators. Operands are read from HBM
// with 16-byte vector loads into registers, written to LDS in a
// K-contiguous layout (an operand whose storage is M- or N-contiguous is
// transposed in registers on the way), and fed to v_mfma_f32_16x16x32_bf16
// (bf16) or v_mfma_f32_16x16x4_f32 (fp32). The next K-tile's loads are in
// flight while the current one is multiplied.
//
// Accumulator layout of a 16x16 MFMA tile (all 16x16 variants): lane l holds
// rows 4*(l/16) + v (v = 0..3) of column l % 16. The k order inside a
// fragment only has to agree between A and B, which it does by construction.
#pragma once

#include "lr_common.hpp"

namespace lr {

template <int BM_, int BN_, int BK_, int NWM_, int NWN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NWM = NWM_, NWN = NWN_;
  static constexpr int NT = 64 * NWM * NWN;
  static constexpr int WTM = BM / NWM, WTN = BN / NWN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
};

enum EpiKind : int {
  EPI_STORE = 0,       // out = acc [/ rowdiv[row]] [+ res]
  EPI_ORMS = 1,        // Online RMSNorm: out = acc / rms_g (or acc, partial mode)
  EPI_SWIGLU = 2,      // out = SiLU(acc0) * acc1
  EPI_SWIGLU_BWD = 3,  // acc0 = g, acc1 = u, acc2 = dm -> m, dg, du
  EPI_RMSBWD = 4,      // out = res + gamma[col]*acc - coef[row]*H; colsum(acc*H)
  EPI_WGRAD = 5,       // fp32 out = acc [* colscale[col]]
  EPI_SWIGLU_BWD2 = 6, // acc0 = g, acc1 = u, res = dm -> m, dg, du (pipelined engine)
};

struct GemmArgs {
  int M, N, K;
  int tiles_m, tiles_n;
  // Operand slots: the pair index for multi-pair kernels, the group index
  // (blockIdx.z) for grouped kernels.
  const void* a[3];
  int64_t lda[3];
  const void* b[3];
  int64_t ldb[3];
  void* c[3];
  int64_t ldc[3];
  const void* res;      // residual (EPI_STORE) or upstream gradient (EPI_RMSBWD)
  int64_t ldres;
  const void* hsrc;     // H of EPI_RMSBWD
  int64_t ldh;
  const float* rowdiv;  // EPI_STORE: divide each row by rowdiv[row]
  const float* rowcoef; // EPI_RMSBWD: per-row coefficient of H
  const void* colscale; // gamma: EPI_RMSBWD, EPI_WGRAD
  float* colsum;        // EPI_RMSBWD: per-M-tile column sums [tiles_m][N]
  // Online RMSNorm
  float* rms_out;       // [M] global RMS (normal mode, written by N-tile 0)
  float* ss_out;        // [P][M] per-panel sums of squares (N-tile 0)
  int n_panels;
  int panel_ktiles;     // K-tiles per panel
  float inv_D;
  float eps;
  int emit_partial;
  // Split-K (pipelined engine): blockIdx.z = slot + groups * split; split s
  // covers k-tiles [s * ktiles_split, (s + 1) * ktiles_split) and writes its
  // output at c[slot] + s * c_split_stride.
  int groups;
  int ktiles_split;
  int64_t c_split_stride;
  // Side job of the pipelined engine, run by every workgroup after its own
  // outputs: cs_out[c] = sum over r = 0 .. cs_rows - 1 of
  // cs_part[r * cs_n + c] in a fixed order (the gamma-gradient column sums
  // of an RMSNorm backward launched before this kernel). Off when cs_out is
  // null.
  const float* cs_part;
  int cs_rows, cs_n;
  float* cs_out;
  // Up to three problems of different M, N (same K) in one launch (weight
  // gradients, pipelined engine), when nprob > 0: after the XCD remapping
  // the workgroups [prob_base[p], prob_base[p + 1]) run problem p's
  // tiles_mp[p] x tiles_np[p] tiles, and slot p of the operand arrays is
  // problem p's, with its own M, N, column scale and element stride
  // between split-K slices. blockIdx.z is then the split.
  int nprob;
  int Mp[3], Np[3], tiles_mp[3], tiles_np[3], prob_base[4];
  const void* colscales[3];
  int64_t csplit[3];
  // Persistent launches (pipelined engine, kernels that walk their tiles):
  // tiles_m x tiles_n x groups tiles, workgroup b running tiles b,
  // b + gridDim.x, ...
  int vtiles;
};

// ---------------------------------------------------------------------------
// Operand staging: HBM -> registers -> LDS [R][PITCH] (K contiguous).
// KC: element (i, k) at p[i*ld + k]; otherwise at p[k*ld + i].
// ---------------------------------------------------------------------------
template <typename T, int R, int BK, int NT, bool KC>
struct Stage {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int PITCH = BK + VEC;
  static constexpr int KB = BK / VEC;  // 16-byte vectors along k per row
  static constexpr int TOTAL = KC ? R * KB : KB * (R / VEC);
  static constexpr int NPER = (TOTAL + NT - 1) / NT;
  static constexpr int NREG = KC ? NPER : NPER * VEC;
  static_assert(BK % VEC == 0 && R % VEC == 0, "tile not a multiple of the vector");
  u32x4 reg[NREG];

  __device__ __forceinline__ void load(const T* __restrict__ p, int64_t ld, int r0, int Rtot,
                                       int k0, int K, int tid) {
#pragma unroll
    for (int v = 0; v < NPER; ++v) {
      const int idx = tid + v * NT;
      const bool live = (TOTAL % NT == 0) || idx < TOTAL;
      if constexpr (KC) {
        const int row = idx / KB, kv = idx % KB;
        const int gr = r0 + row, gk = k0 + kv * VEC;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (live && gr < Rtot) {
          const T* src = p + (int64_t)gr * ld + gk;
          if (gk + VEC <= K) {
            x = *reinterpret_cast<const u32x4*>(src);
          } else if (gk < K) {
            x = load_partial(src, K - gk, 1);
          }
        }
        reg[v] = x;
      } else {
        const int kb = idx % KB, mb = idx / KB;
        const int gm = r0 + mb * VEC;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int gk = k0 + kb * VEC + j;
          u32x4 x = {0u, 0u, 0u, 0u};
          if (live && gk < K && gm < Rtot) {
            const T* src = p + (int64_t)gk * ld + gm;
            if (gm + VEC <= Rtot) {
              x = *reinterpret_cast<const u32x4*>(src);
            } else {
              x = load_partial(src, Rtot - gm, 1);
            }
          }
          reg[v * VEC + j] = x;
        }
      }
    }
  }

  // Fewer than VEC valid elements at src (stride 1): element-wise loads.
  __device__ __forceinline__ static u32x4 load_partial(const T* src, int n, int) {
    float f[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) f[e] = (e < n) ? Elem<T>::load(src + e) : 0.0f;
    return pack16<T>(f);
  }

  __device__ __forceinline__ void store(T* __restrict__ s, int tid) const {
#pragma unroll
    for (int v = 0; v < NPER; ++v) {
      const int idx = tid + v * NT;
      const bool live = (TOTAL % NT == 0) || idx < TOTAL;
      if (!live) continue;
      if constexpr (KC) {
        const int row = idx / KB, kv = idx % KB;
        *reinterpret_cast<u32x4*>(s + row * PITCH + kv * VEC) = reg[v];
      } else {
        const int kb = idx % KB, mb = idx / KB;
        u32x4 out[VEC];
        transpose(&reg[v * VEC], out);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
          *reinterpret_cast<u32x4*>(s + (mb * VEC + i) * PITCH + kb * VEC) = out[i];
      }
    }
  }

  // in[j] holds VEC consecutive m at k = j; out[i] holds VEC consecutive k at m = i.
  __device__ __forceinline__ static void transpose(const u32x4* in, u32x4* out) {
    if constexpr (VEC == 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t a = in[2 * q][i >> 1], b = in[2 * q + 1][i >> 1];
          out[i][q] = (i & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) out[i][j] = in[j][i];
    }
  }

  // Online RMSNorm: add the squares of this thread's (KC) vectors to part[v].
  __device__ __forceinline__ void sum_squares(float* part) const {
    static_assert(KC, "row statistics need the K-contiguous layout");
#pragma unroll
    for (int v = 0; v < NPER; ++v) {
      if constexpr (VEC == 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_lo(reg[v][q]), hi = bf16_hi(reg[v][q]);
          part[v] = __builtin_fmaf(lo, lo, part[v]);
          part[v] = __builtin_fmaf(hi, hi, part[v]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x = __uint_as_float(reg[v][q]);
          part[v] = __builtin_fmaf(x, x, part[v]);
        }
      }
    }
  }
};

// One 16-byte fragment step of MFMAs on an accumulator tile.
template <typename T>
__device__ __forceinline__ void mfma_step(const u32x4& a, const u32x4& b, f32x4& c);

template <>
__device__ __forceinline__ void mfma_step<bf16_t>(const u32x4& a, const u32x4& b, f32x4& c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<float>(const u32x4& a, const u32x4& b, f32x4& c) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c,
                                             0, 0, 0);
}

// Map the linear workgroup id to an output tile: ids on the same XCD (the
// hardware deals workgroups to the 8 XCDs round-robin) get consecutive
// logical ids, which walk GROUP_M M-tiles before the next N-tile so that the
// XCD's L2 serves both operands' tiles to several workgroups.
__device__ __forceinline__ int xcd_logical_of(int pid, int nwg) {
  constexpr int NXCD = 8;
  const int q = nwg / NXCD, rem = nwg % NXCD;
  const int x = pid % NXCD;
  return x * q + (x < rem ? x : rem) + pid / NXCD;
}
__device__ __forceinline__ int xcd_logical(int nwg) { return xcd_logical_of((int)blockIdx.x, nwg); }
template <int GROUP_M = 8>
__device__ __forceinline__ void group_tile(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int in_group = GROUP_M * tiles_n;
  const int gid = logical / in_group;
  const int first_m = gid * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int l = logical % in_group;
  tm = first_m + l % gsize;
  tn = l / gsize;
}
template <int GROUP_M = 8>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  group_tile<GROUP_M>(xcd_logical(tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// LDS bytes used by the main loop.
template <class TL, typename T, int NPAIR>
constexpr int mainloop_lds_bytes() {
  return NPAIR * (TL::BM + TL::BN) * (TL::BK + Elem<T>::VEC) * (int)sizeof(T);
}

template <class TL>
constexpr int stage_c_lds_bytes() {
  return TL::BM * (TL::BN + 4) * 4;
}

template <class TL, typename T, int NPAIR>
constexpr int gemm_lds_bytes() {
  constexpr int a = mainloop_lds_bytes<TL, T, NPAIR>();
  constexpr int b = stage_c_lds_bytes<TL>();
  return (a > b ? a : b) + 8 * TL::BM * 4 /* row stats */ + 4 * TL::BM * 4;
}

// ---------------------------------------------------------------------------
// The K loop. acc[p] accumulates pair p. With ORMS, pair 0's A operand is
// X and its per-row sums of squares are reduced per K-panel into sSS[P][BM].
// ---------------------------------------------------------------------------
template <class TL, typename T, int NPAIR, uint32_t MCMASK, bool ORMS>
__device__ __forceinline__ void mainloop(const GemmArgs& g, int slot0, int m0, int n0,
                                         f32x4 (&acc)[NPAIR][TL::FM][TL::FN], T* smem,
                                         float* sSS) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, NT = TL::NT;
  constexpr int VEC = Elem<T>::VEC, PITCH = BK + VEC, FRAG_K = Elem<T>::FRAG_K;
  static_assert(BK % FRAG_K == 0, "BK must be a multiple of the fragment k");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::NWN, wn = wave % TL::NWN;

  // Stagers per pair (compile-time layouts).
  Stage<T, BM, BK, NT, !(MCMASK & 1u)> sa0;
  Stage<T, BN, BK, NT, !(MCMASK & 2u)> sb0;
  Stage<T, BM, BK, NT, !(MCMASK & 4u)> sa1;
  Stage<T, BN, BK, NT, !(MCMASK & 8u)> sb1;
  Stage<T, BM, BK, NT, !(MCMASK & 16u)> sa2;
  Stage<T, BN, BK, NT, !(MCMASK & 32u)> sb2;

  T* sA[3];
  T* sB[3];
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    sA[p] = smem + p * (BM + BN) * PITCH;
    sB[p] = sA[p] + BM * PITCH;
  }

#pragma unroll
  for (int p = 0; p < NPAIR; ++p)
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) acc[p][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int M = g.M, N = g.N, K = g.K;
  auto load_all = [&](int k0) {
    sa0.load(static_cast<const T*>(g.a[slot0]), g.lda[slot0], m0, M, k0, K, tid);
    sb0.load(static_cast<const T*>(g.b[slot0]), g.ldb[slot0], n0, N, k0, K, tid);
    if constexpr (NPAIR > 1) {
      sa1.load(static_cast<const T*>(g.a[1]), g.lda[1], m0, M, k0, K, tid);
      sb1.load(static_cast<const T*>(g.b[1]), g.ldb[1], n0, N, k0, K, tid);
    }
    if constexpr (NPAIR > 2) {
      sa2.load(static_cast<const T*>(g.a[2]), g.lda[2], m0, M, k0, K, tid);
      sb2.load(static_cast<const T*>(g.b[2]), g.ldb[2], n0, N, k0, K, tid);
    }
  };
  auto store_all = [&]() {
    sa0.store(sA[0], tid);
    sb0.store(sB[0], tid);
    if constexpr (NPAIR > 1) {
      sa1.store(sA[1], tid);
      sb1.store(sB[1], tid);
    }
    if constexpr (NPAIR > 2) {
      sa2.store(sA[2], tid);
      sb2.store(sB[2], tid);
    }
  };

  constexpr int NSS = ORMS ? Stage<T, BM, BK, NT, true>::NPER : 1;
  float ss_part[NSS];
#pragma unroll
  for (int v = 0; v < NSS; ++v) ss_part[v] = 0.f;
  int panel = 0, in_panel = 0;

  const int nk = (K + BK - 1) / BK;
  load_all(0);
  for (int kt = 0; kt < nk; ++kt) {
    store_all();
    if constexpr (ORMS) {
      sa0.sum_squares(ss_part);
      if (++in_panel == g.panel_ktiles || kt == nk - 1) {
        // Reduce each row's partial sums over the KB lanes that share it.
        constexpr int KB = BK / VEC;
#pragma unroll
        for (int v = 0; v < NSS; ++v) {
          float x = ss_part[v];
#pragma unroll
          for (int off = 1; off < KB; off <<= 1) x += __shfl_xor(x, off, 64);
          const int idx = tid + v * NT;
          if ((idx % KB) == 0 && idx < BM * KB) sSS[panel * BM + idx / KB] = x;
          ss_part[v] = 0.f;
        }
        ++panel;
        in_panel = 0;
      }
    }
    __syncthreads();
    if (kt + 1 < nk) load_all((kt + 1) * BK);

#pragma unroll
    for (int f = 0; f < BK / FRAG_K; ++f) {
      const int koff = f * FRAG_K + (VEC * (lane >> 4));
#pragma unroll
      for (int p = 0; p < NPAIR; ++p) {
        u32x4 af[TL::FM], bfr[TL::FN];
#pragma unroll
        for (int i = 0; i < TL::FM; ++i)
          af[i] = *reinterpret_cast<const u32x4*>(
              sA[p] + (wm * TL::WTM + i * 16 + (lane & 15)) * PITCH + koff);
#pragma unroll
        for (int j = 0; j < TL::FN; ++j)
          bfr[j] = *reinterpret_cast<const u32x4*>(
              sB[p] + (wn * TL::WTN + j * 16 + (lane & 15)) * PITCH + koff);
#pragma unroll
        for (int i = 0; i < TL::FM; ++i)
#pragma unroll
          for (int j = 0; j < TL::FN; ++j) mfma_step<T>(af[i], bfr[j], acc[p][i][j]);
      }
    }
    __syncthreads();
  }
}

// Write one accumulator set into the fp32 LDS staging tile [BM][BN + 4].
template <class TL>
__device__ __forceinline__ void stage_acc(const f32x4 (&acc)[TL::FM][TL::FN], float* sC) {
  constexpr int CP = TL::BN + 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::NWN, wn = wave % TL::NWN;
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * TL::WTM + i * 16 + 4 * (lane >> 4) + v;
        const int col = wn * TL::WTN + j * 16 + (lane & 15);
        sC[row * CP + col] = acc[i][j][v];
      }
}

// Read 8 consecutive staged columns.
template <class TL>
__device__ __forceinline__ void read8(const float* sC, int row, int c8, float* v) {
  constexpr int CP = TL::BN + 4;
  const f32x4 a = *reinterpret_cast<const f32x4*>(sC + row * CP + c8);
  const f32x4 b = *reinterpret_cast<const f32x4*>(sC + row * CP + c8 + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = a[e];
    v[4 + e] = b[e];
  }
}

// Load / store 8 consecutive elements of a row-major matrix with a column
// tail of n < 8 valid elements.
template <typename T>
__device__ __forceinline__ void gload8(const T* p, int n, float* v) {
  if constexpr (sizeof(T) == 2) {
    if (n >= 8) {
      unpack16<T>(*reinterpret_cast<const u32x4*>(p), v);
      return;
    }
  } else {
    if (n >= 8) {
      unpack16<T>(*reinterpret_cast<const u32x4*>(p), v);
      unpack16<T>(*reinterpret_cast<const u32x4*>(p + 4), v + 4);
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (e < n) ? Elem<T>::load(p + e) : 0.0f;
}

template <typename T>
__device__ __forceinline__ void gstore8(T* p, int n, const float* v) {
  // Outputs are streamed (non-temporal): no later access of this kernel
  // reads them, and they are far larger than the L2.
  if constexpr (sizeof(T) == 2) {
    if (n >= 8) {
      __builtin_nontemporal_store(pack16<T>(v), reinterpret_cast<u32x4*>(p));
      return;
    }
  } else {
    if (n >= 8) {
      __builtin_nontemporal_store(pack16<T>(v), reinterpret_cast<u32x4*>(p));
      __builtin_nontemporal_store(pack16<T>(v + 4), reinterpret_cast<u32x4*>(p + 4));
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e < n) Elem<T>::store(p + e, v[e]);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <class TL, typename T, int NPAIR, uint32_t MCMASK, int EPI>
__global__ __launch_bounds__(TL::NT) void gemm_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BN = TL::BN, NT = TL::NT;
  constexpr bool ORMS = (EPI == EPI_ORMS);
  extern __shared__ __align__(16) unsigned char lds_raw[];
  T* smem = reinterpret_cast<T*>(lds_raw);
  constexpr int MAIN = mainloop_lds_bytes<TL, T, NPAIR>();
  constexpr int STG = stage_c_lds_bytes<TL>();
  constexpr int BODY = MAIN > STG ? MAIN : STG;
  float* sSS = reinterpret_cast<float*>(lds_raw + BODY);  // [8][BM]
  float* sRow = sSS + 8 * BM;                              // [4][BM]
  float* sC = reinterpret_cast<float*>(lds_raw);

  int tm, tn;
  tile_coords(g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int slot = (NPAIR == 1) ? (int)blockIdx.z : 0;

  f32x4 acc[NPAIR][TL::FM][TL::FN];
  mainloop<TL, T, NPAIR, MCMASK, ORMS>(g, slot, m0, n0, acc, smem, sSS);

  const int tid = threadIdx.x;
  const int M = g.M, N = g.N;

  // Per-row quantities into sRow.
  if constexpr (ORMS) {
    for (int r = tid; r < BM; r += NT) {
      float ss = 0.f;
      for (int p = 0; p < g.n_panels; ++p) ss += sSS[p * BM + r];
      const float rmsg = sqrtf(ss * g.inv_D + g.eps);
      sRow[r] = g.emit_partial ? 1.0f : 1.0f / rmsg;
      const int gr = m0 + r;
      if (tn == 0 && gr < M) {
        if (g.rms_out && !g.emit_partial) g.rms_out[gr] = rmsg;
        if (g.ss_out) {
          if (g.emit_partial) {
            g.ss_out[gr] = ss;
          } else {
            for (int p = 0; p < g.n_panels; ++p) g.ss_out[(int64_t)p * M + gr] = sSS[p * BM + r];
          }
        }
      }
    }
  }

  constexpr int CH = BN / 8;
  constexpr int NOUT = (EPI == EPI_SWIGLU_BWD) ? 3 : 1;

  if constexpr (EPI == EPI_SWIGLU) {
    // m = SiLU(g) * u, element by element in the accumulator layout.
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gg = acc[0][i][j][v];
          acc[0][i][j][v] = gg * sigmoid_f<T>(gg) * acc[1][i][j][v];
        }
  }
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    // m = SiLU(g) u;  dg = dm u sig(g)(1 + g(1 - sig(g)));  du = dm SiLU(g)
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gg = acc[0][i][j][v], uu = acc[1][i][j][v], dm = acc[2][i][j][v];
          const float sg = sigmoid_f<T>(gg);
          const float sl = gg * sg;
          acc[0][i][j][v] = sl * uu;
          acc[1][i][j][v] = dm * uu * sg * (1.0f + gg * (1.0f - sg));
          acc[2][i][j][v] = dm * sl;
        }
  }

  float colacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) colacc[e] = 0.f;

#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    __syncthreads();  // LDS of the main loop (or the previous output) is free
    stage_acc<TL>(acc[(EPI == EPI_SWIGLU_BWD) ? o : 0], sC);
    __syncthreads();
    for (int e = tid; e < BM * CH; e += NT) {
      const int row = e / CH, c8 = (e % CH) * 8;
      const int gr = m0 + row, gc = n0 + c8;
      if (gr >= M || gc >= N) continue;
      const int nv = N - gc;
      float v[8];
      read8<TL>(sC, row, c8, v);
      if constexpr (EPI == EPI_STORE) {
        if (g.rowdiv) {
          const float s = 1.0f / g.rowdiv[gr];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] *= s;
        }
        if (g.res) {
          float rv[8];
          gload8<T>(static_cast<const T*>(g.res) + (int64_t)gr * g.ldres + gc, nv, rv);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] += rv[q];
        }
        gstore8<T>(static_cast<T*>(g.c[slot]) + (int64_t)gr * g.ldc[slot] + gc, nv, v);
      } else if constexpr (EPI == EPI_ORMS) {
        const float s = sRow[row];
        if (g.emit_partial) {
          gstore8<T>(static_cast<T*>(g.c[0]) + (int64_t)gr * g.ldc[0] + gc, nv, v);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] *= s;
          gstore8<T>(static_cast<T*>(g.c[0]) + (int64_t)gr * g.ldc[0] + gc, nv, v);
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
        gstore8<T>(static_cast<T*>(g.c[0]) + (int64_t)gr * g.ldc[0] + gc, nv, v);
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        gstore8<T>(static_cast<T*>(g.c[o]) + (int64_t)gr * g.ldc[o] + gc, nv, v);
      } else if constexpr (EPI == EPI_RMSBWD) {
        float hv[8], rv[8], gm[8];
        gload8<T>(static_cast<const T*>(g.hsrc) + (int64_t)gr * g.ldh + gc, nv, hv);
        gload8<T>(static_cast<const T*>(g.res) + (int64_t)gr * g.ldres + gc, nv, rv);
        gload8<T>(static_cast<const T*>(g.colscale) + gc, nv, gm);
        const float cf = g.rowcoef[gr];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          colacc[q] += v[q] * hv[q];
          v[q] = rv[q] + gm[q] * v[q] - cf * hv[q];
        }
        gstore8<T>(static_cast<T*>(g.c[0]) + (int64_t)gr * g.ldc[0] + gc, nv, v);
      } else if constexpr (EPI == EPI_WGRAD) {
        if (g.colscale) {
          float gm[8];
          gload8<T>(static_cast<const T*>(g.colscale) + gc, nv, gm);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] *= gm[q];
        }
        gstore8<float>(static_cast<float*>(g.c[slot]) + (int64_t)gr * g.ldc[slot] + gc, nv, v);
      }
    }
  }

  if constexpr (EPI == EPI_RMSBWD) {
    // Column sums over this tile's rows, reduced in a fixed order.
    static_assert(NT % CH == 0, "threads must tile the columns");
    constexpr int RG = NT / CH;  // row groups
    __syncthreads();
    float* sCol = sC;  // [RG][BN]
    const int c8 = (tid % CH) * 8, rg = tid / CH;
#pragma unroll
    for (int q = 0; q < 8; ++q) sCol[rg * BN + c8 + q] = colacc[q];
    __syncthreads();
    for (int c = tid; c < BN; c += NT) {
      float s = 0.f;
      for (int q = 0; q < RG; ++q) s += sCol[q * BN + c];
      if (n0 + c < N) g.colsum[(int64_t)tm * N + n0 + c] = s;
    }
  }
}

}  // namespace lr
