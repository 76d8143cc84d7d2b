// Causal self-attention with rotary position embedding (RoPE) for the
// LLaMA-2-style block, head dimension 128, bf16 operands, fp32 accumulation,
// gfx950 (MI355X).
//
// The BOOST pages keep the attention core outside the method: their block
// diagram runs the factorised linear layers around it, their related work
// cites FlashAttention and grouped-query attention, and the project page's
// scope section names grouped-query attention as a case the design is argued
// for. These kernels compute the textbook operation the LLaMA-2 family uses:
// half-split RoPE (pair (x_i, x_{i+64}) of a token at position p rotated by
// p * base^(-2i/128)), softmax(q k^T / sqrt(128)) v with causal masking per
// sequence, query head h reading key/value head h / (H / H_kv).
//
// Kernels:
//   rope_kernel       rotates (or counter-rotates) one [T][heads*128] tensor
//   attn_fwd_kernel   O and the per-row log-sum-exp (LSE), online softmax
//   attn_dq_kernel    dQ (and the row sums D = rowsum(dO * O) used by dK/dV)
//   attn_dkdv_kernel  dK, dV; query heads of a group accumulate in registers
// The backward kernels apply the transposed rotation to dQ and dK in their
// epilogues (both halves of a pair sit in the same lane).
//
// Layout of the MFMA tiles (v_mfma_f32_16x16x32_bf16, D = A B). Lane l
// supplies row l & 15 of A and column l & 15 of B, k = 8g .. 8g + 7 with
// g = l >> 4; it receives D[4g + v][l & 15], v = 0..3. Every score tile is
// formed with the keys (forward, dQ) or the queries (dK/dV) as A, so a lane
// holds one query (key) and four keys (queries) of each 16 x 16 block and
// the softmax statistics of its rows live in the lane itself. The
// probabilities then feed the next product directly as the B operand: its
// k-slots 8g + e are mapped to score columns 16 (2t + e / 4) + 4g + e % 4,
// and the A operand (V^T, K^T, dO^T or Q^T) is read with the same mapping
// by two transposing LDS reads (ds_read_b64_tr_b16, 4 rows each, 16 rows
// apart).
//
// Key/value (or query/dO) tiles of 64 rows x 256 bytes go from HBM to LDS
// with buffer_load_dwordx4 ... lds, double-buffered, their 16-byte chunks
// XOR-swizzled by row (swz below) so that both fragment reads are free of
// bank conflicts. Rows past the end of a sequence lie outside the buffer
// range and read as zeros.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <type_traits>

#include "lr_common.hpp"
#include "lr_gemm2.hpp"
#include "lr_internal.hpp"
#include "lr_attn.hpp"

namespace lr {
namespace {

constexpr int DH = 128;                // head dimension
constexpr int ROWB = DH * 2;           // bytes of one row of a head slice
constexpr int TR = 64;                 // rows of a streamed tile
constexpr int TILEB = TR * ROWB;       // 16 KB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMasked = -1.0e30f;    // score of a masked key (finite: no inf - inf)

__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Reductions over the four lane groups that share a row (lanes l, l ^ 16,
// l ^ 32, l ^ 48): each swap pairs a lane with its partner group, so the
// two outputs hold the lane's value and the partner's.
__device__ __forceinline__ float xg_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xg_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Turns (fractions of 2 pi) per position of rotation pair i:
// base^(-2i/128) / (2 pi), in fp64.
__device__ __forceinline__ double rope_tpp(int i, double log2_base) {
  return exp2(-(double)(2 * i) / DH * log2_base) * 0.15915494309189535;
}
// cos and sin of the angle pos * base^(-2i/128): the angle is formed and
// reduced to a fraction of a turn in fp64, then the hardware sine and cosine
// (which take turns) finish in fp32.
__device__ __forceinline__ void rope_cs(double tpp, int pos, float& c, float& s) {
  double t = (double)pos * tpp;
  t -= floor(t);
  const float f = (float)t;
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

// Blocks are dispatched round-robin over the 8 XCDs. Work item `logical`
// is given to consecutive blocks of one XCD, so the tiles of one
// (sequence, head) run on the same XCD and share their streamed operand
// through its L2.
__device__ __forceinline__ int xcd_item(int nwg) {
  constexpr int NXCD = 8;
  const int pid = blockIdx.x;
  const int q = nwg / NXCD, rem = nwg % NXCD, x = pid % NXCD;
  return x * q + (x < rem ? x : rem) + pid / NXCD;
}

// 16-byte chunk c of row r of a streamed tile sits at chunk c ^ swz(r).
// Measured with the LDS bank-conflict counter on this hardware: with
// 2 (r & 7) both the 16-byte row-fragment reads (16 rows, one logical
// chunk per lane group) and the transposing reads (rows 4g + s/4, 32 bytes
// each) are conflict-free; c ^ (r & 15) leaves the transposing reads 2-way
// conflicted and c ^ (2 (r & 7) + (r >> 3)) the 16-byte reads.
__device__ __forceinline__ int swz(int r) { return 2 * (r & 7); }

// HBM-to-LDS copy of 64-row tiles of a [rows][128] bf16 head slice with
// row stride ld: 16 blocks of 1 KB (4 rows each), shared by NW waves. The
// per-lane offsets depend only on ld; the buffer resource (base and the
// slice's extent, so rows past the end read zeros) is set per slice.
template <int NW>
struct TileDmaT {
  static constexpr int PER = 16 / NW;  // 1 KB blocks per wave
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t rs;
#endif
  uint32_t off[PER];
  uint32_t step;  // bytes between consecutive tiles
  __device__ __forceinline__ void init(int64_t ld, int lane, int wave) {
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      const int blk = NW * v + wave;
      const int r = 4 * blk + (lane >> 4);
      const int c = (lane & 15) ^ swz(r);
      off[v] = (uint32_t)(2 * ((int64_t)r * ld + 8 * c));
    }
    step = (uint32_t)wave_uniform((int)(2 * (int64_t)TR * ld));
  }
  __device__ __forceinline__ void set(const bf16_t* base, int64_t ld, int rows) {
    const int64_t nb = rows > 0 ? 2 * ((int64_t)(rows - 1) * ld + DH) : 0;
#if defined(__HIP_DEVICE_COMPILE__)
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), (short)0, (int)nb,
                                           0x00020000);
#else
    (void)base; (void)nb;
#endif
  }
  __device__ __forceinline__ void issue(int tile, unsigned char* dst, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int v = 0; v < PER; ++v)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LR_LPTR(dst + (NW * v + wave) * 1024), 16,
                                               off[v] + (uint32_t)tile * step, 0, 0, 0);
#else
    (void)tile; (void)dst; (void)wave;
#endif
  }
};

using TileDma = TileDmaT<4>;

// HBM-to-LDS copy of 64 consecutive fp32 values (one per row of a tile),
// issued by one wave; values past `n` read as zeros.
__device__ __forceinline__ void row_dma(const float* base, int n, int tile, unsigned char* dst,
                                        int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(base), (short)0, 4 * n, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LR_LPTR(dst), 4, (uint32_t)(4 * (TR * tile + lane)),
                                           0, 0, 0);
#else
  (void)base; (void)n; (void)tile; (void)dst; (void)lane;
#endif
}

// Per-lane byte offsets inside a tile. Row fragments: lane (g, s) reads
// row 16 kf + s, logical chunk 4 st + g, at rowoff[st] + 4096 kf.
__device__ __forceinline__ void row_offsets(int g, int s, uint32_t (&o)[4]) {
#pragma unroll
  for (int st = 0; st < 4; ++st) o[st] = (uint32_t)(s * ROWB + 16 * ((4 * st + g) ^ swz(s)));
}
// Column fragments: lane (g, s) reads columns 16 i + 4 (s & 3) .. + 3 of
// rows 32 t + 4g + s / 4 and 16 rows below, at coloff[i] + 8192 t (+ 4096).
__device__ __forceinline__ void col_offsets(int g, int s, uint32_t (&o)[8]) {
  const int r0 = 4 * g + (s >> 2);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    o[i] = (uint32_t)(r0 * ROWB + 16 * ((2 * i + ((s >> 1) & 1)) ^ swz(r0)) + 8 * (s & 1));
}

// 16-byte row fragment: `tile` points at the tile (plus 4096 kf for row
// block kf), `off` is the lane's row offset (rowoff[st]).
__device__ __forceinline__ u32x4 frag_rows(const unsigned char* tile, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(tile + off);
}

// Transposed fragment: lane (g, s) receives column 16 i + s of tile rows
// 32 t + 4g .. + 3 and 32 t + 16 + 4g .. + 3 (the permuted k-slots); addr
// is the lane's LDS address of column block i (coloff), IMM the tile's
// offset plus 8192 t.
template <int IMM>
__device__ __forceinline__ u32x4 frag_cols(uint32_t addr) {
  bf16x4 lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(addr), "n"(IMM));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(addr), "n"(IMM + 16 * ROWB));
  u32x4 r4;
  r4[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
  r4[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
  r4[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
  r4[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
  return r4;
}

// Wait for this wave's LDS reads and tie the wait to the fragments it
// delivers: the transposing reads are inline assembly, so without the tie
// the compiler could schedule a product that uses a fragment before the
// wait.
__device__ __forceinline__ void lds_wait(u32x4 (&x)[2]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1])::"memory");
}
// The same, leaving the N most recent LDS reads in flight (LDS reads
// return in order, so the older group's fragments have arrived). Scalar
// loads share this counter and may return out of order; in these loops the
// compiler has waited for its scalar loads before the fragment reads start.
template <int N>
__device__ __forceinline__ void lds_wait_keep(u32x4 (&x)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])
               : "n"(N)
               : "memory");
}

// B operand of k-step t from score blocks 2t and 2t + 1 of one row set.
__device__ __forceinline__ u32x4 pack_b(const f32x4& x0, const f32x4& x1) {
  u32x4 r;
  r[0] = pack_bf16x2(x0[0], x0[1]);
  r[1] = pack_bf16x2(x0[2], x0[3]);
  r[2] = pack_bf16x2(x1[0], x1[1]);
  r[3] = pack_bf16x2(x1[2], x1[3]);
  return r;
}

template <int V>
using IC = std::integral_constant<int, V>;

// Sixteen bytes of a row of a global [rows][ld] tensor, zero past `rows`.
__device__ __forceinline__ u32x4 load_row16(const bf16_t* base, int64_t ld, int row, int rows,
                                            int col) {
  u32x4 z = {0u, 0u, 0u, 0u};
  if (row < rows) z = *reinterpret_cast<const u32x4*>(base + (int64_t)row * ld + col);
  return z;
}

__device__ __forceinline__ void store_row8(bf16_t* base, int64_t ld, int row, int col, float a,
                                           float b, float c, float d) {
  u32x2 w;
  w[0] = pack_bf16x2(a, b);
  w[1] = pack_bf16x2(c, d);
  *reinterpret_cast<u32x2*>(base + (int64_t)row * ld + col) = w;
}

// Transposed rotation of the accumulators of one row set: acc[i][v] holds
// column 16 i + 4g + v; pair p = 16 i + 4g + v (i < 4) partners column
// p + 64 = acc[i + 4][v]. tpp[i][v] are the pairs' turns per position.
__device__ __forceinline__ void rope_inverse_acc(f32x4 (&acc)[8], const double (&tpp)[4][4],
                                                 int pos, float scale) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float c, s;
      rope_cs(tpp[i][v], pos, c, s);
      const float x1 = acc[i][v] * scale, x2 = acc[i + 4][v] * scale;
      acc[i][v] = x1 * c + x2 * s;
      acc[i + 4][v] = x2 * c - x1 * s;
    }
}

// ---------------------------------------------------------------------------
// RoPE on one tensor. Thread: 8 pairs (16 bytes of each half) of one head
// for RT tokens; consecutive threads cover a token's heads contiguously.
// ---------------------------------------------------------------------------
constexpr int RT = 8;

__global__ __launch_bounds__(256) void rope_kernel(const bf16_t* __restrict__ x,
                                                   bf16_t* __restrict__ y, int T, int heads,
                                                   int seq_len, double log2_base, float sgn) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int j = (int)(gid & 7);
  const int64_t hh = (gid >> 3) % heads;
  const int64_t tb = (gid >> 3) / heads;
  const int64_t ld = (int64_t)heads * DH;
  double tpp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) tpp[e] = rope_tpp(8 * j + e, log2_base);
  for (int k = 0; k < RT; ++k) {
    const int64_t t = tb * RT + k;
    if (t >= T) break;
    const int pos = (int)(t % seq_len);
    const bf16_t* src = x + t * ld + hh * DH + 8 * j;
    const u32x4 a = *reinterpret_cast<const u32x4*>(src);
    const u32x4 b = *reinterpret_cast<const u32x4*>(src + DH / 2);
    float x1[8], x2[8], y1[8], y2[8];
    unpack16<bf16_t>(a, x1);
    unpack16<bf16_t>(b, x2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, s;
      rope_cs(tpp[e], pos, c, s);
      s *= sgn;
      y1[e] = x1[e] * c - x2[e] * s;
      y2[e] = x2[e] * c + x1[e] * s;
    }
    bf16_t* dst = y + t * ld + hh * DH + 8 * j;
    *reinterpret_cast<u32x4*>(dst) = pack16<bf16_t>(y1);
    *reinterpret_cast<u32x4*>(dst + DH / 2) = pack16<bf16_t>(y2);
  }
}

// ---------------------------------------------------------------------------
// Forward. Block: 128 queries of one (sequence, head), 4 waves of 32;
// key/value tiles of 64 rows stream through two LDS stages.
// ---------------------------------------------------------------------------
struct FwdArgs {
  const bf16_t* q;  // rotated, [T][H * 128]
  const bf16_t* k;  // rotated, [T][Hkv * 128]
  const bf16_t* v;  // [T][Hkv * 128]
  bf16_t* o;        // [T][H * 128]
  float* lse;       // [H][T]
  int T, seq_len, H, Hkv;
  int ntiles;       // query tiles per sequence
  int nbh;          // sequences x heads
  float c;          // log2(e) / sqrt(128)
};

constexpr int FBM = 128;
constexpr int FWD_LDS = 4 * TILEB;  // K stages 0, 1; V stages 0, 1
// The running row maximum is raised (and O and the row sum rescaled) only
// when a tile's maximum exceeds it by more than this many powers of two;
// probabilities then stay below 2^8, and the final normalisation uses the
// same maximum, so the result is unchanged.
constexpr float kRescaleLog2 = 8.0f;

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int g = lane >> 4, s16 = lane & 15;
  const int item = xcd_item(a.ntiles * a.nbh);
  const int bh = item / a.ntiles;
  const int qt = a.ntiles - 1 - item % a.ntiles;  // longest rows first
  const int b = bh / a.H, h = bh % a.H, hk = h / (a.H / a.Hkv);
  const int64_t ldq = (int64_t)a.H * DH, ldk = (int64_t)a.Hkv * DH;
  const int64_t tok0 = (int64_t)b * a.seq_len;
  const int q0 = qt * FBM, qw = q0 + 32 * wave;
  const int qend = min(q0 + FBM, a.seq_len);
  const int nkt = (qend + TR - 1) / TR;

  TileDma dk, dv;
  dk.init(ldk, lane, wave);
  dv.init(ldk, lane, wave);
  dk.set(a.k + tok0 * ldk + hk * DH, ldk, a.seq_len);
  dv.set(a.v + tok0 * ldk + hk * DH, ldk, a.seq_len);
  dk.issue(0, lds, wave);
  dv.issue(0, lds + 2 * TILEB, wave);

  uint32_t roff[4], caddr[8];
  row_offsets(g, s16, roff);
  col_offsets(g, s16, caddr);
  const uint32_t lbase = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < 8; ++i) caddr[i] += lbase;

  const bf16_t* qbase = a.q + tok0 * ldq + h * DH;
  u32x4 qf[2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      qf[f][st] = load_row16(qbase, ldq, qw + 16 * f + s16, a.seq_len, 32 * st + 8 * g);

  // o[f][8] accumulates the row sums of P: its A operand is a block whose
  // row 0 is all ones, so row 0 of the result (lanes of group 0, element 0)
  // is the sum over the tile's keys, and rescaling it with O keeps it
  // consistent.
  f32x4 o[2][9];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int i = 0; i < 9; ++i) o[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t one2 = s16 == 0 ? 0x3F803F80u : 0u;  // two bf16 ones in row 0
  const u32x4 ones = {one2, one2, one2, one2};
  float m[2] = {kMasked, kMasked};
  const float c = a.c;
  const bool live = qw < a.seq_len;
  // Tile j holds a key at or before this wave's last query.
  auto needed = [&](int j) { return live && j * TR <= qw + 31; };

  // Scores of a key tile from the K stage at byte offset KO.
  auto scores = [&](auto koc, f32x4 (&s)[2][4]) {
    constexpr int KO = decltype(koc)::value;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int kf = 0; kf < 4; ++kf) s[f][kf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int stp = 0; stp < 4; ++stp)
#pragma unroll
      for (int kf = 0; kf < 4; ++kf) {
        const u32x4 kr = frag_rows(lds + KO + 4096 * kf, roff[stp]);
#pragma unroll
        for (int f = 0; f < 2; ++f) s[f][kf] = mma(kr, qf[f][stp], s[f][kf]);
      }
  };
  // Online softmax of one tile's scores: raises the running maximum when
  // needed (alpha: the factor O and the row sums are rescaled by) and packs
  // the probabilities as B operands.
  auto softmax = [&](f32x4 (&s)[2][4], float (&alpha)[2], u32x4 (&pb)[2][2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      float mx = m[f];
#pragma unroll
      for (int kf = 0; kf < 4; ++kf)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[f][kf][v]);
      mx = xg_max(mx);
      const bool grow = (mx - m[f]) * c > kRescaleLog2;
      alpha[f] = grow ? fexp2((m[f] - mx) * c) : 1.0f;
      m[f] = grow ? mx : m[f];
      const float mc = m[f] * c;
#pragma unroll
      for (int kf = 0; kf < 4; ++kf)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[f][kf][v] = fexp2(fmaf(s[f][kf][v], c, -mc));
#pragma unroll
      for (int t = 0; t < 2; ++t) pb[t][f] = pack_b(s[f][2 * t], s[f][2 * t + 1]);
    }
  };

  // Step j: K and V of tile j are in LDS stage j & 1; loads tile j + 1
  // into the other stage, then scores, softmax and P V.
  auto tile = [&](auto stc, int j) {
    constexpr int ST = decltype(stc)::value;
    constexpr int KO = ST * TILEB, VO = 2 * TILEB + ST * TILEB;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    block_barrier();
    if (j + 1 < nkt) {
      dk.issue(j + 1, lds + (ST ^ 1) * TILEB, wave);
      dv.issue(j + 1, lds + 2 * TILEB + (ST ^ 1) * TILEB, wave);
    }
    if (!needed(j)) return;
    const int k0 = j * TR;
    f32x4 sc[2][4];
    scores(IC<KO>{}, sc);
    if (k0 + TR - 1 > qw) {  // the tile crosses this wave's diagonal
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int kf = 0; kf < 4; ++kf)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (k0 + 16 * kf + 4 * g + v > qw + 16 * f + s16) sc[f][kf][v] = kMasked;
    }
    float alpha[2];
    u32x4 pb[2][2];
    softmax(sc, alpha, pb);
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int i = 0; i < 9; ++i) o[f][i] *= alpha[f];
    }
    // V^T fragments of four column blocks per group, two buffers: the next
    // group's reads are in flight while this group's products run.
    auto load = [&](auto tc, u32x4 (&vt)[4], int i0) {
      constexpr int t = decltype(tc)::value;
#pragma unroll
      for (int u = 0; u < 4; ++u) vt[u] = frag_cols<VO + 8192 * t>(caddr[i0 + u]);
    };
    auto pv = [&](int t, u32x4 (&vt)[4], int i0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int f = 0; f < 2; ++f) o[f][i0 + u] = mma(vt[u], pb[t][f], o[f][i0 + u]);
    };
    u32x4 va[4], vb[4];
    load(IC<0>{}, va, 0);
    load(IC<0>{}, vb, 4);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int f = 0; f < 2; ++f) o[f][8] = mma(ones, pb[t][f], o[f][8]);
    lds_wait_keep<8>(va);
    pv(0, va, 0);
    load(IC<1>{}, va, 0);
    lds_wait_keep<8>(vb);
    pv(0, vb, 4);
    load(IC<1>{}, vb, 4);
    lds_wait_keep<8>(va);
    pv(1, va, 0);
    lds_wait_keep<0>(vb);
    pv(1, vb, 4);
  };
  for (int j = 0; j < nkt; j += 2) {
    tile(IC<0>{}, j);
    if (j + 1 < nkt) tile(IC<1>{}, j + 1);
  }

  if (!live) return;
  bf16_t* obase = a.o + tok0 * ldq + h * DH;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int row = qw + 16 * f + s16;
    const float lt = xg_sum(o[f][8][0]);  // only group 0 holds row 0 of the sums
    if (row >= a.seq_len) continue;
    const float inv = 1.0f / lt;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      store_row8(obase, ldq, row, 16 * i + 4 * g, o[f][i][0] * inv, o[f][i][1] * inv,
                 o[f][i][2] * inv, o[f][i][3] * inv);
    if (g == 0) a.lse[(int64_t)h * a.T + tok0 + row] = (m[f] * c + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Backward, dQ. Block: 128 queries of one (sequence, head), 4 waves of 32;
// key/value tiles stream as in the forward. First writes, for its rows,
// D = rowsum(dO * O) and LSE * log2(e) for the dK/dV kernel.
// ---------------------------------------------------------------------------
struct BwdArgs {
  const bf16_t* q;     // rotated, [T][H * 128]
  const bf16_t* k;     // rotated, [T][Hkv * 128]
  const bf16_t* v;     // [T][Hkv * 128]
  const bf16_t* o;     // forward output [T][H * 128]
  const bf16_t* dout;  // its gradient [T][H * 128]
  const float* lse;    // [H][T]
  float* dsum;         // [H][T]: rowsum(dO * O)
  float* lse2;         // [H][T]: LSE * log2(e)
  bf16_t* dq;          // [T][H * 128]
  bf16_t* dk;          // [T][Hkv * 128]
  bf16_t* dv;          // [T][Hkv * 128]
  int T, seq_len, H, Hkv;
  int ntiles, nbh;
  float c;             // log2(e) / sqrt(128)
  float scale;         // 1 / sqrt(128)
  double log2_base;
};

constexpr int DQ_LDS = 4 * TILEB;

__global__ __launch_bounds__(256, 2) void attn_dq_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int g = lane >> 4, s16 = lane & 15;
  const int item = xcd_item(a.ntiles * a.nbh);
  const int bh = item / a.ntiles;
  const int qt = a.ntiles - 1 - item % a.ntiles;
  const int b = bh / a.H, h = bh % a.H, hk = h / (a.H / a.Hkv);
  const int64_t ldq = (int64_t)a.H * DH, ldk = (int64_t)a.Hkv * DH;
  const int64_t tok0 = (int64_t)b * a.seq_len;
  const int q0 = qt * FBM, qw = q0 + 32 * wave;
  const int qend = min(q0 + FBM, a.seq_len);
  const int nkt = (qend + TR - 1) / TR;

  TileDma dk, dv;
  dk.init(ldk, lane, wave);
  dv.init(ldk, lane, wave);
  dk.set(a.k + tok0 * ldk + hk * DH, ldk, a.seq_len);
  dv.set(a.v + tok0 * ldk + hk * DH, ldk, a.seq_len);
  dk.issue(0, lds, wave);
  dv.issue(0, lds + 2 * TILEB, wave);

  uint32_t roff[4], caddr[8];
  row_offsets(g, s16, roff);
  col_offsets(g, s16, caddr);
  const uint32_t lbase = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < 8; ++i) caddr[i] += lbase;

  const int64_t hoff = tok0 * ldq + h * DH;
  u32x4 qf[2][4], df[2][4];
  float lse2[2], dsum[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int row = qw + 16 * f + s16;
    float part = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      qf[f][st] = load_row16(a.q + hoff, ldq, row, a.seq_len, 32 * st + 8 * g);
      df[f][st] = load_row16(a.dout + hoff, ldq, row, a.seq_len, 32 * st + 8 * g);
      const u32x4 ov = load_row16(a.o + hoff, ldq, row, a.seq_len, 32 * st + 8 * g);
      float x[8], y[8];
      unpack16<bf16_t>(df[f][st], x);
      unpack16<bf16_t>(ov, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(x[e], y[e], part);
    }
    dsum[f] = xg_sum(part);
    const bool ok = row < a.seq_len;
    lse2[f] = ok ? a.lse[(int64_t)h * a.T + tok0 + row] * kLog2e : 0.f;
    if (ok && g == 0) {
      a.dsum[(int64_t)h * a.T + tok0 + row] = dsum[f];
      a.lse2[(int64_t)h * a.T + tok0 + row] = lse2[f];
    }
  }

  f32x4 acc[2][8];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c = a.c;
  const bool live = qw < a.seq_len;

  auto tile = [&](auto stc, int j) {
    constexpr int ST = decltype(stc)::value;
    constexpr int KO = ST * TILEB, VO = 2 * TILEB + ST * TILEB;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    block_barrier();
    if (j + 1 < nkt) {
      dk.issue(j + 1, lds + (ST ^ 1) * TILEB, wave);
      dv.issue(j + 1, lds + 2 * TILEB + (ST ^ 1) * TILEB, wave);
    }
    const int k0 = j * TR;
    if (!live || k0 > qw + 31) return;

    f32x4 sc[2][4], dp[2][4];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int kf = 0; kf < 4; ++kf) {
        sc[f][kf] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[f][kf] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int stp = 0; stp < 4; ++stp)
#pragma unroll
      for (int kf = 0; kf < 4; ++kf) {
        const u32x4 kr = frag_rows(lds + KO + 4096 * kf, roff[stp]);
        const u32x4 vr = frag_rows(lds + VO + 4096 * kf, roff[stp]);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          sc[f][kf] = mma(kr, qf[f][stp], sc[f][kf]);
          dp[f][kf] = mma(vr, df[f][stp], dp[f][kf]);
        }
      }

#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int kf = 0; kf < 4; ++kf)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[f][kf][v] = fexp2(fmaf(sc[f][kf][v], c, -lse2[f]));
    if (k0 + TR - 1 > qw) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int kf = 0; kf < 4; ++kf)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (k0 + 16 * kf + 4 * g + v > qw + 16 * f + s16) sc[f][kf][v] = 0.f;
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int kf = 0; kf < 4; ++kf)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[f][kf][v] *= dp[f][kf][v] - dsum[f];  // dS

    auto dqk = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      u32x4 sb[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) sb[f] = pack_b(sc[f][2 * t], sc[f][2 * t + 1]);
#pragma unroll
      for (int i0 = 0; i0 < 8; i0 += 2) {
        u32x4 kt[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) kt[u] = frag_cols<KO + 8192 * t>(caddr[i0 + u]);
        lds_wait(kt);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int f = 0; f < 2; ++f) acc[f][i0 + u] = mma(kt[u], sb[f], acc[f][i0 + u]);
      }
    };
    dqk(IC<0>{});
    dqk(IC<1>{});
  };
  for (int j = 0; j < nkt; j += 2) {
    tile(IC<0>{}, j);
    if (j + 1 < nkt) tile(IC<1>{}, j + 1);
  }

  if (!live) return;
  double tpp[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) tpp[i][v] = rope_tpp(16 * i + 4 * g + v, a.log2_base);
  bf16_t* dst = a.dq + hoff;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int row = qw + 16 * f + s16;
    if (row >= a.seq_len) continue;
    rope_inverse_acc(acc[f], tpp, row, a.scale);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      store_row8(dst, ldq, row, 16 * i + 4 * g, acc[f][i][0], acc[f][i][1], acc[f][i][2],
                 acc[f][i][3]);
  }
}

// ---------------------------------------------------------------------------
// Backward, dK and dV. Block: 128 keys of one (sequence, key/value head),
// 4 waves of 32; for every query head of the group, query/dO tiles of 64
// rows (with their LSE * log2(e) and D values) stream through two LDS
// stages, from the tile holding the block's first key to the end of the
// sequence. Each 64-query tile is taken in two halves of 32 queries, so the
// score and dP accumulators of only one half are live at a time.
// ---------------------------------------------------------------------------
constexpr int KBN = 128;
constexpr int KV_STAGE = 2 * TILEB + 2 * 256;  // Q, dO, LSE * log2(e), D
constexpr int DKV_LDS = 2 * KV_STAGE;
constexpr int kDkdvWaves = 8;  // 8 waves of 16 keys (2 per SIMD) or 4 of 32

template <int NWK>
__global__ __launch_bounds__(64 * NWK, 1) void attn_dkdv_kernel(BwdArgs a) {
  constexpr int FK = KBN / (16 * NWK);  // 16-key fragments per wave
  constexpr int KPW = 16 * FK;          // keys per wave
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int g = lane >> 4, s16 = lane & 15;
  const int item = xcd_item(a.ntiles * a.nbh);  // nbh = sequences x key/value heads here
  const int bh = item / a.ntiles;
  const int kt = item % a.ntiles;  // the first key blocks see the most queries
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int grp = a.H / a.Hkv;
  const int64_t ldq = (int64_t)a.H * DH, ldk = (int64_t)a.Hkv * DH;
  const int64_t tok0 = (int64_t)b * a.seq_len;
  const int k0 = kt * KBN, kw = k0 + KPW * wave;
  const int qt0 = k0 / TR;
  const int nqt = (a.seq_len + TR - 1) / TR;
  const int nq = nqt - qt0;  // query tiles per head
  const int nit = grp * nq;  // (head, query tile) steps

  const int64_t koff = tok0 * ldk + hk * DH;
  u32x4 kf[FK][4], vf[FK][4];
#pragma unroll
  for (int f = 0; f < FK; ++f)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      kf[f][st] = load_row16(a.k + koff, ldk, kw + 16 * f + s16, a.seq_len, 32 * st + 8 * g);
      vf[f][st] = load_row16(a.v + koff, ldk, kw + 16 * f + s16, a.seq_len, 32 * st + 8 * g);
    }

  uint32_t roff[4], caddr[8];
  row_offsets(g, s16, roff);
  col_offsets(g, s16, caddr);
  const uint32_t lbase = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < 8; ++i) caddr[i] += lbase;

  TileDmaT<NWK> dq, dd;
  dq.init(ldq, lane, wave);
  dd.init(ldq, lane, wave);
  // Next (head, query tile) to load.
  int nh = hk * grp, nt = qt0;
  auto issue = [&](unsigned char* stage) {
    const int64_t qoff = tok0 * ldq + (int64_t)nh * DH;
    dq.set(a.q + qoff, ldq, a.seq_len);
    dd.set(a.dout + qoff, ldq, a.seq_len);
    dq.issue(nt, stage, wave);
    dd.issue(nt, stage + TILEB, wave);
    if (wave == 0)
      row_dma(a.lse2 + (int64_t)nh * a.T + tok0, a.seq_len, nt, stage + 2 * TILEB, lane);
    else if (wave == 1)
      row_dma(a.dsum + (int64_t)nh * a.T + tok0, a.seq_len, nt, stage + 2 * TILEB + 256, lane);
    if (++nt == nqt) {
      nt = qt0;
      ++nh;
    }
  };

  f32x4 dka[FK][8], dva[FK][8];
#pragma unroll
  for (int f = 0; f < FK; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dka[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      dva[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const float c = a.c;
  const bool live = kw < a.seq_len;
  if (nit > 0) issue(lds);
  int cur_t = qt0;  // query tile of the current step

  auto step = [&](auto stc, int it) {
    constexpr int ST = decltype(stc)::value;
    constexpr int QO = ST * KV_STAGE, DO = QO + TILEB, LO = QO + 2 * TILEB, SO = LO + 256;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    block_barrier();
    if (it + 1 < nit) issue(lds + (ST ^ 1) * KV_STAGE);
    const int qs = cur_t * TR;
    if (++cur_t == nqt) cur_t = qt0;
    if (!live || qs + TR - 1 < kw) return;  // every query before every key of this wave
    const float* lrow = reinterpret_cast<const float*>(lds + LO);
    const float* drow = reinterpret_cast<const float*>(lds + SO);

    // Scores and dP of query half t (queries qs + 32t .. + 31).
    auto sdp = [&](auto tc, f32x4 (&sc)[FK][2], f32x4 (&dp)[FK][2]) {
      constexpr int t = decltype(tc)::value;
#pragma unroll
      for (int f = 0; f < FK; ++f)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          sc[f][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[f][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int stp = 0; stp < 4; ++stp)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int qf = 2 * t + qq;
          const u32x4 qr = frag_rows(lds + QO + 4096 * qf, roff[stp]);
          const u32x4 dr = frag_rows(lds + DO + 4096 * qf, roff[stp]);
#pragma unroll
          for (int f = 0; f < FK; ++f) {
            sc[f][qq] = mma(qr, kf[f][stp], sc[f][qq]);
            dp[f][qq] = mma(dr, vf[f][stp], dp[f][qq]);
          }
        }
    };
    // P and dS of half t, packed as B operands; masked when the half
    // crosses this wave's diagonal.
    auto soft = [&](auto tc, f32x4 (&sc)[FK][2], const f32x4 (&dp)[FK][2],
                    u32x4 (&pb)[FK], u32x4 (&sb)[FK], bool diag) {
      constexpr int t = decltype(tc)::value;
      const int qb = qs + 32 * t;
      f32x4 lv[2], dv4[2];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        lv[qq] = *reinterpret_cast<const f32x4*>(lrow + 32 * t + 16 * qq + 4 * g);
        dv4[qq] = *reinterpret_cast<const f32x4*>(drow + 32 * t + 16 * qq + 4 * g);
      }
#pragma unroll
      for (int f = 0; f < FK; ++f)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[f][qq][v] = fexp2(fmaf(sc[f][qq][v], c, -lv[qq][v]));
      if (diag) {
#pragma unroll
        for (int f = 0; f < FK; ++f)
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (kw + 16 * f + s16 > qb + 16 * qq + 4 * g + v) sc[f][qq][v] = 0.f;
      }
#pragma unroll
      for (int f = 0; f < FK; ++f) {
        pb[f] = pack_b(sc[f][0], sc[f][1]);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[f][qq][v] *= dp[f][qq][v] - dv4[qq][v];  // dS
        sb[f] = pack_b(sc[f][0], sc[f][1]);
      }
    };
    // dV += P^T dO and dK += dS^T Q for half t. dO^T and Q^T fragments of
    // column blocks i0, i0 + 1 go through two buffers: the reads of the
    // next pair are in flight while this pair's products run.
    auto grads = [&](auto tc, const u32x4 (&pb)[FK], const u32x4 (&sb)[FK]) {
      constexpr int t = decltype(tc)::value;
      auto load = [&](u32x4 (&fr)[4], int i0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          fr[2 * u] = frag_cols<DO + 8192 * t>(caddr[i0 + u]);
          fr[2 * u + 1] = frag_cols<QO + 8192 * t>(caddr[i0 + u]);
        }
      };
      auto prod = [&](u32x4 (&fr)[4], int i0) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int f = 0; f < FK; ++f) {
            dva[f][i0 + u] = mma(fr[2 * u], pb[f], dva[f][i0 + u]);
            dka[f][i0 + u] = mma(fr[2 * u + 1], sb[f], dka[f][i0 + u]);
          }
      };
      u32x4 fa[4], fb[4];
      load(fa, 0);
      load(fb, 2);
      lds_wait_keep<8>(fa);
      prod(fa, 0);
      load(fa, 4);
      lds_wait_keep<8>(fb);
      prod(fb, 2);
      load(fb, 6);
      lds_wait_keep<8>(fa);
      prod(fa, 4);
      lds_wait_keep<0>(fb);
      prod(fb, 6);
    };

    auto half = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      f32x4 sc[FK][2], dp[FK][2];
      u32x4 pb[FK], sb[FK];
      sdp(tc, sc, dp);
      soft(tc, sc, dp, pb, sb, qs + 32 * t < kw + KPW - 1);
      grads(tc, pb, sb);
    };
    half(IC<0>{});
    half(IC<1>{});
  };
  for (int it = 0; it < nit; it += 2) {
    step(IC<0>{}, it);
    if (it + 1 < nit) step(IC<1>{}, it + 1);
  }

  if (!live) return;
  double tpp[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) tpp[i][v] = rope_tpp(16 * i + 4 * g + v, a.log2_base);
#pragma unroll
  for (int f = 0; f < FK; ++f) {
    const int row = kw + 16 * f + s16;
    if (row >= a.seq_len) continue;
    rope_inverse_acc(dka[f], tpp, row, a.scale);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      store_row8(a.dk + koff, ldk, row, 16 * i + 4 * g, dka[f][i][0], dka[f][i][1],
                 dka[f][i][2], dka[f][i][3]);
      store_row8(a.dv + koff, ldk, row, 16 * i + 4 * g, dva[f][i][0], dva[f][i][1],
                 dva[f][i][2], dva[f][i][3]);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
hipError_t run_rope(const void* x, void* y, int T, int heads, int seq_len, double rope_base,
                    bool inverse, hipStream_t s) {
  const int64_t threads = (int64_t)((T + RT - 1) / RT) * heads * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const bf16_t*>(x), static_cast<bf16_t*>(y), T, heads, seq_len,
                     std::log2(rope_base), inverse ? -1.0f : 1.0f);
  return hipGetLastError();
}

hipError_t run_attn_fwd(const AttnDesc& d, hipStream_t s) {
  FwdArgs a;
  a.q = static_cast<const bf16_t*>(d.q);
  a.k = static_cast<const bf16_t*>(d.k);
  a.v = static_cast<const bf16_t*>(d.v);
  a.o = static_cast<bf16_t*>(d.o);
  a.lse = d.lse;
  a.T = d.T;
  a.seq_len = d.seq_len;
  a.H = d.H;
  a.Hkv = d.Hkv;
  a.ntiles = (d.seq_len + FBM - 1) / FBM;
  a.nbh = (d.T / d.seq_len) * d.H;
  a.c = kLog2e / std::sqrt((float)DH);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(a.ntiles * a.nbh), dim3(256), FWD_LDS, s, a);
  return hipGetLastError();
}

static BwdArgs bwd_args(const AttnDesc& d) {
  BwdArgs a;
  a.q = static_cast<const bf16_t*>(d.q);
  a.k = static_cast<const bf16_t*>(d.k);
  a.v = static_cast<const bf16_t*>(d.v);
  a.o = static_cast<const bf16_t*>(d.o);
  a.dout = static_cast<const bf16_t*>(d.dout);
  a.lse = d.lse;
  a.dsum = d.dsum;
  a.lse2 = d.lse2;
  a.dq = static_cast<bf16_t*>(d.dq);
  a.dk = static_cast<bf16_t*>(d.dk);
  a.dv = static_cast<bf16_t*>(d.dv);
  a.T = d.T;
  a.seq_len = d.seq_len;
  a.H = d.H;
  a.Hkv = d.Hkv;
  a.c = kLog2e / std::sqrt((float)DH);
  a.scale = 1.0f / std::sqrt((float)DH);
  a.log2_base = std::log2(d.rope_base);
  return a;
}

hipError_t run_attn_dq(const AttnDesc& d, hipStream_t s) {
  BwdArgs a = bwd_args(d);
  a.ntiles = (d.seq_len + FBM - 1) / FBM;
  a.nbh = (d.T / d.seq_len) * d.H;
  hipLaunchKernelGGL(attn_dq_kernel, dim3(a.ntiles * a.nbh), dim3(256), DQ_LDS, s, a);
  return hipGetLastError();
}

hipError_t run_attn_dkdv(const AttnDesc& d, hipStream_t s) {
  BwdArgs a = bwd_args(d);
  a.ntiles = (d.seq_len + KBN - 1) / KBN;
  a.nbh = (d.T / d.seq_len) * d.Hkv;
  auto kern = &attn_dkdv_kernel<kDkdvWaves>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, DKV_LDS);
  });
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3(a.ntiles * a.nbh), dim3(64 * kDkdvWaves), DKV_LDS, s, a);
  return hipGetLastError();
}

}  // namespace lr
