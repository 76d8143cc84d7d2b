// Pipelined bf16 MFMA GEMM engine for gfx950 (the path for aligned shapes).
//
// Operand tiles go from HBM straight into LDS with buffer_load_dwordx4 ... lds
// (16 bytes per lane; a wave's instruction fills one contiguous 1 KB block),
// through a ring of NSTAGE LDS stages: the loads of K-tile kt + NSTAGE - 1
// are issued while K-tile kt is multiplied, and one barrier per K-tile
// separates reuse of a stage. No operand passes through registers on its
// way to LDS. Both operand storage orders are consumed directly:
//
//  * K-contiguous operands ([rows][k]) sit in LDS as rows of BK elements.
//    The 16-byte chunks of a row are XOR-swizzled so that the lanes of an
//    MFMA fragment read (consecutive rows, one chunk) spread over distinct
//    4-bank groups: chunk ^ ((row >> 1) & 7) for 128-byte rows (BK = 64),
//    chunk ^ ((row >> 1) & 3) for 64-byte rows (BK = 32). For the latter the
//    LDS bank-conflict counters read 47% with the 16-row pattern
//    chunk ^ ((row >> 2) & 3) and 5% with this 8-row one. Fragments are read
//    with ds_read_b128.
//  * M/N-contiguous operands ([k][rows]) sit in LDS as k-rows; fragments are
//    read with ds_read_b64_tr_b16, the transposing LDS read: within a
//    16-lane group, result lane i element e is element (i & 3) of the
//    8 bytes addressed by lane 4e + (i >> 2). Pointing lane s at k-row
//    kb + s/4, columns m0 + 4(s & 3) gives lane i the four values
//    A[m0 + i][kb .. kb + 3]; two such reads make an MFMA fragment. Chunks
//    are XOR-swizzled by k-row so the four k-rows of a group and the two
//    groups read together fall on distinct banks.
//
// Requirements (checked by the host): K % BK == 0, N % 8 == 0, 16-byte
// aligned operands, leading dimensions multiples of 8; M/N-contiguous
// operands have a row count that is a multiple of 8. Rows beyond M or N
// read zeros or the last row: they only feed outputs that are never stored.
//
// MFMA: v_mfma_f32_16x16x32_bf16. Lane group g = lane / 16 holds
// k = 8g .. 8g + 7 of each 32-wide k step in both operands; the accumulator
// of a 16 x 16 tile holds rows 4g + v (v = 0..3) of column lane % 16.
#pragma once

#include "lr_common.hpp"
#include "lr_gemm.hpp"

namespace lr {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define LR_GPTR(p) ((__attribute__((address_space(1))) void*)(p))
#define LR_LPTR(p) ((__attribute__((address_space(3))) void*)(p))
#ifndef LR_SPLIT_AB
#define LR_SPLIT_AB 1
#endif

// NSPLIT = 2: a two-pair tile whose B rows hold pair 0's BN / 2 rows, then
// pair 1's; waves of the first NWN / 2 columns multiply pair 0, the others
// pair 1. Each wave runs one pair, so the LDS reads per MFMA are those of a
// one-pair tile twice the size; the epilogue pairs up the two halves.
// BDIAG_ = 1: a two-pair tile whose pairs share the output tile and run one
// after the other along K (a block-diagonal product): the K loop multiplies
// pair 0 (A0, B0) into the first accumulator set, then pair 1 into the
// second, so every wave holds both results of its elements and a stage
// holds one pair's A and B tiles.
template <int BM_, int BN_, int BK_, int NWM_, int NWN_, int NSTAGE_, int NSPLIT_ = 1,
          int NSTAGE_A_ = 0, int BDIAG_ = 0>
struct Tile2 {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NWM = NWM_, NWN = NWN_;
  static constexpr int NSTAGE = NSTAGE_;
  static constexpr bool BDIAG = BDIAG_ != 0;
  // BDIAG_ = 2: the first pair's results (the gate) are packed to bf16 once
  // its K loop is done, and the second pair accumulates in the same
  // registers: half the accumulator registers of BDIAG_ = 1 for the gate.
  static constexpr bool BDPACK = BDIAG_ == 2;
  // NSTAGE_A_ > 0: the A operand (the streamed activation of a one-pair
  // product) gets a ring of its own with NSTAGE_A_ stages and B keeps
  // NSTAGE, so A's loads are issued NSTAGE_A_ - 1 K-tiles ahead.
  static constexpr bool ASYM = NSTAGE_A_ > 0;
  static constexpr int NSTAGE_A = ASYM ? NSTAGE_A_ : NSTAGE_;
  static constexpr int NSPLIT = NSPLIT_;
  static constexpr int BNO = BN / NSPLIT;  // output columns of a block tile
  static_assert(NSPLIT == 1 || (NSPLIT == 2 && NWN % 2 == 0), "split tiles need an even NWN");
  static constexpr int NT = 64 * NWM * NWN;
  static constexpr int NWAVE = NWM * NWN;
  static constexpr int WTM = BM / NWM, WTN = BN / NWN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int NSTEP = BK / 32;
  static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
};

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The compiler schedules no instruction across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}).
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// A value that is the same in every lane of a wave, moved to a scalar register.
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Scheduling hint for one sub-step: NVM HBM-to-LDS loads, then NDS
// fragment reads, each followed by an equal share of the NMF MFMAs, then
// the rest of the MFMAs. One memory instruction between every few MFMAs
// keeps the memory queues short and the matrix pipe busy.
template <int NDS, int NVM, int NMF>
__device__ __forceinline__ void interleave() {
  constexpr int per = (NDS + NVM) ? NMF / (NDS + NVM) : 0;
#pragma unroll
  for (int k = 0; k < NVM; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMA
  }
#pragma unroll
  for (int k = 0; k < NDS; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NMF - (NDS + NVM) * per, 0);
}

// Wait until at most n vector-memory operations of this wave are pending;
// n is a compile-time constant once the caller's loop is unrolled, and the
// switch folds to one wait. Counts above 24 wait for 24 (more than needed).
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 21: wait_vmcnt<21>(); break;
    case 22: wait_vmcnt<22>(); break;
    case 23: wait_vmcnt<23>(); break;
    default: wait_vmcnt<24>(); break;
  }
}

// Epilogue bands. A band is 16 rows of a wave tile; with 64 columns it is
// held in LDS as 16 rows of 128 bytes whose 16-byte chunks are XOR-swizzled
// by row, so that the 8-byte accesses of the accumulator layout (lane l:
// row l & 15, columns 16 j + 4 (l >> 4) .. + 3) and the 16-byte accesses of
// whole rows both spread over the banks.
__device__ __forceinline__ int epi_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ uint32_t epi_acc_off(int j, int lane) {
  const int r = lane & 15, c = 2 * j + (lane >> 5), h = (lane >> 4) & 1;
  return (uint32_t)(r * 128 + 16 * (c ^ epi_swz(r)) + 8 * h);
}

// Buffer resource over rows [m0, M) x columns [n0, N) of a row-major bf16 or
// fp32 matrix (the range ends at its last element; empty for a null base).
// The range check applies to the per-lane offset only, so every access puts
// its whole offset there.
__device__ __forceinline__ void epi_range(const void* base, int esz, int64_t ld, int m0, int n0,
                                          int M, int N, const unsigned char*& p, int& bytes) {
  const bool live = base != nullptr && m0 < M && n0 < N;
  p = static_cast<const unsigned char*>(base) + (live ? esz * ((int64_t)m0 * ld + n0) : 0);
  int64_t nb = live ? esz * ((int64_t)(M - m0 - 1) * ld + (N - n0)) : 0;
  bytes = (int)(nb > 0x7FFFFFFF ? 0x7FFFFFFF : nb);
}

// One bf16 input of the epilogue (residual, upstream gradient, H, dm). A
// band (16 x 64) is copied by two 1 KB HBM-to-LDS loads, each covering 8
// whole 128-byte rows, into a wave-private LDS slot in the band layout.
// Rows past M, and columns past N in the last row, read as zeros; columns
// past N elsewhere read the next row and are never stored.
struct EpiDma {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t rs;
#endif
  uint32_t voff[2];  // this lane's byte offsets of the two halves of band 0
  uint32_t band;     // bytes between bands
  __device__ __forceinline__ void init(const bf16_t* base, int64_t ld, int m0, int n0, int M, int N,
                                       int row0, int col0, int lane) {
    const unsigned char* p;
    int bytes;
    epi_range(base, 2, ld, m0, n0, M, N, p, bytes);
#if defined(__HIP_DEVICE_COMPILE__)
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(p), (short)0, bytes, 0x00020000);
#endif
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + lane / 8, c = (lane & 7) ^ epi_swz(r);
      voff[h] = (uint32_t)(2 * ((int64_t)(row0 + r) * ld + col0 + 8 * c));
    }
    band = (uint32_t)wave_uniform((int)(2 * 16 * ld));
  }
  // Band i into the 2 KB slot `dst` (the same in every lane).
  __device__ __forceinline__ void issue(int i, unsigned char* dst) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LR_LPTR(dst + 1024 * h), 16, voff[h] + i * band, 0, 0, 0);
#else
    (void)i; (void)dst;
#endif
  }
};

// One fp32 value per row of the block tile (rows past the end, or a null
// array, read as zero).
struct EpiRow {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t rs;
#endif
  uint32_t voff;
  __device__ __forceinline__ void init(const float* base, int m0, int M, int row) {
    const unsigned char* p;
    int bytes;
    epi_range(base, 4, 1, m0, 0, M, 1, p, bytes);
#if defined(__HIP_DEVICE_COMPILE__)
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(p), (short)0, bytes, 0x00020000);
#endif
    voff = (uint32_t)(4 * row);
  }
  __device__ __forceinline__ float load(int i) const {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 64 * i, 0, 0));
#else
    return 0.f;
#endif
  }
};

// Stores of one bf16 output, band by band: 16-byte buffer stores of whole
// staged rows with the non-temporal hint. Lanes whose chunk starts past the
// last column get an offset outside the range and rows past the end fall
// outside it, so every lane issues the same stores.
template <int PERL>
struct EpiOut {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t rs;
#endif
  uint32_t voff[PERL];
  uint32_t band;
  __device__ __forceinline__ void init(void* base, int64_t ld, int m0, int n0, int M, int N, int row0,
                                       int col0, int lane, int CH) {
    const unsigned char* p;
    int bytes;
    epi_range(base, 2, ld, m0, n0, M, N, p, bytes);
#if defined(__HIP_DEVICE_COMPILE__)
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(p), (short)0, bytes, 0x00020000);
#endif
#pragma unroll
    for (int q = 0; q < PERL; ++q) {
      const int id = lane + 64 * q, rr = id / CH, cc = id % CH;
      const bool ok = n0 + col0 + 8 * cc < N;
      voff[q] = ok ? (uint32_t)(2 * ((int64_t)(row0 + rr) * ld + col0 + 8 * cc)) : 0x80000000u;
    }
    band = (uint32_t)wave_uniform((int)(2 * 16 * ld));
  }
  __device__ __forceinline__ void store(int i, int q, u32x4 x) const {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, voff[q] + i * band, 0, 2 /* nt */);
#else
    (void)i; (void)q; (void)x;
#endif
  }
};

// Element i (0..2, the same in every lane) of a three-entry argument array.
template <typename T>
__device__ __forceinline__ T pick3(const T (&a)[3], int i) {
  return i == 0 ? a[0] : (i == 1 ? a[1] : a[2]);
}

// 32-bit LDS address of a pointer into the kernel's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wait until every LDS read of this wave has returned its data. The
// builtin (not inline asm) lets the compiler's own wait insertion see it.
// Encoding: vmcnt = 63 (bits 3:0 and 15:14), expcnt = 7, lgkmcnt = 0.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ---------------------------------------------------------------------------
// One operand's DMA loader and fragment reader.
//   R   rows of the operand tile (BM for A, BN for B)
//   KC  true: storage [rows][k]; false: storage [k][rows]
// ---------------------------------------------------------------------------
template <int R, int BK, int NWAVE, bool KC>
struct Opnd {
  static constexpr int BYTES = R * BK * 2;
  static constexpr int BLOCKS = BYTES / 1024;
  static_assert(BYTES % 1024 == 0, "tile must be whole 1 KB blocks");
  static_assert(BLOCKS % NWAVE == 0, "blocks must split over the waves");
  static constexpr int PER = BLOCKS / NWAVE;  // DMA instructions per lane per stage
  // KC geometry
  static constexpr int CPR = BK / 8;          // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;        // rows per 1 KB block
  // MC geometry
  static constexpr int CPK = R / 8;           // 16-byte chunks per k-row
  static constexpr int KPB = KC ? 1 : 64 / CPK;
  static_assert(KC || (R >= 128 && 64 % CPK == 0) || (KC), "M-contiguous tiles need R >= 128");

  // Consecutive loads of a lane step through rows (KC) or k-rows (MC) by
  // VROWS. The chunk swizzle repeats every SWP rows, so loads v and
  // v + NOFF share their swizzle: NOFF per-lane offsets serve all loads of
  // a lane, the rest of the load index moving the base of the buffer
  // resource (KC) or going into the scalar offset (MC). This keeps vector
  // registers free for fragments.
  static constexpr int VROWS = NWAVE * (KC ? RPB : KPB);
  static constexpr int SWP = KC ? (BK == 64 ? 16 : 8) : 16;
  static constexpr int gcd_(int a, int b) { return b ? gcd_(b, a % b) : a; }
  static constexpr int NOFF = SWP / gcd_(VROWS, SWP) < PER ? SWP / gcd_(VROWS, SWP) : PER;
  uint32_t off[NOFF];  // per-lane byte offsets of loads 0 .. NOFF-1 (tile origin, k0 = 0)
  uint32_t vstep;      // bytes between loads v and v + NOFF

  // Elements from the operand's first element to one past its last one.
  __device__ static __forceinline__ int64_t extent(int64_t ld, int Rtot, int K) {
    return KC ? (int64_t)(Rtot - 1) * ld + K : (int64_t)(K - 1) * ld + Rtot;
  }

  // Swizzle of a K-contiguous row: flips the chunk index so that
  // consecutive rows at one logical chunk hit distinct bank groups.
  __device__ static __forceinline__ int swz_kc(int row) {
    return (BK == 64) ? ((row >> 1) & 7) : ((row >> 1) & 3);
  }
  // Swizzle of a k-row of an M-contiguous tile (flips chunk bits 1..3).
  __device__ static __forceinline__ int swz_mc(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }

  // K-contiguous rows past Rtot are not clamped: their offsets lie past the
  // operand's extent, so the buffer range check returns zeros for them (they
  // only feed outputs that are never stored). M-contiguous column chunks
  // past Rtot are clamped to the last one.
  __device__ __forceinline__ void init(int64_t ld, int r0, int Rtot, int lane, int wave) {
    static_assert((NOFF * VROWS) % SWP == 0 || NOFF == PER, "loads v and v + NOFF must share a swizzle");
    // The same in every lane; kept in a scalar register so the buffer
    // resources built from it are scalar too.
    vstep = (uint32_t)wave_uniform((int)(2 * (int64_t)NOFF * VROWS * ld));
#pragma unroll
    for (int v = 0; v < NOFF; ++v) {
      const int b = v * NWAVE + wave;
      int64_t e;
      if constexpr (KC) {
        const int row = b * RPB + lane / CPR;
        const int c = (lane % CPR) ^ swz_kc(row);
        e = (int64_t)(r0 + row) * ld + 8 * c;
      } else {
        const int k = b * KPB + lane / CPK;
        const int c = (lane % CPK) ^ swz_mc(k);
        int gc = r0 / 8 + c;
        const int last = Rtot / 8 - 1;
        gc = gc < last ? gc : last;
        e = (int64_t)k * ld + 8 * gc;
      }
      off[v] = (uint32_t)(2 * e);
    }
  }

  // Issue this stage's loads: `src` points at the tile's k0 (element (r, k0)
  // for KC, (k0, r) for MC) and `nbytes` bytes from it are the operand's;
  // `dst` is the stage's LDS tile. The loads go through buffer resources
  // (base and size in scalar registers, one 32-bit offset per lane): a lane
  // whose offset falls outside the range reads zeros, never memory beyond
  // the operand.
  __device__ __forceinline__ void issue(const bf16_t* src, uint32_t nbytes, unsigned char* dst,
                                        int wave) const {
    // The buffer-resource type exists only for the GPU target; the host
    // pass (which emits the launch stubs) must not see it.
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      const int b = v * NWAVE + wave;
      const uint32_t vo = off[v % NOFF];
      const uint32_t step = (uint32_t)(v / NOFF) * vstep;
      if constexpr (KC) {
        const uint32_t adv = (uint32_t)wave_uniform((int)step);
        const int rem = wave_uniform((int)(nbytes > adv ? nbytes - adv : 0u));
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(src)) + adv, (short)0,
            rem, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LR_LPTR(dst + b * 1024), 16, vo, 0, 0, 0);
      } else {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(src), (short)0, (int)nbytes, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LR_LPTR(dst + b * 1024), 16, vo, step, 0, 0);
      }
    }
#else
    (void)src; (void)nbytes; (void)dst; (void)wave;
#endif
  }

  // Per-lane byte offsets of fragment reads inside a stage tile, for the
  // 16-row group starting at row `w0` (a multiple of 16) and k-step `st`.
  // KC: one ds_read_b128; MC: two ds_read_b64_tr_b16 (4 k-rows apart).
  __device__ static __forceinline__ int frag_off(int w0, int st, int lane) {
    const int g = lane >> 4, s = lane & 15;
    if constexpr (KC) {
      const int row = w0 + s;
      const int c = 4 * st + g;
      return row * (BK * 2) + 16 * (c ^ swz_kc(row));
    } else {
      const int k = 32 * st + 8 * g + (s >> 2);
      const int m = w0 + 4 * (s & 3);
      return k * (R * 2) + 16 * ((m >> 3) ^ swz_mc(k)) + 2 * (m & 7);
    }
  }

  // IMM: a constant byte offset, an immediate of the transposing reads.
  template <int IMM = 0>
  __device__ static __forceinline__ u32x4 read_frag(const unsigned char* tile, int off) {
    if constexpr (KC)
      return *reinterpret_cast<const u32x4*>(tile + off + IMM);
    else
      return read_tr<IMM>(lds_addr(tile + off));
  }
  // The two transposing reads of an M-contiguous fragment at LDS address a.
  // The second read is 4 k-rows further down; its swizzle is the same (k & 3
  // and (k >> 3) & 1 do not change when k grows by 4 within a lane's 8-row
  // group). The reads are issued as inline assembly: the compiler would
  // otherwise make each wait for every pending HBM-to-LDS load, which
  // serialises the pipeline. The caller waits for them (wait_lgkmcnt0)
  // before the fragments are used.
  template <int IMM>
  __device__ static __forceinline__ u32x4 read_tr(uint32_t a) {
    static_assert(!KC, "transposing reads are for M-contiguous tiles");
    static_assert(IMM >= 0 && IMM + 4 * R * 2 < 65536, "LDS instruction offsets are 16-bit");
    bf16x4 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(a), "n"(IMM));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(a), "n"(IMM + 4 * R * 2));
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
    return r;
  }

  // Fragment of rows w0 .. w0 + 15 at the 32-wide k-step ST of the tile.
  // An M-contiguous fragment one k-step on lies 32 k-rows further down with
  // the same swizzle (k & 3 and (k >> 3) & 1 do not change by 32): the step
  // is an immediate of the read instruction, not an address computation.
  template <int ST>
  __device__ static __forceinline__ u32x4 read_step(const unsigned char* tile, int w0, int lane) {
    if constexpr (KC)
      return read_frag(tile, frag_off(w0, ST, lane));
    else
      return read_tr<ST * 32 * R * 2>(lds_addr(tile) + frag_off(w0, 0, lane));
  }
  // The same for an M-contiguous tile at LDS address base (the same in every
  // lane, in a scalar register): one vector add per fragment.
  template <int ST>
  __device__ static __forceinline__ u32x4 read_step_at(uint32_t base, int w0, int lane) {
    return read_tr<ST * 32 * R * 2>(base + frag_off(w0, 0, lane));
  }
};

template <class TL, int NPAIR>
constexpr int stage_bytes() {
  return (TL::NSPLIT == 2 ? 2 * TL::BM + TL::BN
                          : (TL::BDIAG ? 1 : NPAIR) * (TL::BM + TL::BN)) * TL::BK * 2;
}
// The operand ring: NSTAGE stages, or with separate rings NSTAGE_A A tiles
// followed by NSTAGE B tiles.
template <class TL, int NPAIR>
constexpr int ring_bytes() {
  return TL::ASYM ? (TL::NSTAGE_A * TL::BM + TL::NSTAGE * TL::BN) * TL::BK * 2
                  : TL::NSTAGE * stage_bytes<TL, NPAIR>();
}

// Wave-private epilogue staging: one 16-row band of a wave tile in bf16.
template <class TL>
constexpr int epi_wave_bytes() {
  return 16 * TL::WTN * 2;
}

// Staging bands (one per wave) and the column sums of the RMSNorm backward.
template <class TL>
constexpr int epi_area_bytes() {
  return TL::NWAVE * epi_wave_bytes<TL>() + TL::NWM * TL::BN * 4;
}
template <int EPI>
constexpr int epi_nin() {
  return ((EPI == EPI_STORE || EPI == EPI_RMSBWD || EPI == EPI_SWIGLU_BWD2) ? 1 : 0) +
         (EPI == EPI_RMSBWD ? 1 : 0);
}
// Split tiles hand half of their accumulators over through LDS: in one
// round, or in two rounds of a quarter each when the band-input slots would
// not fit beside a one-round exchange area in the ring.
template <class TL, int EPI>
constexpr int epi_xch_rounds() {
  constexpr int one = TL::NWAVE * (TL::FM / 2) * TL::FN * 4 * 64 * 4;
  constexpr int fme = TL::FM / 2;
  constexpr int pds = (epi_nin<EPI>() == 2 ? 3 : 4) < fme ? (epi_nin<EPI>() == 2 ? 3 : 4) : fme;
  constexpr int slots = TL::NWAVE * pds * epi_nin<EPI>() * 2048;
  return (epi_nin<EPI>() > 0 && one + slots > TL::NSTAGE * (2 * TL::BM + TL::BN) * TL::BK * 2) ? 2 : 1;
}
template <class TL, int EPI>
constexpr int epi_xch_bytes() {
  return TL::NSPLIT == 2 ? TL::NWAVE * (TL::FM / 2 / epi_xch_rounds<TL, EPI>()) * TL::FN * 4 * 64 * 4 : 0;
}
// First byte of the band-input slots (1 KB aligned, after both areas above).
template <class TL, int EPI>
constexpr int epi_in0() {
  constexpr int a = epi_area_bytes<TL>() > epi_xch_bytes<TL, EPI>() ? epi_area_bytes<TL>()
                                                                     : epi_xch_bytes<TL, EPI>();
  return (a + 1023) / 1024 * 1024;
}
template <class TL, int EPI>
constexpr int epi_pds() {
  constexpr int fme = TL::NSPLIT == 2 ? TL::FM / 2 : TL::FM;
  constexpr int want = epi_nin<EPI>() == 2 ? 3 : 4;
  return want < fme ? want : fme;
}
template <class TL, int NPAIR, int EPI>
constexpr int gemm2_body_bytes() {
  constexpr int ring = ring_bytes<TL, NPAIR>();
  constexpr int in_end = epi_in0<TL, EPI>() + TL::NWAVE * epi_pds<TL, EPI>() * epi_nin<EPI>() * 2048;
  constexpr int epi = in_end > epi_area_bytes<TL>() ? in_end : epi_area_bytes<TL>();
  return ring > epi ? ring : epi;
}
// The Online RMSNorm's per-row totals and row scales (two floats per row)
// live in the ring once the main loop is done, after the staging area.
template <class TL>
constexpr int orms_off() {
  return (epi_area_bytes<TL>() + 1023) / 1024 * 1024;
}

// Persistent workgroups: the 8-wave one-pair and block-diagonal tiles of the
// storing epilogues run one workgroup per CU that walks its tiles. Once a
// tile's main loop is done, the next tile's first K-tiles (the loads the
// prologue issues before its barrier) go into their stages while the
// epilogue runs from LDS areas outside them; the launch gap, the argument
// loads and the pipeline fill of every tile but the first then overlap the
// epilogue's stores.
// (The Online RMSNorm tile, at 256 VGPRs, would spill with the tile loop's
// state, and its long-K launches have few tiles per CU.)
template <class TL, int NPAIR, int EPI>
constexpr bool gemm2_persist() {
  return TL::NWAVE == 8 && TL::NSPLIT == 1 &&
         (EPI == EPI_STORE || EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD2) &&
         (TL::BDIAG || (NPAIR == 1 && TL::BM == 256 && TL::BN == 256));
}

// LDS places of the epilogue: the staging bands (and the RMSNorm-backward
// column sums after them), the Online RMSNorm row totals and scales, and the
// band-input slots, slot p of wave w at slot_off(p) + w * NIN * 2 KB.
// Without persistence they start at the ring's origin. With it they avoid
// the stages that hold the next tile's first K-tiles: shared ring, stages
// 0 .. NSTAGE - 2 (the areas follow them); separate rings, A stages 0 and 1
// and B stage 0 (staging and row sums in B stage 1, slots 0 and 1 in A
// stage 2, slot 2 in the rest of B stage 1).
template <class TL, int NPAIR, int EPI>
struct EpiLds {
  static constexpr bool P = gemm2_persist<TL, NPAIR, EPI>();
  static constexpr int NIN = epi_nin<EPI>();
  static constexpr int EW = TL::NWAVE * epi_wave_bytes<TL>();
  static constexpr int SLOT = TL::NWAVE * NIN * 2048;  // one slot of every wave
  static constexpr int AB = TL::BM * TL::BK * 2, BB = TL::BNO * TL::BK * 2;
  static constexpr int ST = !P ? 0 : TL::ASYM ? TL::NSTAGE_A * AB + BB
                                              : (TL::NSTAGE - 1) * stage_bytes<TL, NPAIR>();
  static constexpr int ORM = !P ? orms_off<TL>() : ST + EW;
  static constexpr int RS = EPI == EPI_ORMS ? 8 * TL::BM : 0;  // row totals and scales
  static constexpr int IN0 = !P ? epi_in0<TL, EPI>() : TL::ASYM ? 2 * AB : ST + EW + RS;
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int PDS0 = epi_pds<TL, EPI>();
  static constexpr int PDS_FIT = SLOT ? (LDS_MAX - IN0) / SLOT : PDS0;
  static constexpr int PDS = !P ? PDS0 : TL::ASYM ? (PDS0 < 3 ? PDS0 : 3)
                                       : (PDS0 < PDS_FIT ? PDS0 : PDS_FIT);
  static constexpr int slot_off(int p) {
    return (P && TL::ASYM && p == 2) ? ST + EW : IN0 + p * SLOT;
  }
  static constexpr int end_() {
    int e = ST + EW + RS;
    for (int p = 0; p < (NIN ? PDS : 0); ++p) e = slot_off(p) + SLOT > e ? slot_off(p) + SLOT : e;
    return e;
  }
  static constexpr int END = end_();
  static_assert(!P || NIN == 0 || PDS >= 2, "persistent epilogue needs two band-input slots");
  static_assert(!P || !TL::ASYM || (TL::NSTAGE_A == 3 && TL::NSTAGE == 2 && AB >= 2 * SLOT &&
                                    BB >= EW + (RS > SLOT ? RS : SLOT)),
                "separate-ring epilogue places");
  static_assert(!P || END <= LDS_MAX, "persistent epilogue areas exceed LDS");
};

template <class TL, int NPAIR, int EPI>
constexpr int gemm2_lds_bytes() {
  if constexpr (gemm2_persist<TL, NPAIR, EPI>()) {
    constexpr int ring = ring_bytes<TL, NPAIR>(), e = EpiLds<TL, NPAIR, EPI>::END;
    return ring > e ? ring : e;
  } else {
    return gemm2_body_bytes<TL, NPAIR, EPI>();
  }
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// The 4-wave packed block-diagonal tile runs two workgroups per CU, so its
// registers are held to two waves per SIMD (256).
template <class TL>
constexpr int gemm2_min_waves() {
  return (TL::BDPACK && TL::NWAVE == 4) ? 2 : 1;
}
template <class TL, int NPAIR, uint32_t MCMASK, int EPI>
__global__ __launch_bounds__(TL::NT, gemm2_min_waves<TL>()) void gemm2_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, S = TL::NSTAGE;
  constexpr int FM = TL::FM, FN = TL::FN;
  constexpr bool ORMS = (EPI == EPI_ORMS);
  constexpr bool SPLITN = (TL::NSPLIT == 2);
  static_assert(!SPLITN || (NPAIR == 2 && MCMASK == 0u && !ORMS && EPI != EPI_RMSBWD),
                "split tiles are for K-contiguous two-pair products");
  constexpr bool BD = TL::BDIAG;
  static_assert(!BD || (NPAIR == 2 && MCMASK == 0u && !ORMS && !SPLITN && !TL::ASYM &&
                        (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD2)),
                "block-diagonal tiles are for the K-contiguous gate/up pair");
  constexpr int BNO = TL::BNO;
  constexpr int SB = stage_bytes<TL, NPAIR>();
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int RING = ring_bytes<TL, NPAIR>();
  static_assert(!TL::ASYM || (NPAIR == 1 && !SPLITN), "separate rings are for one-pair tiles");
  constexpr int SA = TL::NSTAGE_A;
  // Epilogue areas (the ring is free by then): staging bands and column
  // sums, the split-tile exchange, the band-input slots.
  constexpr int EPIB = epi_area_bytes<TL>();
  constexpr int XCH = epi_xch_bytes<TL, EPI>();
  constexpr int IN0 = epi_in0<TL, EPI>();
  constexpr int BODY = gemm2_body_bytes<TL, NPAIR, EPI>();
  using EL = EpiLds<TL, NPAIR, EPI>;
  constexpr bool PST = EL::P;
  constexpr int LDSB = gemm2_lds_bytes<TL, NPAIR, EPI>();
  // Online RMSNorm, after the main loop: per-row sums of squares, row scales.
  float* sTot = reinterpret_cast<float*>(lds + EL::ORM);  // [BM]
  float* sRow = sTot + BM;                                      // [BM]
  static_assert(!ORMS || EL::ORM + 8 * BM <= LDSB, "row sums exceed the ring");

  // The wave index is uniform across a wave: keep it in a scalar register.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int wm = wave / TL::NWN, wn = wave % TL::NWN;
  int tm, tn;
  // An XCD's 32 concurrent tiles span 4 M-tiles x 8 N-tiles. For the split
  // tile, whose rows carry two A operands, that is 7.3 MB of operands at the
  // 7B shape against 8.4 MB for 8 x 4 (measured: 6% faster SwiGLU tiles,
  // 2-6% faster one-pair tiles, 5% fewer L2 misses).
  // With several problems in one launch (nprob > 0) the workgroup's problem
  // is its slot: shape, column scale and split stride come from its entry.
  int slot, M, N;
  const void* colscale = g.colscale;
  int64_t csplit = g.c_split_stride;
  if (NPAIR == 1 && g.nprob > 0) {
    const int lg = xcd_logical((int)gridDim.x);
    slot = wave_uniform(lg >= g.prob_base[2] ? 2 : (lg >= g.prob_base[1] ? 1 : 0));
    M = pick3(g.Mp, slot);
    N = pick3(g.Np, slot);
    const int base = slot == 0 ? 0 : (slot == 1 ? g.prob_base[1] : g.prob_base[2]);
    group_tile<4>(lg - base, pick3(g.tiles_mp, slot), pick3(g.tiles_np, slot), tm, tn);
    colscale = pick3(g.colscales, slot);
    csplit = pick3(g.csplit, slot);
  } else {
    tile_coords<4>(g.tiles_m, g.tiles_n, tm, tn);
    slot = (NPAIR == 1) ? (int)blockIdx.z % g.groups : 0;
    M = g.M;
    N = g.N;
  }
  // Persistent launches: tile v of tiles_m x tiles_n x groups (the groups
  // after one another), through the same XCD remapping with v in place of
  // the workgroup id (the grid is a multiple of 8 whenever a workgroup runs
  // more than one tile, so v and its workgroup sit on the same XCD).
  int vt = (int)blockIdx.x;
  auto vcoords = [&](int vv, int& tm_, int& tn_, int& slot_) {
    const int tmn = g.tiles_m * g.tiles_n;
    const int lg = xcd_logical_of(vv, g.vtiles);
    slot_ = NPAIR == 1 ? lg / tmn : 0;
    group_tile<4>(lg - slot_ * tmn, g.tiles_m, g.tiles_n, tm_, tn_);
  };
  if constexpr (PST) vcoords(vt, tm, tn, slot);
  int m0 = tm * BM, n0 = tn * BNO;
  const int split = (int)blockIdx.z / g.groups;

  // With two waves per SIMD the SIMD serves the older wave's MFMAs first,
  // so the younger one (waves NWAVE / 2 ..) ends each K-tile alone while
  // the older one waits at the barrier. When every operand is K-contiguous
  // the older waves therefore issue all HBM-to-LDS loads (measured: 7%
  // faster 256 x 256 tiles; no gain measured with M/N-contiguous operands,
  // which keep every wave issuing its share). Split tiles load 1.25 times
  // the bytes per MFMA: there the older waves stall behind their loads (the
  // younger ones then wait at the barrier for half the loop), and every
  // wave issues its share (measured: 6-9% faster). Block-diagonal tiles,
  // which load 1.5 times the bytes per MFMA of a one-pair 256 x 256 tile
  // through three stages, are faster with the older half issuing (measured:
  // all eight waves issuing made the SwiGLU tiles 3-5% slower).
  constexpr int NDMA = (TL::NWAVE == 8 && MCMASK == 0u && !SPLITN) ? TL::NWAVE / 2 : TL::NWAVE;
  // Separate rings with half the waves loading: the older half loads the B
  // tiles (after the barrier of K-tile k, B of k + 2) and the younger half
  // the A tiles (at the start of K-tile k, A of k + 2, into the stage K-tile
  // k - 1 freed). A wave stalls while its loads enter the load path; split
  // so, each wave has half the loads, and the two waves of a SIMD stall at
  // different points of the K-tile, each while the other issues MFMAs.
  // (Not the Online RMSNorm tile: at 256 VGPRs already, it spilled so.)
  constexpr bool SPLIT_AB = LR_SPLIT_AB && TL::ASYM && 2 * NDMA == TL::NWAVE && !ORMS;
  // A loader's wave index among the waves that issue its loads.
  const int dwave = SPLIT_AB ? wave % NDMA : wave;
  const bool a_iss = SPLIT_AB ? wave >= NDMA : (NDMA == TL::NWAVE || wave < NDMA);
  const bool b_iss = SPLIT_AB ? wave < NDMA : (NDMA == TL::NWAVE || wave < NDMA);
  using OA0 = Opnd<BM, BK, NDMA, !(MCMASK & 1u)>;
  using OB0 = Opnd<BNO, BK, NDMA, !(MCMASK & 2u)>;
  using OA1 = Opnd<BM, BK, NDMA, !(MCMASK & 4u)>;
  using OB1 = Opnd<BNO, BK, NDMA, !(MCMASK & 8u)>;
  using OA2 = Opnd<BM, BK, NDMA, !(MCMASK & 16u)>;
  using OB2 = Opnd<BN, BK, NDMA, !(MCMASK & 32u)>;
  OA0 a0;
  OB0 b0;
  OA1 a1;
  OB1 b1;
  OA2 a2;
  OB2 b2;
  const bf16_t* pa[3];
  const bf16_t* pb[3];
  int64_t sa[3], sb[3];  // element step of the source pointer per K-tile
  int64_t ea[3], eb[3];  // elements of the operand from pa / pb on
  // The operands' loaders for the tile at rows m0_, columns n0_ of slot_.
  auto init_ops = [&](int m0_, int n0_, int M_, int N_, int slot_) {
    const int p0 = slot_;
    // Selected with constant indices (not g.a[p0]): a run-time index into
    // the argument arrays would go through private memory, and the values
    // would no longer be known to be the same in every lane.
    pa[0] = static_cast<const bf16_t*>(pick3(g.a, p0));
    pb[0] = static_cast<const bf16_t*>(pick3(g.b, p0));
    const int64_t lda0 = pick3(g.lda, p0), ldb0 = pick3(g.ldb, p0);
    a0.init(lda0, m0_, M_, lane, dwave);
    b0.init(ldb0, n0_, N_, lane, dwave);
    ea[0] = OA0::extent(lda0, M_, g.K);
    eb[0] = OB0::extent(ldb0, N_, g.K);
    sa[0] = (MCMASK & 1u) ? (int64_t)BK * lda0 : BK;
    sb[0] = (MCMASK & 2u) ? (int64_t)BK * ldb0 : BK;
    if constexpr (NPAIR > 1) {
      pa[1] = static_cast<const bf16_t*>(g.a[1]);
      pb[1] = static_cast<const bf16_t*>(g.b[1]);
      a1.init(g.lda[1], m0_, M_, lane, wave);
      b1.init(g.ldb[1], n0_, N_, lane, wave);
      ea[1] = OA1::extent(g.lda[1], M_, g.K);
      eb[1] = OB1::extent(g.ldb[1], N_, g.K);
      sa[1] = (MCMASK & 4u) ? (int64_t)BK * g.lda[1] : BK;
      sb[1] = (MCMASK & 8u) ? (int64_t)BK * g.ldb[1] : BK;
    }
    if constexpr (NPAIR > 2) {
      pa[2] = static_cast<const bf16_t*>(g.a[2]);
      pb[2] = static_cast<const bf16_t*>(g.b[2]);
      a2.init(g.lda[2], m0_, M_, lane, wave);
      b2.init(g.ldb[2], n0_, N_, lane, wave);
      ea[2] = OA2::extent(g.lda[2], M_, g.K);
      eb[2] = OB2::extent(g.ldb[2], N_, g.K);
      sa[2] = (MCMASK & 16u) ? (int64_t)BK * g.lda[2] : BK;
      sb[2] = (MCMASK & 32u) ? (int64_t)BK * g.ldb[2] : BK;
    }
    // The per-lane offsets hold the (clamped) rows / chunks relative to the
    // matrix start; a split starts its sources at its first k-tile.
    const int64_t kt0 = (int64_t)split * g.ktiles_split;
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) {
      pa[p] += kt0 * sa[p];
      pb[p] += kt0 * sb[p];
      ea[p] -= kt0 * sa[p];
      eb[p] -= kt0 * sb[p];
    }
  };
  init_ops(m0, n0, M, N, slot);
  auto stage_ptr = [&](int s) { return lds + s * SB; };
  // Stage tiles of K-tile kt: [A][B] stages, or the two rings.
  auto a_stage = [&](int kt) {
    return TL::ASYM ? lds + (kt % SA) * (BM * BK * 2) : stage_ptr(kt % S);
  };
  auto b_stage = [&](int kt) {
    return TL::ASYM ? lds + SA * (BM * BK * 2) + (kt % S) * (BNO * BK * 2)
                    : stage_ptr(kt % S) + BM * BK * 2;
  };
  // Separate rings: one operand's loads of K-tile kt (the same empty range
  // past the last K-tile as below).
  auto issue_a = [&](int kt) {
    if (!a_iss) return;
    const uint32_t n = kt < g.ktiles_split ? (uint32_t)(2 * (ea[0] - kt * sa[0])) : 0u;
    a0.issue(pa[0] + kt * sa[0], n, a_stage(kt), dwave);
  };
  auto issue_b = [&](int kt) {
    if (!b_iss) return;
    const uint32_t n = kt < g.ktiles_split ? (uint32_t)(2 * (eb[0] - kt * sb[0])) : 0u;
    b0.issue(pb[0] + kt * sb[0], n, b_stage(kt), dwave);
  };
  auto issue = [&](int kt) {
    if (NDMA < TL::NWAVE && wave >= NDMA) return;
    unsigned char* st = stage_ptr(kt % S);
    // A K-tile past the last one loads nothing: an empty buffer range
    // reads zeros without touching memory, so the loop issues its loads
    // without branches.
    const bool live = kt < g.ktiles_split;
    auto nb = [&](int64_t e, int64_t step) { return live ? (uint32_t)(2 * (e - kt * step)) : 0u; };
    if constexpr (BD) {
      // [A][B] of pair 0 for the first ktiles_split K-tiles, then of pair 1.
      const int nkh = g.ktiles_split;
      const bool second = kt >= nkh;
      const int lk = second ? kt - nkh : kt;
      const bool on = kt < 2 * nkh;
      auto nbd = [&](int64_t e, int64_t step) { return on ? (uint32_t)(2 * (e - lk * step)) : 0u; };
      if (!second) {
        a0.issue(pa[0] + lk * sa[0], nbd(ea[0], sa[0]), st, wave);
        b0.issue(pb[0] + lk * sb[0], nbd(eb[0], sb[0]), st + BM * BK * 2, wave);
      } else {
        a1.issue(pa[1] + lk * sa[1], nbd(ea[1], sa[1]), st, wave);
        b1.issue(pb[1] + lk * sb[1], nbd(eb[1], sb[1]), st + BM * BK * 2, wave);
      }
      return;
    }
    if constexpr (SPLITN) {
      // [A0][A1][B0][B1]: the two B tiles form one BN-row tile.
      a0.issue(pa[0] + kt * sa[0], nb(ea[0], sa[0]), st, wave);
      a1.issue(pa[1] + kt * sa[1], nb(ea[1], sa[1]), st + BM * BK * 2, wave);
      b0.issue(pb[0] + kt * sb[0], nb(eb[0], sb[0]), st + 2 * BM * BK * 2, wave);
      b1.issue(pb[1] + kt * sb[1], nb(eb[1], sb[1]), st + (2 * BM + BNO) * BK * 2, wave);
      return;
    }
    a0.issue(pa[0] + kt * sa[0], nb(ea[0], sa[0]), st, wave);
    b0.issue(pb[0] + kt * sb[0], nb(eb[0], sb[0]), st + BM * BK * 2, wave);
    if constexpr (NPAIR > 1) {
      a1.issue(pa[1] + kt * sa[1], nb(ea[1], sa[1]), st + (BM + BN) * BK * 2, wave);
      b1.issue(pb[1] + kt * sb[1], nb(eb[1], sb[1]), st + (2 * BM + BN) * BK * 2, wave);
    }
    if constexpr (NPAIR > 2) {
      a2.issue(pa[2] + kt * sa[2], nb(ea[2], sa[2]), st + 2 * (BM + BN) * BK * 2, wave);
      b2.issue(pb[2] + kt * sb[2], nb(eb[2], sb[2]), st + (3 * BM + 2 * BN) * BK * 2, wave);
    }
  };
  constexpr int L = BD ? OA0::PER + OB0::PER
                      : OA0::PER + OB0::PER + (NPAIR > 1 ? OA1::PER + OB1::PER : 0) +
                            (NPAIR > 2 ? OA2::PER + OB2::PER : 0);
  static_assert(!BD || (OA0::PER == OA1::PER && OB0::PER == OB1::PER),
                "both pairs of a block-diagonal tile load alike");
  static_assert(L * (S - 1) < 64, "too many loads in flight for vmcnt");

  constexpr bool BDP = TL::BDPACK;
  static_assert(!BDP || BD, "packing is for block-diagonal tiles");
  constexpr int NACC = (SPLITN || BDP) ? 1 : NPAIR;
  f32x4 acc[NACC][FM][FN];
  u32x2 gpk[BDP ? FM : 1][BDP ? FN : 1];  // the first pair's results, bf16
#pragma unroll
  for (int p = 0; p < NACC; ++p)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[p][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane fragment offsets (k-step 0; step 1 adds a constant).
  const int w0m = wm * TL::WTM, w0n = wn * TL::WTN;
  const int pw = SPLITN ? wn / (TL::NWN / 2) : 0;  // the pair a split-tile wave runs
  // Byte shift of FM/2 row bands in an A stage tile (the swizzle pattern
  // repeats every 16 rows, so shifted offsets stay valid).
  const int srot = SPLITN ? pw * (FM / 2) * 16 * BK * 2 : 0;
  static_assert(!SPLITN || FM % 2 == 0, "split tiles hand over half of the row bands");

  // Online RMSNorm: the waves of one row band (same wm) read the same A
  // fragments; wave wn sums the squares of bands wn, wn + NWN, ... . Its
  // fragment slots hold the bands rotated by wn (slot i: band (i + wn) mod
  // FM, accumulators alike), so that those bands sit in the fixed slots 0,
  // NWN, ...: a choice by wn at run time among the slots would cost vector
  // instructions beside every sub-step's MFMAs.
  constexpr int FSS = (FM + TL::NWN - 1) / TL::NWN;
  constexpr bool ROT = ORMS && MCMASK == 0u && !SPLITN && !BD && FM % TL::NWN == 0 && (FM & (FM - 1)) == 0;
  static_assert(!ORMS || (ROT && !PST), "Online RMSNorm tiles take rotated bands, one tile per workgroup");
  auto band_of = [&](int i) { return ROT ? (i + wn) & (FM - 1) : i; };
  // ssp: this lane's part of the current panel's sums; tot: the sums of the
  // finished panels, added in panel order (lanes 0..15 hold rows 0..15 of
  // the fragment after the cross-lane sums).
  float ssp[FSS], tot[FSS];
#pragma unroll
  for (int i = 0; i < FSS; ++i) ssp[i] = tot[i] = 0.f;
  // Per-panel sums are written as each panel ends (by the first column tile
  // of a row band only) unless the caller asked for the total.
  bool ss_panels = ORMS && g.ss_out != nullptr && !g.emit_partial && tn == 0;
  int panel = 0, in_panel = 0;
  // The panel length is pinned in a scalar register: reloaded from the
  // kernel arguments inside the K loop, its wait would also wait for every
  // LDS read in flight (scalar loads and LDS reads share one counter).
  int panel_kt = g.panel_ktiles;
  if constexpr (ORMS) asm volatile("" : "+s"(panel_kt));

  // Fragment registers are double-buffered: the LDS reads of sub-step q + 1
  // (a sub-step is one 32-wide k step of one operand pair) are in flight
  // while the MFMAs of sub-step q run. The stage barrier sits before the
  // last sub-step of a K-tile, once its fragments are in registers, so the
  // first fragments of the next K-tile load under that sub-step's MFMAs.
  constexpr int Q = ((SPLITN || BD) ? 1 : NPAIR) * TL::NSTEP;
  u32x4 fa[2][FM], fb[2][FN];
  // st: the stage of K-tile kt (one ring); separate rings use kt.
  auto read_q = [&](int kt, const unsigned char* st, auto q_tag, int buf) {
    constexpr int q = decltype(q_tag)::value;
    constexpr int p = q / TL::NSTEP, s = q % TL::NSTEP;
    const unsigned char* tA = TL::ASYM ? a_stage(kt)
                              : SPLITN ? st + pw * BM * BK * 2 : st + p * (BM + BN) * BK * 2;
    const unsigned char* tB = TL::ASYM ? b_stage(kt)
                              : SPLITN ? st + 2 * BM * BK * 2 : tA + BM * BK * 2;
    const bool amc = (MCMASK >> (2 * p)) & 1u;
    const bool bmc = (MCMASK >> (2 * p + 1)) & 1u;
    // The tiles' LDS addresses as one scalar each: left to itself the
    // compiler splits the ring offset into parts and spends two vector
    // instructions per transposing fragment read on them.
    uint32_t ta = lds_addr(tA), tb = lds_addr(tB);
    if constexpr ((MCMASK & 0x15u) != 0u && !SPLITN) asm volatile("" : "+s"(ta));
    if constexpr ((MCMASK & 0x2Au) != 0u) asm volatile("" : "+s"(tb));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // Split tiles: the up-pair waves hold row bands in rotated order
      // (slot i holds band (i + FM/2) mod FM), so that every wave keeps
      // slots 0 .. FM/2 - 1 and hands over the rest.
      const unsigned char* tAi = SPLITN ? (i < FM / 2 ? tA + srot : tA - srot) : tA;
      if constexpr (ROT) {
        // The swizzle repeats every 16 rows: band b is 16 rows (2 KB per
        // 64-wide K-tile row block) further on.
        fa[buf][i] = Opnd<BM, BK, NDMA, true>::read_frag(
            tAi + band_of(i) * (16 * BK * 2), Opnd<BM, BK, NDMA, true>::frag_off(w0m, s, lane));
      } else if constexpr (MCMASK == 0u) {
        fa[buf][i] = Opnd<BM, BK, NDMA, true>::template read_step<s>(tAi, w0m + 16 * i, lane);
      } else if (amc) {
        fa[buf][i] = SPLITN ? Opnd<BM, BK, NDMA, false>::template read_step<s>(tAi, w0m + 16 * i, lane)
                            : Opnd<BM, BK, NDMA, false>::template read_step_at<s>(ta, w0m + 16 * i, lane);
      } else {
        fa[buf][i] = Opnd<BM, BK, NDMA, true>::template read_step<s>(tAi, w0m + 16 * i, lane);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (bmc)
        fb[buf][j] = Opnd<BN, BK, NDMA, false>::template read_step_at<s>(tb, w0n + 16 * j, lane);
      else
        fb[buf][j] = Opnd<BN, BK, NDMA, true>::template read_step<s>(tB, w0n + 16 * j, lane);
    }
  };
  // ph: the pair a block-diagonal tile's current K-tile belongs to.
  auto compute_q = [&](int q, int buf, auto ph_tag) {
    const int p = BD ? decltype(ph_tag)::value : q / TL::NSTEP;
    if constexpr (ORMS) {
      if (p == 0) {
#pragma unroll
        for (int i = 0; i < FM; i += TL::NWN) {  // the slots of bands wn, wn + NWN, ...
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // Both squares of a bf16 pair in one v_dot2c_f32_bf16 (a bf16
            // square is exact in fp32): a quarter of the vector
            // instructions of unpacking and two FMAs, beside the MFMAs.
            const bf16x8 all = __builtin_bit_cast(bf16x8, fa[buf][i]);
            const bf16x2 v = {all[2 * c], all[2 * c + 1]};
            ssp[i / TL::NWN] = __builtin_amdgcn_fdot2_f32_bf16(v, v, ssp[i / TL::NWN], false);
          }
        }
        // The sums are taken in this sub-step: left alone, the compiler
        // sinks them into the next one, whose fragment reads must then wait
        // for them.
#pragma unroll
        for (int j = 0; j < FSS; ++j) asm volatile("" : "+v"(ssp[j]));
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_step<bf16_t>(fb[buf][j], fa[buf][i], acc[BDP ? 0 : p][i][j]);
  };
  // K-tile kt has landed in LDS when at most (K-tiles issued after it) x L
  // loads of this lane remain; `after` is that count of K-tiles.
  // Every K-tile index is issued (past the last one with an empty range),
  // so K-tile kt has landed once at most (S - 2) x L loads of this lane
  // are in flight.
  constexpr int VM_AFTER = (S - 2) * L;
  // DS reads of one sub-step of pair 0 (K-contiguous fragments; the
  // transposing reads of M-contiguous ones are inline assembly the
  // scheduler cannot group).
  constexpr int NDS = ((MCMASK & 1u) ? 0 : FM) + ((MCMASK & 2u) ? 0 : FN);

  const int nk = g.ktiles_split;
  // Separate rings (A: SA = 3 stages, B: S = 2): at the barrier of K-tile kt
  // B of K-tile kt + 2 is issued, then A of kt + 3, so the loads issued
  // after K-tile kt + 1's are A's of kt + 2 alone.
  static_assert(!TL::ASYM || (SA == 3 && S == 2), "separate rings: 3 A stages, 2 B stages");
  constexpr int LA = OA0::PER;
  static_assert(!TL::ASYM || 2 * LA + OB0::PER < 64, "too many loads in flight for vmcnt");
  // The prologue: the loads issued before its barrier (pro_pre), then the
  // wait for K-tile 0, the barrier and the loads of the stages it frees
  // (pro_post). A persistent workgroup runs the next tile's pro_pre before
  // the epilogue and its pro_post after; AF is the number of vector-memory
  // operations the wave issued in between (a lower bound: waiting for
  // fewer in flight is never too early), which may still be in flight
  // since operations retire in order.
  auto pro_pre = [&]() {
    if constexpr (TL::ASYM) {
      issue_a(0);
      issue_b(0);
      issue_a(1);
    } else {
#pragma unroll
      for (int s = 0; s < S - 1; ++s) issue(s);
    }
  };
  auto pro_post = [&](auto after_tag) {
    constexpr int AF = decltype(after_tag)::value;
    constexpr int W = (TL::ASYM ? LA : VM_AFTER) + AF;
    if constexpr (SPLIT_AB) {
      // B loaders: B of K-tile 0 has landed with at most AF operations
      // pending; A loaders: A of K-tile 0 with at most LA + AF (A of 1).
      if (b_iss)
        wait_vmcnt<(AF < 63 ? AF : 63)>();
      else
        wait_vmcnt<(W < 63 ? W : 63)>();
    } else {
      wait_vmcnt<(W < 63 ? W : 63)>();
    }
    wait_lgkmcnt0();  // every wave's epilogue is done with its LDS areas
    block_barrier();
    if constexpr (TL::ASYM) {
      issue_b(1);
      if constexpr (!SPLIT_AB) issue_a(2);  // (split: at the start of K-tile 0)
    } else {
      issue(S - 1);
    }
  };
  pro_pre();
  pro_post(std::integral_constant<int, 0>{});

  for (;;) {  // the tiles of a persistent workgroup (one otherwise)
  read_q(0, stage_ptr(0), std::integral_constant<int, 0>{}, 0);
  // Fragment reads are in flight only inside the loop body, between a
  // sub-step's start and the next sub-step's wait: every path into and out
  // of the loop has them landed, so code the compiler places at the loop's
  // edges cannot touch registers still being written.
  sched_fence();
  wait_lgkmcnt0();
  sched_fence();

  // One K-tile. Fragment buffer of sub-step q of K-tile kt: (kt Q + q) & 1,
  // i.e. (q + B0) & 1 with B0 = (kt Q) & 1; with an odd sub-step count the
  // loop runs K-tiles in pairs so that B0 stays a constant.
  auto ktile = [&](int kt, auto b0_tag, auto ph_tag) {
    constexpr int B0 = decltype(b0_tag)::value;
    const unsigned char* st = stage_ptr(kt % S);
    static_for<Q>([&](auto q_tag) {
      constexpr int q = decltype(q_tag)::value;
      const int buf = (q + B0) & 1;
      // Nothing is scheduled across this wait in either direction: the
      // fragments of sub-step q (some read by inline assembly the compiler
      // does not track) are in registers only after it.
      sched_fence();
      wait_lgkmcnt0();
      sched_fence();
      if constexpr (SPLIT_AB && q == 0) issue_a(kt + 2);
      if constexpr (q + 1 < Q) {
        read_q(kt, st, std::integral_constant<int, q + 1>{}, buf ^ 1);
        compute_q(q, buf, ph_tag);
        interleave<NDS, 0, FM * FN>();
      } else {
        // Every wave has its fragments of K-tile kt in registers once it
        // passes the barrier; the stage of K-tile kt is then free for
        // K-tile kt + S, and K-tile kt + 1 has landed. (On the last K-tile
        // this reads a stage no MFMA uses.)
        if constexpr (SPLIT_AB) {
          // B loaders: B of K-tile kt + 1 (issued one K-tile ago) is their
          // only load in flight; A loaders: A of kt + 1 and of kt + 2.
          if (b_iss)
            wait_vmcnt<0>();
          else
            wait_vmcnt<LA>();
          block_barrier();
          issue_b(kt + 2);
        } else if constexpr (TL::ASYM) {
          wait_vmcnt<LA>();
          block_barrier();
          issue_b(kt + 2);
          issue_a(kt + 3);
        } else {
          wait_vmcnt<VM_AFTER>();
          block_barrier();
          issue(kt + S);
        }
        read_q(kt + 1, stage_ptr((kt + 1) % S), std::integral_constant<int, 0>{}, buf ^ 1);
        compute_q(q, buf, ph_tag);
        interleave<NDS, L, FM * FN>();
      }
    });
    if constexpr (ORMS) {
      if (++in_panel == panel_kt || kt == nk - 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          if (i % TL::NWN == wn) {
            float x = ssp[i / TL::NWN];
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            tot[i / TL::NWN] += x;
            const int gr = m0 + w0m + 16 * i + lane;
            // One vector store among the ring's loads: a wait for at most n
            // operations in flight then waits for one load more than it
            // would have (operations retire in order), never for fewer.
            if (ss_panels && lane < 16 && gr < M) g.ss_out[(int64_t)panel * M + gr] = x;
            ssp[i / TL::NWN] = 0.f;
          }
        ++panel;
        in_panel = 0;
      }
    }
    sched_fence();
    wait_lgkmcnt0();
    sched_fence();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (BD) {
    // nk K-tiles of pair 0, then nk of pair 1 (nk = ktiles_split each).
    static_assert(!(Q & 1), "block-diagonal tiles take an even sub-step count");
    for (int kt = 0; kt < nk; ++kt) ktile(kt, I0{}, I0{});
    if constexpr (BDP) {
      // The gate is final: keep it as bf16 (half the registers) and clear
      // the accumulators for the up pair.
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          gpk[i][j] = u32x2{pack_bf16x2(acc[0][i][j][0], acc[0][i][j][1]),
                            pack_bf16x2(acc[0][i][j][2], acc[0][i][j][3])};
          acc[0][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    for (int kt = nk; kt < 2 * nk; ++kt) ktile(kt, I0{}, I1{});
  } else if constexpr (Q & 1) {
    for (int kt = 0; kt < nk; kt += 2) {
      ktile(kt, I0{}, I0{});
      if (kt + 1 < nk) ktile(kt + 1, I1{}, I0{});
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) ktile(kt, I0{}, I0{});
  }
  // The last fragment reads (of a stage no MFMA uses, or before the loop
  // with no K-tile at all) and the empty-range loads past the last K-tile
  // are still in flight; nothing may reuse their registers or LDS before
  // they land.
  sched_fence();
  wait_lgkmcnt0();
  wait_vmcnt<0>();
  sched_fence();
  __syncthreads();  // every wave is done with the ring
  if constexpr (ORMS) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i % TL::NWN == wn && lane < 16) sTot[w0m + 16 * i + lane] = tot[i / TL::NWN];
    __syncthreads();
  }
  // Persistent: the next tile's coordinates, loaders and first loads; the
  // epilogue's LDS areas lie outside the stages these fill.
  bool more = false;
  int tm1 = 0, tn1 = 0, slot1 = 0;
  if constexpr (PST) {
    if (vt + (int)gridDim.x < g.vtiles) {
      more = true;
      vcoords(vt + (int)gridDim.x, tm1, tn1, slot1);
      init_ops(tm1 * BM, tn1 * BNO, M, N, slot1);
      pro_pre();
    }
  }

  // Epilogue geometry. Split tiles: the wave running pair 0 (gate) and its
  // partner in the same row band running pair 1 (up) each finish half of the
  // bands, handing the other half of their accumulators over through LDS;
  // afterwards acc[0][i] holds the gate and acc[0][FME + i] the up values of
  // band keep0 + i. LR_E(p, i, j) names pair p of epilogue band i. Band i
  // covers rows rb + 16 i .. + 15 and columns cb .. cb + WTN - 1 of the tile.
  constexpr int FME = SPLITN ? FM / 2 : FM;
  const int keep0 = pw * FME;
  const int rb = w0m + 16 * keep0;                                  // first row
  const int cb = SPLITN ? (wn % (TL::NWN / 2)) * TL::WTN : w0n;  // first column
  // The MFMA takes the B fragment as its first operand, so fragment (i, j)
  // of lane l holds row rb + 16 i + (l & 15) of the block tile at the four
  // consecutive columns cb + 16 j + 4 (l >> 4) + v, v = 0..3.
  // (The lane index is recomputed here, behind an empty asm statement the
  // compiler cannot move, so that it keeps no values derived from it alive
  // across the main loop, nor hoists them out of a persistent tile loop.)
  int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(elane));
  const int lane = elane;  // the epilogue's lane index
  const int fr = elane & 15, fc = 4 * (elane >> 4);

  // HBM inputs of the epilogue, requested before anything else: gamma and
  // the row scalars into registers, the bf16 element inputs (NIN of them)
  // band by band into wave-private LDS slots, PDS bands ahead.
  constexpr bool HAS_RES = (EPI == EPI_STORE || EPI == EPI_RMSBWD || EPI == EPI_SWIGLU_BWD2);
  constexpr bool HAS_H = (EPI == EPI_RMSBWD);
  constexpr bool HAS_GAMMA = (EPI == EPI_RMSBWD || EPI == EPI_WGRAD);
  constexpr bool HAS_ROW = (EPI == EPI_STORE || EPI == EPI_RMSBWD);
  constexpr int NIN = (HAS_RES ? 1 : 0) + (HAS_H ? 1 : 0);
  constexpr int PDS = EL::PDS;
  static_assert(NIN == epi_nin<EPI>(), "input count");
  static_assert(NIN == 0 || TL::WTN == 64, "band inputs need 64-column wave tiles");
  static_assert(NIN == 0 || EL::slot_off(PDS - 1) + EL::SLOT <= LDSB, "input slots exceed LDS");
  const bf16_t* resp = static_cast<const bf16_t*>(g.res);
  const bf16_t* hp = static_cast<const bf16_t*>(g.hsrc);

  float gmv[FN][4];  // gamma of this lane's columns
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) gmv[j][v] = 1.0f;
  if constexpr (HAS_GAMMA) {
#if defined(__HIP_DEVICE_COMPILE__)
    // Columns past the end read as zero; no gamma array means gamma = 1.
    const bool gon = colscale != nullptr;
    const unsigned char* gp;
    int gbytes;
    epi_range(colscale, 2, 0, 0, n0, 1, N, gp, gbytes);
    const __amdgpu_buffer_rsrc_t grs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(gp), (short)0, gbytes, 0x00020000);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      // Without a gamma array the load reads zeros and the 1 comes from
      // `one`: no branch, so the loads need not be waited for here.
      const float one = gon ? 0.0f : 1.0f;
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(grs, 2 * (cb + 16 * j + fc), 0, 0);
      gmv[j][0] = bf16_lo(w[0]) + one;
      gmv[j][1] = bf16_hi(w[0]) + one;
      gmv[j][2] = bf16_lo(w[1]) + one;
      gmv[j][3] = bf16_hi(w[1]) + one;
    }
#endif
  }
  // Per-row scalars: the RMSNorm-backward coefficient, or the divisor of a
  // plain store (rows past the end read zero; they are never stored).
  float rowv[FME];
  if constexpr (HAS_ROW) {
    EpiRow in_row;
    in_row.init(EPI == EPI_RMSBWD ? g.rowcoef : g.rowdiv, m0, M, rb + fr);
#pragma unroll
    for (int i = 0; i < FME; ++i) rowv[i] = in_row.load(i);
  }
  // The band inputs' loads are counted by hand below: no other HBM access
  // may be issued after them but the epilogue's stores.
  asm volatile("" ::: "memory");
  sched_fence();
  EpiDma in_res, in_h;
  if constexpr (HAS_RES) in_res.init(resp, g.ldres, m0, n0, M, N, rb, cb, lane);
  if constexpr (HAS_H) in_h.init(hp, g.ldh, m0, n0, M, N, rb, cb, lane);
  unsigned char* sIn = lds + wave * (NIN * 2048);  // + slot_off(p): [NIN][2 KB]
  // A plain store without a residual has no band inputs.
  const bool in_on = NIN > 0 && (EPI != EPI_STORE || resp != nullptr);
  auto issue_band = [&](int i) {
    unsigned char* slot = sIn + EL::slot_off(i % PDS);
    if constexpr (HAS_RES) in_res.issue(i, slot);
    if constexpr (HAS_H) in_h.issue(i, slot + 2048);
  };
  if constexpr (NIN > 0) {
    if (in_on) {
#pragma unroll
      for (int i = 0; i < PDS; ++i) issue_band(i);
    }
  }

  if constexpr (ORMS) {
    for (int r = tid; r < BM; r += TL::NT) {
      const float ss = sTot[r];
      const float rmsg = sqrtf(ss * g.inv_D + g.eps);
      sRow[r] = g.emit_partial ? 1.0f : 1.0f / rmsg;
      const int gr = m0 + r;
      if (tn == 0 && gr < M) {
        if (g.rms_out && !g.emit_partial) g.rms_out[gr] = rmsg;
        // (per-panel sums were written as their panels ended)
        if (g.ss_out && g.emit_partial) g.ss_out[gr] = ss;
      }
    }
    if constexpr (PST) {
      // A bare barrier: __syncthreads would also wait for the next tile's
      // loads in flight.
      wait_lgkmcnt0();
      block_barrier();
    } else {
      __syncthreads();
    }
  }

  if constexpr (SPLITN) {
    constexpr int NRD = epi_xch_rounds<TL, EPI>();
    static_assert(XCH <= IN0, "the exchange area overlaps the input slots");
    static_assert(FME % NRD == 0, "exchange rounds split the bands");
    static_assert(XCH <= RING, "exchange area exceeds the ring");
    constexpr int NR = FME / NRD;
    const int partner = wm * TL::NWN + (wn + TL::NWN / 2) % TL::NWN;
    // [NWAVE][NR][FN][64 lanes][4]: a lane's four values of a fragment are
    // one 16-byte access, a wave's instruction one contiguous 1 KB.
    f32x4* xch = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int rd = 0; rd < NRD; ++rd) {
#pragma unroll
      for (int ii = 0; ii < NR; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          xch[((wave * NR + ii) * FN + j) * 64 + lane] = acc[0][FME + rd * NR + ii][j];
      // A bare barrier: __syncthreads would also wait for the band-input
      // loads in flight.
      wait_lgkmcnt0();
      block_barrier();
      // Slot i: own pair, band keep0 + i; slot FME + i: the partner's pair,
      // same band. Put the gate in slot i and the up values in slot FME + i.
#pragma unroll
      for (int ii = 0; ii < NR; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int i = rd * NR + ii;
          const f32x4 oth = xch[((partner * NR + ii) * FN + j) * 64 + lane];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float own = acc[0][i][j][v];
            acc[0][i][j][v] = pw ? oth[v] : own;
            acc[0][FME + i][j][v] = pw ? own : oth[v];
          }
        }
      wait_lgkmcnt0();
      block_barrier();  // the next round and the staging area reuse the exchange area
    }
  }
#define LR_E(p, i, j) acc[SPLITN ? 0 : (p)][SPLITN ? (p) * FME + (i) : (i)][j]
  // The gate value g of element v of band i, fragment j, as it enters the
  // SiLU: a bf16 value in every tile of this engine (the packed gate, or the
  // accumulator rounded alike, as a bf16 GEMM would store it), so that the
  // forward and the recompute in the backward agree bitwise whichever of
  // these tiles they run. (A shape's forward gate/up product runs on this
  // engine exactly when its recompute does: the same K, N and extents.)
  auto gate_of = [&](int i, int j, int v) -> float {
    if constexpr (BDP) {
      const uint32_t w = gpk[i][j][v >> 1];
      return (v & 1) ? bf16_hi(w) : bf16_lo(w);
    } else {
      return bf16_lo(pack_bf16x2(LR_E(0, i, j)[v], 0.f));
    }
  };

  // Elementwise combination of the accumulators.
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < FME; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gg = gate_of(i, j, v);
          if constexpr (BDP)  // the up values in the accumulators
            acc[0][i][j][v] = gg * sigmoid_f<bf16_t>(gg) * acc[0][i][j][v];
          else
            LR_E(0, i, j)[v] = gg * sigmoid_f<bf16_t>(gg) * LR_E(1, i, j)[v];
        }
  }

  // Staging of one band's bf16 outputs for whole-row stores.
  static_assert(TL::WTN == 64 || TL::WTN == 32, "staging supports 32- and 64-column wave tiles");
  constexpr int RB = TL::WTN * 2;     // bytes per staged row
  constexpr int CH = TL::WTN / 8;     // 16-byte chunks per row
  constexpr int PERL = 16 * CH / 64;  // chunks per lane per band
  auto swz_st = [](int row) { return RB == 128 ? epi_swz(row) : ((row >> 2) & 3); };
  unsigned char* sWb = lds + EL::ST + wave * epi_wave_bytes<TL>();
  constexpr int NOUT = (EPI == EPI_SWIGLU_BWD2) ? 3 : 1;
  void* cq[NOUT];
  int64_t lq[NOUT];
  EpiOut<PERL> outs[NOUT];
#pragma unroll
  for (int q = 0; q < NOUT; ++q) {
    cq[q] = (EPI == EPI_STORE) ? pick3(g.c, slot) : pick3(g.c, q);
    lq[q] = (EPI == EPI_STORE) ? pick3(g.ldc, slot) : pick3(g.ldc, q);
    if constexpr (NIN > 0 || PST) outs[q].init(cq[q], lq[q], m0, n0, M, N, rb, cb, lane, CH);
  }
  // With band inputs in flight every lane must issue the same stores (the
  // waits count them), so they go through the buffer range check; without,
  // plain stores of the lanes in range.
  auto put_band = [&](int i, const u32x2 (&w)[FN], const EpiOut<PERL>& out, void* cbase, int64_t ldc,
                      auto uniform_tag) {
    constexpr bool UNIFORM = decltype(uniform_tag)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = 2 * j + (lane >> 5), h = (lane >> 4) & 1;  // logical chunk, 8-byte half
      *reinterpret_cast<u32x2*>(sWb + fr * RB + 16 * (c ^ swz_st(fr)) + 8 * h) = w[j];
    }
#pragma unroll
    for (int q = 0; q < PERL; ++q) {
      const int id = lane + 64 * q, rr = id / CH, cc = id % CH;
      const u32x4 x = *reinterpret_cast<const u32x4*>(sWb + rr * RB + 16 * (cc ^ swz_st(rr)));
      if constexpr (UNIFORM) {
        out.store(i, q, x);
      } else {
        const int gr = m0 + rb + 16 * band_of(i) + rr, gc = n0 + cb + 8 * cc;
        if (gr < M && gc < N)
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(static_cast<bf16_t*>(cbase) +
                                                                 (int64_t)gr * ldc + gc));
      }
    }
  };
  auto unpack4 = [](u32x2 w, float* x) {
    x[0] = bf16_lo(w[0]);
    x[1] = bf16_hi(w[0]);
    x[2] = bf16_lo(w[1]);
    x[3] = bf16_hi(w[1]);
  };
  float colacc[FN][4];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) colacc[j][v] = 0.f;

  // Band by band: wait for the band's inputs, read them in the accumulator
  // layout, hand the slot to the band PDS ahead, combine, pack to bf16 and
  // store through the staging area. The hardware retires loads and stores
  // of a wave in order through one counter; the wait for band i allows
  // exactly the operations issued after band i's input loads to be pending.
  auto run_bands = [&](auto in_tag) {
    constexpr bool IN = decltype(in_tag)::value;
    constexpr int DM = IN ? 2 * NIN : 0;  // input loads per band
    constexpr int ST = NOUT * PERL;       // stores per band
#pragma unroll
    for (int i = 0; i < FME; ++i) {
      u32x2 rin[FN], hin[FN];
      if constexpr (IN) {
        // Operations issued after band i's loads: the bands issued at the
        // start after it, then per earlier band its successor's loads (if
        // any) and its stores.
        int after = 0;
        if (i < PDS) {
          for (int b2 = i + 1; b2 < PDS; ++b2) after += DM;
          for (int k = 0; k < i; ++k) after += (k + PDS < FME ? DM : 0) + ST;
        } else {
          after = ST;
          for (int k = i - PDS + 1; k < i; ++k) after += (k + PDS < FME ? DM : 0) + ST;
        }
        sched_fence();
        wait_vmcnt_le(after);
        sched_fence();
        const unsigned char* slot = sIn + EL::slot_off(i % PDS);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (HAS_RES) rin[j] = *reinterpret_cast<const u32x2*>(slot + epi_acc_off(j, lane));
          if constexpr (HAS_H) hin[j] = *reinterpret_cast<const u32x2*>(slot + 2048 + epi_acc_off(j, lane));
        }
        if (i + PDS < FME) {
          wait_lgkmcnt0();  // the slot's reads have returned before it is refilled
          issue_band(i + PDS);
        }
      }
      float rs = 1.0f;  // 1 / rms_g, 1 / rowdiv, or the RMSNorm-backward coefficient
      if constexpr (ORMS) rs = sRow[rb + 16 * band_of(i) + fr];
      if constexpr (EPI == EPI_STORE) rs = 1.0f / rowv[i];
      if constexpr (EPI == EPI_RMSBWD) rs = rowv[i];
      u32x2 pk[NOUT][FN];  // this band's packed bf16 outputs
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float o[NOUT][4];
        float rv[4] = {0.f, 0.f, 0.f, 0.f}, hv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (IN && HAS_RES) unpack4(rin[j], rv);
        if constexpr (IN && HAS_H) unpack4(hin[j], hv);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float x = (EPI == EPI_SWIGLU_BWD2) ? gate_of(i, j, v) : LR_E(0, i, j)[v];
          if constexpr (EPI == EPI_STORE) {
            o[0][v] = (g.rowdiv ? x * rs : x) + rv[v];
          } else if constexpr (EPI == EPI_ORMS) {
            o[0][v] = x * rs;
          } else if constexpr (EPI == EPI_SWIGLU) {
            o[0][v] = x;  // already combined
          } else if constexpr (EPI == EPI_RMSBWD) {
            // dX = dY + gamma (dZ_n A) - coef H; gamma-gradient sums of acc H
            colacc[j][v] += x * hv[v];
            o[0][v] = rv[v] + gmv[j][v] * x - rs * hv[v];
          } else if constexpr (EPI == EPI_SWIGLU_BWD2) {
            // g, u recomputed in the accumulators, dm from HBM:
            // m = SiLU(g) u; dg = dm u sig(g)(1 + g(1 - sig(g))); du = dm SiLU(g)
            // (SiLU'(g) = sig(g) + SiLU(g) (1 - sig(g)): one FMA on values
            // already at hand; the epilogue is bound by its vector work.)
            const float uu = LR_E(BDP ? 0 : 1, i, j)[v], dm = rv[v];  // (packed: up in acc[0])
            const float sg = sigmoid_f<bf16_t>(x);
            const float sl = x * sg;
            const float ds = __builtin_fmaf(sl, 1.0f - sg, sg);
            o[0][v] = sl * uu;
            o[1][v] = (dm * uu) * ds;
            o[2][v] = dm * sl;
          }
        }
#pragma unroll
        for (int q = 0; q < NOUT; ++q)
          pk[q][j] = u32x2{pack_bf16x2(o[q][0], o[q][1]), pack_bf16x2(o[q][2], o[q][3])};
        // Left to itself the compiler sinks the column sums to their use
        // after the last band and holds the H values of every band until then.
        if constexpr (HAS_H) {
#pragma unroll
          for (int v = 0; v < 4; ++v) asm volatile("" : "+v"(colacc[j][v]));
        }
      }
#pragma unroll
      for (int q = 0; q < NOUT; ++q)
        put_band(i, pk[q], outs[q], cq[q], lq[q], std::integral_constant<bool, IN || PST>{});
    }
  };
  if constexpr (EPI != EPI_WGRAD) {
    if constexpr (NIN == 0) {
      run_bands(std::false_type{});
    } else if constexpr (EPI == EPI_STORE) {
      if (in_on)
        run_bands(std::true_type{});
      else
        run_bands(std::false_type{});
    } else {
      run_bands(std::true_type{});
    }
  }

  if constexpr (EPI == EPI_RMSBWD) {
    // This wave's column sums: the 16 lanes holding the same columns add
    // theirs (a butterfly over lane bits 0..3); the NWM waves of a column
    // band are then added through LDS in wave order (fixed order).
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = colacc[j][v];
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        colacc[j][v] = x;
      }
    float* sCol = reinterpret_cast<float*>(lds + EL::ST + EL::EW);  // [NWM][BN]
    if (fr == 0) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) sCol[wm * BN + cb + 16 * j + fc + v] = colacc[j][v];
    }
  }

  if constexpr (EPI == EPI_WGRAD) {
    // fp32 weight gradients straight from the accumulators: 16 bytes per
    // lane, 16 rows x 64 bytes per store.
#pragma unroll
    for (int i = 0; i < FME; ++i) {
      const int gr = m0 + rb + 16 * i + fr;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int gc = n0 + cb + 16 * j + fc;
        if (gr < M && gc < N) {
          const f32x4 x = LR_E(0, i, j);
          __builtin_nontemporal_store(
              f32x4{x[0] * gmv[j][0], x[1] * gmv[j][1], x[2] * gmv[j][2], x[3] * gmv[j][3]},
              reinterpret_cast<f32x4*>(static_cast<float*>(pick3(g.c, slot)) + split * csplit +
                                       (int64_t)gr * pick3(g.ldc, slot) + gc));
        }
      }
    }
  }

  if constexpr (EPI == EPI_RMSBWD) {
    const float* sCol = reinterpret_cast<const float*>(lds + EL::ST + EL::EW);
    // A bare barrier: the column sums are in LDS; the band stores may
    // still be in flight.
    wait_lgkmcnt0();
    block_barrier();
    for (int c = tid; c < BN; c += TL::NT) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < TL::NWM; ++q) sum += sCol[q * BN + c];
      if (n0 + c < N) g.colsum[(int64_t)tm * N + n0 + c] = sum;
    }
  }

  // Side job: a share of the columns of an earlier kernel's per-tile column
  // sums. A wave takes one column at a time: lane l adds rows l, l + 64, ...
  // in order, then a fixed butterfly adds the 64 lanes (deterministic).
  if (g.cs_out != nullptr) {
    const int nwg = (int)(gridDim.x * gridDim.z);
    const int wid = (int)(blockIdx.x + gridDim.x * blockIdx.z);
    const int per = (g.cs_n + nwg - 1) / nwg;
    const int cend = min(g.cs_n, (wid + 1) * per);
    for (int c = wid * per + wave; c < cend; c += TL::NWAVE) {
      float sum = 0.f;
      for (int r = lane; r < g.cs_rows; r += 64) sum += g.cs_part[(int64_t)r * g.cs_n + c];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
      if (lane == 0) g.cs_out[c] = sum;
    }
  }

  if (!more) break;
  // The next tile. The vector-memory operations this wave issued after the
  // next tile's first loads: the row scalars, the band inputs and the
  // stores (uniform in a persistent workgroup), a count known per path.
  vt += (int)gridDim.x;
  tm = tm1;
  tn = tn1;
  slot = slot1;
  m0 = tm * BM;
  n0 = tn * BNO;
  // The loaders again (a few scalar and vector operations): their values
  // from before the epilogue need not stay live across it.
  init_ops(m0, n0, M, N, slot);
  if constexpr (ORMS) ss_panels = g.ss_out != nullptr && !g.emit_partial && tn == 0;
#pragma unroll
  for (int p = 0; p < NACC; ++p)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[p][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < FSS; ++i) ssp[i] = tot[i] = 0.f;
  panel = 0;
  in_panel = 0;
  {
    constexpr int E_OUT = (HAS_ROW ? FME : 0) + FME * NOUT * PERL;
    constexpr int E_IN = E_OUT + FME * 2 * NIN;
    if (in_on)
      pro_post(std::integral_constant<int, E_IN>{});
    else
      pro_post(std::integral_constant<int, E_OUT>{});
  }
  }  // tiles
#undef LR_E
}

}  // namespace lr
