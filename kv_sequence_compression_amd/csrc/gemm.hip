// Projection GEMM and fused compressor on the gfx950 matrix cores.
//
// The projection ("序列压缩注意力", eq. attn-seqcomp-csa-proj) is the one
// dense contraction of the compressor: Y = H Wt^T with K = d.  One workgroup
// computes a 256 x 256 tile of Y with 4 wavefronts (2 x 2, each 128 x 128 as
// 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators in registers).  Under sustained
// load the chip's power limit sets the rate: a kernel built the same way on
// v_mfma_f32_16x16x32_bf16 (8 waves of 128 x 64, two per SIMD) drew less
// power per MFMA and ran at a higher clock, but its matrix cores were
// correspondingly less busy, and it measured the same throughput.  K advances in
// 128-byte slabs (64 bf16 / 32 fp32 of every tile row: whole cache lines, so
// every L2 request is a full line) that are copied global -> LDS directly
// (global_load_lds_dwordx4, no register staging).  The LDS holds a ring of
// 3 slabs of H and 2 of Wt (5 x 32 KiB = 160 KiB): H, streamed from HBM,
// is requested two slabs ahead, the weights, which hit in L2 or the
// last-level cache, one slab ahead.
//
// The fused kernels keep that accumulator tile in registers and pool it
// there, so C and Z never reach HBM:
//  * the 32x32 MFMA accumulator gives every lane four runs of 4 consecutive
//    token rows of one channel (rows 8q + 4h + 0..3 of a 32-row subtile,
//    h = lane / 32), i.e. whole CSA blocks of m = 4 rows;
//  * the N tile is laid out so that each wavefront holds the SAME channels of
//    every stream (CSA: 32 channels x [C^a | C^b | Z^a | Z^b]; HCA: 64
//    channels x [C | Z]);
//  * CSA (eq. attn-seqcomp-csa-softmax / -pool): a lane folds its block's
//    a-rows into (max, sum, weighted sum) and its b-rows into the partial of
//    the NEXT entry; one exchange between lanes l and l ^ 32 hands the
//    b-partial to the entry that needs it (eq. attn-seqcomp-overlap-bound for the first block of a
//    sequence).  The first entry of a tile that continues a sequence needs
//    the previous tile's last block: both partials go to a small halo buffer
//    and a fix-up kernel merges them (log-sum-exp merge, exact up to
//    rounding);
//  * HCA (eq. attn-seqcomp-hca): a wave row of 128 tokens is one block of
//    m' = 128; lanes fold 64 rows each, then one exchange merges the halves.
// Tiles are rows of one sequence (tile table from the planner); the grid is
// remapped so that all N tiles of an M panel run on the same XCD (shared L2).
#include "amdgcn.hpp"
#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;                      // BM = BN = 256
constexpr int kRowBytes = 128;                  // bytes of one tile row per K slab (64 bf16 / 32 fp32)
constexpr int kSlabBytes = kTile * kRowBytes;   // 32 KiB: one operand's slab
constexpr int kStagesA = 3;                     // H slabs in the ring
constexpr int kStagesB = 2;                     // Wt slabs in the ring
constexpr int kLdsB = kStagesA * kSlabBytes;    // offset of the Wt slots
constexpr int kLdsBytes = (kStagesA + kStagesB) * kSlabBytes;   // 160 KiB: all of a CU's LDS
constexpr int kLoadsPerSlab = kTile / 4 / 8;    // global_load_lds per wave and operand slab (8 rows each)

enum : int { MODE_PROJECT = 0, MODE_CSA = 1, MODE_HCA = 2, MODE_CSA_APPEND = 3 };

// Slot of 16-byte chunk kc (0..7) in 128-byte tile row r: kc ^ f(r) with
// f(r) = (r ^ (r >> 3)) & 7.  A fragment read takes one chunk of 32
// consecutive rows; the LDS serves it without bank conflicts whether it
// handles 8 lanes (128 bytes) or 16 lanes (256 bytes) per pass: any 8
// consecutive rows get 8 distinct slots, and of 16 consecutive rows from a
// multiple of 16 the 8 even rows (one half of a 256-byte bank window) get 8
// distinct slots, as do the 8 odd rows.
__device__ __forceinline__ int swz_f(int r) { return (r ^ (r >> 3)) & 7; }

// XCD-aware tile order: hardware hands workgroup w to XCD (w mod 8); give
// each XCD one contiguous range of logical tiles (N fastest), so the N tiles
// sharing an M panel of H run on one XCD and its L2.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  const int q = G >> 3, r = G & 7, x = w & 7, k = w >> 3;
  return x * q + min(x, r) + k;
}

struct Args {
  const char* H;        // [rows x d] in-dtype
  const char* Wt;       // [n_w x d]  in-dtype
  int64_t lda;          // bytes per H / Wt row (= d * es)
  int nk;               // K slabs
  // projection
  int64_t T;
  int n_out;
  char* Y;
  int64_t ld_y;         // elements
  // fused
  int c;
  const float* Ba;
  const float* Bb;
  const TileRec* tiles;
  float* halo;
  char* out;
  // CSA append: state of every block's previous block (b-stream partial)
  const float* state_in;   // [nb][3][c]: M, S, A planes
  float* state_out;        // [nb][3][c]
  int64_t nb;              // blocks (= entries)
  // grid
  int n_mt, n_nt;
  // fused kernels built with LOOKUP: tiles found from the sequence offsets
  // (tile_lookup) instead of the planner's table; batch <= kTileLookupMaxBatch
  const int64_t* cu;
  int batch;
  int m;
};

template <int DIN>
struct Frag;

// Accumulator tile of one wave: [4 M subtiles][4 N subtiles] of 32 x 32.
// Lane l holds column l % 32 and rows 8 q + 4 (l / 32) + r (element 4 q + r).
typedef f32x16_t WaveAcc[4][4];

// A K slab (128 bytes of every tile row) is consumed in 4 steps; step s reads
// 4 A and 4 B fragments of 16 bytes per lane from LDS (lane l: row l % 32 of
// each 32-row subtile, chunk 2 s + l / 32 of the row) and issues the MFMAs
// over them.  Rows 32 i + (l % 32) of subtile i have f = x0 ^ 4 (i & 1) with
// x0 = (l & 7) ^ ((l >> 3) & 3), so chunk 2 s + h sits at byte
// 16 (h ^ x0) ^ 32 (s ^ 2 (i & 1)) of the row: ro[k] holds the lane's row
// start plus 16 (h ^ x0) ^ 32 k.
struct Frags {
  f32x4_t a[4], b[4];
};

template <int S>
__device__ __forceinline__ void read_frags(const char* As, const char* Bs, const int (&ro)[4], int wm, int wn,
                                           Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = S ^ (2 * (i & 1));
    f.a[i] = *reinterpret_cast<const f32x4_t*>(As + (wm * 128 + i * 32) * kRowBytes + ro[k]);
    f.b[i] = *reinterpret_cast<const f32x4_t*>(Bs + (wn * 128 + i * 32) * kRowBytes + ro[k]);
  }
}

template <>
struct Frag<DT_BF16> {
  static __device__ __forceinline__ void mma1(const Frags& f, WaveAcc& acc, int i, int j) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.a[i]),
                                                         __builtin_bit_cast(bf16x8_t, f.b[j]), acc[i][j], 0, 0, 0);
  }
  // Step s: lane l feeds row l % 32 and the 8 consecutive k of chunk 2 s + l / 32.
  // MFMAs of M subtiles [I0, I1) over all 4 N subtiles.
  template <int I0 = 0, int I1 = 4>
  static __device__ __forceinline__ void mma(const Frags& f, WaveAcc& acc) {
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.a[i]),
                                                             __builtin_bit_cast(bf16x8_t, f.b[j]), acc[i][j], 0, 0, 0);
  }
};

template <>
struct Frag<DT_F32> {
  static __device__ __forceinline__ void mma1(const Frags& f, WaveAcc& acc, int i, int j) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][t], f.b[j][t], acc[i][j], 0, 0, 0);
  }
  // Step s: chunk 2 s + h holds the 4 fp32 k = 8 s + 4 h + t, t = 0..3; four
  // 32x32x2 MFMAs per (i, j), where at MFMA t lane half h feeds k = 8 s + 4 h + t.
  // The same permutation of k on both operands leaves the dot products unchanged.
  template <int I0 = 0, int I1 = 4>
  static __device__ __forceinline__ void mma(const Frags& f, WaveAcc& acc) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][t], f.b[j][t], acc[i][j], 0, 0, 0);
  }
};

// Copy one 128-byte-wide K slab of 256 rows of one operand into LDS.  Wave w
// fills rows [64 w, 64 w + 64) with 8 instructions of 1 KiB (8 rows) each;
// lane p writes LDS slot p & 7 of row p >> 3 of its 8, which holds chunk
// (p & 7) ^ f(row) -- an XOR, so reads find chunk kc at kc ^ f(row).  The 8
// lanes of a row read its 128 bytes: one full cache line.  Buffer loads take
// the operand base from a descriptor, the lane's row offset from a 32-bit
// register and the slab's K offset from a scalar register.
__device__ __forceinline__ void load_slab(__amdgpu_buffer_rsrc_t src, const uint32_t (&off)[kLoadsPerSlab],
                                          uint32_t k_bytes, char* lds_slab, int w) {
#pragma unroll
  for (int i = 0; i < kLoadsPerSlab; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)(lds_slab + (w * 8 + i) * 1024), 16, off[i], k_bytes,
                                             0, 0);
}

// State of the K loop of one wave.
struct Ring {
  __amdgpu_buffer_rsrc_t a_src;
  __amdgpu_buffer_rsrc_t b_src;
  char* lds;
  int sa, sb;        // ring slots of the slab being multiplied
  int w;
};

// Fragment r (0..7) of step S: A subtile r for r < 4, else B subtile r - 4.
template <int S, int R>
__device__ __forceinline__ void read_frag(const char* As, const char* Bs, const int (&ro)[4], int wm, int wn,
                                          Frags& f) {
  constexpr int i = R & 3;
  constexpr int k = S ^ (2 * (i & 1));
  if (R < 4) f.a[i] = *reinterpret_cast<const f32x4_t*>(As + (wm * 128 + i * 32) * kRowBytes + ro[k]);
  else f.b[i] = *reinterpret_cast<const f32x4_t*>(Bs + (wn * 128 + i * 32) * kRowBytes + ro[k]);
}

// Slab copies of one iteration: copy q < 8 is row group q of the Wt slab,
// q >= 8 row group q - 8 of the H slab.
struct Copies {
  __amdgpu_buffer_rsrc_t a_src, b_src;
  char* a_dst;
  char* b_dst;
  uint32_t a_k, b_k;
};

template <int Q>
__device__ __forceinline__ void issue_copy(const Copies& c, const uint32_t (&a_off)[kLoadsPerSlab],
                                           const uint32_t (&b_off)[kLoadsPerSlab], int w) {
  // The activations are read once per tile column and stream through, so
  // their copies are non-temporal (aux = 2): measured on the c = 128 key
  // compressor, whose panels feed only 2 tile columns, 8% faster; the same or
  // slightly faster for CSA (c = 512) and HCA.  The weights, re-read by every
  // panel, keep the default policy.
  if (Q < 8)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.b_src, (lds_void_t*)(c.b_dst + (w * 8 + Q) * 1024), 16, b_off[Q & 7],
                                             c.b_k, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.a_src, (lds_void_t*)(c.a_dst + (w * 8 + (Q & 7)) * 1024), 16,
                                             a_off[Q & 7], c.a_k, 0, 2);
}

// One step: the 16 MFMAs over fragments `cur` (M subtile outer, N inner),
// with the 8 reads of the next step's fragments (in the order that step
// consumes them: a0 b0 b1 b2 b3 a1 a2 a3) issued after the MFMAs whose bit is
// set in RMASK, and slab copies Q0, Q0 + 1, ... after those set in CMASK.  A
// copy occupies the issuing wave for ~16 cycles (64 lanes x 16 bytes through
// the address unit), so copies and reads go into different MFMA shadows.
__host__ __device__ constexpr int popc16(int x) {
  return ((x >> 0) & 1) + ((x >> 1) & 1) + ((x >> 2) & 1) + ((x >> 3) & 1) + ((x >> 4) & 1) + ((x >> 5) & 1) +
         ((x >> 6) & 1) + ((x >> 7) & 1) + ((x >> 8) & 1) + ((x >> 9) & 1) + ((x >> 10) & 1) + ((x >> 11) & 1) +
         ((x >> 12) & 1) + ((x >> 13) & 1) + ((x >> 14) & 1) + ((x >> 15) & 1);
}

template <int DIN, int SN, int RMASK, int Q0, int CMASK>
__device__ __forceinline__ void step(const Frags& cur, Frags& nxt, WaveAcc& acc, const char* As, const char* Bs,
                                     const int (&ro)[4], int wm, int wn, const Copies& cp,
                                     const uint32_t (&a_off)[kLoadsPerSlab], const uint32_t (&b_off)[kLoadsPerSlab],
                                     int w) {
  static_assert(RMASK == 0 || popc16(RMASK) == 8, "a step reads 8 fragments");
  constexpr int kOrder[8] = {0, 4, 5, 6, 7, 1, 2, 3};
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    Frag<DIN>::mma1(cur, acc, q >> 2, q & 3);
    if ((RMASK >> q) & 1) {
      switch (popc16(RMASK & ((1 << q) - 1))) {
        case 0: read_frag<SN, kOrder[0]>(As, Bs, ro, wm, wn, nxt); break;
        case 1: read_frag<SN, kOrder[1]>(As, Bs, ro, wm, wn, nxt); break;
        case 2: read_frag<SN, kOrder[2]>(As, Bs, ro, wm, wn, nxt); break;
        case 3: read_frag<SN, kOrder[3]>(As, Bs, ro, wm, wn, nxt); break;
        case 4: read_frag<SN, kOrder[4]>(As, Bs, ro, wm, wn, nxt); break;
        case 5: read_frag<SN, kOrder[5]>(As, Bs, ro, wm, wn, nxt); break;
        case 6: read_frag<SN, kOrder[6]>(As, Bs, ro, wm, wn, nxt); break;
        default: read_frag<SN, kOrder[7]>(As, Bs, ro, wm, wn, nxt); break;
      }
    }
    if ((CMASK >> q) & 1) {
      switch (Q0 + popc16(CMASK & ((1 << q) - 1))) {
#define SEQCOMP_COPY_CASE(n) \
  case n:                    \
    issue_copy<n>(cp, a_off, b_off, w); \
    break;
        SEQCOMP_COPY_CASE(0) SEQCOMP_COPY_CASE(1) SEQCOMP_COPY_CASE(2) SEQCOMP_COPY_CASE(3)
        SEQCOMP_COPY_CASE(4) SEQCOMP_COPY_CASE(5) SEQCOMP_COPY_CASE(6) SEQCOMP_COPY_CASE(7)
        SEQCOMP_COPY_CASE(8) SEQCOMP_COPY_CASE(9) SEQCOMP_COPY_CASE(10) SEQCOMP_COPY_CASE(11)
        SEQCOMP_COPY_CASE(12) SEQCOMP_COPY_CASE(13) SEQCOMP_COPY_CASE(14)
        default: issue_copy<15>(cp, a_off, b_off, w); break;
#undef SEQCOMP_COPY_CASE
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// MFMA slots of the fragment reads and of the 4 copies of a step.
constexpr int kReadSlots = 0x00ff;    // after MFMAs 0..7
constexpr int kCopySlots = 0x5500;    // after MFMAs 8, 10, 12, 14

// One K slab j.  Slab j - 1 was finished by every wave before the barrier
// that opened this iteration, so its slots take the copies of H slab j + 2
// (3-slot ring) and Wt slab j + 1 (2-slot ring).  Per-wave copy order is
// ... A(j+1) B(j+1) A(j+2)[0..3] | barrier | A(j+2)[4..7]: before the barrier
// vmcnt(4) (the 4 copies of step 2 left open) means A(j+1) and B(j+1) have
// landed.
//   step 0 MFMAs | reads of step 1, then Wt copies 0-3, in between
//   step 1 MFMAs | reads of step 2, then Wt copies 4-7, in between
//   step 2 MFMAs | reads of step 3, then H copies 0-3, in between
//   wait copies + own reads | barrier
//   step 3 MFMAs | reads of step 0 of slab j + 1, then H copies 4-7, in between
// The H copies issued after the barrier go to the slot of slab j - 1 too,
// which every wave had finished before this iteration began.
template <int DIN, bool ISSUE_B, bool ISSUE_A, bool LAST>
__device__ __forceinline__ void k_iter(Ring& R, int j, const uint32_t (&a_off)[kLoadsPerSlab],
                                       const uint32_t (&b_off)[kLoadsPerSlab], const int (&ro)[4], int wm, int wn,
                                       Frags& f0, Frags& f1, WaveAcc& acc) {
  const char* As = R.lds + R.sa * kSlabBytes;
  const char* Bs = R.lds + kLdsB + R.sb * kSlabBytes;
  Copies cp;
  cp.a_src = R.a_src;
  cp.b_src = R.b_src;
  cp.b_dst = R.lds + kLdsB + (R.sb ^ 1) * kSlabBytes;
  cp.a_dst = R.lds + (R.sa == 0 ? kStagesA - 1 : R.sa - 1) * kSlabBytes;
  cp.b_k = (uint32_t)(j + 1) * kRowBytes;
  cp.a_k = (uint32_t)(j + 2) * kRowBytes;
  // Wt copies (needed at the end of this iteration) in steps 0 and 1, H
  // copies (needed at the end of the next one) in steps 2 and 3.
  constexpr int CB = ISSUE_B ? kCopySlots : 0;
  constexpr int CA = ISSUE_A ? kCopySlots : 0;
  constexpr int NA = popc16(CA);                    // H copies issued before the barrier
  __builtin_amdgcn_sched_barrier(0);
  step<DIN, 1, kReadSlots, 0, CB>(f0, f1, acc, As, Bs, ro, wm, wn, cp, a_off, b_off, R.w);
  step<DIN, 2, kReadSlots, popc16(CB), CB>(f1, f0, acc, As, Bs, ro, wm, wn, cp, a_off, b_off, R.w);
  step<DIN, 3, kReadSlots, 8, CA>(f0, f1, acc, As, Bs, ro, wm, wn, cp, a_off, b_off, R.w);
  if (!LAST) {
    wait_vmcnt_lgkm0<NA>();                         // A(j+1), B(j+1) landed; the step-2 H copies may be open
    lds_barrier();
    R.sa = R.sa == kStagesA - 1 ? 0 : R.sa + 1;
    R.sb ^= 1;
    step<DIN, 0, kReadSlots, 8 + NA, CA>(f1, f0, acc, R.lds + R.sa * kSlabBytes, R.lds + kLdsB + R.sb * kSlabBytes,
                                         ro, wm, wn, cp, a_off, b_off, R.w);
  } else {
    wait_lgkmcnt0();   // every wave is done with the ring before the epilogue reuses the LDS
    lds_barrier();
    step<DIN, 0, 0, 0, 0>(f1, f0, acc, As, Bs, ro, wm, wn, cp, a_off, b_off, R.w);
  }
}

template <int DIN>
__device__ __forceinline__ void mainloop(const char* a_base, const uint32_t (&a_off)[kLoadsPerSlab],
                                         const char* b_base, const uint32_t (&b_off)[kLoadsPerSlab], int nk,
                                         char* lds, int w, int lane, int wm, int wn, WaveAcc& acc) {
  const __amdgpu_buffer_rsrc_t a_src = raw_rsrc(a_base), b_src = raw_rsrc(b_base);
  int ro[4];
  {
    const int h = lane >> 5;
    const int x0 = (lane & 7) ^ ((lane >> 3) & 3);
#pragma unroll
    for (int k = 0; k < 4; ++k) ro[k] = (lane & 31) * kRowBytes + ((16 * (h ^ x0)) ^ (32 * k));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  Ring R{a_src, b_src, lds, 0, 0, w};
  load_slab(a_src, a_off, 0, lds, w);
  load_slab(b_src, b_off, 0, lds + kLdsB, w);
  if (nk > 1) {
    load_slab(a_src, a_off, kRowBytes, lds + kSlabBytes, w);
    wait_vmcnt<kLoadsPerSlab>();                    // A(0), B(0) landed; A(1) in flight
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  Frags f0, f1;
  read_frags<0>(lds, lds + kLdsB, ro, wm, wn, f0);
  int j = 0;
  for (; j + 2 < nk; ++j) k_iter<DIN, true, true, false>(R, j, a_off, b_off, ro, wm, wn, f0, f1, acc);
  if (j + 1 < nk) {
    k_iter<DIN, true, false, false>(R, j, a_off, b_off, ro, wm, wn, f0, f1, acc);
    ++j;
  }
  k_iter<DIN, false, false, true>(R, j, a_off, b_off, ro, wm, wn, f0, f1, acc);
}

// Per-thread source rows of the two operands: thread (wave w, lane p) loads
// tile rows r_i = 64 w + 8 i + (p >> 3), i = 0..7, at chunk (p & 7) ^ f(r_i).
template <int MODE>
__device__ __forceinline__ int b_row_of(int n, int nt, int c, int n_out) {
  if (MODE == MODE_PROJECT) return min(nt * kTile + n, n_out - 1);
  const int half = n >> 7;                 // which wave column
  if (MODE == MODE_CSA || MODE == MODE_CSA_APPEND) {   // 4 streams x 32 channels per wave column
    const int s = (n & 127) >> 5, j = n & 31;
    const int ch = nt * 64 + half * 32 + j;
    return s * c + min(ch, c - 1);
  } else {                                 // 2 streams x 64 channels per wave column
    const int s = (n & 127) >> 6, j = n & 63;
    const int ch = nt * 128 + half * 64 + j;
    return s * c + min(ch, c - 1);
  }
}

// Softmax partial of the 4 rows of run q (elements 4 q .. 4 q + 3) of one
// accumulator: logits z + B in log2 units (bias2 = log2(e) * B), values v.
__device__ __forceinline__ SoftAcc partial_rows4(const float (&z)[4], const float (&v)[4], const float (&bias2)[4]) {
  float l[4];
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    l[j] = fmaf(z[j], kLog2e, bias2[j]);
    M = fmaxf(M, l[j]);
  }
  SoftAcc s;
  s.M = M;
  s.S = 0.f;
  s.A = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float w = exp2_hw(l[j] - M);
    s.S += w;
    s.A = fmaf(w, v[j], s.A);
  }
  return s;
}
__device__ __forceinline__ SoftAcc partial4(const f32x16_t& z, const f32x16_t& v, int q, const float (&bias2)[4]) {
  const float zq[4] = {z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]};
  const float vq[4] = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
  return partial_rows4(zq, vq, bias2);
}

// The partial of lane l ^ 32 (the other lane half, same column), through the
// gfx950 half-swap: v_permlane32_swap(v, v) leaves lanes 0..31 of its second
// result holding v of lanes 32..63 and lanes 32..63 of its first result
// holding v of lanes 0..31 -- no LDS round trip.
__device__ __forceinline__ float xor32(float v, bool upper) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(upper ? r[0] : r[1]);
}

__device__ __forceinline__ SoftAcc xor32_acc(const SoftAcc& s, bool upper) {
  return SoftAcc{xor32(s.M, upper), xor32(s.S, upper), xor32(s.A, upper)};
}

template <int DOUT>
__device__ __forceinline__ void store1(char* out, int64_t idx, float v) {
  if (DOUT == DT_BF16) reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits(v);
  else reinterpret_cast<float*>(out)[idx] = v;
}

// Projection epilogue: every accumulator element goes straight to Y through
// a buffer descriptor over the tile's rows; rows past T fall outside the
// descriptor's range and columns past n_out get an offset outside it, so the
// hardware drops those stores and no branch splits the epilogue (branches
// would let the compiler copy all 256 accumulators to VGPRs at once).
template <int DOUT>
__device__ void epilogue_project(const Args& a, WaveAcc& acc, int mt, int nt, int lane, int wm, int wn) {
  constexpr int es = DOUT == DT_BF16 ? 2 : 4;
  const int64_t row0 = (int64_t)mt * kTile;
  const int64_t rows = min<int64_t>(kTile, a.T - row0);
  const uint32_t range = (uint32_t)(rows * a.ld_y * es);   // < 2^31: checked by the host
  const __amdgpu_buffer_rsrc_t dst =
      __builtin_amdgcn_make_buffer_rsrc(a.Y + row0 * a.ld_y * es, (short)0, (int)range, 0x00020000);
  const int col = lane & 31, h = lane >> 5;
  const uint32_t ld_bytes = (uint32_t)(a.ld_y * es);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nt * kTile + wn * 128 + j * 32 + col;
      // 2^31 + (row offset < 2^31: checked by the host) is past the range
      const uint32_t cbase = n < a.n_out ? (uint32_t)n * es : 0x80000000u;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t r = wm * 128 + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        const uint32_t off = r * ld_bytes + cbase;
        if (DOUT == DT_BF16) {
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_bits(acc[i][j][e]), dst, off, 0, 0);
        } else {
          // Pass the element through a VGPR: folding the accumulator register
          // straight into the store's data operand stored element 0 sixteen
          // times with this compiler.
          float v = acc[i][j][e];
          asm volatile("" : "+v"(v));
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), dst, off, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // bounds the accumulator values held in VGPRs
  }
}

// CSA epilogue.  Wave (wm, wn), lane (h = lane / 32, col = lane % 32):
// accumulator [ms][s] holds stream s (C^a, C^b, Z^a, Z^b) at channel
// 64 nt + 32 wn + col; its run q covers rows 128 wm + 32 ms + 8 q + 4 h + 0..3,
// i.e. block (entry) 32 wm + 8 ms + 2 q + h of the tile.
// B^a / B^b of the lane's channel, log2(e)-scaled; loaded before the K loop
// so their latency hides behind it.
__device__ __forceinline__ void csa_bias(const Args& a, int nt, int lane, int wn, float (&ba)[4], float (&bb)[4]) {
  const int ch = nt * 64 + wn * 32 + (lane & 31);
  const bool ok = ch < a.c;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ba[r] = ok ? a.Ba[r * a.c + ch] * kLog2e : 0.f;
    bb[r] = ok ? a.Bb[r * a.c + ch] * kLog2e : 0.f;
  }
}

template <int DOUT>
__device__ void epilogue_csa(const Args& a, WaveAcc& acc, const TileRec& t, int tile, int nt, int lane, int wm,
                             int wn, char* lds, const float (&ba)[4], const float (&bb)[4]) {
  const int col = lane & 31, h = lane >> 5;
  const int c = a.c;
  const int ch = nt * 64 + wn * 32 + col;
  const bool ok = ch < c;
  float* xfer = reinterpret_cast<float*>(lds);       // [wn][col][3]: wave row 0 -> wave row 1
  float* halo = a.halo + (int64_t)tile * 6 * c;       // [Ma Sa Aa Mb Sb Ab] x c
  // b-partial of each wave row's last block (ms 3, run 3, lanes h = 1).
  {
    const SoftAcc pb = partial4(acc[3][3], acc[3][1], 3, bb);
    if (h == 1 && wm == 0) {
      float* x = xfer + (wn * 32 + col) * 3;
      x[0] = pb.M;
      x[1] = pb.S;
      x[2] = pb.A;
    }
    if (h == 1 && wm == 1 && t.n_rows == kTile && ok) {   // the next tile continues the sequence
      halo[3 * c + ch] = pb.M;
      halo[4 * c + ch] = pb.S;
      halo[5 * c + ch] = pb.A;
    }
  }
  __syncthreads();
  SoftAcc carry;                                      // b-partial of the block before (run q, h = 0)
  softacc_init(carry);
  if (wm == 1) {
    const float* x = xfer + (wn * 32 + col) * 3;
    carry.M = x[0];
    carry.S = x[1];
    carry.A = x[2];
  }
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const SoftAcc pa = partial4(acc[ms][2], acc[ms][0], q, ba);
      const SoftAcc pb = partial4(acc[ms][3], acc[ms][1], q, bb);
      // Lane l ^ 32 holds the other half of this run pair: for h = 1 it is
      // the previous block (h = 0, same q); for h = 0 it is run (q, h = 1),
      // the previous block of run (q + 1, h = 0) -- carried to the next step.
      const SoftAcc px = xor32_acc(pb, h != 0);
      const SoftAcc prev = h ? px : carry;
      carry = px;
      const int blk = wm * 32 + ms * 8 + q * 2 + h;  // block (= entry) index inside the tile
      // The tile's block 0 has no b-partial here (lane h = 0 of wave row 0
      // carries the empty partial), so the merge returns its a-partial: the
      // whole entry when the tile starts its sequence (eq.
      // attn-seqcomp-overlap-bound), else the halo's a-part.  Only the stores
      // are predicated, so the arithmetic stays in one basic block.
      const SoftAcc m = softacc_merge(pa, prev);
      const bool first = (ms == 0 && q == 0) && blk == 0;
      const bool tile_first = (t.flags & TILE_FIRST) != 0;
      if (ok && blk * 4 < t.n_rows && (!first || tile_first))
        store1<DOUT>(a.out, ((int64_t)t.entry_start + blk) * c + ch, m.A / m.S);
      if (ms == 0 && q == 0) {
        if (ok && first && !tile_first) {
          halo[0 * c + ch] = pa.M;
          halo[1 * c + ch] = pa.S;
          halo[2 * c + ch] = pa.A;
        }
      }
    }
    // Keep the accumulator reads of the next subtile row after this one:
    // hoisted all at once they would need 256 VGPRs and spill.
    __builtin_amdgcn_sched_barrier(0);
  }
}

// CSA append epilogue (decode): the tile's rows are 64 independent blocks of
// m = 4 tokens, block j being the newest block of its own sequence.  Its
// entry merges the block's a-partial with the b-partial of the sequence's
// previous block, which the caller carries from the previous append in
// state_in (M = -inf, S = A = 0 for a sequence's first block: the entry-0
// rule of eq. attn-seqcomp-overlap-bound); the block's own b-partial becomes
// the state for its successor.  Same accumulator layout as epilogue_csa: run
// q of lane half h is block 32 wm + 8 ms + 2 q + h of the tile.
// One append entry: block j's a-partial merged with its previous block's
// b-partial gives the entry; block j's own b-partial becomes the new state.
template <int DOUT>
__device__ __forceinline__ void append_store(const Args& a, const SoftAcc& pa, const SoftAcc& pb, const SoftAcc& prev,
                                             int64_t j, bool ok, int ch) {
  const SoftAcc m = softacc_merge(pa, prev);
  if (ok && j < a.nb) {
    store1<DOUT>(a.out, j * a.c + ch, m.A / m.S);
    float* so = a.state_out + j * 3 * a.c + ch;
    so[0] = pb.M;
    so[a.c] = pb.S;
    so[2 * a.c] = pb.A;
  }
}

template <int DOUT>
__device__ void epilogue_csa_append(const Args& a, WaveAcc& acc, int mt, int nt, int lane, int wm, int wn,
                                    const float (&ba)[4], const float (&bb)[4]) {
  const int col = lane & 31, h = lane >> 5;
  const int c = a.c;
  const int ch = nt * 64 + wn * 32 + col;
  const bool ok = ch < c;
  const int64_t j0 = (int64_t)mt * 64;
  // the 16 previous-block partials this lane merges, loaded up front
  SoftAcc prev[16];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t j = min(j0 + wm * 32 + ms * 8 + q * 2 + h, a.nb - 1);
      const float* st = a.state_in + j * 3 * c + min(ch, c - 1);
      prev[ms * 4 + q] = SoftAcc{st[0], st[c], st[2 * c]};
    }
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const SoftAcc pa = partial4(acc[ms][2], acc[ms][0], q, ba);
      const SoftAcc pb = partial4(acc[ms][3], acc[ms][1], q, bb);
      append_store<DOUT>(a, pa, pb, prev[ms * 4 + q], j0 + wm * 32 + ms * 8 + q * 2 + h, ok, ch);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// HCA epilogue (m' = 128): wave row wm is block wm of the tile; accumulator
// [ms][qq] holds C and [ms][2 + qq] holds Z at channel 128 nt + 64 wn + 32 qq + col.
// The tile's bias slice B[0:128][128 nt : 128 nt + 128] is first staged in
// LDS (log2(e)-scaled, 64 KiB, coalesced 16-byte loads by the whole
// workgroup); the K loop is done with the LDS ring at this point.
template <int DOUT>
__device__ void epilogue_hca(const Args& a, WaveAcc& acc, const TileRec& t, int nt, int tid, int wm, int wn,
                             char* lds) {
  const int lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int c = a.c;
  float* sb = reinterpret_cast<float*>(lds);          // [128 rows][128 channels]
  {
    // 16 independent 16-byte loads per thread, all in flight before the stores.
    float4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = tid + k * kThreads;
      const int r = i >> 5, c4 = (i & 31) * 4;
      const int ch = min(nt * 128 + c4, c - 4);     // c % 16 == 0: in bounds; columns past c unused
      v[k] = *reinterpret_cast<const float4*>(a.Ba + (int64_t)r * c + ch);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = tid + k * kThreads;
      const int r = i >> 5, c4 = (i & 31) * 4;
      *reinterpret_cast<float4*>(sb + r * 128 + c4) =
          make_float4(v[k].x * kLog2e, v[k].y * kLog2e, v[k].z * kLog2e, v[k].w * kLog2e);
    }
  }
  __syncthreads();
  const bool block_ok = (wm + 1) * 128 <= t.n_rows;
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int cl = wn * 64 + qq * 32 + col;            // channel within the tile's slice
    const int ch = nt * 128 + cl;
    const bool ok = ch < c;
    SoftAcc s;
    softacc_init(s);
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = sb[(ms * 32 + q * 8 + h * 4 + r) * 128 + cl];
        s = softacc_merge(s, partial4(acc[ms][2 + qq], acc[ms][qq], q, b));
      }
    }
    s = softacc_merge(s, xor32_acc(s, h != 0));
    if (ok && block_ok && h == 0) store1<DOUT>(a.out, ((int64_t)t.entry_start + wm) * c + ch, s.A / s.S);
  }
}

// One logical tile.  The thread index is passed through an empty asm
// statement so the compiler cannot hoist lane-derived values out of the
// persistent loop (they would stay live across the K loop and crowd out the
// accumulators).  LOOKUP: the tile record comes from the sequence offsets,
// not from the planner's table (a separate instantiation, so the kernels
// that read the table are built exactly as without it).
template <int DIN, int MODE, int DOUT, bool LOOKUP>
__device__ __forceinline__ void run_tile(const Args& a, int L, char* lds) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int mt = L / a.n_nt, nt = L - mt * a.n_nt;
  const int wm = w >> 1, wn = w & 1;

  int64_t row0;
  int nvalid;
  TileRec t{};
  if (MODE == MODE_PROJECT || MODE == MODE_CSA_APPEND) {
    row0 = (int64_t)mt * kTile;
    nvalid = (int)min<int64_t>(kTile, a.T - row0);
  } else {
    t = LOOKUP ? tile_lookup(a.cu, a.batch, a.m, kTile, mt) : a.tiles[mt];
    row0 = t.row_start;
    nvalid = t.n_rows;
  }
  // Byte offsets from uniform bases; they fit 32 bits because a tile of H is
  // 256 rows of at most 64 KiB and the host rejects a Wt of 4 GiB or more.
  const char* a_base = a.H + row0 * a.lda;
  uint32_t a_off[kLoadsPerSlab], b_off[kLoadsPerSlab];
#pragma unroll
  for (int i = 0; i < kLoadsPerSlab; ++i) {
    const int r = w * 64 + i * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ swz_f(r);
    a_off[i] = (uint32_t)(min(r, nvalid - 1) * a.lda + kc * 16);
    b_off[i] = (uint32_t)((int64_t)b_row_of<MODE>(r, nt, a.c, a.n_out) * a.lda + kc * 16);
  }
  float ba[4] = {0.f, 0.f, 0.f, 0.f}, bb[4] = {0.f, 0.f, 0.f, 0.f};
  if (MODE == MODE_CSA || MODE == MODE_CSA_APPEND) csa_bias(a, nt, lane, wn, ba, bb);
  WaveAcc acc;
  mainloop<DIN>(a_base, a_off, a.Wt, b_off, a.nk, lds, w, lane, wm, wn, acc);
  if (MODE == MODE_PROJECT) epilogue_project<DOUT>(a, acc, mt, nt, lane, wm, wn);
  else if (MODE == MODE_CSA) epilogue_csa<DOUT>(a, acc, t, mt, nt, lane, wm, wn, lds, ba, bb);
  else if (MODE == MODE_CSA_APPEND) epilogue_csa_append<DOUT>(a, acc, mt, nt, lane, wm, wn, ba, bb);
  else epilogue_hca<DOUT>(a, acc, t, nt, tid, wm, wn, lds);
}

// Persistent grid: one workgroup per CU walks rounds of gridDim.x logical
// tiles.  In every round each XCD owns one contiguous range of logical tiles
// (N fastest), so the workgroups that share an M panel of H start it
// together and advance through K in step: their H slabs hit in the XCD's L2.
template <int DIN, int MODE, int DOUT, bool LOOKUP = false>
__global__ __launch_bounds__(kThreads, 1) void tile_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int G = a.n_mt * a.n_nt;
  const int P = gridDim.x;
  for (int L = xcd_remap(blockIdx.x, P); L < G; L += P) {
    run_tile<DIN, MODE, DOUT, LOOKUP>(a, L, lds);
    __syncthreads();   // the epilogue's LDS use ends before the next tile's loads
  }
}

// First entry of every tile that continues a sequence: merge the tile's
// first-block a-partial with the previous tile's last-block b-partial.
template <int DOUT>
__global__ __launch_bounds__(256) void csa_fixup_kernel(const TileRec* __restrict__ tiles, const int64_t* __restrict__ cu,
                                                        int batch, int c, const float* __restrict__ halo,
                                                        char* __restrict__ out) {
  const int tile = blockIdx.x;
  const TileRec t = tiles ? tiles[tile] : tile_lookup(cu, batch, 4, kTile, tile);
  if (t.flags & TILE_FIRST) return;
  const float* ha = halo + (int64_t)tile * 6 * c;
  const float* hb = halo + (int64_t)(tile - 1) * 6 * c;
  for (int ch = threadIdx.x; ch < c; ch += blockDim.x) {
    SoftAcc pa, pb;
    pa.M = ha[ch];
    pa.S = ha[c + ch];
    pa.A = ha[2 * c + ch];
    pb.M = hb[3 * c + ch];
    pb.S = hb[4 * c + ch];
    pb.A = hb[5 * c + ch];
    const SoftAcc m = softacc_merge(pa, pb);
    store1<DOUT>(reinterpret_cast<char*>(out), (int64_t)t.entry_start * c + ch, m.A / m.S);
  }
}

// Split-K form of the big-tile CSA append, for mid-size batches whose
// 256 x 256 tiles fill a quarter to all but one of 256 workgroups (1024
// blocks are 16 x 8 tiles).  Workgroup (L, s) multiplies K slabs
// [s nk / S, (s + 1) nk / S) of logical tile L and stores its accumulators as
// they sit in registers; append_reduce_kernel adds the S partials of one
// wave's 32-row M subtile and runs the append epilogue on the sum.  Partial
// layout, in float4: [L][s][wave][ms][N subtile][element quad][lane], so
// every store and load is one coalesced 1 KiB row.
constexpr int kPartialQuads = 4 * 4 * 64;      // float4 per (L, s, wave, ms) block: 16 KiB

__device__ __forceinline__ int64_t partial_base(int64_t L, int S, int s, int w, int ms) {
  return (((L * S + s) * 4 + w) * 4 + ms) * kPartialQuads;
}

template <int DIN>
__global__ __launch_bounds__(kThreads, 1) void append_splitk_kernel(Args a, int S, float4* __restrict__ partial) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int L = blockIdx.x / S, sp = blockIdx.x - L * S;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int mt = L / a.n_nt, nt = L - mt * a.n_nt;
  const int wm = w >> 1, wn = w & 1;
  const int64_t row0 = (int64_t)mt * kTile;
  const int nvalid = (int)min<int64_t>(kTile, a.T - row0);
  const int k0 = (int)((int64_t)sp * a.nk / S), k1 = (int)((int64_t)(sp + 1) * a.nk / S);   // S <= nk: k1 > k0
  uint32_t a_off[kLoadsPerSlab], b_off[kLoadsPerSlab];
#pragma unroll
  for (int i = 0; i < kLoadsPerSlab; ++i) {
    const int r = w * 64 + i * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ swz_f(r);
    a_off[i] = (uint32_t)(min(r, nvalid - 1) * a.lda + kc * 16);
    b_off[i] = (uint32_t)((int64_t)b_row_of<MODE_CSA_APPEND>(r, nt, a.c, a.n_out) * a.lda + kc * 16);
  }
  WaveAcc acc;
  mainloop<DIN>(a.H + row0 * a.lda + (int64_t)k0 * kRowBytes, a_off, a.Wt + (int64_t)k0 * kRowBytes, b_off, k1 - k0,
                lds, w, lane, wm, wn, acc);
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    float4* dst = partial + partial_base(L, S, sp, w, ms) + lane;
#pragma unroll
    for (int jn = 0; jn < 4; ++jn)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // each element through a VGPR: a store fed straight from an
        // accumulator register has been miscompiled (see epilogue_project)
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[ms][jn][4 * q4 + e];
          asm volatile("" : "+v"(v[e]));
        }
        dst[(jn * 4 + q4) * 64] = make_float4(v[0], v[1], v[2], v[3]);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Workgroup = one wave: (tile L, wave w, M subtile ms).  Four splits' loads
// are in flight at a time; the sum runs in split order, so it is the same on
// every call.
// Adds the U >= S splits' partials of one (tile, wave, row block) in split
// order, every load issued before the first add (splits past S load split
// S - 1 again and add nothing).
template <int U>
__device__ __forceinline__ void sum_big_partials(const float4* __restrict__ partial, int64_t L, int S, int w, int ms,
                                                 int lane, f32x16_t (&acc)[4]) {
  float4 v[U][16];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float4* src = partial + partial_base(L, S, min(u, S - 1), w, ms) + lane;
#pragma unroll
    for (int k = 0; k < 16; ++k) v[u][k] = src[k * 64];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool in = u < S;
#pragma unroll
    for (int jn = 0; jn < 4; ++jn)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = v[u][jn * 4 + q4];
        acc[jn][4 * q4 + 0] += in ? x.x : 0.f;
        acc[jn][4 * q4 + 1] += in ? x.y : 0.f;
        acc[jn][4 * q4 + 2] += in ? x.z : 0.f;
        acc[jn][4 * q4 + 3] += in ? x.w : 0.f;
      }
  }
}

// Reduce of the big-tile split-K (S <= 4 splits): one wave per (tile, wave
// of the tile, row block of 8 blocks); the epilogue inputs are loaded before
// the partials.
template <int DOUT>
__global__ __launch_bounds__(64) void append_reduce_kernel(Args a, int S, const float4* __restrict__ partial) {
  const int L = blockIdx.x >> 4, w = (blockIdx.x >> 2) & 3, ms = blockIdx.x & 3;
  const int lane = threadIdx.x;
  const int mt = L / a.n_nt, nt = L - mt * a.n_nt;
  const int wm = w >> 1, wn = w & 1;
  const int col = lane & 31, h = lane >> 5;
  const int ch = nt * 64 + wn * 32 + col;
  const bool ok = ch < a.c;
  const int chc = min(ch, a.c - 1);
  const int64_t j0 = (int64_t)mt * 64 + wm * 32 + ms * 8 + h;
  float ba[4], bb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ba[r] = a.Ba[r * a.c + chc];   // scaled by log2(e) after the sums
    bb[r] = a.Bb[r * a.c + chc];
  }
  SoftAcc prev[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t j = min(j0 + q * 2, a.nb - 1);
    const float* st = a.state_in + j * 3 * a.c + chc;
    prev[q] = SoftAcc{st[0], st[a.c], st[2 * a.c]};
  }
  f32x16_t acc[4];
#pragma unroll
  for (int jn = 0; jn < 4; ++jn) acc[jn] = f32x16_t{};
  if (S <= 2)
    sum_big_partials<2>(partial, L, S, w, ms, lane, acc);
  else
    sum_big_partials<4>(partial, L, S, w, ms, lane, acc);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ba[r] = ok ? ba[r] * kLog2e : 0.f;
    bb[r] = ok ? bb[r] * kLog2e : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const SoftAcc pa = partial4(acc[2], acc[0], q, ba);
    const SoftAcc pb = partial4(acc[3], acc[1], q, bb);
    append_store<DOUT>(a, pa, pb, prev[q], j0 + q * 2, ok, ch);
  }
}

// Decode append for batches too small to fill the chip with 256 x 256 tiles.
// A narrower tile of 128 rows (32 blocks) x 128 columns (32 channels x the 4
// streams C^a | C^b | Z^a | Z^b) is split over K when even those tiles are
// too few.  The fp32 partial products of a call take 4 bytes x tile area x
// splits per tile, and the splits that fill 256 workgroups fall as the tile
// grows, so the bytes grow with the tile area: 16 MiB at 64 blocks with
// these tiles against 32 MiB (at half the workgroups) with 256 x 256 ones.
// Eight waves, two per SIMD: wave w holds rows [32 (w % 4), 32 (w % 4) + 32)
// of the tile and all four streams of the tile's 32 channels (one 32 x 32
// accumulator per stream, so its lanes see whole blocks of every stream, the
// layout of the fused epilogue), over the even (w < 4) or odd (w >= 4)
// k-steps of every slab; the odd half is added to the even one through LDS
// at the end.  With two waves per SIMD each hides the other's LDS and
// barrier waits, which a slab of only 512 MFMA cycles per SIMD exposes.  K
// advances in the 128-byte slabs of the big kernel, copied global -> LDS
// through a 4-stage ring three slabs ahead.
constexpr int kSkThreads = 512;
constexpr int kSkTile = 128;                           // tile rows and columns
constexpr int kSkSlab = kSkTile * kRowBytes;           // 16 KiB: one operand's slab
constexpr int kSkStages = 4;
constexpr int kSkLdsBytes = kSkStages * 2 * kSkSlab;   // 128 KiB
constexpr int kSkLoads = kSkTile / 8 / 8;              // copies per wave and operand slab (8 rows each): 2
constexpr int kAppendMaxSplits = 32;
constexpr int kAppendWorkgroups = 256;                 // workgroups to aim for: one per CU of an MI355X
constexpr int kSkPartialQuads = 4 * 4 * 64;            // float4 per (tile, split, row block): 16 KiB

// Tiles of the two append forms.
__host__ __device__ inline int64_t big_append_tiles(int64_t nb, int c) {
  return ((4 * nb + kTile - 1) / kTile) * ((c + 63) / 64);
}
__host__ __device__ inline int64_t skinny_append_tiles(int64_t nb, int c) {
  return ((4 * nb + kSkTile - 1) / kSkTile) * ((c + 31) / 32);
}

template <int DIN>
__device__ __forceinline__ void sk_mma(const f32x4_t& a, const f32x4_t& b, f32x16_t& acc) {
  if (DIN == DT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
  } else {
    // chunk 2 s + h holds fp32 k = 8 s + 4 h + t; the same permutation of k on
    // both operands leaves the dot products unchanged
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc, 0, 0, 0);
  }
}

// Copy K slab `slab` of both operands into ring stage `stage`: wave w fills
// rows [16 w, 16 w + 16) of each with 2 copies of 8 rows (1 KiB).
__device__ __forceinline__ void sk_copy(__amdgpu_buffer_rsrc_t a_src, __amdgpu_buffer_rsrc_t b_src,
                                        const uint32_t (&a_off)[kSkLoads], const uint32_t (&b_off)[kSkLoads],
                                        char* lds, int stage, int slab, int w) {
  char* as = lds + stage * 2 * kSkSlab;
  char* bs = as + kSkSlab;
  const uint32_t k = (uint32_t)slab * kRowBytes;
#pragma unroll
  for (int i = 0; i < kSkLoads; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_src, (lds_void_t*)(as + (w * kSkLoads + i) * 1024), 16, a_off[i], k,
                                             0, 2);
#pragma unroll
  for (int i = 0; i < kSkLoads; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b_src, (lds_void_t*)(bs + (w * kSkLoads + i) * 1024), 16, b_off[i], k,
                                             0, 0);
}

// K slabs [k0, k1) of tile (mt, nt): wave w adds its k-steps (parity w / 4)
// of row block w % 4 into acc[stream].  Ends with every wave past its last
// LDS read and a barrier, so the caller may reuse the LDS.
template <int DIN>
__device__ __forceinline__ void sk_mainloop(const Args& a, int mt, int nt, int k0, int k1, char* lds, int w, int lane,
                                            f32x16_t (&acc)[4]) {
  const int64_t row0 = (int64_t)mt * kSkTile;
  const int nvalid = (int)min<int64_t>(kSkTile, a.T - row0);
  uint32_t a_off[kSkLoads], b_off[kSkLoads];
#pragma unroll
  for (int i = 0; i < kSkLoads; ++i) {
    const int r = w * 16 + i * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ swz_f(r);
    a_off[i] = (uint32_t)(min(r, nvalid - 1) * a.lda + kc * 16);
    const int s = r >> 5, ch = min(nt * 32 + (r & 31), a.c - 1);
    b_off[i] = (uint32_t)((int64_t)(s * a.c + ch) * a.lda + kc * 16);
  }
  const __amdgpu_buffer_rsrc_t a_src = raw_rsrc(a.H + row0 * a.lda + (int64_t)k0 * kRowBytes);
  const __amdgpu_buffer_rsrc_t b_src = raw_rsrc(a.Wt + (int64_t)k0 * kRowBytes);
  // fragment offsets as in the big kernel: subtile i's rows have swizzle
  // x0 ^ 4 (i & 1), so chunk 2 s + h of row (lane % 32) sits at ro[s ^ 2 (i & 1)]
  int ro[4];
  {
    const int h = lane >> 5;
    const int x0 = (lane & 7) ^ ((lane >> 3) & 3);
#pragma unroll
    for (int k = 0; k < 4; ++k) ro[k] = (lane & 31) * kRowBytes + ((16 * (h ^ x0)) ^ (32 * k));
  }
  const int rb = w & 3, kh = w >> 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
  const int nks = k1 - k0;
  for (int p = 0; p < min(3, nks); ++p) sk_copy(a_src, b_src, a_off, b_off, lds, p, p, w);
  for (int j = 0; j < nks; ++j) {
    const int ahead = min(2, nks - 1 - j);            // slabs issued after slab j
    if (ahead == 2) wait_vmcnt<2 * 2 * kSkLoads>();
    else if (ahead == 1) wait_vmcnt<2 * kSkLoads>();
    else wait_vmcnt<0>();
    lds_barrier();                                    // slab j in LDS; every wave is done with slab j - 1
    if (j + 3 < nks) sk_copy(a_src, b_src, a_off, b_off, lds, (j + 3) & 3, j + 3, w);
    const char* as = lds + (j & 3) * 2 * kSkSlab + (rb * 32) * kRowBytes;
    const char* bs = lds + (j & 3) * 2 * kSkSlab + kSkSlab;
    f32x4_t fa[2], fb[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int s = 2 * t + kh;
      fa[t] = *reinterpret_cast<const f32x4_t*>(as + ro[s ^ (2 * (rb & 1))]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        fb[t][q] = *reinterpret_cast<const f32x4_t*>(bs + (q * 32) * kRowBytes + ro[s ^ (2 * (q & 1))]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) sk_mma<DIN>(fa[t], fb[t][q], acc[q]);
  }
  wait_lgkmcnt0();
  lds_barrier();                                      // the ring's LDS is free
}

// Adds the odd-k-step half (waves 4..7) into the even half (waves 0..3)
// through LDS, in the same order on every call.  Returns true in the waves
// that hold the sum.
__device__ __forceinline__ bool sk_combine(f32x16_t (&acc)[4], char* lds, int w, int lane) {
  float4* x = reinterpret_cast<float4*>(lds) + (w & 3) * kSkPartialQuads + lane;
  if (w >= 4) {
#pragma unroll
    for (int jn = 0; jn < 4; ++jn)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[jn][4 * q4 + e];
          asm volatile("" : "+v"(v[e]));
        }
        x[(jn * 4 + q4) * 64] = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
  __syncthreads();
  if (w >= 4) return false;
#pragma unroll
  for (int jn = 0; jn < 4; ++jn)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 o = x[(jn * 4 + q4) * 64];
      acc[jn][4 * q4 + 0] += o.x;
      acc[jn][4 * q4 + 1] += o.y;
      acc[jn][4 * q4 + 2] += o.z;
      acc[jn][4 * q4 + 3] += o.w;
    }
  return true;
}

// Append epilogue of row block rb of a skinny tile: its run q of lane half h
// is block 32 mt + 8 rb + 2 q + h.
template <int DOUT>
__device__ __forceinline__ void sk_epilogue(const Args& a, const f32x16_t (&acc)[4], int mt, int nt, int rb, int lane) {
  const int col = lane & 31, h = lane >> 5;
  const int ch = nt * 32 + col;
  const bool ok = ch < a.c;
  const int chc = min(ch, a.c - 1);
  float ba[4], bb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ba[r] = a.Ba[r * a.c + chc] * kLog2e;
    bb[r] = a.Bb[r * a.c + chc] * kLog2e;
  }
  const int64_t j0 = (int64_t)mt * 32 + rb * 8 + h;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t j = j0 + 2 * q;
    const float* st = a.state_in + min(j, a.nb - 1) * 3 * a.c + chc;
    const SoftAcc prev{st[0], st[a.c], st[2 * a.c]};
    const SoftAcc pa = partial4(acc[2], acc[0], q, ba);
    const SoftAcc pb = partial4(acc[3], acc[1], q, bb);
    append_store<DOUT>(a, pa, pb, prev, j, ok, ch);
  }
}

// Workgroup (tile L, split sp): K slabs [sp nk / S, (sp + 1) nk / S).  With
// S = 1 it finishes the entries itself; otherwise it stores its accumulators
// as they sit in registers ([L][sp][row block][stream][element quad][lane]
// float4: every store one coalesced 1 KiB row) for
// append_skinny_reduce_kernel.
template <int DIN, int DOUT>
__global__ __launch_bounds__(kSkThreads, 1) void append_skinny_kernel(Args a, int S, float4* __restrict__ partial) {
  __shared__ __attribute__((aligned(1024))) char lds[kSkLdsBytes];
  const int L = blockIdx.x / S, sp = blockIdx.x - L * S;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int mt = L / a.n_nt, nt = L - mt * a.n_nt;
  const int k0 = (int)((int64_t)sp * a.nk / S), k1 = (int)((int64_t)(sp + 1) * a.nk / S);   // S <= nk: k1 > k0
  f32x16_t acc[4];
  sk_mainloop<DIN>(a, mt, nt, k0, k1, lds, w, lane, acc);
  if (!sk_combine(acc, lds, w, lane)) return;
  if (S == 1) {
    sk_epilogue<DOUT>(a, acc, mt, nt, w, lane);
    return;
  }
  if ((int64_t)mt * 32 + w * 8 >= a.nb) return;           // no block of row block w: nothing reads it
  float4* dst = partial + (((int64_t)L * S + sp) * 4 + w) * kSkPartialQuads + lane;
#pragma unroll
  for (int jn = 0; jn < 4; ++jn)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // each element through a VGPR: a store fed straight from an
      // accumulator register has been miscompiled (see epilogue_project)
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = acc[jn][4 * q4 + e];
        asm volatile("" : "+v"(v[e]));
      }
      dst[(jn * 4 + q4) * 64] = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// Workgroup = (tile L, row block w) of the split form, eight waves: wave u
// adds splits u, u + 8, ... in increasing order, then the waves' sums meet in
// a fixed tree through LDS ((4..7 into 0..3), (2, 3 into 0, 1), 1 into 0 --
// the same sum on every call) and wave 0 runs the append epilogue.
// Reduce of the skinny split-K.  Workgroup (tile L, row block rb, run q)
// owns blocks j = 32 mt + 8 rb + 2 q + h (h = lane / 32) of the tile's 32
// channels: wave u adds stream u's float4 (the 4 rows of the lane's block)
// over the S splits in split order, every load issued before the first add;
// waves 1..3 hand their sums to wave 0 through LDS, and wave 0, whose
// epilogue inputs were loaded before the partials, finishes the run.
constexpr int kSkReduceThreads = 256;
constexpr int kSkReduceUnroll = 8;
template <int DOUT>
__global__ __launch_bounds__(kSkReduceThreads) void append_skinny_reduce_kernel(Args a, int S,
                                                                                const float4* __restrict__ partial) {
  __shared__ float4 xch[3][64];
  const int q = blockIdx.x & 3, rb = (blockIdx.x >> 2) & 3, L = blockIdx.x >> 4;
  const int u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int mt = L / a.n_nt, nt = L - mt * a.n_nt;
  const int64_t jrun = (int64_t)mt * 32 + rb * 8 + 2 * q;
  if (jrun >= a.nb) return;                                // both blocks of the run are past the batch
  const int col = lane & 31, h = lane >> 5;
  const int ch = nt * 32 + col;
  const int chc = min(ch, a.c - 1);
  const int64_t j = jrun + h;
  float ba[4] = {}, bb[4] = {}, st[3] = {};   // scaled by log2(e) after the sums: no wait before the partials
  if (u == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ba[r] = a.Ba[r * a.c + chc];
      bb[r] = a.Bb[r * a.c + chc];
    }
    const float* sp = a.state_in + min(j, a.nb - 1) * 3 * a.c + chc;
    st[0] = sp[0];
    st[1] = sp[a.c];
    st[2] = sp[2 * a.c];
  }
  // split sp of this (tile, row block) sits at + sp * 4 * kSkPartialQuads
  const float4* src = partial + ((int64_t)L * S * 4 + rb) * kSkPartialQuads + (u * 4 + q) * 64 + lane;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += kSkReduceUnroll) {
    float4 v[kSkReduceUnroll];
#pragma unroll
    for (int i = 0; i < kSkReduceUnroll; ++i)   // unconditional (clamped) loads: no wait between them
      v[i] = src[(int64_t)min(s0 + i, S - 1) * 4 * kSkPartialQuads];
#pragma unroll
    for (int i = 0; i < kSkReduceUnroll; ++i) {
      const bool in = s0 + i < S;
      sum.x += in ? v[i].x : 0.f;
      sum.y += in ? v[i].y : 0.f;
      sum.z += in ? v[i].z : 0.f;
      sum.w += in ? v[i].w : 0.f;
    }
  }
  if (u > 0) xch[u - 1][lane] = sum;
  __syncthreads();
  if (u != 0) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ba[r] *= kLog2e;
    bb[r] *= kLog2e;
  }
  const float4 cb = xch[0][lane], za4 = xch[1][lane], zb4 = xch[2][lane];
  const float va[4] = {sum.x, sum.y, sum.z, sum.w}, vb[4] = {cb.x, cb.y, cb.z, cb.w};
  const float za[4] = {za4.x, za4.y, za4.z, za4.w}, zb[4] = {zb4.x, zb4.y, zb4.z, zb4.w};
  append_store<DOUT>(a, partial_rows4(za, va, ba), partial_rows4(zb, vb, bb), SoftAcc{st[0], st[1], st[2]}, j,
                     ch < a.c, ch);
}

// Form of a decode append of nb blocks:
//  * BIG: the 256 x 256 tiles alone fill 256 workgroups;
//  * BIG_SPLIT: they fill at least 64, and the K loop is split S ways so
//    that about 256 run (measured at 1024 blocks: 101 + 19 us, against
//    160 us for the unsplit 128 x 128 tiles, whose copies move twice the
//    bytes per MFMA);
//  * SKINNY: smaller batches, 128 x 128 tiles split S >= 1 ways (S = 1: no
//    partials; measured at 64 blocks: 16 + 7.5 us, against 18.5 + 12 us for
//    256 x 256 tiles split 16 ways).
// S is capped at the K loop's slab count nk.  A function of nb, c and nk
// only, so the workspace size does not depend on the device.
// Decode append for one or two sequences (4 nb <= 8 rows of H): no tiles
// and no partial products, one launch.  A workgroup of 8 waves owns
// channels 2 g and 2 g + 1; wave w dots weight row (w % 4) c + 2 g + w / 4
// (stream w % 4 of its channel, in the row order C^a, C^b, Z^a, Z^b of Wt)
// with every row of H.  K advances in pieces of 16 KiB of each row: H's
// piece is staged in LDS once for the 8 waves, lane l of a wave takes the
// 16-byte chunks l + 64 i of the piece, and every load of a piece is issued
// before the first is used.  The 8 x R dot products meet in LDS and 2 nb
// threads run the append epilogue.  At c = 512 the 256 workgroups stream
// the weights once; the MFMA tiles would read 16 to 32 x as many H rows as
// there are and need a split-K round trip to fill the chip.
constexpr int kGvThreads = 512;
constexpr int kGvPieceChunks = 16;                        // 16-byte chunks per lane and piece
constexpr int kGvPieceRowChunks = kGvPieceChunks * 64;    // 16 KiB of each row per piece
constexpr int kGvMaxBlocks = 2;

// acc + <w, h> over one 16-byte chunk (8 bf16 or 4 fp32 of each operand).
template <int DIN>
__device__ __forceinline__ float dot_chunk(const f32x4_t& w, const f32x4_t& h, float acc) {
  if (DIN == DT_BF16) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // the elements go through scalars: hipcc bit-casts a subscripted vector
      // element as if it were element 0
      const float wt = w[t], ht = h[t];
      // v_dot2c_f32_bf16: acc + w0 h0 + w1 h1 (bf16 products are exact in fp32)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wt), __builtin_bit_cast(bf16x2_t, ht), acc,
                                            false);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = fmaf(w[t], h[t], acc);
  }
  return acc;
}

template <int DIN, int DOUT, int R>
__global__ __launch_bounds__(kGvThreads, 1) void append_gemv_kernel(Args a) {
  __shared__ f32x4_t hs[R][kGvPieceRowChunks];              // R x 16 KiB
  __shared__ float red[8][R];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ch = 2 * blockIdx.x + (w >> 2);                // c is even: ch < c
  const int nck = (int)(a.lda >> 4);                       // 16-byte chunks per row
  const f32x4_t* wrow = reinterpret_cast<const f32x4_t*>(a.Wt + (int64_t)((w & 3) * a.c + ch) * a.lda);
  const f32x4_t* hsrc = reinterpret_cast<const f32x4_t*>(a.H);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  for (int p0 = 0; p0 < nck; p0 += kGvPieceRowChunks) {
    const int pn = min(kGvPieceRowChunks, nck - p0);       // chunks of each row in this piece
    // H first, then this wave's weight chunks, all unconditional (a chunk
    // past the piece reads the row's last one: branches around the loads
    // would serialise them), so the H stores below wait for the H loads only
    f32x4_t hv[2 * R];
#pragma unroll
    for (int i = 0; i < 2 * R; ++i) {
      const int f = tid + kGvThreads * i, r = f / kGvPieceRowChunks, k = f % kGvPieceRowChunks;
      hv[i] = hsrc[(int64_t)r * nck + p0 + min(k, pn - 1)];
    }
    f32x4_t wv[kGvPieceChunks];
#pragma unroll
    for (int i = 0; i < kGvPieceChunks; ++i)
      wv[i] = __builtin_nontemporal_load(wrow + p0 + min(lane + 64 * i, pn - 1));
#pragma unroll
    for (int i = 0; i < kGvPieceChunks; ++i)   // chunks past the piece add 0 x (a finite copy of an H chunk)
      if (lane + 64 * i >= pn) wv[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (p0 > 0) __syncthreads();                           // every wave is done with the previous piece
#pragma unroll
    for (int i = 0; i < 2 * R; ++i) {
      const int f = tid + kGvThreads * i;
      hs[f / kGvPieceRowChunks][f % kGvPieceRowChunks] = hv[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kGvPieceChunks; ++i) {
      const int k = lane + 64 * i;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = dot_chunk<DIN>(wv[i], hs[r][k], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float v = acc[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[w][r] = v;
  }
  __syncthreads();
  if (tid >= 2 * a.nb) return;
  const int j = tid >> 1, cc = tid & 1;                    // block j of channel 2 g + cc
  const int chj = 2 * blockIdx.x + cc;
  float za[4], va[4], zb[4], vb[4], ba[4], bb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    va[t] = red[cc * 4 + 0][4 * j + t];
    vb[t] = red[cc * 4 + 1][4 * j + t];
    za[t] = red[cc * 4 + 2][4 * j + t];
    zb[t] = red[cc * 4 + 3][4 * j + t];
    ba[t] = a.Ba[t * a.c + chj] * kLog2e;
    bb[t] = a.Bb[t * a.c + chj] * kLog2e;
  }
  const float* st = a.state_in + (int64_t)j * 3 * a.c + chj;
  const SoftAcc prev{st[0], st[a.c], st[2 * a.c]};
  append_store<DOUT>(a, partial_rows4(za, va, ba), partial_rows4(zb, vb, bb), prev, j, true, chj);
}

enum AppendForm { APPEND_BIG = 0, APPEND_BIG_SPLIT = 1, APPEND_SKINNY = 2, APPEND_GEMV = 3 };
struct AppendPlan {
  int form;
  int S;
  int64_t tiles;
};

AppendPlan append_plan(int64_t nb, int c, int nk) {
  AppendPlan p{};
  const int64_t gb = big_append_tiles(nb, c);
  int64_t S;
  if (nb <= kGvMaxBlocks) {
    p.form = APPEND_GEMV;
    p.tiles = c / 2;
    S = 1;
  } else if (gb >= kAppendWorkgroups) {
    p.form = APPEND_BIG;
    p.tiles = gb;
    S = 1;
  } else if (gb * 4 >= kAppendWorkgroups) {
    p.form = APPEND_BIG_SPLIT;
    p.tiles = gb;
    S = kAppendWorkgroups / gb;
  } else {
    p.form = APPEND_SKINNY;
    p.tiles = skinny_append_tiles(nb, c);
    S = kAppendWorkgroups / p.tiles;
  }
  S = S < 1 ? 1 : S > kAppendMaxSplits ? kAppendMaxSplits : S;
  p.S = (int)(S > nk ? nk : S);
  return p;
}

template <int DIN, int MODE, int DOUT, bool LOOKUP = false>
hipError_t launch_tile(const Args& a, hipStream_t stream) {
  const int G = a.n_mt * a.n_nt;
  const int P = min(G, device_cu_count());   // one workgroup of the tile kernels fits per CU
  hipLaunchKernelGGL((tile_kernel<DIN, MODE, DOUT, LOOKUP>), dim3(P), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int MODE, bool LOOKUP = false>
hipError_t dispatch(int in_dt, int out_dt, const Args& a, hipStream_t stream) {
  if (in_dt == DT_BF16)
    return out_dt == DT_BF16 ? launch_tile<DT_BF16, MODE, DT_BF16, LOOKUP>(a, stream)
                             : launch_tile<DT_BF16, MODE, DT_F32, LOOKUP>(a, stream);
  return out_dt == DT_BF16 ? launch_tile<DT_F32, MODE, DT_BF16, LOOKUP>(a, stream)
                           : launch_tile<DT_F32, MODE, DT_F32, LOOKUP>(a, stream);
}

}  // namespace

hipError_t launch_project(int in_dt, int out_dt, const void* H, int64_t T, int d, const void* Wt, int n_out,
                          void* Y, int64_t ld_y, hipStream_t stream) {
  Args a{};
  const int es = in_dt == DT_BF16 ? 2 : 4;
  a.H = static_cast<const char*>(H);
  a.Wt = static_cast<const char*>(Wt);
  a.lda = (int64_t)d * es;
  a.nk = d * es / kRowBytes;
  a.T = T;
  a.n_out = n_out;
  a.Y = static_cast<char*>(Y);
  a.ld_y = ld_y;
  a.c = 1;
  a.n_mt = (int)((T + kTile - 1) / kTile);
  a.n_nt = (n_out + kTile - 1) / kTile;
  return dispatch<MODE_PROJECT>(in_dt, out_dt, a, stream);
}

hipError_t launch_fused(int mode, int in_dt, int out_dt, const void* H, int d, const void* Wt, int c,
                        const float* Ba, const float* Bb, const TileRec* tiles, const int64_t* cu_dev, int batch,
                        int n_tiles, void* out, float* halo, hipStream_t stream) {
  Args a{};
  const int es = in_dt == DT_BF16 ? 2 : 4;
  a.H = static_cast<const char*>(H);
  a.Wt = static_cast<const char*>(Wt);
  a.lda = (int64_t)d * es;
  a.nk = d * es / kRowBytes;
  a.c = c;
  a.Ba = Ba;
  a.Bb = Bb;
  a.tiles = tiles;
  a.cu = cu_dev;
  a.batch = batch;
  a.m = mode == 0 ? 4 : 128;
  a.halo = halo;
  a.out = static_cast<char*>(out);
  a.n_mt = n_tiles;
  a.n_out = 1;
  if (mode == 0) {   // CSA: 64 channels x 4 streams per N tile
    a.n_nt = (c + 63) / 64;
    return tiles ? dispatch<MODE_CSA>(in_dt, out_dt, a, stream) : dispatch<MODE_CSA, true>(in_dt, out_dt, a, stream);
  }
  a.n_nt = (c + 127) / 128;   // HCA: 128 channels x 2 streams per N tile
  return tiles ? dispatch<MODE_HCA>(in_dt, out_dt, a, stream) : dispatch<MODE_HCA, true>(in_dt, out_dt, a, stream);
}

size_t append_partial_bytes(int64_t nb, int c) {
  // sized for the uncapped split count, so the size depends on nb and c
  // only; a call whose K has fewer slabs than that uses less of it
  const AppendPlan p = append_plan(nb, c, 1 << 30);
  if (p.S <= 1) return 0;
  const size_t per = p.form == APPEND_BIG_SPLIT ? (size_t)4 * 4 * kPartialQuads : (size_t)4 * kSkPartialQuads;
  return (size_t)p.tiles * p.S * per * sizeof(float4);
}

hipError_t launch_csa_append(int in_dt, int out_dt, const void* H, int64_t nb, int d, const void* Wt, int c,
                             const float* Ba, const float* Bb, const float* state_in, float* state_out, void* out,
                             void* partial, hipStream_t stream) {
  Args a{};
  const int es = in_dt == DT_BF16 ? 2 : 4;
  a.H = static_cast<const char*>(H);
  a.Wt = static_cast<const char*>(Wt);
  a.lda = (int64_t)d * es;
  a.nk = d * es / kRowBytes;
  a.T = nb * 4;
  a.c = c;
  a.Ba = Ba;
  a.Bb = Bb;
  a.out = static_cast<char*>(out);
  a.state_in = state_in;
  a.state_out = state_out;
  a.nb = nb;
  a.n_out = 1;
  const AppendPlan p = append_plan(nb, c, a.nk);
  const int G = (int)p.tiles, S = p.S;
  if (S > 1 && partial == nullptr) return hipErrorInvalidValue;
  float4* part = static_cast<float4*>(partial);
  if (p.form == APPEND_GEMV) {
    auto gemv = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(G), dim3(kGvThreads), 0, stream, a); };
    if (nb == 1) {
      if (in_dt == DT_BF16) out_dt == DT_BF16 ? gemv(append_gemv_kernel<DT_BF16, DT_BF16, 4>)
                                              : gemv(append_gemv_kernel<DT_BF16, DT_F32, 4>);
      else out_dt == DT_BF16 ? gemv(append_gemv_kernel<DT_F32, DT_BF16, 4>) : gemv(append_gemv_kernel<DT_F32, DT_F32, 4>);
    } else {
      if (in_dt == DT_BF16) out_dt == DT_BF16 ? gemv(append_gemv_kernel<DT_BF16, DT_BF16, 8>)
                                              : gemv(append_gemv_kernel<DT_BF16, DT_F32, 8>);
      else out_dt == DT_BF16 ? gemv(append_gemv_kernel<DT_F32, DT_BF16, 8>) : gemv(append_gemv_kernel<DT_F32, DT_F32, 8>);
    }
    return hipGetLastError();
  }
  if (p.form != APPEND_SKINNY) {
    a.n_mt = (int)((a.T + kTile - 1) / kTile);
    a.n_nt = (c + 63) / 64;
    if (S == 1) return dispatch<MODE_CSA_APPEND>(in_dt, out_dt, a, stream);
    if (S > 4) return hipErrorInvalidValue;   // 64 <= tiles < 256 give S <= 4, all append_reduce_kernel adds
    if (in_dt == DT_BF16)
      hipLaunchKernelGGL(append_splitk_kernel<DT_BF16>, dim3(G * S), dim3(kThreads), 0, stream, a, S, part);
    else
      hipLaunchKernelGGL(append_splitk_kernel<DT_F32>, dim3(G * S), dim3(kThreads), 0, stream, a, S, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (out_dt == DT_BF16)
      hipLaunchKernelGGL(append_reduce_kernel<DT_BF16>, dim3(G * 16), dim3(64), 0, stream, a, S, part);
    else
      hipLaunchKernelGGL(append_reduce_kernel<DT_F32>, dim3(G * 16), dim3(64), 0, stream, a, S, part);
    return hipGetLastError();
  }
  a.n_mt = (int)((a.T + kSkTile - 1) / kSkTile);
  a.n_nt = (c + 31) / 32;
  auto split = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(G * S), dim3(kSkThreads), 0, stream, a, S, part); };
  if (in_dt == DT_BF16) out_dt == DT_BF16 ? split(append_skinny_kernel<DT_BF16, DT_BF16>)
                                          : split(append_skinny_kernel<DT_BF16, DT_F32>);
  else out_dt == DT_BF16 ? split(append_skinny_kernel<DT_F32, DT_BF16>) : split(append_skinny_kernel<DT_F32, DT_F32>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  if (out_dt == DT_BF16)
    hipLaunchKernelGGL(append_skinny_reduce_kernel<DT_BF16>, dim3(G * 16), dim3(kSkReduceThreads), 0, stream, a, S,
                       part);
  else
    hipLaunchKernelGGL(append_skinny_reduce_kernel<DT_F32>, dim3(G * 16), dim3(kSkReduceThreads), 0, stream, a, S,
                       part);
  return hipGetLastError();
}

hipError_t launch_csa_fixup(int out_dt, const TileRec* tiles, const int64_t* cu_dev, int batch, int n_tiles, int c,
                            const float* halo, void* out, hipStream_t stream) {
  if (out_dt == DT_BF16)
    hipLaunchKernelGGL(csa_fixup_kernel<DT_BF16>, dim3(n_tiles), dim3(256), 0, stream, tiles, cu_dev, batch, c,
                       halo, static_cast<char*>(out));
  else
    hipLaunchKernelGGL(csa_fixup_kernel<DT_F32>, dim3(n_tiles), dim3(256), 0, stream, tiles, cu_dev, batch, c,
                       halo, static_cast<char*>(out));
  return hipGetLastError();
}

}  // namespace seqcomp
