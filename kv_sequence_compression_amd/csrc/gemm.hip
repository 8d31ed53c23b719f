// Projection GEMM and fused compressor on the gfx950 matrix cores.
//
// The projection ("序列压缩注意力", eq. attn-seqcomp-csa-proj) is the one
// dense contraction of the compressor: Y = H Wt^T with K = d.  One workgroup
// computes a 256 x 256 tile of Y with 4 wavefronts (2 x 2, each 128 x 128 as
// 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators in registers: with one wave per
// SIMD that instruction sustains ~94% of the bf16 peak on gfx950, the 16x16x32
// form only ~56%, as measured with back-to-back independent MFMAs).  K advances in
// 128-byte slabs (64 bf16 / 32 fp32) that are copied global -> LDS directly
// (global_load_lds_dwordx4, no register staging) into a 2-stage ring.
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
#include "launch.hpp"

namespace seqcomp {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kTile = 256;                      // BM = BN = 256
constexpr int kRowBytes = 64;                   // bytes of one tile row per K slab (32 bf16 / 16 fp32)
constexpr int kTileBytes = kTile * kRowBytes;   // 16 KiB per operand per stage
constexpr int kStages = 5;                      // ring depth: 4 slabs of loads in flight
constexpr int kStageBytes = 2 * kTileBytes;     // A and B
constexpr int kLdsBytes = kStages * kStageBytes;  // 160 KiB: all of a CU's LDS

enum : int { MODE_PROJECT = 0, MODE_CSA = 1, MODE_HCA = 2 };

// 16-byte slot of k-chunk kc (0..3) in 64-byte tile row r.  With g(r) =
// ((r >> 1) ^ (r >> 2)) & 3 the 16 lanes reading one k-chunk of 16
// consecutive rows hit distinct 16-byte bank groups whether the LDS services
// 8 lanes (128 bytes) or 16 lanes (256 bytes) per pass: within any 8 rows the
// even and the odd rows take distinct slots, and rows r, r+4, r+8, r+12
// (same bank offset r*64 mod 256) take four distinct slots.
__device__ __forceinline__ int swz_g(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int swz(int r, int kc) { return kc ^ swz_g(r); }

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
  // grid
  int n_mt, n_nt;
};

template <int DIN>
struct Frag;

// Accumulator tile of one wave: [4 M subtiles][4 N subtiles] of 32 x 32.
// Lane l holds column l % 32 and rows 8 q + 4 (l / 32) + r (element 4 q + r).
typedef f32x16_t WaveAcc[4][4];

// One K slab (64 bytes of every tile row) is consumed in two halves; a half
// reads 4 A and 4 B fragments of 16 bytes per lane from LDS and issues the
// MFMAs over them.  The 16-byte chunk a lane reads is chunk 2 half + l / 32
// (bf16) or l / 32 * 2 + half (fp32) of its row, found at slot chunk ^ x.
struct Frags {
  f32x4_t a[4], b[4];
};

template <>
struct Frag<DT_BF16> {
  // k16 step `half` of the 32 bf16 of a slab: lane l feeds row l % 32 and the
  // 8 consecutive k of chunk 2 half + l / 32.
  static __device__ __forceinline__ void load(const char* As, const char* Bs, int lane_off, int x, int h, int wm,
                                              int wn, int half, Frags& f) {
    const int slot = ((half * 2 + h) ^ x) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = *reinterpret_cast<const f32x4_t*>(As + (wm * 128 + i * 32) * kRowBytes + lane_off + slot);
      f.b[i] = *reinterpret_cast<const f32x4_t*>(Bs + (wn * 128 + i * 32) * kRowBytes + lane_off + slot);
    }
  }
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
  // Half `half` of the 16 fp32 of a slab: four 32x32x2 MFMAs per (i, j).  At
  // step t lane l feeds k = 8 (l / 32) + 4 half + t, so the two lane halves
  // cover k and k + 8; the same permutation of k on both operands leaves the
  // dot products unchanged.
  static __device__ __forceinline__ void load(const char* As, const char* Bs, int lane_off, int x, int h, int wm,
                                              int wn, int half, Frags& f) {
    const int slot = ((h * 2 + half) ^ x) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = *reinterpret_cast<const f32x4_t*>(As + (wm * 128 + i * 32) * kRowBytes + lane_off + slot);
      f.b[i] = *reinterpret_cast<const f32x4_t*>(Bs + (wn * 128 + i * 32) * kRowBytes + lane_off + slot);
    }
  }
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

// Copy one 64-byte-wide K slab of 256 rows of one operand into LDS.  Wave w
// fills rows [64 w, 64 w + 64) with 4 instructions of 1 KiB (16 rows) each;
// lane p writes LDS slot p & 3 of row p >> 2, which holds k-chunk
// swz(row, p & 3) -- an XOR, so reads find chunk kc at swz(row, kc).
__device__ __forceinline__ void load_slab(const char* base, const uint32_t (&off)[4], int64_t k_bytes, char* lds_tile,
                                          int w) {
  const char* kb = base + k_bytes;                  // uniform
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(kb + off[i]), (lds_void_t*)(lds_tile + (w * 4 + i) * 1024), 16,
                                     0, 0);
}

// s_waitcnt with vmcnt(n) and the other counters left open (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt left open.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left open.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Wait until at most `n` slab loads (8 instructions each per wave: 4 for A,
// 4 for B) are still in flight.
__device__ __forceinline__ void wait_slabs_in_flight(int n) {
  if (n >= 3) wait_vmcnt<24>();
  else if (n == 2) wait_vmcnt<16>();
  else if (n == 1) wait_vmcnt<8>();
  else wait_vmcnt<0>();
}

// Workgroup barrier for the K loop.  __syncthreads() also fences global
// memory, which makes the compiler wait for EVERY outstanding load (vmcnt(0))
// and would drain the slab ring; here the caller waits for exactly the slab
// it needs, and the empty asm statements keep the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// K loop over a ring of kStages LDS slabs: slab kt + kStages - 1 is
// requested while slab kt is multiplied, so up to kStages - 1 slabs of
// global -> LDS copies overlap the matrix work.  Within an iteration:
//   copy request for slab kt + 4 | read half 1 of slab kt | MFMAs of half 0
//   wait for slab kt + 1 (own copies) and own LDS reads | barrier
//   read half 0 of slab kt + 1   | MFMAs of half 1
// so LDS reads always overlap MFMAs.  After the barrier every wave's copies
// of slab kt + 1 have landed and every wave has finished reading slab kt,
// whose stage the next iteration refills.
template <int DIN>
__device__ __forceinline__ void mainloop(const char* a_base, const uint32_t (&a_off)[4], const char* b_base,
                                         const uint32_t (&b_off)[4], int nk, char* lds, int w, int lane, int wm,
                                         int wn, WaveAcc& acc) {
  const int lane_off = (lane & 31) * kRowBytes;
  const int x = swz_g(lane & 31);                   // swz() of rows 32 k + (lane & 31)
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  const int pro = min(kStages - 1, nk);
  for (int s = 0; s < pro; ++s) {
    load_slab(a_base, a_off, (int64_t)s * kRowBytes, lds + s * kStageBytes, w);
    load_slab(b_base, b_off, (int64_t)s * kRowBytes, lds + s * kStageBytes + kTileBytes, w);
  }
  wait_slabs_in_flight(pro - 1);                    // slab 0 has landed
  lds_barrier();
  Frags f0, f1;
  Frag<DIN>::load(lds, lds + kTileBytes, lane_off, x, h, wm, wn, 0, f0);
  int stage = 0;
  int kt = 0;
  // steady state: slab kt + kStages - 1 exists (so does slab kt + 1).  The
  // compiler waits for all LDS reads before the first MFMA that uses the
  // fragments carried over the loop edge (f0), so half 1 is read only after
  // that first MFMA group: the forced wait then covers reads issued a whole
  // MFMA block earlier, and the half-1 reads overlap 12 MFMAs.
  for (; kt + kStages - 1 < nk; ++kt) {
    char* cur = lds + stage * kStageBytes;
    const int nxt_stage = stage + 1 == kStages ? 0 : stage + 1;
    char* dst = lds + (stage == 0 ? kStages - 1 : stage - 1) * kStageBytes;   // read in iteration kt - 1
    const int64_t kb = (int64_t)(kt + kStages - 1) * kRowBytes;
    load_slab(a_base, a_off, kb, dst, w);
    load_slab(b_base, b_off, kb, dst + kTileBytes, w);
    __builtin_amdgcn_sched_barrier(0);
    Frag<DIN>::template mma<0, 1>(f0, acc);
    __builtin_amdgcn_sched_barrier(0);
    Frag<DIN>::load(cur, cur + kTileBytes, lane_off, x, h, wm, wn, 1, f1);
    __builtin_amdgcn_sched_barrier(0);
    Frag<DIN>::template mma<1, 4>(f0, acc);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_lgkm0<8 * (kStages - 2)>();          // slab kt + 1 landed (kt + 2 .. kt + 4 in flight), own reads done
    lds_barrier();
    char* nx = lds + nxt_stage * kStageBytes;
    Frag<DIN>::load(nx, nx + kTileBytes, lane_off, x, h, wm, wn, 0, f0);
    __builtin_amdgcn_sched_barrier(0);
    Frag<DIN>::mma(f1, acc);
    __builtin_amdgcn_sched_barrier(0);
    stage = nxt_stage;
  }
  // drain: every slab has been requested
  for (; kt < nk; ++kt) {
    char* cur = lds + stage * kStageBytes;
    const int nxt_stage = stage + 1 == kStages ? 0 : stage + 1;
    Frag<DIN>::load(cur, cur + kTileBytes, lane_off, x, h, wm, wn, 1, f1);
    Frag<DIN>::mma(f0, acc);
    wait_slabs_in_flight(nk - 2 - kt);
    wait_lgkmcnt0();
    lds_barrier();
    if (kt + 1 < nk) {
      char* nx = lds + nxt_stage * kStageBytes;
      Frag<DIN>::load(nx, nx + kTileBytes, lane_off, x, h, wm, wn, 0, f0);
    }
    Frag<DIN>::mma(f1, acc);
    stage = nxt_stage;
  }
}

// Per-thread source rows of the two operands: thread (wave w, lane p) loads
// tile rows r_i = 64 w + 16 i + (p >> 2), i = 0..3, at k-chunk swz(r_i, p & 3).
template <int MODE>
__device__ __forceinline__ int b_row_of(int n, int nt, int c, int n_out) {
  if (MODE == MODE_PROJECT) return min(nt * kTile + n, n_out - 1);
  const int half = n >> 7;                 // which wave column
  if (MODE == MODE_CSA) {                  // 4 streams x 32 channels per wave column
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
__device__ __forceinline__ SoftAcc partial4(const f32x16_t& z, const f32x16_t& v, int q, const float (&bias2)[4]) {
  float l[4];
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    l[j] = fmaf(z[4 * q + j], kLog2e, bias2[j]);
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
    s.A = fmaf(w, v[4 * q + j], s.A);
  }
  return s;
}

__device__ __forceinline__ SoftAcc shfl_acc(const SoftAcc& s, int src) {
  SoftAcc r;
  r.M = __shfl(s.M, src, 64);
  r.S = __shfl(s.S, src, 64);
  r.A = __shfl(s.A, src, 64);
  return r;
}

__device__ __forceinline__ SoftAcc shfl_xor_acc(const SoftAcc& s, int mask) {
  SoftAcc r;
  r.M = __shfl_xor(s.M, mask, 64);
  r.S = __shfl_xor(s.S, mask, 64);
  r.A = __shfl_xor(s.A, mask, 64);
  return r;
}

template <int DOUT>
__device__ __forceinline__ void store1(char* out, int64_t idx, float v) {
  if (DOUT == DT_BF16) reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits(v);
  else reinterpret_cast<float*>(out)[idx] = v;
}

template <int DOUT>
__device__ void epilogue_project(const Args& a, WaveAcc& acc, int mt, int nt, int lane, int wm, int wn) {
  const int col = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nt * kTile + wn * 128 + j * 32 + col;
      if (n >= a.n_out) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = (int64_t)mt * kTile + wm * 128 + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        if (row < a.T) store1<DOUT>(a.Y, row * a.ld_y + n, acc[i][j][e]);
      }
    }
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
      const SoftAcc px = shfl_xor_acc(pb, 32);
      const SoftAcc prev = h ? px : carry;
      carry = px;
      const int blk = wm * 32 + ms * 8 + q * 2 + h;  // block (= entry) index inside the tile
      if (ok && blk * 4 < t.n_rows) {
        const int64_t e = (int64_t)t.entry_start + blk;
        if (blk == 0) {
          if (t.flags & TILE_FIRST) {
            store1<DOUT>(a.out, e * c + ch, pa.A / pa.S);   // entry 0: no b rows
          } else {
            halo[0 * c + ch] = pa.M;
            halo[1 * c + ch] = pa.S;
            halo[2 * c + ch] = pa.A;
          }
        } else {
          const SoftAcc m = softacc_merge(pa, prev);
          store1<DOUT>(a.out, e * c + ch, m.A / m.S);
        }
      }
    }
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
    s = softacc_merge(s, shfl_xor_acc(s, 32));
    if (ok && block_ok && h == 0) store1<DOUT>(a.out, ((int64_t)t.entry_start + wm) * c + ch, s.A / s.S);
  }
}

// One logical tile.  The thread index is passed through an empty asm
// statement so the compiler cannot hoist lane-derived values out of the
// persistent loop (they would stay live across the K loop and crowd out the
// accumulators).
template <int DIN, int MODE, int DOUT>
__device__ __forceinline__ void run_tile(const Args& a, int L, char* lds) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int w = tid >> 6, lane = tid & 63;
  const int mt = L / a.n_nt, nt = L - mt * a.n_nt;
  const int wm = w >> 1, wn = w & 1;

  int64_t row0;
  int nvalid;
  TileRec t{};
  if (MODE == MODE_PROJECT) {
    row0 = (int64_t)mt * kTile;
    nvalid = (int)min<int64_t>(kTile, a.T - row0);
  } else {
    t = a.tiles[mt];
    row0 = t.row_start;
    nvalid = t.n_rows;
  }
  // Byte offsets from uniform bases; they fit 32 bits because a tile of H is
  // 256 rows of at most 64 KiB and the host rejects a Wt of 4 GiB or more.
  const char* a_base = a.H + row0 * a.lda;
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = w * 64 + i * 16 + (lane >> 2);
    const int kc = swz(r, lane & 3);
    a_off[i] = (uint32_t)(min(r, nvalid - 1) * a.lda + kc * 16);
    b_off[i] = (uint32_t)((int64_t)b_row_of<MODE>(r, nt, a.c, a.n_out) * a.lda + kc * 16);
  }
  float ba[4] = {0.f, 0.f, 0.f, 0.f}, bb[4] = {0.f, 0.f, 0.f, 0.f};
  if (MODE == MODE_CSA) csa_bias(a, nt, lane, wn, ba, bb);
  WaveAcc acc;
  mainloop<DIN>(a_base, a_off, a.Wt, b_off, a.nk, lds, w, lane, wm, wn, acc);
  if (MODE == MODE_PROJECT) epilogue_project<DOUT>(a, acc, mt, nt, lane, wm, wn);
  else if (MODE == MODE_CSA) epilogue_csa<DOUT>(a, acc, t, mt, nt, lane, wm, wn, lds, ba, bb);
  else epilogue_hca<DOUT>(a, acc, t, nt, tid, wm, wn, lds);
}

// Persistent grid: one workgroup per CU walks rounds of gridDim.x logical
// tiles.  In every round each XCD owns one contiguous range of logical tiles
// (N fastest), so the workgroups that share an M panel of H start it
// together and advance through K in step: their H slabs hit in the XCD's L2.
template <int DIN, int MODE, int DOUT>
__global__ __launch_bounds__(kThreads, 1) void tile_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int G = a.n_mt * a.n_nt;
  const int P = gridDim.x;
  for (int L = xcd_remap(blockIdx.x, P); L < G; L += P) {
    run_tile<DIN, MODE, DOUT>(a, L, lds);
    __syncthreads();   // the epilogue's LDS use ends before the next tile's loads
  }
}

// First entry of every tile that continues a sequence: merge the tile's
// first-block a-partial with the previous tile's last-block b-partial.
template <int DOUT>
__global__ __launch_bounds__(256) void csa_fixup_kernel(const TileRec* __restrict__ tiles, int c,
                                                        const float* __restrict__ halo, char* __restrict__ out) {
  const int tile = blockIdx.x;
  const TileRec t = tiles[tile];
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

// Compute units of the current device (one workgroup of the tile kernels fits per CU).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int DIN, int MODE, int DOUT>
hipError_t launch_tile(const Args& a, hipStream_t stream) {
  const int G = a.n_mt * a.n_nt;
  const int P = min(G, cu_count());
  hipLaunchKernelGGL((tile_kernel<DIN, MODE, DOUT>), dim3(P), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(int in_dt, int out_dt, const Args& a, hipStream_t stream) {
  if (in_dt == DT_BF16)
    return out_dt == DT_BF16 ? launch_tile<DT_BF16, MODE, DT_BF16>(a, stream)
                             : launch_tile<DT_BF16, MODE, DT_F32>(a, stream);
  return out_dt == DT_BF16 ? launch_tile<DT_F32, MODE, DT_BF16>(a, stream)
                           : launch_tile<DT_F32, MODE, DT_F32>(a, stream);
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
                        const float* Ba, const float* Bb, const TileRec* tiles, int n_tiles, void* out, float* halo,
                        hipStream_t stream) {
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
  a.halo = halo;
  a.out = static_cast<char*>(out);
  a.n_mt = n_tiles;
  a.n_out = 1;
  if (mode == 0) {   // CSA: 64 channels x 4 streams per N tile
    a.n_nt = (c + 63) / 64;
    return dispatch<MODE_CSA>(in_dt, out_dt, a, stream);
  }
  a.n_nt = (c + 127) / 128;   // HCA: 128 channels x 2 streams per N tile
  return dispatch<MODE_HCA>(in_dt, out_dt, a, stream);
}

hipError_t launch_csa_fixup(int out_dt, const TileRec* tiles, int n_tiles, int c, const float* halo, void* out,
                            hipStream_t stream) {
  if (out_dt == DT_BF16)
    hipLaunchKernelGGL(csa_fixup_kernel<DT_BF16>, dim3(n_tiles), dim3(256), 0, stream, tiles, c, halo,
                       static_cast<char*>(out));
  else
    hipLaunchKernelGGL(csa_fixup_kernel<DT_F32>, dim3(n_tiles), dim3(256), 0, stream, tiles, c, halo,
                       static_cast<char*>(out));
  return hipGetLastError();
}

}  // namespace seqcomp
