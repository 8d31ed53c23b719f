// Projection GEMM and fused compressor on the gfx950 matrix cores.
//
// The projection ("序列压缩注意力", eq. attn-seqcomp-csa-proj) is the one
// dense contraction of the compressor: Y = H Wt^T with K = d.  One workgroup
// computes a 256 x 256 tile of Y with 4 wavefronts (2 x 2, each 128 x 128 as
// 8 x 8 v_mfma_f32_16x16x32_bf16 accumulators in registers).  K advances in
// 128-byte slabs (64 bf16 / 32 fp32) that are copied global -> LDS directly
// (global_load_lds_dwordx4, no register staging) into a 2-stage ring.
//
// The fused kernels keep that accumulator tile in registers and pool it
// there, so C and Z never reach HBM:
//  * the 16x16 MFMA accumulator gives every lane 4 consecutive token rows of
//    one channel, i.e. exactly one CSA block of m = 4 rows;
//  * the N tile is laid out so that each wavefront holds the SAME channels of
//    every stream (CSA: 32 channels x [C^a | C^b | Z^a | Z^b]; HCA: 64
//    channels x [C | Z]);
//  * CSA (eq. attn-seqcomp-csa-softmax / -pool): a lane folds its block's
//    a-rows into (max, sum, weighted sum) and its b-rows into the partial of
//    the NEXT entry; one 16-lane rotation hands the b-partial to the entry
//    that needs it (eq. attn-seqcomp-overlap-bound for the first block of a
//    sequence).  The first entry of a tile that continues a sequence needs
//    the previous tile's last block: both partials go to a small halo buffer
//    and a fix-up kernel merges them (log-sum-exp merge, exact up to
//    rounding);
//  * HCA (eq. attn-seqcomp-hca): a wave row of 128 tokens is one block of
//    m' = 128; lanes fold 32 rows each, then two butterfly merges combine the
//    four lane groups.
// Tiles are rows of one sequence (tile table from the planner); the grid is
// remapped so that all N tiles of an M panel run on the same XCD (shared L2).
#include "launch.hpp"

namespace seqcomp {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kTile = 256;                      // BM = BN = 256
constexpr int kRowBytes = 128;                  // bytes of one tile row per K slab
constexpr int kTileBytes = kTile * kRowBytes;   // 32 KiB per operand per stage
constexpr int kStages = 2;
constexpr int kLdsBytes = kStages * 2 * kTileBytes;

enum : int { MODE_PROJECT = 0, MODE_CSA = 1, MODE_HCA = 2 };

// 16-byte slot of k-chunk kc (0..7) in tile row r.  XOR swizzle so that the
// 16 lanes reading one k-chunk of 16 consecutive rows hit distinct LDS banks
// whether the banks are serviced in groups of 8 or of 16 lanes.
__device__ __forceinline__ int swz(int r, int kc) { return kc ^ (r & 7) ^ ((r >> 3) & 1); }

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

template <>
struct Frag<DT_BF16> {
  // one K slab = 64 bf16 = two k32 steps; a lane feeds 8 consecutive k.  The
  // eight B fragments of a step stay in registers; A fragments are read one
  // M subtile at a time so the 256 accumulators keep the AGPR file to themselves.
  static __device__ __forceinline__ void compute(const char* As, const char* Bs, int lane_off, int x, int lg,
                                                 int wm, int wn, f32x4_t (&acc)[8][8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int slot = ((h * 4 + lg) ^ x) * 16;
      bf16x8_t b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 128 + j * 16) * kRowBytes + lane_off + slot);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(As + (wm * 128 + i * 16) * kRowBytes + lane_off + slot);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
  }
};

template <>
struct Frag<DT_F32> {
  // one K slab = 32 fp32 = one k32 step made of eight 16x16x4 MFMAs; lane
  // (row, g = lane/16) feeds k = 8 g + t at step t, the same permutation of
  // k on both operands, so the dot products are unchanged.
  static __device__ __forceinline__ void compute(const char* As, const char* Bs, int lane_off, int x, int lg,
                                                 int wm, int wn, f32x4_t (&acc)[8][8]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int slot = ((lg * 2 + half) ^ x) * 16;
      f32x4_t a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i] = *reinterpret_cast<const f32x4_t*>(As + (wm * 128 + i * 16) * kRowBytes + lane_off + slot);
        b[i] = *reinterpret_cast<const f32x4_t*>(Bs + (wn * 128 + i * 16) * kRowBytes + lane_off + slot);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][t], b[j][t], acc[i][j], 0, 0, 0);
    }
  }
};

// Copy one 128-byte-wide K slab of 256 rows of one operand into LDS.  Wave w
// fills rows [64 w, 64 w + 64) with 8 instructions of 1 KiB (8 rows) each;
// lane p writes LDS slot p & 7 of row p >> 3, which holds k-chunk
// swz(row, p & 7) -- the same XOR, so reads find chunk kc at swz(row, kc).
__device__ __forceinline__ void load_slab(const char* base, const uint32_t (&off)[8], int64_t k_bytes, char* lds_tile,
                                          int w) {
  const char* kb = base + k_bytes;                  // uniform
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(kb + off[i]), (lds_void_t*)(lds_tile + (w * 8 + i) * 1024), 16,
                                     0, 0);
}

template <int DIN>
__device__ __forceinline__ void mainloop(const char* a_base, const uint32_t (&a_off)[8], const char* b_base,
                                         const uint32_t (&b_off)[8], int nk, char* lds, int w, int lane, int wm,
                                         int wn, f32x4_t (&acc)[8][8]) {
  const int lane_off = (lane & 15) * kRowBytes;
  const int x = (lane & 7) ^ ((lane >> 3) & 1);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_slab(a_base, a_off, 0, lds, w);
  load_slab(b_base, b_off, 0, lds + kTileBytes, w);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = lds + (kt & 1) * 2 * kTileBytes;
    if (kt + 1 < nk) {
      char* nxt = lds + ((kt + 1) & 1) * 2 * kTileBytes;
      load_slab(a_base, a_off, (int64_t)(kt + 1) * kRowBytes, nxt, w);
      load_slab(b_base, b_off, (int64_t)(kt + 1) * kRowBytes, nxt + kTileBytes, w);
    }
    Frag<DIN>::compute(cur, cur + kTileBytes, lane_off, x, lane >> 4, wm, wn, acc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

// Per-thread source rows of the two operands: thread (wave w, lane p) loads
// tile rows r_i = 64 w + 8 i + (p >> 3), i = 0..7, at k-chunk swz(r_i, p & 7).
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

__device__ __forceinline__ SoftAcc partial4(const f32x4_t& z, const f32x4_t& v, const float (&bias)[4]) {
  float l[4];
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    l[j] = (z[j] + bias[j]) * kLog2e;
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
__device__ void epilogue_project(const Args& a, f32x4_t (&acc)[8][8], int mt, int nt, int lane, int wm, int wn) {
  const int col = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = nt * kTile + wn * 128 + j * 16 + col;
      if (n >= a.n_out) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = (int64_t)mt * kTile + wm * 128 + i * 16 + g * 4 + r;
        if (row < a.T) store1<DOUT>(a.Y, row * a.ld_y + n, acc[i][j][r]);
      }
    }
  }
}

// CSA epilogue.  Wave (wm, wn), lane (g = lane / 16, col = lane % 16):
// accumulator [ms][2 s + h] holds rows 128 wm + 16 ms + 4 g + (0..3) of
// stream s (C^a, C^b, Z^a, Z^b) at channel 64 nt + 32 wn + 16 h + col.
template <int DOUT>
__device__ void epilogue_csa(const Args& a, f32x4_t (&acc)[8][8], const TileRec& t, int tile, int nt, int lane,
                             int wm, int wn, char* lds) {
  const int col = lane & 15, g = lane >> 4;
  const int c = a.c;
  float* xfer = reinterpret_cast<float*>(lds);       // [wn][h][col][3]: wave row 0 -> wave row 1
  float* halo = a.halo + (int64_t)tile * 6 * c;       // [Ma Sa Aa Mb Sb Ab] x c
  float ba[2][4], bb[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ch = nt * 64 + wn * 32 + h * 16 + col;
    const bool ok = ch < c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ba[h][r] = ok ? a.Ba[r * c + ch] : 0.f;
      bb[h][r] = ok ? a.Bb[r * c + ch] : 0.f;
    }
  }
  // The b-partial of each wave row's last block (block 31 / 63 of the tile).
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ch = nt * 64 + wn * 32 + h * 16 + col;
    const SoftAcc pb = partial4(acc[7][6 + h], acc[7][2 + h], bb[h]);
    if (g == 3 && wm == 0) {
      float* x = xfer + ((wn * 2 + h) * 16 + col) * 3;
      x[0] = pb.M;
      x[1] = pb.S;
      x[2] = pb.A;
    }
    if (g == 3 && wm == 1 && t.n_rows == kTile && ch < c) {   // the next tile continues the sequence
      halo[3 * c + ch] = pb.M;
      halo[4 * c + ch] = pb.S;
      halo[5 * c + ch] = pb.A;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ch = nt * 64 + wn * 32 + h * 16 + col;
    const bool ok = ch < c;
    SoftAcc carry;
    softacc_init(carry);
    if (wm == 1) {
      const float* x = xfer + ((wn * 2 + h) * 16 + col) * 3;
      carry.M = x[0];
      carry.S = x[1];
      carry.A = x[2];
    }
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) {
      const SoftAcc pa = partial4(acc[ms][4 + h], acc[ms][h], ba[h]);
      const SoftAcc pb = partial4(acc[ms][6 + h], acc[ms][2 + h], bb[h]);
      // Lane l takes the b-partial of lane l - 16 (the previous block); lanes
      // 0..15 receive lanes 48..63 = this subtile's last block, which is the
      // previous block for the first lanes of the NEXT subtile.
      const SoftAcc br = shfl_acc(pb, (lane + 48) & 63);
      const SoftAcc prev = g == 0 ? carry : br;
      carry = br;
      const int blk = wm * 32 + ms * 4 + g;            // block (= entry) index inside the tile
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
// [ms][q] holds C and [ms][4 + q] holds Z at channel 128 nt + 64 wn + 16 q + col.
template <int DOUT>
__device__ void epilogue_hca(const Args& a, f32x4_t (&acc)[8][8], const TileRec& t, int nt, int lane, int wm,
                             int wn) {
  const int col = lane & 15, g = lane >> 4;
  const int c = a.c;
  const bool block_ok = (wm + 1) * 128 <= t.n_rows;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ch = nt * 128 + wn * 64 + q * 16 + col;
    const bool ok = ch < c;
    SoftAcc s;
    softacc_init(s);
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) {
      float b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = ok ? a.Ba[(ms * 16 + g * 4 + r) * c + ch] : 0.f;
      s = softacc_merge(s, partial4(acc[ms][4 + q], acc[ms][q], b));
    }
    s = softacc_merge(s, shfl_xor_acc(s, 16));
    s = softacc_merge(s, shfl_xor_acc(s, 32));
    if (ok && block_ok && g == 0) store1<DOUT>(a.out, ((int64_t)t.entry_start + wm) * c + ch, s.A / s.S);
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
  uint32_t a_off[8], b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = w * 64 + i * 8 + (lane >> 3);
    const int kc = swz(r, lane & 7);
    a_off[i] = (uint32_t)(min(r, nvalid - 1) * a.lda + kc * 16);
    b_off[i] = (uint32_t)((int64_t)b_row_of<MODE>(r, nt, a.c, a.n_out) * a.lda + kc * 16);
  }
  f32x4_t acc[8][8];
  mainloop<DIN>(a_base, a_off, a.Wt, b_off, a.nk, lds, w, lane, wm, wn, acc);
  if (MODE == MODE_PROJECT) epilogue_project<DOUT>(a, acc, mt, nt, lane, wm, wn);
  else if (MODE == MODE_CSA) epilogue_csa<DOUT>(a, acc, t, mt, nt, lane, wm, wn, lds);
  else epilogue_hca<DOUT>(a, acc, t, nt, lane, wm, wn);
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
