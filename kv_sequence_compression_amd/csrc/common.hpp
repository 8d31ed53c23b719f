// Device-side helpers shared by the seqcomp kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seqcomp {

// One tile of rows of ONE sequence.  Tiles never cross sequences; a tile's
// rows all belong to complete blocks of m rows.
struct TileRec {
  int32_t row_start;    // first row (packed-batch row index)
  int32_t n_rows;       // rows of complete blocks in this tile (multiple of m, > 0)
  int32_t entry_start;  // packed index of the tile's first entry
  int32_t flags;        // TILE_FIRST: the tile starts its sequence
};
static_assert(sizeof(TileRec) == 16, "tile record is one 16-byte load");
enum : int32_t { TILE_FIRST = 1 };
// flags bits 1..31: index of the tile's sequence in the packed batch
__host__ __device__ inline int tile_seq(int32_t flags) { return (int)((uint32_t)flags >> 1); }

// Tile k of a packed batch of at most kTileLookupMaxBatch sequences, the
// record the planner would write, computed by one wave from the sequence
// offsets: lane b takes sequence b (floor(L_b / m) entries, their rows cut
// into tiles of tile_rows), two inclusive scans over the lanes give every
// sequence's first tile and first entry, and tile k belongs to the first
// sequence whose tiles end past k.  Every lane of the wave must take part;
// the result is wave-uniform.  k must be below the batch's tile count.
constexpr int kTileLookupMaxBatch = 64;
__device__ __forceinline__ TileRec tile_lookup(const int64_t* __restrict__ cu, int batch, int m, int tile_rows,
                                               int k) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));   // keep the scans inside a caller's persistent loop
  int row0 = 0, ne = 0;
  if (lane < batch) {
    const int64_t start = cu[lane];
    row0 = (int)start;
    ne = (int)((cu[lane + 1] - start) / m);
  }
  const int nt = (int)(((int64_t)ne * m + tile_rows - 1) / tile_rows);
  int tend = nt, eend = ne;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(tend, off, 64);
    const int e = __shfl_up(eend, off, 64);
    if (lane >= off) {
      tend += a;
      eend += e;
    }
  }
  const unsigned long long past = __ballot(tend > k);
  const int s = past ? __ffsll(past) - 1 : 0;
  const int t0 = __shfl(tend - nt, s, 64);
  const int e0 = __shfl(eend - ne, s, 64);
  const int r0 = __shfl(row0, s, 64);
  const int rows = __shfl(ne * m, s, 64);
  const int j = k - t0;
  TileRec r;
  r.row_start = __builtin_amdgcn_readfirstlane(r0 + j * tile_rows);
  r.n_rows = __builtin_amdgcn_readfirstlane(min(tile_rows, rows - j * tile_rows));
  r.entry_start = __builtin_amdgcn_readfirstlane(e0 + j * (tile_rows / m));
  r.flags = __builtin_amdgcn_readfirstlane((j == 0 ? TILE_FIRST : 0) | (s << 1));
  return r;
}

enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

// log2(e): exp(x) = 2^(x * log2 e); v_exp_f32 evaluates 2^x.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// bfloat16 round-to-nearest-even of a finite float (the compressor produces
// no NaN or infinity): add half an ulp of the kept part, plus one if the
// kept part is odd, then truncate.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// The same packing through gfx950's conversion instruction
// (v_cvt_pk_bf16_f32, round to nearest even): one instruction for two values.
// Equal to pack_bf16x2 on finite inputs.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Cross-lane exchanges in registers, with no LDS round trip (__shfl_xor
// compiles to ds_bpermute).  Lane index = threadIdx.x % 64 (blocks of whole
// waves).  gfx950: DPP row_ror:8 within each row of 16 lanes;
// v_permlane16_swap exchanges rows 0 <-> 1 and 2 <-> 3; v_permlane32_swap
// the two halves.  Each swap returns the pair (first operand, second operand)
// after the exchange: with both operands x, a lane of an even row (lower
// half) finds its partner's value in the second, of an odd row (upper half)
// in the first.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v);
__device__ __forceinline__ float lane_xor8(float x) { return dpp_f32<0x128>(x); }   // row_ror:8
__device__ __forceinline__ float lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Maximum over the 64 lanes of a wave, in every lane: DPP quad swaps and
// row mirrors give each row of 16 its maximum, the two swaps combine rows.
// Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));      // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f32<0x4E>(x));      // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f32<0x141>(x));     // row_half_mirror
  x = fmaxf(x, dpp_f32<0x140>(x));     // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Four OCP E4M3FN codes packed little-endian in a word: v_cvt_pk_fp8_f32
// rounds to nearest even into the OCP E4M3FN grid on gfx950 (a sweep of every
// fp32 magnitude below 512, both signs, gave the same codes as f32_to_e4m3
// below); clamping to +-448 first gives the saturating encoding.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const auto sat = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

// OCP E4M3FN encoding of a float: saturate |x| to 448 (the largest finite
// value, 1.75 * 2^8), round to nearest even.  Below 2^-6 the grid is the
// subnormal step 2^-9, so the code is rint(|x| * 512) (8 is the smallest
// normal, whose fields are exponent 1, mantissa 0).  Above, keep 3 of the 23
// mantissa bits with round-half-even on the fp32 bit pattern and rebias the
// exponent from 127 to 7.  The sign bit is copied, so -0 encodes as 0x80.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
  }
  return sign | code;
}

// Online softmax accumulator of one channel: running max M (in log2 units),
// running sum S of 2^(l - M) and running weighted sum A of 2^(l - M) * v.
struct SoftAcc {
  float M, S, A;
};

__device__ __forceinline__ void softacc_init(SoftAcc& s) {
  s.M = -INFINITY;
  s.S = 0.f;
  s.A = 0.f;
}

// Merge two partial accumulators (exact up to rounding: rescale both to the
// larger maximum).  Either side may be empty (M = -inf, S = A = 0).
// One exponential: the side with the larger maximum keeps factor 1 (what
// 2^(M - M) gives exactly), the other gets 2^-|x.M - y.M|.
__device__ __forceinline__ SoftAcc softacc_merge(SoftAcc x, SoftAcc y) {
#pragma clang fp contract(off)
  const float M = fmaxf(x.M, y.M);
  if (M == -INFINITY) return x;
  const float dm = x.M - y.M;                       // +-inf when one side is empty
  const float e = exp2_hw(-fabsf(dm));
  const bool x_top = dm >= 0.f;
  const float fx = x_top ? 1.f : e;
  const float fy = x_top ? e : 1.f;
  SoftAcc r;
  r.M = M;
  r.S = x.S * fx + y.S * fy;
  r.A = x.A * fx + y.A * fy;
  return r;
}

template <int N>
struct Vec {
  float v[N];
};

// 16-byte vector load / store through the vector memory path.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Load 8 consecutive channels of one row as floats.
template <int DT>
__device__ __forceinline__ void load8(const void* row_ptr, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<DT_BF16>(const void* p, float (&x)[8]) {
  const uint4 u = ld16(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<DT_F32>(const void* p, float (&x)[8]) {
  const uint4 a = ld16(p);
  const uint4 b = ld16(reinterpret_cast<const char*>(p) + 16);
  x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
  x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
  x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
  x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
}

// Store 8 consecutive channels (bf16 or fp32).
template <int DT>
__device__ __forceinline__ void store8(void* p, const float (&x)[8]);

template <>
__device__ __forceinline__ void store8<DT_BF16>(void* p, const float (&x)[8]) {
  st16(p, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                     pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
}

template <>
__device__ __forceinline__ void store8<DT_F32>(void* p, const float (&x)[8]) {
  st16(p, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])));
  st16(reinterpret_cast<char*>(p) + 16,
       make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])));
}

template <int DT>
struct DTypeSize;
template <>
struct DTypeSize<DT_F32> { static constexpr int value = 4; };
template <>
struct DTypeSize<DT_BF16> { static constexpr int value = 2; };

}  // namespace seqcomp
