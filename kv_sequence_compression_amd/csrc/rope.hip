// Partial RoPE and mixed-precision store of compressed entries into a cache.
//
// "Ch 05 · HCA — 长上下文的全景镜" (section on partial RoPE): rotary position
// encoding turns adjacent pairs of dimensions by a position-dependent angle,
// on the last r (= 64 of 512) dimensions of an entry only; the entry's
// position is carried by the RoPE of the segment centre.  "混合压缩注意力双方
// 案解析" (section 3, mixed-precision storage): the RoPE dimensions are kept
// in bf16, the other KV values in fp8.
//
// Entry e of sequence b, compressing block i of that sequence, sits at
// position pos0[b] + m i + (m - 1) / 2.  Pair k of the RoPE part, columns
// (c - r + 2k, c - r + 2k + 1), turns by pos * base^(-2k / r).  The c - r
// position-free dimensions are stored as OCP E4M3 codes with the per-entry
// scale s = max |x| / 448 over those dimensions (1 if all zero), the r
// rotated ones as bf16 (round to nearest even).
//
// Workgroup = one tile of up to 64 entries of one sequence (tile table from
// the planner); lane l handles 8 consecutive channels.  The fp8 codes are
// those of x * (1 / s), which can differ by one code from rounding x / s
// only when x / s lies within an ulp of a rounding midpoint.
#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kRopeThreads = 256;

// Angle of pair `kp` at position `pos`, reduced to [-pi, pi] in double
// precision (positions of 10^6 tokens and more keep their accuracy), then
// sin / cos in single precision.
__device__ __forceinline__ void rope_sincos(double pos, double theta, float& sn, float& cs) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = pos * theta;
  a -= two_pi * rint(a / two_pi);
  sincosf((float)a, &sn, &cs);
}

// Encode and store one entry chunk (8 channels at ch0) of lane data x; a
// RoPE chunk turns its 4 pairs by the angles whose cos / sin are given.
template <int DIN>
__device__ __forceinline__ void store_chunk(const float (&x)[8], int ch0, int cn, float inv_s, const float (&cs)[4],
                                            const float (&sn)[4], bool store, int64_t slot, int r,
                                            uint8_t* __restrict__ nope, uint16_t* __restrict__ rope) {
  if (ch0 < cn) {
    uint2 q;
    q.x = pack_e4m3x4(x[0] * inv_s, x[1] * inv_s, x[2] * inv_s, x[3] * inv_s);
    q.y = pack_e4m3x4(x[4] * inv_s, x[5] * inv_s, x[6] * inv_s, x[7] * inv_s);
    if (store) *reinterpret_cast<uint2*>(nope + slot * cn + ch0) = q;
  } else {
    float y[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      y[2 * p] = x[2 * p] * cs[p] - x[2 * p + 1] * sn[p];
      y[2 * p + 1] = x[2 * p] * sn[p] + x[2 * p + 1] * cs[p];
    }
    if (store)
      *reinterpret_cast<uint4*>(rope + slot * r + (ch0 - cn)) =
          make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
  }
}

// c <= 512: a lane holds the 8 channels 8 l of G entries at a time, all their
// loads in flight together; wave w takes entries G w + g, G w + g + 4 G, ...
// Larger c: one entry at a time, 8 channels 8 l + 512 j per lane, two passes
// over the row (the second hits the cache).
// Entries are read exactly once: non-temporal 16-byte loads.
typedef unsigned int rope_u32x4_t __attribute__((ext_vector_type(4)));
template <int DIN>
__device__ __forceinline__ void load8_stream(const char* p, float (&x)[8]) {
  const rope_u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const rope_u32x4_t*>(p));
  if (DIN == DT_BF16) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const rope_u32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const rope_u32x4_t*>(p + 16));
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y); x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y); x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  }
}

// LOOKUP: the workgroup finds its tile from the sequence offsets (tile_lookup,
// at most kTileLookupMaxBatch sequences) instead of the planner's table; a
// separate instantiation, so the kernel that reads the table is unchanged.
template <int DIN, bool LOOKUP = false>
__global__ __launch_bounds__(kRopeThreads) void rope_store_kernel(
    const char* __restrict__ entries, int c, int m, const int64_t* __restrict__ cu, const int64_t* __restrict__ pos0,
    int r, double log2_base, const int64_t* __restrict__ slots, int64_t n_slots, const TileRec* __restrict__ tiles,
    uint8_t* __restrict__ nope, float* __restrict__ scale, uint16_t* __restrict__ rope, int batch) {
  constexpr int ES = DTypeSize<DIN>::value;
  constexpr int G = 4;
  const TileRec t = LOOKUP ? tile_lookup(cu, batch, m, m * kRopeTileEntries, blockIdx.x) : tiles[blockIdx.x];
  const int seq = tile_seq(t.flags);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ne = t.n_rows / m;
  const int cn = c - r;                                   // position-free dimensions
  // tokens from the sequence start to the tile's first block centre, plus the offset
  const double base_pos = (double)(t.row_start - cu[seq]) + (pos0 ? (double)pos0[seq] : 0.0) + 0.5 * (m - 1);
  if (c <= 512) {
    const int ch0 = 8 * lane;
    const bool active = ch0 < c;
    const bool rope_lane = active && ch0 >= cn;
    // the lane's 4 pair frequencies and the turn of one block (m tokens):
    // consecutive entries of a group follow by one complex multiplication
    double theta[4];
    float step_c[4], step_s[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      theta[p] = rope_lane ? exp2(-2.0 * ((ch0 - cn) / 2 + p) / r * log2_base) : 0.0;
      rope_sincos((double)m, theta[p], step_s[p], step_c[p]);
    }
    for (int k0 = G * w; k0 < ne; k0 += 4 * G) {
      float x[G][8];
      int64_t slot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int k = min(k0 + g, ne - 1);                // past the tile end: re-read the last entry, store nothing
        const int64_t e = (int64_t)t.entry_start + k;
        slot[g] = slots ? slots[e] : e;
        if (active) load8_stream<DIN>(entries + (e * c + ch0) * ES, x[g]);
        else
#pragma unroll
          for (int j = 0; j < 8; ++j) x[g][j] = 0.f;
      }
      float cs[4], sn[4];
      if (rope_lane)
#pragma unroll
        for (int p = 0; p < 4; ++p) rope_sincos(base_pos + (double)k0 * m, theta[p], sn[p], cs[p]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float amax = 0.f;
        if (ch0 < cn)
#pragma unroll
          for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[g][j]));
        amax = wave_max_f32(amax);
        const float s = amax > 0.f ? amax / 448.0f : 1.0f;
        const bool store = k0 + g < ne && slot[g] >= 0 && slot[g] < n_slots;   // out-of-range rows are not stored
        if (store && lane == 0) scale[slot[g]] = s;
        if (active) store_chunk<DIN>(x[g], ch0, cn, 1.0f / s, cs, sn, store, slot[g], r, nope, rope);
        if (rope_lane)
#pragma unroll
          for (int p = 0; p < 4; ++p) {                   // advance to the next entry: angle + m theta
            const float c2 = cs[p] * step_c[p] - sn[p] * step_s[p];
            sn[p] = sn[p] * step_c[p] + cs[p] * step_s[p];
            cs[p] = c2;
          }
      }
    }
    return;
  }
  for (int k = w; k < ne; k += 4) {
    const int64_t e = (int64_t)t.entry_start + k;
    const int64_t slot = slots ? slots[e] : e;
    const bool store = slot >= 0 && slot < n_slots;
    const char* row = entries + e * c * ES;
    float amax = 0.f;
    for (int ch0 = 8 * lane; ch0 < cn; ch0 += 512) {
      float x[8];
      load8<DIN>(row + (int64_t)ch0 * ES, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
    }
    amax = wave_max_f32(amax);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    if (store && lane == 0) scale[slot] = s;
    const double pos = base_pos + (double)k * m;
    for (int ch0 = 8 * lane; ch0 < c; ch0 += 512) {
      float x[8];
      load8<DIN>(row + (int64_t)ch0 * ES, x);
      float cs[4], sn[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const double theta = ch0 >= cn ? exp2(-2.0 * ((ch0 - cn) / 2 + p) / r * log2_base) : 0.0;
        rope_sincos(pos, theta, sn[p], cs[p]);
      }
      store_chunk<DIN>(x, ch0, cn, 1.0f / s, cs, sn, store, slot, r, nope, rope);
    }
  }
}

}  // namespace

hipError_t launch_rope_store(int in_dt, const void* entries, int c, int m, const int64_t* cu_dev, int batch,
                             const int64_t* pos0_dev, int r, double rope_base, const int64_t* slots_dev,
                             int64_t n_slots, const TileRec* tiles, int n_tiles, uint8_t* nope, float* scale,
                             uint16_t* rope, hipStream_t stream) {
  const double lb = log2(rope_base);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(n_tiles), dim3(kRopeThreads), 0, stream, static_cast<const char*>(entries), c, m,
                       cu_dev, pos0_dev, r, lb, slots_dev, n_slots, tiles, nope, scale, rope, batch);
  };
  if (in_dt == DT_BF16) tiles ? args(rope_store_kernel<DT_BF16>) : args(rope_store_kernel<DT_BF16, true>);
  else tiles ? args(rope_store_kernel<DT_F32>) : args(rope_store_kernel<DT_F32, true>);
  return hipGetLastError();
}

}  // namespace seqcomp
