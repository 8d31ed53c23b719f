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
// the planner); wave w stores entries w, w + 4, ...; lane l handles 8
// consecutive channels 8 l + 512 j.  The angle is reduced modulo 2 pi in
// double precision (positions reach 10^6 tokens and more) before sin / cos.
#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kRopeThreads = 256;

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

template <int DIN>
__global__ __launch_bounds__(kRopeThreads) void rope_store_kernel(
    const char* __restrict__ entries, int c, int m, const int64_t* __restrict__ cu, const int64_t* __restrict__ pos0,
    int r, double log2_base, const int64_t* __restrict__ slots, int64_t n_slots, const TileRec* __restrict__ tiles,
    uint8_t* __restrict__ nope, float* __restrict__ scale, uint16_t* __restrict__ rope) {
  constexpr int ES = DTypeSize<DIN>::value;
  const TileRec t = tiles[blockIdx.x];
  const int seq = tile_seq(t.flags);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ne = t.n_rows / m;
  const int cn = c - r;                                   // position-free dimensions
  // tokens from the sequence start to the tile's first block, plus the offset
  const double base_pos = (double)(t.row_start - cu[seq]) + (pos0 ? (double)pos0[seq] : 0.0) + 0.5 * (m - 1);
  const double two_pi = 6.283185307179586476925286766559;
  for (int k = w; k < ne; k += 4) {
    const int64_t e = (int64_t)t.entry_start + k;
    const int64_t slot = slots ? slots[e] : e;
    const bool store = slot >= 0 && slot < n_slots;       // out-of-range slots are not stored
    const char* row = entries + e * c * ES;
    // absolute maximum of the position-free part
    float amax = 0.f;
    for (int ch0 = 8 * lane; ch0 < cn; ch0 += 512) {
      float x[8];
      load8<DIN>(row + (int64_t)ch0 * ES, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
    }
    amax = wave_max_f(amax);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    if (store && lane == 0) scale[slot] = s;
    const double pos = base_pos + (double)k * m;
    for (int ch0 = 8 * lane; ch0 < c; ch0 += 512) {
      float x[8];
      load8<DIN>(row + (int64_t)ch0 * ES, x);           // the amax pass left it in the cache
      if (ch0 < cn) {
        uint2 q;
        q.x = f32_to_e4m3(x[0] / s) | (f32_to_e4m3(x[1] / s) << 8) | (f32_to_e4m3(x[2] / s) << 16) |
              (f32_to_e4m3(x[3] / s) << 24);
        q.y = f32_to_e4m3(x[4] / s) | (f32_to_e4m3(x[5] / s) << 8) | (f32_to_e4m3(x[6] / s) << 16) |
              (f32_to_e4m3(x[7] / s) << 24);
        if (store) *reinterpret_cast<uint2*>(nope + slot * cn + ch0) = q;
      } else {
        float y[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int kp = (ch0 - cn) / 2 + p;                          // pair index in the RoPE part
          const double theta = exp2(-2.0 * kp / r * log2_base);
          double a = pos * theta;
          a -= two_pi * rint(a / two_pi);
          double sn, cs;
          sincos(a, &sn, &cs);
          const double x0 = x[2 * p], x1 = x[2 * p + 1];
          y[2 * p] = (float)(x0 * cs - x1 * sn);
          y[2 * p + 1] = (float)(x0 * sn + x1 * cs);
        }
        if (store)
          *reinterpret_cast<uint4*>(rope + slot * r + (ch0 - cn)) =
              make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                         pack_bf16x2(y[6], y[7]));
      }
    }
  }
}

}  // namespace

hipError_t launch_rope_store(int in_dt, const void* entries, int c, int m, const int64_t* cu_dev,
                             const int64_t* pos0_dev, int r, double rope_base, const int64_t* slots_dev,
                             int64_t n_slots, const TileRec* tiles, int n_tiles, uint8_t* nope, float* scale,
                             uint16_t* rope, hipStream_t stream) {
  const double lb = log2(rope_base);
  if (in_dt == DT_BF16)
    hipLaunchKernelGGL(rope_store_kernel<DT_BF16>, dim3(n_tiles), dim3(kRopeThreads), 0, stream,
                       static_cast<const char*>(entries), c, m, cu_dev, pos0_dev, r, lb, slots_dev, n_slots, tiles,
                       nope, scale, rope);
  else
    hipLaunchKernelGGL(rope_store_kernel<DT_F32>, dim3(n_tiles), dim3(kRopeThreads), 0, stream,
                       static_cast<const char*>(entries), c, m, cu_dev, pos0_dev, r, lb, slots_dev, n_slots, tiles,
                       nope, scale, rope);
  return hipGetLastError();
}

}  // namespace seqcomp
