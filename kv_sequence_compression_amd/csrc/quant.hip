// Per-entry scaled FP8 (OCP E4M3FN) encoding of compressed entries.
//
// The mixed-precision KV storage described in "混合压缩注意力双方案解析"
// (section on the shared design: fp8 for the non-RoPE KV values) is taken
// here as: s_i = max_ch |x[i, ch]| / 448 (1 for an all-zero entry) and
// code[i, ch] = E4M3(x[i, ch] / s_i), saturating, round to nearest even.
//
// One wavefront per entry: lanes read 4-float chunks of the fp32 row,
// reduce the absolute maximum across the 64 lanes, then encode and store 4
// codes per chunk.  HBM-bound (4 bytes read + 1 written per element).
#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void quant_fp8_kernel(const float* __restrict__ src, int64_t E, int c,
                                                                  uint8_t* __restrict__ out,
                                                                  float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * kQuantThreads) >> 6;
  const int nq = c >> 2;                       // float4 chunks per entry
  for (int64_t e = wave; e < E; e += n_waves) {
    const float4* row = reinterpret_cast<const float4*>(src + e * c);
    float amax = 0.f;
    for (int q = lane; q < nq; q += 64) {
      const float4 x = row[q];
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
    amax = wave_max_f32(amax);          // in registers: DPP and lane swaps
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    uint32_t* orow = reinterpret_cast<uint32_t*>(out + e * c);
    for (int q = lane; q < nq; q += 64) {
      const float4 x = row[q];                 // second read hits the cache
      orow[q] = pack_e4m3x4(x.x / s, x.y / s, x.z / s, x.w / s);
    }
    if (lane == 0) scale[e] = s;
  }
}

}  // namespace

hipError_t launch_quant_fp8(const float* src, int64_t E, int c, uint8_t* out, float* scale, hipStream_t stream) {
  const int64_t waves_needed = E;
  int64_t blocks = (waves_needed + (kQuantThreads / 64) - 1) / (kQuantThreads / 64);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quant_fp8_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, src, E, c, out,
                     scale);
  return hipGetLastError();
}

}  // namespace seqcomp
