// Measurement only (loaded by bench.py, not by the library): ceilings the
// library's kernels are held against.
//
// 1. seqcomp_probe_stream_mix: the memory traffic of the CSA pooling call
// with no arithmetic.
// Entry e reads rows 4e..4e+3 of Z^a and C^a and rows 4e-4..4e-1 of Z^b and
// C^b (its own rows again for e = 0), 1 KiB each, with non-temporal loads,
// in the order the pooling kernel uses: every wave of the chip takes entries
// w, w + W, w + 2W, ... (W waves in all).  With `write` set it stores one
// 1 KiB row per entry (the XOR of what it read), 16 bytes read per byte
// written as in the pooling call with bf16 output; without, it stores only
// under a condition the data never meets, so the loads cannot be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ uint4 ld_stream(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(256) void stream_mix_kernel(const char* __restrict__ Ca, const char* __restrict__ Cb,
                                                         const char* __restrict__ Za, const char* __restrict__ Zb,
                                                         int64_t n_entries, char* __restrict__ out, int write) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + w, nw = (int64_t)gridDim.x * 4;
  const int64_t col = lane * 16;
  for (int64_t e = gw; e < n_entries; e += nw) {
    const int64_t ra = e * 4;
    uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t rb = e > 0 ? ra - 4 + k : ra + k;
      const uint4 a = ld_stream(Za + (ra + k) * 1024 + col), b = ld_stream(Ca + (ra + k) * 1024 + col);
      const uint4 c = ld_stream(Zb + rb * 1024 + col), d = ld_stream(Cb + rb * 1024 + col);
      acc.x ^= a.x ^ b.y ^ c.z ^ d.w;
      acc.y ^= a.y ^ b.z ^ c.w ^ d.x;
      acc.z ^= a.z ^ b.w ^ c.x ^ d.y;
      acc.w ^= a.w ^ b.x ^ c.y ^ d.z;
    }
    if (write || acc.x == 0x9E3779B9u) *reinterpret_cast<uint4*>(out + e * 1024 + col) = acc;
  }
}

// 2. The bf16 matrix cores with nothing else to do: each wave keeps 16
// independent 32x32 accumulators and feeds v_mfma_f32_32x32x16_bf16 from 8
// A and 8 B fragments of random bf16 data held in registers, rotating them
// so that every instruction sees other operands (as in a GEMM, where the
// operands change every k-step).  One wave per SIMD, as in the tile kernels.
// The sustained rate under load is the power-limited ceiling of that
// instruction on this chip.
__global__ __launch_bounds__(256, 1) void mfma_kernel(const uint4* __restrict__ data, int iters,
                                                      float* __restrict__ out) {
  const uint4* src = data + ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  f32x4_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 x = src[i], y = src[8 + i];
    a[i] = __builtin_bit_cast(f32x4_t, x);
    b[i] = __builtin_bit_cast(f32x4_t, y);
  }
  f32x16_t acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = f32x16_t{};
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[(q + u) & 7]),
                                                         __builtin_bit_cast(bf16x8_t, b[(3 * q + u) & 7]), acc[q],
                                                         0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[q][e];
  if (s == 1234.5f) out[blockIdx.x * 256 + threadIdx.x] = s;   // never met; keeps the loop
}

}  // namespace

// data: 256 x (#CUs) x 256 lanes x 256 bytes of random bf16 (one workgroup
// per CU reads its own), iters a multiple of 8; out: one float per thread,
// written only under a condition the data never meets.  FLOPs of a call:
// iters x 16 x 32768 x 4 waves x #CUs.
extern "C" int seqcomp_probe_mfma(const void* data, int iters, float* out, void* stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  hipLaunchKernelGGL(mfma_kernel, dim3(cus), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(data), iters, out);
  return (int)hipGetLastError();
}

// Streams: [4 n_entries x 512] bf16 each (1 KiB rows), out: [n_entries x 512]
// bf16.  Returns 0, or the HIP error code of the launch.
extern "C" int seqcomp_probe_stream_mix(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                                        int64_t n_entries, void* out, int write, void* stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  hipLaunchKernelGGL(stream_mix_kernel, dim3(4 * cus), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(Ca), static_cast<const char*>(Cb), static_cast<const char*>(Za),
                     static_cast<const char*>(Zb), n_entries, static_cast<char*>(out), write);
  return (int)hipGetLastError();
}
