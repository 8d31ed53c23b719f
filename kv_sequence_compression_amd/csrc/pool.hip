// Pooling-only kernels: the compressor's softmax pooling over streams that
// are already in HBM (the unfused path).  HBM-bound: every input element is
// read exactly once, every entry written once.
//
// CSA ("序列压缩注意力", eq. attn-seqcomp-csa-softmax / -pool / -overlap-bound):
//   entry i, channel ch:  softmax over the 2m logits
//     Z^a[m i + r] + B^a[r]      (r < m, block i, a-stream)
//     Z^b[m(i-1) + r] + B^b[r]   (r < m, block i-1, b-stream; -inf for i = 0)
//   applied to C^a / C^b of the same rows.
// HCA (eq. attn-seqcomp-hca): softmax over Z[m i + r] + B[r], r < m, on C.
//
// Work split: a workgroup takes one tile (rows of one sequence); a thread
// takes (entry, 8-channel vector) items and streams the entry's rows with an
// online max / sum (fp32, base-2 exponent on logits pre-scaled by log2 e).
#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kPoolThreads = 256;

// Fold up to R rows (row k valid iff k < nvalid) into 8 per-channel online
// softmax accumulators.  z, v: logit and value rows; bias: B rows (fp32, row
// stride c floats) for the same rows.
template <int R>
__device__ __forceinline__ void fold_rows(SoftAcc (&acc)[8], const float (&z)[R][8], const float (&v)[R][8],
                                          const float (&bias)[R][8], int nvalid) {
  // No FMA contraction: the normaliser S and the numerator A take the same
  // roundings, so value rows of ones give entries of exactly one.
#pragma clang fp contract(off)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float l[R];
    float top = acc[j].M;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      l[k] = k < nvalid ? (z[k][j] + bias[k][j]) * kLog2e : -INFINITY;
      top = fmaxf(top, l[k]);
    }
    if (top == -INFINITY) continue;            // no valid row yet
    const float scale = exp2_hw(acc[j].M - top);
    float S = acc[j].S * scale;
    float A = acc[j].A * scale;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (k < nvalid) {                        // rows past nvalid were not loaded
        const float w = exp2_hw(l[k] - top);
        S += w;
        A = fmaf(w, v[k][j], A);
      }
    }
    acc[j].M = top;
    acc[j].S = S;
    acc[j].A = A;
  }
}

template <int DOUT>
__device__ __forceinline__ void finish_store(const SoftAcc (&acc)[8], char* dst) {
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = acc[j].A / acc[j].S;
  store8<DOUT>(dst, o);
}

template <int DIN, int DOUT>
__global__ __launch_bounds__(kPoolThreads) void pool_csa_kernel(
    const char* __restrict__ Ca, const char* __restrict__ Cb, const char* __restrict__ Za,
    const char* __restrict__ Zb, int64_t ld_bytes, const float* __restrict__ Ba, const float* __restrict__ Bb,
    int m, int c, const TileRec* __restrict__ tiles, char* __restrict__ out) {
  constexpr int ES = DTypeSize<DIN>::value;
  constexpr int OS = DTypeSize<DOUT>::value;
  const TileRec t = tiles[blockIdx.x];
  const int nv = c >> 3;
  const int ne = t.n_rows / m;
  const int items = ne * nv;
  for (int it = threadIdx.x; it < items; it += kPoolThreads) {
    const int e = it / nv;
    const int v = it - e * nv;
    const int64_t ra = (int64_t)t.row_start + (int64_t)e * m;   // first a-stream row
    const bool has_b = e > 0 || !(t.flags & TILE_FIRST);        // entry 0 of a sequence has no b rows
    const int64_t col = (int64_t)v * 8 * ES;
    SoftAcc acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) softacc_init(acc[j]);
    for (int r0 = 0; r0 < m; r0 += 4) {
      const int na = min(4, m - r0);
      const int nb = has_b ? na : 0;
      float za[4][8], ca[4][8], ba[4][8], zb[4][8], cb[4][8], bb[4][8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < na) {
          const int64_t row = ra + r0 + k;
          load8<DIN>(Za + row * ld_bytes + col, za[k]);
          load8<DIN>(Ca + row * ld_bytes + col, ca[k]);
          load8<DT_F32>(Ba + (int64_t)(r0 + k) * c + v * 8, ba[k]);
        }
        if (k < nb) {
          const int64_t row = ra - m + r0 + k;
          load8<DIN>(Zb + row * ld_bytes + col, zb[k]);
          load8<DIN>(Cb + row * ld_bytes + col, cb[k]);
          load8<DT_F32>(Bb + (int64_t)(r0 + k) * c + v * 8, bb[k]);
        }
      }
      fold_rows<4>(acc, za, ca, ba, na);
      fold_rows<4>(acc, zb, cb, bb, nb);
    }
    finish_store<DOUT>(acc, out + ((int64_t)(t.entry_start + e) * c + v * 8) * OS);
  }
}

template <int DIN, int DOUT>
__global__ __launch_bounds__(kPoolThreads) void pool_hca_kernel(
    const char* __restrict__ C, const char* __restrict__ Z, int64_t ld_bytes, const float* __restrict__ B, int m,
    int c, const TileRec* __restrict__ tiles, char* __restrict__ out) {
  constexpr int ES = DTypeSize<DIN>::value;
  constexpr int OS = DTypeSize<DOUT>::value;
  constexpr int R = 8;
  const TileRec t = tiles[blockIdx.x];
  const int nv = c >> 3;
  const int ne = t.n_rows / m;
  const int items = ne * nv;
  for (int it = threadIdx.x; it < items; it += kPoolThreads) {
    const int e = it / nv;
    const int v = it - e * nv;
    const int64_t r_first = (int64_t)t.row_start + (int64_t)e * m;
    const int64_t col = (int64_t)v * 8 * ES;
    SoftAcc acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) softacc_init(acc[j]);
    for (int r0 = 0; r0 < m; r0 += R) {
      const int nr = min(R, m - r0);
      float z[R][8], x[R][8], b[R][8];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (k < nr) {
          const int64_t row = r_first + r0 + k;
          load8<DIN>(Z + row * ld_bytes + col, z[k]);
          load8<DIN>(C + row * ld_bytes + col, x[k]);
          load8<DT_F32>(B + (int64_t)(r0 + k) * c + v * 8, b[k]);
        }
      }
      fold_rows<R>(acc, z, x, b, nr);
    }
    finish_store<DOUT>(acc, out + ((int64_t)(t.entry_start + e) * c + v * 8) * OS);
  }
}

}  // namespace

hipError_t launch_pool_csa(int in_dt, int out_dt, const void* Ca, const void* Cb, const void* Za, const void* Zb,
                           int64_t ld_in, const float* Ba, const float* Bb, int m, int c, const TileRec* tiles,
                           int n_tiles, void* out, hipStream_t stream) {
  const int64_t ldb = ld_in * (in_dt == DT_BF16 ? 2 : 4);
  const dim3 grid(n_tiles), block(kPoolThreads);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, (const char*)Ca, (const char*)Cb, (const char*)Za,
                       (const char*)Zb, ldb, Ba, Bb, m, c, tiles, (char*)out);
  };
  if (in_dt == DT_BF16 && out_dt == DT_BF16) args(pool_csa_kernel<DT_BF16, DT_BF16>);
  else if (in_dt == DT_BF16 && out_dt == DT_F32) args(pool_csa_kernel<DT_BF16, DT_F32>);
  else if (in_dt == DT_F32 && out_dt == DT_BF16) args(pool_csa_kernel<DT_F32, DT_BF16>);
  else args(pool_csa_kernel<DT_F32, DT_F32>);
  return hipGetLastError();
}

hipError_t launch_pool_hca(int in_dt, int out_dt, const void* C, const void* Z, int64_t ld_in, const float* B,
                           int m, int c, const TileRec* tiles, int n_tiles, void* out, hipStream_t stream) {
  const int64_t ldb = ld_in * (in_dt == DT_BF16 ? 2 : 4);
  const dim3 grid(n_tiles), block(kPoolThreads);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, (const char*)C, (const char*)Z, ldb, B, m, c, tiles,
                       (char*)out);
  };
  if (in_dt == DT_BF16 && out_dt == DT_BF16) args(pool_hca_kernel<DT_BF16, DT_BF16>);
  else if (in_dt == DT_BF16 && out_dt == DT_F32) args(pool_hca_kernel<DT_BF16, DT_F32>);
  else if (in_dt == DT_F32 && out_dt == DT_BF16) args(pool_hca_kernel<DT_F32, DT_BF16>);
  else args(pool_hca_kernel<DT_F32, DT_F32>);
  return hipGetLastError();
}

}  // namespace seqcomp
