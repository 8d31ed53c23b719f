// Pooling-only kernels: the compressor's softmax pooling over streams that
// are already in HBM (the unfused path).  HBM-bound: every input element is
// read exactly once and every entry written once, so the design goal is bytes
// in flight: few registers per lane (high occupancy), 16-byte loads issued
// back to back, biases served from LDS.
//
// CSA ("序列压缩注意力", eq. attn-seqcomp-csa-softmax / -pool / -overlap-bound):
//   entry i, channel ch:  softmax over the 2m logits
//     Z^a[m i + r] + B^a[r]      (r < m, block i, a-stream)
//     Z^b[m(i-1) + r] + B^b[r]   (r < m, block i-1, b-stream; -inf for i = 0)
//   applied to C^a / C^b of the same rows.
// HCA (eq. attn-seqcomp-hca): softmax over Z[m i + r] + B[r], r < m, on C.
//
// Logits are kept in log2 units (bias pre-scaled by log2 e in LDS, so the
// logit is one fma) and exponentiated with v_exp_f32; the per-channel online
// softmax state is (max, sum, weighted sum) in fp32.
#include <algorithm>

#include "launch.hpp"

namespace seqcomp {

namespace {

typedef __attribute__((address_space(3))) float lds_f32;   // LDS pointer: ds_read, 32-bit address

constexpr int kPoolThreads = 256;
constexpr int kCsaSlice = 512;    // channels per CSA workgroup
constexpr int kHcaSlice = 64;     // channels per HCA wave (8 lanes x 8 channels)

// Raw 16-byte row chunk: 8 bf16 or 4 fp32 (an fp32 chunk of 8 channels is two).
template <int DIN>
struct Raw8 {
  uint4 u[DIN == DT_BF16 ? 1 : 2];
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streamed input: every byte is read exactly once, so the loads are
// non-temporal (measured on MI355X: ~6.8 TB/s for such reads against
// ~6.1 TB/s for ordinary loads).
__device__ __forceinline__ uint4 ld16_stream(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int DIN>
__device__ __forceinline__ void ld_raw(Raw8<DIN>& r, const char* p) {
  r.u[0] = ld16_stream(p);
  if (DIN == DT_F32) r.u[DIN == DT_F32 ? 1 : 0] = ld16_stream(p + 16);
}

template <int DIN>
__device__ __forceinline__ float raw_get(const Raw8<DIN>& r, int j) {
  if (DIN == DT_BF16) {
    const uint32_t w = j < 2 ? r.u[0].x : j < 4 ? r.u[0].y : j < 6 ? r.u[0].z : r.u[0].w;
    return (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  } else {
    const uint4& q = r.u[(j >> 2) & (DIN == DT_F32 ? 1 : 0)];
    const int k = j & 3;
    return __uint_as_float(k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w);
  }
}

// Stage rows [0, m) of a bias slice (channels [ch0, ch0 + width)) into LDS as
// log2(e) * B, row stride `width`.  All threads of the block take part; each
// issues 4 independent 16-byte loads (indices past the end re-read the last
// element) before its first store, so the staging costs a few memory
// latencies instead of one per element.
__device__ __forceinline__ void stage_bias(lds_f32* dst, const float* __restrict__ B, int m, int c, int ch0,
                                           int width) {
  const int w4 = width >> 2;                       // c % 16 == 0 and ch0 % 64 == 0: 16-byte aligned
  const int n4 = m * w4;
  for (int base = 0; base < n4; base += 4 * kPoolThreads) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(base + u * kPoolThreads + (int)threadIdx.x, n4 - 1);
      const int r = i / w4, j = i - r * w4;
      v[u] = *reinterpret_cast<const float4*>(B + (int64_t)r * c + ch0 + 4 * j);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * kPoolThreads + (int)threadIdx.x;
      if (i < n4) {
        const int r = i / w4, j = i - r * w4;
        lds_f32* d = dst + r * width + 4 * j;
        d[0] = v[u].x * kLog2e;
        d[1] = v[u].y * kLog2e;
        d[2] = v[u].z * kLog2e;
        d[3] = v[u].w * kLog2e;
      }
    }
  }
}

// Fold 8 rows of 8 channels into the online softmax state with ONE rescale.
// Row k takes part iff bit k of `valid` is set (at least one is); the others
// were loaded from a valid row (finite values) and get logit -inf, hence
// weight exactly 0, so the code has no branches.  Two passes over the rows
// (maximum, then exponentials and sums) recompute the logit from the raw
// 16-byte loads and the LDS bias instead of keeping 64 logits live.
// MASKED = false drops the per-element selects for kernels whose chunks are
// always full (HCA with m' % 64 == 0); a runtime choice between the two in
// one kernel raised the register count past 3 waves per SIMD and was slower.
template <int DIN, bool MASKED = true>
__device__ __forceinline__ void fold_chunk(SoftAcc (&acc)[8], const Raw8<DIN> (&z)[8], const Raw8<DIN> (&v)[8],
                                           const lds_f32* const (&bias)[8], uint32_t valid) {
  // No FMA contraction of the sums: the normaliser S and the numerator A take
  // the same roundings, so value rows of ones give entries of exactly one.
#pragma clang fp contract(off)
  float top[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) top[j] = acc[j].M;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool ok = !MASKED || ((valid >> k) & 1u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float l = fmaf(raw_get<DIN>(z[k], j), kLog2e, bias[k][j]);
      top[j] = fmaxf(top[j], ok ? l : -INFINITY);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float scale = exp2_hw(acc[j].M - top[j]);   // 0 while the state is empty
    acc[j].S *= scale;
    acc[j].A *= scale;
    acc[j].M = top[j];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool ok = !MASKED || ((valid >> k) & 1u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float l = fmaf(raw_get<DIN>(z[k], j), kLog2e, bias[k][j]);
      const float w = exp2_hw((ok ? l : -INFINITY) - top[j]);
      acc[j].S += w;
      acc[j].A = fmaf(w, raw_get<DIN>(v[k], j), acc[j].A);
    }
  }
}

template <int DOUT>
__device__ __forceinline__ void store1_pool(char* out, int64_t idx, float v) {
  if (DOUT == DT_BF16) reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits(v);
  else reinterpret_cast<float*>(out)[idx] = v;
}

template <int DOUT>
__device__ __forceinline__ void store_entry8(const SoftAcc (&acc)[8], char* dst) {
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = acc[j].A / acc[j].S;
  store8<DOUT>(dst, o);
}

// CSA: a persistent grid.  Each workgroup stages the bias of its channel
// slice (512 channels, grid.y) once, then walks tiles blockIdx.x,
// blockIdx.x + gridDim.x, ...; a tile holds 4 * epw entries of one sequence
// and wave w takes entries [w epw, (w + 1) epw) of it, lane = (entry q,
// 8-channel vector v) with epw = 512 / min(c, 512) entries per wave.  So all
// waves of the chip sweep the streams together inside a window of a few
// thousand entries: measured on the long-context workload, 5.69 TB/s against
// 5.40 TB/s when every workgroup owned a 64-entry tile (a window of 192 MB
// per stream), with identical output.  Rows are taken four a-rows plus the
// matching four b-rows at a time.
template <int DIN, int DOUT>
__global__ __launch_bounds__(kPoolThreads) void pool_csa_kernel(
    const char* __restrict__ Ca, const char* __restrict__ Cb, const char* __restrict__ Za,
    const char* __restrict__ Zb, int64_t ld_bytes, const float* __restrict__ Ba, const float* __restrict__ Bb,
    int m, int c, const TileRec* __restrict__ tiles, int n_tiles, char* __restrict__ out) {
  constexpr int ES = DTypeSize<DIN>::value;
  constexpr int OS = DTypeSize<DOUT>::value;
  extern __shared__ float sB_[];                // [2][m][width]: log2e * B^a, log2e * B^b
  lds_f32* sB = (lds_f32*)sB_;
  const int ch0 = blockIdx.y * kCsaSlice;
  const int width = min(kCsaSlice, c - ch0);
  lds_f32* sBa = sB;
  lds_f32* sBb = sB + m * width;
  stage_bias(sBa, Ba, m, c, ch0, width);
  stage_bias(sBb, Bb, m, c, ch0, width);
  __syncthreads();
  const int nv_full = min(c, kCsaSlice) >> 3;         // vectors per entry of a full slice
  const int epw = 64 / nv_full;                       // entries per wave (tile rows: 4 epw m)
  const int nv = width >> 3;                          // vectors of this slice
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane / nv_full, vl = lane - q * nv_full;
  const bool lane_ok = q < epw && vl < nv;
  const int v = lane_ok ? vl : 0;                     // idle lanes re-read vector 0 and store nothing
  const int eq = w * epw + (q < epw ? q : 0);         // entry of the lane within the tile
  const int64_t col = (int64_t)(ch0 + v * 8) * ES;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const TileRec t = tiles[tile];
    const int ne = t.n_rows / m;
    if (w * epw >= ne) continue;                      // wave-uniform: no entry of this wave in the tile
    const int e = min(eq, ne - 1);                    // lanes past the tile's entries re-read its last one
    const bool ok = lane_ok && eq < ne;
    const int64_t ra = (int64_t)t.row_start + (int64_t)e * m;   // first a-stream row
    const bool has_b = e > 0 || !(t.flags & TILE_FIRST);        // entry 0 of a sequence has no b rows
    SoftAcc acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) softacc_init(acc[j]);
#pragma unroll 1
    for (int r0 = 0; r0 < m; r0 += 4) {
      const int na = min(4, m - r0);
      Raw8<DIN> z[8], x[8];
      const lds_f32* bias[8];
      // slots 0..3: a rows r0..r0+3 of block i; slots 4..7: b rows of block
      // i-1.  Missing rows re-read a valid row and are masked off.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = min(r0 + k, m - 1);
        const int64_t row_a = ra + r;
        const int64_t row_b = has_b ? ra - m + r : row_a;
        ld_raw<DIN>(z[k], Za + row_a * ld_bytes + col);
        ld_raw<DIN>(x[k], Ca + row_a * ld_bytes + col);
        ld_raw<DIN>(z[4 + k], Zb + row_b * ld_bytes + col);
        ld_raw<DIN>(x[4 + k], Cb + row_b * ld_bytes + col);
        bias[k] = &sBa[r * width + v * 8];
        bias[4 + k] = &sBb[r * width + v * 8];
      }
      const uint32_t amask = (1u << na) - 1u;
      const uint32_t valid = amask | (has_b ? amask << 4 : 0u);
      fold_chunk<DIN>(acc, z, x, bias, valid);
    }
    if (ok) store_entry8<DOUT>(acc, out + ((int64_t)(t.entry_start + e) * c + ch0 + v * 8) * OS);
  }
}

// HCA: workgroup = (64-channel slice, tile of entries); wave w takes entries
// w, w + 4, ... of the tile (the bias slice is staged once for all of them).  Lane = 8 g + v: vector v (8 channels) of the slice and row
// group g, which folds rows g, g + 8, g + 16, ... (so one load instruction
// reads 8 consecutive rows); three butterfly merges combine the row groups.
template <int DIN, int DOUT, bool FULL>
__global__ __launch_bounds__(kPoolThreads) void pool_hca_kernel(
    const char* __restrict__ C, const char* __restrict__ Z, int64_t ld_bytes, const float* __restrict__ B, int m,
    int c, const TileRec* __restrict__ tiles, int n_tiles, char* __restrict__ out) {
  constexpr int ES = DTypeSize<DIN>::value;
  constexpr int OS = DTypeSize<DOUT>::value;
  extern __shared__ float sB_[];                  // [m][width]: log2e * B slice
  lds_f32* sB = (lds_f32*)sB_;
  // 1-D grid.  The hardware hands workgroup w to XCD w mod 8; XCD x takes
  // tiles x, x + 8, x + 16, ... and all channel slices of a tile one after
  // the other, so the slices of a row are read by one XCD close in time
  // (measured: 63% -> 69% of HBM peak against the slices of a tile spread
  // over all eight XCDs).
  const int n_slices = (c + kHcaSlice - 1) / kHcaSlice;
  const int xw = blockIdx.x & 7, kw = blockIdx.x >> 3;
  const int tile = xw + 8 * (kw / n_slices);
  if (tile >= n_tiles) return;                    // the grid is padded to 8 tiles
  const TileRec t = tiles[tile];
  const int ch0 = (kw % n_slices) * kHcaSlice;
  const int width = min(kHcaSlice, c - ch0);
  stage_bias(sB, B, m, c, ch0, width);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 3, v = lane & 7;
  const bool vok = v * 8 < width;
  const int vv = vok ? v : 0;                     // lanes past the slice re-read vector 0, store nothing
  const int64_t col = (int64_t)(ch0 + vv * 8) * ES;
  const int ne = t.n_rows / m;
  for (int e = w; e < ne; e += 4) {               // entries w, w + 4, ... of the tile
    const int64_t r_first = (int64_t)t.row_start + (int64_t)e * m;
    SoftAcc acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) softacc_init(acc[j]);
#pragma unroll 1
    for (int r0 = g; r0 < m; r0 += 64) {          // this lane's rows r0, r0 + 8, ..., r0 + 56
      Raw8<DIN> z[8], x[8];
      const lds_f32* bias[8];
      uint32_t valid = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = r0 + 8 * k;
        valid |= (r < m ? 1u : 0u) << k;
        const int rr = min(r, m - 1);             // rows past the block re-read its last row, masked off
        const int64_t row = r_first + rr;
        ld_raw<DIN>(z[k], Z + row * ld_bytes + col);
        ld_raw<DIN>(x[k], C + row * ld_bytes + col);
        bias[k] = &sB[rr * width + vv * 8];
      }
      fold_chunk<DIN, !FULL>(acc, z, x, bias, valid);
    }
    // row groups g ^ 1, g ^ 2, g ^ 4 are lanes l ^ 8, l ^ 16, l ^ 32: exchanged
    // in registers (DPP, lane swaps), not through LDS
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      SoftAcc s = acc[j];
      s = softacc_merge(s, SoftAcc{lane_xor8(s.M), lane_xor8(s.S), lane_xor8(s.A)});
      s = softacc_merge(s, SoftAcc{lane_xor16(s.M), lane_xor16(s.S), lane_xor16(s.A)});
      s = softacc_merge(s, SoftAcc{lane_xor32(s.M), lane_xor32(s.S), lane_xor32(s.A)});
      acc[j] = s;
    }
    if (g == 0 && vok) store_entry8<DOUT>(acc, out + ((int64_t)(t.entry_start + e) * c + ch0 + v * 8) * OS);
  }
}

// HCA for m <= 128, reading whole rows: a persistent workgroup of 8 waves
// takes a tile of epe = 8 / wpe entries of one sequence at a time (wpe =
// ceil(m / 16) waves per entry); wave w covers rows [16 (w % wpe),
// 16 (w % wpe) + 16) of entry w / wpe and lane l channels [8 l, 8 l + 8) of
// the workgroup's 512-channel slice, so one load instruction reads a whole
// row of Z or C (the read pattern that streams fastest: 6.6 TB/s in a probe
// against 6.2 TB/s for 8 rows x 128 bytes).  The lane's 16 x 8 biases stay in
// registers for the whole sweep.  A wave folds its rows into (max, sum,
// weighted sum) per channel; the states of an entry's waves meet in LDS and
// thread t merges channel t, in wave order.  Measured on the long-context
// workload: 6.3 TB/s, against 5.9 TB/s for the 64-channel-slice kernel below.
constexpr int kHcaRowThreads = 512;
constexpr int kHcaRowsPerWave = 16;

template <int DIN, int DOUT>
__global__ __launch_bounds__(kHcaRowThreads) void pool_hca_rows_kernel(
    const char* __restrict__ C, const char* __restrict__ Z, int64_t ld_bytes, const float* __restrict__ B, int m,
    int c, const TileRec* __restrict__ tiles, int n_tiles, char* __restrict__ out) {
  // No FMA contraction of the sums: the normaliser and the numerator take the
  // same roundings, so value rows of ones give entries of exactly one.
#pragma clang fp contract(off)
  constexpr int ES = DTypeSize<DIN>::value;
  constexpr int OS = DTypeSize<DOUT>::value;
  constexpr int RC = DIN == DT_BF16 ? 4 : 2;          // rows per load chunk (registers in flight)
  __shared__ float xs[8][3][kCsaSlice];              // 48 KiB: (M, S, A) of every channel, per wave
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ch0 = blockIdx.y * kCsaSlice;
  const int width = min(kCsaSlice, c - ch0);
  const int wpe = (m + kHcaRowsPerWave - 1) / kHcaRowsPerWave;   // waves per entry
  const int epe = 8 / wpe;                                         // entries per tile
  const int q = w / wpe, r0 = (w - q * wpe) * kHcaRowsPerWave;     // the wave's entry and first row
  const bool lane_ok = lane * 8 < width;
  const int v = lane_ok ? lane : 0;
  const int64_t col = (int64_t)(ch0 + v * 8) * ES;
  float bias[kHcaRowsPerWave][8];
#pragma unroll
  for (int r = 0; r < kHcaRowsPerWave; ++r) {
    const int rr = min(r0 + r, m - 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) bias[r][j] = B[(int64_t)rr * c + ch0 + v * 8 + j] * kLog2e;
  }
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const TileRec t = tiles[tile];
    const int ne = t.n_rows / m;
    const bool active = q < epe && q < ne;            // wave-uniform
    SoftAcc acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) softacc_init(acc[j]);
    if (active) {
      const int64_t row0 = (int64_t)t.row_start + (int64_t)q * m;
#pragma unroll
      for (int h = 0; h < kHcaRowsPerWave / RC; ++h) {
        Raw8<DIN> z[RC], x[RC];
#pragma unroll
        for (int k = 0; k < RC; ++k) {
          const int r = min(r0 + h * RC + k, m - 1);  // rows past the block re-read its last row, masked off
          ld_raw<DIN>(z[k], Z + (row0 + r) * ld_bytes + col);
          ld_raw<DIN>(x[k], C + (row0 + r) * ld_bytes + col);
        }
        float top[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) top[j] = acc[j].M;
#pragma unroll
        for (int k = 0; k < RC; ++k) {
          const bool ok = r0 + h * RC + k < m;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            top[j] = fmaxf(top[j], ok ? fmaf(raw_get<DIN>(z[k], j), kLog2e, bias[h * RC + k][j]) : -INFINITY);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float sc = exp2_hw(acc[j].M - top[j]);   // 0 while the state is empty
          acc[j].S *= sc;
          acc[j].A *= sc;
          acc[j].M = top[j];
        }
#pragma unroll
        for (int k = 0; k < RC; ++k) {
          const bool ok = r0 + h * RC + k < m;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float l = fmaf(raw_get<DIN>(z[k], j), kLog2e, bias[h * RC + k][j]);
            const float wt = exp2_hw((ok ? l : -INFINITY) - top[j]);
            acc[j].S += wt;
            acc[j].A = fmaf(wt, raw_get<DIN>(x[k], j), acc[j].A);
          }
        }
      }
    }
    __syncthreads();                                   // the previous tile's merges have read xs
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xs[w][0][lane * 8 + j] = acc[j].M;
      xs[w][1][lane * 8 + j] = acc[j].S;
      xs[w][2][lane * 8 + j] = acc[j].A;
    }
    __syncthreads();
    const int ch = threadIdx.x;                        // 512 threads: one channel of the slice each
    if (ch < width) {
      for (int e = 0; e < min(epe, ne); ++e) {
        SoftAcc mg{xs[e * wpe][0][ch], xs[e * wpe][1][ch], xs[e * wpe][2][ch]};
        for (int u = 1; u < wpe; ++u)
          mg = softacc_merge(mg, SoftAcc{xs[e * wpe + u][0][ch], xs[e * wpe + u][1][ch], xs[e * wpe + u][2][ch]});
        store1_pool<DOUT>(out, ((int64_t)(t.entry_start + e) * c + ch0 + ch), mg.A / mg.S);
      }
    }
  }
}

}  // namespace

hipError_t launch_pool_csa(int in_dt, int out_dt, const void* Ca, const void* Cb, const void* Za, const void* Zb,
                           int64_t ld_in, const float* Ba, const float* Bb, int m, int c, const TileRec* tiles,
                           int n_tiles, void* out, hipStream_t stream) {
  const int64_t ldb = ld_in * (in_dt == DT_BF16 ? 2 : 4);
  // two workgroups per compute unit walk the tiles (measured: 5.69 TB/s, against
  // 5.62 with three and 5.63 with four)
  const int P = (int)std::min<int64_t>(n_tiles, 2 * (int64_t)device_cu_count());
  const dim3 grid(P, (c + kCsaSlice - 1) / kCsaSlice), block(kPoolThreads);
  const size_t lds = (size_t)2 * m * min(c, kCsaSlice) * sizeof(float);   // <= 64 KiB for m <= 16
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, lds, stream, (const char*)Ca, (const char*)Cb, (const char*)Za,
                       (const char*)Zb, ldb, Ba, Bb, m, c, tiles, n_tiles, (char*)out);
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
  if (m <= kPoolHcaRowsMaxM) {
    // one workgroup of 8 waves per compute unit walks the tiles
    const dim3 grid((unsigned)std::min<int64_t>(n_tiles, device_cu_count()), (c + kCsaSlice - 1) / kCsaSlice),
        block(kHcaRowThreads);
    auto args = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, stream, (const char*)C, (const char*)Z, ldb, B, m, c, tiles, n_tiles,
                         (char*)out);
    };
    if (in_dt == DT_BF16 && out_dt == DT_BF16) args(pool_hca_rows_kernel<DT_BF16, DT_BF16>);
    else if (in_dt == DT_BF16 && out_dt == DT_F32) args(pool_hca_rows_kernel<DT_BF16, DT_F32>);
    else if (in_dt == DT_F32 && out_dt == DT_BF16) args(pool_hca_rows_kernel<DT_F32, DT_BF16>);
    else args(pool_hca_rows_kernel<DT_F32, DT_F32>);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((int64_t)(n_tiles + 7) / 8 * 8 * ((c + kHcaSlice - 1) / kHcaSlice))),
      block(kPoolThreads);
  const size_t lds = (size_t)m * min(c, kHcaSlice) * sizeof(float);      // <= 64 KiB for m <= 256
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, lds, stream, (const char*)C, (const char*)Z, ldb, B, m, c, tiles,
                       n_tiles, (char*)out);
  };
  // every fold step of a lane is 8 valid rows when m is a multiple of 64
  const bool full = m % 64 == 0;
  if (in_dt == DT_BF16 && out_dt == DT_BF16)
    full ? args(pool_hca_kernel<DT_BF16, DT_BF16, true>) : args(pool_hca_kernel<DT_BF16, DT_BF16, false>);
  else if (in_dt == DT_BF16 && out_dt == DT_F32)
    full ? args(pool_hca_kernel<DT_BF16, DT_F32, true>) : args(pool_hca_kernel<DT_BF16, DT_F32, false>);
  else if (in_dt == DT_F32 && out_dt == DT_BF16)
    full ? args(pool_hca_kernel<DT_F32, DT_BF16, true>) : args(pool_hca_kernel<DT_F32, DT_BF16, false>);
  else
    full ? args(pool_hca_kernel<DT_F32, DT_F32, true>) : args(pool_hca_kernel<DT_F32, DT_F32, false>);
  return hipGetLastError();
}

}  // namespace seqcomp
