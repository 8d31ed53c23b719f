// Tile planner (one or more workgroups): splits every sequence of a packed batch into tiles of at most
// `tile_rows` rows made of complete blocks of m rows (a sequence of L tokens
// has floor(L/m) entries; the tail block is dropped), and records where each
// tile's entries go in the packed output.
#include <algorithm>

#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void plan_tiles_kernel(const int64_t* __restrict__ cu, int batch,
                                                                  int m, int tile_rows,
                                                                  TileRec* __restrict__ tiles, int capacity) {
  __shared__ int s_tile_end[kPlanThreads];   // inclusive prefix of tiles per sequence (this chunk)
  __shared__ int s_ent_end[kPlanThreads];    // inclusive prefix of entries per sequence
  __shared__ int s_row0[kPlanThreads];
  __shared__ int s_rows[kPlanThreads];
  __shared__ int s_base_tile, s_base_ent;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_base_tile = 0;
    s_base_ent = 0;
  }
  __syncthreads();
  for (int b0 = 0; b0 < batch; b0 += kPlanThreads) {
    const int b = b0 + tid;
    int nt = 0, ne = 0, row0 = 0;
    if (b < batch) {
      const int64_t start = cu[b];
      const int64_t len = cu[b + 1] - start;
      ne = (int)(len / m);
      nt = (ne * m + tile_rows - 1) / tile_rows;
      row0 = (int)start;
    }
    s_tile_end[tid] = nt;
    s_ent_end[tid] = ne;
    s_row0[tid] = row0;
    s_rows[tid] = ne * m;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {   // Hillis-Steele inclusive scan
      const int a = tid >= off ? s_tile_end[tid - off] : 0;
      const int e = tid >= off ? s_ent_end[tid - off] : 0;
      __syncthreads();
      s_tile_end[tid] += a;
      s_ent_end[tid] += e;
      __syncthreads();
    }
    const int chunk_tiles = s_tile_end[kPlanThreads - 1];
    const int base_tile = s_base_tile, base_ent = s_base_ent;
    // Cooperative write: tile k of this chunk belongs to the first sequence
    // whose inclusive tile prefix exceeds k.  Every workgroup runs the same
    // scan; workgroup g writes the g-th of gridDim.x equal ranges of the
    // chunk's tiles.
    const int n_seq = min(kPlanThreads, batch - b0);      // sequences of this chunk
    const int per_wg = (chunk_tiles + (int)gridDim.x - 1) / (int)gridDim.x;
    const int k_lo = (int)blockIdx.x * per_wg, k_hi = min(chunk_tiles, k_lo + per_wg);
    for (int k = k_lo + tid; k < k_hi; k += kPlanThreads) {
      int lo = 0, hi = n_seq - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_tile_end[mid] > k) hi = mid; else lo = mid + 1;
      }
      const int seq_tile0 = lo ? s_tile_end[lo - 1] : 0;
      const int j = k - seq_tile0;
      const int ent0 = lo ? s_ent_end[lo - 1] : 0;
      TileRec r;
      r.row_start = s_row0[lo] + j * tile_rows;
      r.n_rows = min(tile_rows, s_rows[lo] - j * tile_rows);
      r.entry_start = base_ent + ent0 + j * (tile_rows / m);
      r.flags = (j == 0 ? TILE_FIRST : 0) | ((b0 + lo) << 1);
      const int idx = base_tile + k;
      if (idx < capacity) tiles[idx] = r;
    }
    __syncthreads();
    if (tid == 0) {
      s_base_tile += chunk_tiles;
      s_base_ent += s_ent_end[kPlanThreads - 1];
    }
    __syncthreads();
  }
}

}  // namespace

int device_cu_count() {
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

int64_t count_tiles(const int64_t* cu, int64_t batch, int64_t m, int64_t tile_rows) {
  int64_t n = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t rows = ((cu[b + 1] - cu[b]) / m) * m;
    n += (rows + tile_rows - 1) / tile_rows;
  }
  return n;
}

hipError_t launch_plan(const int64_t* cu_dev, int batch, int m, int tile_rows, TileRec* tiles, int n_tiles,
                       hipStream_t stream) {
  // one workgroup per 1024 tile records (at most 128): a single workgroup took
  // 40-55 us to write the 65536 records of the long-context CSA pooling call
  const int wgs = std::max(1, std::min(128, (n_tiles + 1023) / 1024));
  hipLaunchKernelGGL(plan_tiles_kernel, dim3(wgs), dim3(kPlanThreads), 0, stream, cu_dev, batch, m, tile_rows,
                     tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace seqcomp
