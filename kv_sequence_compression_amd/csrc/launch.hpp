// Host-side launchers of the seqcomp kernels.  Arguments are validated by
// the C ABI layer (abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace seqcomp {

// Rows per tile of the CSA pooling kernel: 4 waves x epw entries of m rows,
// epw = 512 / min(c, 512) entries per wave (64 lanes x 8 channels).
inline int pool_csa_tile_rows(int m, int64_t c) { return 4 * (512 / (int)(c < 512 ? c : 512)) * m; }
// Rows per tile of the HCA pooling kernels.  m <= 128: the whole-row kernel,
// 8 / ceil(m / 16) entries per tile (one workgroup of 8 waves, ceil(m / 16)
// waves per entry); 128 < m <= 256: whole blocks of about 1024 rows, a
// multiple of 4 blocks (the 4 waves of a workgroup share them and the bias
// slice staged once for all of them).
constexpr int kPoolHcaRowsMaxM = 128;
inline int pool_hca_tile_rows(int m) {
  return m <= kPoolHcaRowsMaxM ? (8 / ((m + 15) / 16)) * m : m * 4 * ((1024 / m + 3) / 4);
}
constexpr int kPoolCsaMaxM = 16;
constexpr int kPoolHcaMaxM = 256;
constexpr int kFusedTileRows = 256;   // MFMA macro-tile height (tokens)

// Compute units of the current device (cached per device).
int device_cu_count();

// Host mirror of the device planner: number of tiles of a packed batch.
int64_t count_tiles(const int64_t* cu, int64_t batch, int64_t m, int64_t tile_rows);

// Writes the tile table of a packed batch (one workgroup).
hipError_t launch_plan(const int64_t* cu_dev, int batch, int m, int tile_rows,
                       TileRec* tiles, int n_tiles, hipStream_t stream);

// CSA pooling over tiles; out is [E x c] of out_dt (DT_F32 or DT_BF16).
hipError_t launch_pool_csa(int in_dt, int out_dt, const void* Ca, const void* Cb, const void* Za,
                           const void* Zb, int64_t ld_in, const float* Ba, const float* Bb, int m, int c,
                           const TileRec* tiles, int n_tiles, void* out, hipStream_t stream);

// HCA pooling over tiles; out is [E x c] of out_dt (DT_F32 or DT_BF16).
hipError_t launch_pool_hca(int in_dt, int out_dt, const void* C, const void* Z, int64_t ld_in,
                           const float* B, int m, int c, const TileRec* tiles, int n_tiles, void* out,
                           hipStream_t stream);

// Per-entry scaled OCP E4M3 encoding of fp32 entries [E x c].
hipError_t launch_quant_fp8(const float* src, int64_t E, int c, uint8_t* out, float* scale,
                            hipStream_t stream);

// Y[T x n_out] = H[T x d] * Wt[n_out x d]^T.
hipError_t launch_project(int in_dt, int out_dt, const void* H, int64_t T, int d, const void* Wt,
                          int n_out, void* Y, int64_t ld_y, hipStream_t stream);

// Fused compressor.  `out` receives DT_F32 or DT_BF16 entries.  For CSA,
// `halo` holds per tile the fp32 (M, S, A) triples of the first block's
// a-stream and the last block's b-stream (6 * c floats per tile); the fix-up
// kernel then writes the first entry of every tile that continues a sequence.
// `tiles` is the planner's table, or NULL for batches of at most
// kTileLookupMaxBatch sequences: the kernels then find their tiles from
// cu_dev themselves (tile_lookup), and no planner launch is needed.
hipError_t launch_fused(int mode, int in_dt, int out_dt, const void* H, int d, const void* Wt, int c,
                        const float* Ba, const float* Bb, const TileRec* tiles, const int64_t* cu_dev, int batch,
                        int n_tiles, void* out, float* halo, hipStream_t stream);

// CSA decode append: nb independent blocks of 4 rows of H; entry j merges
// block j's a-partial with state_in[j] (the previous block's b-partial, fp32
// [nb][3][c]) and block j's b-partial goes to state_out[j].  One or two
// blocks run a kernel with a wave per weight row; batches whose 256 x 256
// tiles fill the chip run the big-tile kernel; the others run 128 x 128
// tiles with the K loop split over up to 32 workgroups per tile,
// `partial` (append_partial_bytes(nb, c) bytes, null when that is 0)
// holding their fp32 products until a reduce kernel adds them and runs the
// same epilogue.
hipError_t launch_csa_append(int in_dt, int out_dt, const void* H, int64_t nb, int d, const void* Wt, int c,
                             const float* Ba, const float* Bb, const float* state_in, float* state_out, void* out,
                             void* partial, hipStream_t stream);
size_t append_partial_bytes(int64_t nb, int c);

// Partial RoPE + mixed store of packed entries [E x c] (tiles of 64 entries
// with tile_rows = 64 m: the planner's table, or NULL for batches of at most
// kTileLookupMaxBatch sequences, whose workgroups look their tiles up).
constexpr int kRopeTileEntries = 64;
hipError_t launch_rope_store(int in_dt, const void* entries, int c, int m, const int64_t* cu_dev, int batch,
                             const int64_t* pos0_dev, int r, double rope_base, const int64_t* slots_dev,
                             int64_t n_slots, const TileRec* tiles, int n_tiles, uint8_t* nope, float* scale,
                             uint16_t* rope, hipStream_t stream);

// Lightning indexer: 64 heads of 128 bf16 dimensions; workgroups of 8
// queries of one sequence (tiles from the planner with m = 1, tile_rows = 8).
constexpr int kIndexerHeads = 64;
constexpr int kIndexerDim = 128;
constexpr int kIndexerTileQueries = 8;
constexpr int kIndexerMaxK = 1024;
hipError_t launch_indexer_topk(const void* q, const float* w, const void* keys, const int64_t* cu_k_dev,
                               const int32_t* n_valid, const TileRec* tiles, int n_tiles, int k, int32_t* out_idx,
                               float* out_score, hipStream_t stream);

// Dense shared-KV MQA with an attention sink over compressed entries: 128
// heads of 512 dims; one workgroup per query (tiles from the planner with
// m = 1, tile_rows = 1).  out_dt is DT_BF16 or DT_F32.
constexpr int kMqaHeads = 128;
constexpr int kMqaDim = 512;
hipError_t launch_mqa_sink(int out_dt, const void* q, const void* kv, const int64_t* cu_k_dev, const int32_t* n_valid,
                           const TileRec* tiles, int T, const void* k_sink, const void* v_sink, float scale, void* out,
                           float* lse, hipStream_t stream);

hipError_t launch_csa_fixup(int out_dt, const TileRec* tiles, const int64_t* cu_dev, int batch, int n_tiles, int c,
                            const float* halo, void* out, hipStream_t stream);

}  // namespace seqcomp
