// C ABI of the seqcomp library: argument validation on the host, then the
// kernel launches on the caller's stream.  Declarations and the contract of
// every entry point are in include/seqcomp.h.
#include "seqcomp.h"

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "launch.hpp"

using namespace seqcomp;

namespace {

constexpr int kVersion = 10000;   // 1.0.0
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elt_size(int dt) { return dt == SEQCOMP_F32 ? 4 : dt == SEQCOMP_BF16 ? 2 : 1; }

inline bool valid_in_dtype(int dt) { return dt == SEQCOMP_F32 || dt == SEQCOMP_BF16; }
inline bool valid_out_dtype(int dt) { return dt == SEQCOMP_F32 || dt == SEQCOMP_BF16 || dt == SEQCOMP_FP8_E4M3; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Range {
  uintptr_t lo = 0, hi = 0;   // [lo, hi)
};

inline Range range_of(const void* p, size_t bytes) {
  Range r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + bytes;
  return r;
}

inline bool overlaps(Range a, Range b) {
  return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Rows [0, T) of a strided matrix: the last row ends at (T-1)*ld + cols.
inline size_t strided_bytes(int64_t T, int64_t ld, int64_t cols, int es) {
  if (T <= 0) return 0;
  return (size_t)(((T - 1) * ld + cols) * es);
}

// cu_seqlens: 0-based, non-decreasing, total rows within int32.
int check_cu(const int64_t* cu, int64_t batch, int64_t* total_rows) {
  if (batch < 0 || batch > (int64_t(1) << 30)) return SEQCOMP_E_SHAPE;
  if (!cu) return SEQCOMP_E_NULL;
  if (cu[0] != 0) return SEQCOMP_E_SEQLENS;
  for (int64_t b = 0; b < batch; ++b)
    if (cu[b + 1] < cu[b]) return SEQCOMP_E_SEQLENS;
  if (cu[batch] > kMaxRows) return SEQCOMP_E_SHAPE;
  *total_rows = cu[batch];
  return SEQCOMP_OK;
}

int64_t entries_of(const int64_t* cu, int64_t batch, int64_t m) {
  int64_t e = 0;
  for (int64_t b = 0; b < batch; ++b) e += (cu[b + 1] - cu[b]) / m;
  return e;
}

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return SEQCOMP_OK;
  if (e == hipErrorNotSupported) return SEQCOMP_E_UNSUPPORTED;
  return SEQCOMP_E_HIP;
}

// Workspace layout: [tile table | CSA halo triples (fused CSA) | fp32 staging (fp8 output)].
struct WsLayout {
  size_t tiles_off = 0, halo_off = 0, stage_off = 0, total = 0;
  int64_t n_tiles = 0;
};

WsLayout ws_layout(int op, int mode, int64_t m, int64_t c, const int64_t* cu, int64_t batch, int out_dtype) {
  WsLayout w;
  int64_t tile_rows;
  if (op == SEQCOMP_OP_POOL_CSA) tile_rows = pool_csa_tile_rows((int)m, c);
  else if (op == SEQCOMP_OP_POOL_HCA) tile_rows = pool_hca_tile_rows((int)m);
  else tile_rows = kFusedTileRows;
  w.n_tiles = count_tiles(cu, batch, m, tile_rows);
  const int64_t E = entries_of(cu, batch, m);
  size_t off = 0;
  w.tiles_off = off;
  off = round_up(off + (size_t)w.n_tiles * sizeof(TileRec), 256);
  w.halo_off = off;
  if (op == SEQCOMP_OP_FUSED && mode == SEQCOMP_MODE_CSA) off = round_up(off + (size_t)w.n_tiles * 6 * c * 4, 256);
  w.stage_off = off;
  if (out_dtype == SEQCOMP_FP8_E4M3) off = round_up(off + (size_t)E * c * 4, 256);
  w.total = (E == 0) ? 0 : off;
  return w;
}

// Output checks shared by the pooling and fused calls.
int check_output(int out_dtype, const void* out, const float* out_scale, int64_t E, int64_t c, Range* out_r,
                 Range* scale_r) {
  if (!valid_out_dtype(out_dtype)) return SEQCOMP_E_DTYPE;
  *out_r = Range();
  *scale_r = Range();
  if (E == 0) return SEQCOMP_OK;
  if (!out) return SEQCOMP_E_NULL;
  if (!aligned16(out)) return SEQCOMP_E_ALIGN;
  *out_r = range_of(out, (size_t)E * c * elt_size(out_dtype));
  if (out_dtype == SEQCOMP_FP8_E4M3) {
    if (!out_scale) return SEQCOMP_E_NULL;
    if (!aligned16(out_scale)) return SEQCOMP_E_ALIGN;
    *scale_r = range_of(out_scale, (size_t)E * 4);
    if (overlaps(*out_r, *scale_r)) return SEQCOMP_E_ALIAS;
  }
  return SEQCOMP_OK;
}

int check_workspace(const void* ws, size_t ws_bytes, size_t need, Range* ws_r) {
  *ws_r = Range();
  if (need == 0) return SEQCOMP_OK;
  if (!ws) return SEQCOMP_E_WORKSPACE;
  if (ws_bytes < need) return SEQCOMP_E_WORKSPACE;
  if (!aligned16(ws)) return SEQCOMP_E_ALIGN;
  *ws_r = range_of(ws, need);
  return SEQCOMP_OK;
}

// Any written range (outputs, workspace) overlapping any read range or another written range.
int check_alias(const Range* written, int nw, const Range* read, int nr) {
  for (int i = 0; i < nw; ++i) {
    for (int j = 0; j < nr; ++j)
      if (overlaps(written[i], read[j])) return SEQCOMP_E_ALIAS;
    for (int j = i + 1; j < nw; ++j)
      if (overlaps(written[i], written[j])) return SEQCOMP_E_ALIAS;
  }
  return SEQCOMP_OK;
}

// Pooling (fp32 staging when fp8 output), then the fp8 encoder.
int run_pool(bool csa, const void* const* streams, int64_t ld_in, int in_dtype, const float* Ba, const float* Bb,
             int64_t m, int64_t c, const int64_t* cu_dev, int64_t batch, int64_t E, void* out, int out_dtype,
             float* out_scale, void* ws, const WsLayout& L, hipStream_t st) {
  char* wsb = static_cast<char*>(ws);
  TileRec* tiles = reinterpret_cast<TileRec*>(wsb + L.tiles_off);
  const int op = csa ? SEQCOMP_OP_POOL_CSA : SEQCOMP_OP_POOL_HCA;
  const int tile_rows = op == SEQCOMP_OP_POOL_CSA ? pool_csa_tile_rows((int)m, c) : pool_hca_tile_rows((int)m);
  hipError_t e = launch_plan(cu_dev, (int)batch, (int)m, tile_rows, tiles, (int)L.n_tiles, st);
  if (e != hipSuccess) return hip_status(e);
  const bool fp8 = out_dtype == SEQCOMP_FP8_E4M3;
  void* dst = fp8 ? (void*)(wsb + L.stage_off) : out;
  const int dst_dt = fp8 ? DT_F32 : out_dtype;
  if (csa)
    e = launch_pool_csa(in_dtype, dst_dt, streams[0], streams[1], streams[2], streams[3], ld_in, Ba, Bb, (int)m,
                        (int)c, tiles, (int)L.n_tiles, dst, st);
  else
    e = launch_pool_hca(in_dtype, dst_dt, streams[0], streams[1], ld_in, Ba, (int)m, (int)c, tiles,
                        (int)L.n_tiles, dst, st);
  if (e != hipSuccess) return hip_status(e);
  if (fp8) e = launch_quant_fp8(reinterpret_cast<const float*>(dst), E, (int)c, static_cast<uint8_t*>(out),
                                out_scale, st);
  return hip_status(e);
}

int pool_common(bool csa, const void* const* streams, int n_streams, int64_t ld_in, int in_dtype,
                const float* Ba, const float* Bb, int64_t m, int64_t c, const int64_t* cu_host,
                const int64_t* cu_dev, int64_t batch, void* out, int out_dtype, float* out_scale, void* ws,
                size_t ws_bytes, void* stream) {
  if (!valid_in_dtype(in_dtype)) return SEQCOMP_E_DTYPE;
  if (!valid_out_dtype(out_dtype)) return SEQCOMP_E_DTYPE;
  if (m < 1 || m > (csa ? kPoolCsaMaxM : kPoolHcaMaxM)) return SEQCOMP_E_UNSUPPORTED;
  if (c < 16 || c % 16 != 0 || c > (int64_t(1) << 20)) return SEQCOMP_E_UNSUPPORTED;
  if (ld_in < c || ld_in > (int64_t(1) << 32)) return SEQCOMP_E_SHAPE;   // row offsets and byte ranges in int64
  const int es = elt_size(in_dtype);
  if ((ld_in * es) % 16 != 0) return SEQCOMP_E_ALIGN;
  int64_t T = 0;
  int st = check_cu(cu_host, batch, &T);
  if (st) return st;
  const int64_t E = entries_of(cu_host, batch, m);
  Range out_r, scale_r;
  if ((st = check_output(out_dtype, out, out_scale, E, c, &out_r, &scale_r))) return st;
  if (E == 0) return SEQCOMP_OK;
  for (int i = 0; i < n_streams; ++i) {
    if (!streams[i]) return SEQCOMP_E_NULL;
    if (!aligned16(streams[i])) return SEQCOMP_E_ALIGN;
  }
  if (!Ba || (csa && !Bb) || !cu_dev) return SEQCOMP_E_NULL;
  if (!aligned16(Ba) || (csa && !aligned16(Bb)) || !aligned16(cu_dev)) return SEQCOMP_E_ALIGN;
  const int op = csa ? SEQCOMP_OP_POOL_CSA : SEQCOMP_OP_POOL_HCA;
  const WsLayout L = ws_layout(op, 0, m, c, cu_host, batch, out_dtype);
  // one workgroup per (tile, channel slice of 512 / 64 channels) on a 32-bit grid
  if ((L.n_tiles + 7) / 8 * 8 * (csa ? 1 : (c + 63) / 64) >= (int64_t(1) << 31)) return SEQCOMP_E_UNSUPPORTED;
  Range ws_r;
  if ((st = check_workspace(ws, ws_bytes, L.total, &ws_r))) return st;
  Range reads[7];
  int nr = 0;
  for (int i = 0; i < n_streams; ++i) reads[nr++] = range_of(streams[i], strided_bytes(T, ld_in, c, es));
  reads[nr++] = range_of(Ba, (size_t)m * c * 4);
  if (csa) reads[nr++] = range_of(Bb, (size_t)m * c * 4);
  reads[nr++] = range_of(cu_dev, (size_t)(batch + 1) * 8);
  const Range writes[3] = {out_r, scale_r, ws_r};
  if ((st = check_alias(writes, 3, reads, nr))) return st;
  return run_pool(csa, streams, ld_in, in_dtype, Ba, Bb, m, c, cu_dev, batch, E, out, out_dtype, out_scale, ws, L,
                  static_cast<hipStream_t>(stream));
}

// Scratch of the allocation-free fused entry point: one array per device
// (each device that loads the library holds its own copy until the process
// ends).  Host code never uses the array's name as
// an address: it is a host-side stand-in.  The device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array.
int device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SEQCOMP_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SEQCOMP_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SEQCOMP_E_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return SEQCOMP_OK;
}

// The fused compressor behind both entry points.  With use_scratch the
// workspace arguments are ignored and the call runs in this device's
// file-scope scratch array instead (rejected when it needs more).
int fused_impl(int mode, int64_t m, const void* H, int64_t d, int in_dtype, const void* Wt, int64_t c,
               const float* Ba, const float* Bb, const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
               int64_t batch, void* out, int out_dtype, float* out_scale, void* workspace, size_t workspace_bytes,
               bool use_scratch, void* stream) {
  if (mode != SEQCOMP_MODE_CSA && mode != SEQCOMP_MODE_HCA) return SEQCOMP_E_UNSUPPORTED;
  const bool csa = mode == SEQCOMP_MODE_CSA;
  if ((csa && m != 4) || (!csa && m != 128)) return SEQCOMP_E_UNSUPPORTED;
  if (!valid_in_dtype(in_dtype)) return SEQCOMP_E_DTYPE;
  if (!valid_out_dtype(out_dtype)) return SEQCOMP_E_DTYPE;
  if (d < 64 || d % 64 != 0 || d > (int64_t(1) << 24)) return SEQCOMP_E_UNSUPPORTED;
  if (c < 16 || c % 16 != 0 || c > (int64_t(1) << 20)) return SEQCOMP_E_UNSUPPORTED;
  if (!csa && Bb) return SEQCOMP_E_SHAPE;
  // the kernels address one 256-row tile of H and all of Wt with 32-bit byte offsets
  if ((csa ? 4 : 2) * c * d * elt_size(in_dtype) >= (int64_t(1) << 32) ||
      256 * d * elt_size(in_dtype) >= (int64_t(1) << 32))
    return SEQCOMP_E_UNSUPPORTED;
  int64_t T = 0;
  int st = check_cu(cu_seqlens_host, batch, &T);
  if (st) return st;
  const int64_t E = entries_of(cu_seqlens_host, batch, m);
  Range out_r, scale_r;
  if ((st = check_output(out_dtype, out, out_scale, E, c, &out_r, &scale_r))) return st;
  if (E == 0) return SEQCOMP_OK;
  if (!H || !Wt || !Ba || (csa && !Bb) || !cu_seqlens_dev) return SEQCOMP_E_NULL;
  if (!aligned16(H) || !aligned16(Wt) || !aligned16(Ba) || (csa && !aligned16(Bb)) || !aligned16(cu_seqlens_dev))
    return SEQCOMP_E_ALIGN;
  const WsLayout L = ws_layout(SEQCOMP_OP_FUSED, mode, m, c, cu_seqlens_host, batch, out_dtype);
  const int es = elt_size(in_dtype);
  const int S = csa ? 4 : 2;
  Range reads[5];
  int nr = 0;
  reads[nr++] = range_of(H, (size_t)T * d * es);
  reads[nr++] = range_of(Wt, (size_t)S * c * d * es);
  reads[nr++] = range_of(Ba, (size_t)m * c * 4);
  if (csa) reads[nr++] = range_of(Bb, (size_t)m * c * 4);
  reads[nr++] = range_of(cu_seqlens_dev, (size_t)(batch + 1) * 8);
  if (use_scratch) {
    // the outputs against the inputs, then the scratch size: all host-side
    // checks come before the call's first HIP call (the scratch lookup)
    const Range outs[2] = {out_r, scale_r};
    if ((st = check_alias(outs, 2, reads, nr))) return st;
    if (L.total > kScratchBytes) return SEQCOMP_E_SCRATCH;
    if ((st = device_scratch(&workspace))) return st;
    workspace_bytes = kScratchBytes;
  }
  Range ws_r;
  if ((st = check_workspace(workspace, workspace_bytes, L.total, &ws_r))) return st;
  const Range writes[3] = {out_r, scale_r, ws_r};
  if ((st = check_alias(writes, 3, reads, nr))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(workspace);
  TileRec* tiles = reinterpret_cast<TileRec*>(wsb + L.tiles_off);
  float* halo = csa ? reinterpret_cast<float*>(wsb + L.halo_off) : nullptr;
  const bool fp8 = out_dtype == SEQCOMP_FP8_E4M3;
  void* dst = fp8 ? (void*)(wsb + L.stage_off) : out;
  const int dst_dt = fp8 ? DT_F32 : out_dtype;
  // Calls of at most two rounds of the persistent grid over few sequences:
  // the kernels look their tiles up from the offsets and the planner launch
  // goes (the 8192-token CSA call: 178 -> 175 us).  Longer calls keep the
  // planner's table, one load per tile instead of a lookup per tile.
  const int64_t n_nt = csa ? (c + 63) / 64 : (c + 127) / 128;
  const bool planned = batch > kTileLookupMaxBatch || L.n_tiles * n_nt > 2 * (int64_t)device_cu_count();
  hipError_t e = planned
                     ? launch_plan(cu_seqlens_dev, (int)batch, (int)m, kFusedTileRows, tiles, (int)L.n_tiles, s)
                     : hipSuccess;
  const TileRec* tt = planned ? tiles : nullptr;
  if (e == hipSuccess)
    e = launch_fused(mode, in_dtype, dst_dt, H, (int)d, Wt, (int)c, Ba, Bb, tt, cu_seqlens_dev, (int)batch,
                     (int)L.n_tiles, dst, halo, s);
  if (e == hipSuccess && csa)
    e = launch_csa_fixup(dst_dt, tt, cu_seqlens_dev, (int)batch, (int)L.n_tiles, (int)c, halo, dst, s);
  if (e == hipSuccess && fp8)
    e = launch_quant_fp8(reinterpret_cast<const float*>(dst), E, (int)c, static_cast<uint8_t*>(out), out_scale, s);
  return hip_status(e);
}

}  // namespace

extern "C" {

int seqcomp_version(void) { return kVersion; }

const char* seqcomp_status_string(int status) {
  switch (status) {
    case SEQCOMP_OK: return "ok";
    case SEQCOMP_E_NULL: return "a required pointer is NULL";
    case SEQCOMP_E_SHAPE: return "a size is out of range or sizes disagree";
    case SEQCOMP_E_DTYPE: return "dtype not supported for this argument";
    case SEQCOMP_E_ALIGN: return "pointer or row stride not 16-byte aligned";
    case SEQCOMP_E_ALIAS: return "an output overlaps an input or the workspace";
    case SEQCOMP_E_WORKSPACE: return "workspace missing or too small";
    case SEQCOMP_E_UNSUPPORTED: return "configuration not supported (m, d or c)";
    case SEQCOMP_E_HIP: return "HIP runtime call or kernel launch failed";
    case SEQCOMP_E_SEQLENS: return "cu_seqlens must start at 0 and be non-decreasing";
    case SEQCOMP_E_SCRATCH: return "the call needs more scratch than the allocation-free entry point holds (64 MiB)";
    default: return "unknown status";
  }
}

int64_t seqcomp_num_entries(const int64_t* cu_seqlens_host, int64_t batch, int64_t m) {
  int64_t T;
  if (m < 1 || check_cu(cu_seqlens_host, batch, &T) != SEQCOMP_OK) return -1;
  return entries_of(cu_seqlens_host, batch, m);
}

size_t seqcomp_workspace_bytes(int op, int mode, int64_t m, int64_t c, const int64_t* cu_seqlens_host,
                               int64_t batch, int out_dtype) {
  int64_t T;
  if (op < SEQCOMP_OP_POOL_CSA || op > SEQCOMP_OP_FUSED) return (size_t)-1;
  if (op == SEQCOMP_OP_FUSED && mode != SEQCOMP_MODE_CSA && mode != SEQCOMP_MODE_HCA) return (size_t)-1;
  if (m < 1 || c < 1 || !valid_out_dtype(out_dtype)) return (size_t)-1;
  if (check_cu(cu_seqlens_host, batch, &T) != SEQCOMP_OK) return (size_t)-1;
  return ws_layout(op, mode, m, c, cu_seqlens_host, batch, out_dtype).total;
}

int seqcomp_project(const void* H, int64_t T, int64_t d, int in_dtype, const void* Wt, int64_t n_out, void* Y,
                    int64_t ld_y, int out_dtype, void* stream) {
  if (!valid_in_dtype(in_dtype)) return SEQCOMP_E_DTYPE;
  if (out_dtype != SEQCOMP_F32 && out_dtype != SEQCOMP_BF16) return SEQCOMP_E_DTYPE;
  if (T < 0 || T > kMaxRows || d < 1 || n_out < 1 || ld_y < n_out) return SEQCOMP_E_SHAPE;
  if (d % 64 != 0 || n_out % 16 != 0 || d > (int64_t(1) << 24) || n_out > (int64_t(1) << 24))
    return SEQCOMP_E_UNSUPPORTED;
  if ((ld_y * elt_size(out_dtype)) % 16 != 0) return SEQCOMP_E_ALIGN;
  // the kernels address one 256-row tile of H and all of Wt with 32-bit byte offsets
  if (n_out * d * elt_size(in_dtype) >= (int64_t(1) << 32) || 256 * d * elt_size(in_dtype) >= (int64_t(1) << 32))
    return SEQCOMP_E_UNSUPPORTED;
  // ... and store one 256-row tile of Y through offsets below 2^31
  if (256 * ld_y * elt_size(out_dtype) >= (int64_t(1) << 31)) return SEQCOMP_E_UNSUPPORTED;
  if (T == 0) return SEQCOMP_OK;
  if (!H || !Wt || !Y) return SEQCOMP_E_NULL;
  if (!aligned16(H) || !aligned16(Wt) || !aligned16(Y)) return SEQCOMP_E_ALIGN;
  const int es = elt_size(in_dtype);
  const Range reads[2] = {range_of(H, (size_t)T * d * es), range_of(Wt, (size_t)n_out * d * es)};
  const Range writes[1] = {range_of(Y, strided_bytes(T, ld_y, n_out, elt_size(out_dtype)))};
  int st = check_alias(writes, 1, reads, 2);
  if (st) return st;
  return hip_status(launch_project(in_dtype, out_dtype, H, T, (int)d, Wt, (int)n_out, Y, ld_y,
                                   static_cast<hipStream_t>(stream)));
}

int seqcomp_pool_csa(const void* Ca, const void* Cb, const void* Za, const void* Zb, int64_t ld_in, int in_dtype,
                     const float* Ba, const float* Bb, int64_t m, int64_t c, const int64_t* cu_seqlens_host,
                     const int64_t* cu_seqlens_dev, int64_t batch, void* out, int out_dtype, float* out_scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const void* streams[4] = {Ca, Cb, Za, Zb};
  return pool_common(true, streams, 4, ld_in, in_dtype, Ba, Bb, m, c, cu_seqlens_host, cu_seqlens_dev, batch, out,
                     out_dtype, out_scale, workspace, workspace_bytes, stream);
}

int seqcomp_pool_hca(const void* C, const void* Z, int64_t ld_in, int in_dtype, const float* B, int64_t m, int64_t c,
                     const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev, int64_t batch, void* out,
                     int out_dtype, float* out_scale, void* workspace, size_t workspace_bytes, void* stream) {
  const void* streams[2] = {C, Z};
  return pool_common(false, streams, 2, ld_in, in_dtype, B, nullptr, m, c, cu_seqlens_host, cu_seqlens_dev, batch,
                     out, out_dtype, out_scale, workspace, workspace_bytes, stream);
}

int seqcomp_compress_fused(int mode, int64_t m, const void* H, int64_t d, int in_dtype, const void* Wt, int64_t c,
                           const float* Ba, const float* Bb, const int64_t* cu_seqlens_host,
                           const int64_t* cu_seqlens_dev, int64_t batch, void* out, int out_dtype,
                           float* out_scale, void* workspace, size_t workspace_bytes, void* stream) {
  return fused_impl(mode, m, H, d, in_dtype, Wt, c, Ba, Bb, cu_seqlens_host, cu_seqlens_dev, batch, out, out_dtype,
                    out_scale, workspace, workspace_bytes, false, stream);
}

int seqcomp_compress_fused_noalloc(int mode, int64_t m, const void* H, int64_t d, int in_dtype, const void* Wt,
                                   int64_t c, const float* Ba, const float* Bb, const int64_t* cu_seqlens_host,
                                   const int64_t* cu_seqlens_dev, int64_t batch, void* out, int out_dtype,
                                   float* out_scale, void* stream) {
  return fused_impl(mode, m, H, d, in_dtype, Wt, c, Ba, Bb, cu_seqlens_host, cu_seqlens_dev, batch, out, out_dtype,
                    out_scale, nullptr, 0, true, stream);
}

// Split-K partial products (small batches), then the fp32 staging of an fp8 output.
static size_t append_partial_region(int64_t nb, int64_t c) { return round_up(append_partial_bytes(nb, (int)c), 256); }

size_t seqcomp_append_workspace_bytes(int64_t nb, int64_t c, int out_dtype) {
  if (nb < 0 || nb * 4 > kMaxRows || c < 1 || c > (int64_t(1) << 20) || !valid_out_dtype(out_dtype))
    return (size_t)-1;
  if (nb == 0) return 0;
  const size_t staging = out_dtype == SEQCOMP_FP8_E4M3 ? round_up((size_t)nb * c * 4, 256) : 0;
  return append_partial_region(nb, c) + staging;
}

int seqcomp_csa_append(const void* H, int64_t nb, int64_t d, int in_dtype, const void* Wt, int64_t c,
                       const float* Ba, const float* Bb, const float* state_in, float* state_out, void* out,
                       int out_dtype, float* out_scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_in_dtype(in_dtype)) return SEQCOMP_E_DTYPE;
  if (!valid_out_dtype(out_dtype)) return SEQCOMP_E_DTYPE;
  if (nb < 0 || nb * 4 > kMaxRows) return SEQCOMP_E_SHAPE;
  if (d < 64 || d % 64 != 0 || d > (int64_t(1) << 24)) return SEQCOMP_E_UNSUPPORTED;
  if (c < 16 || c % 16 != 0 || c > (int64_t(1) << 20)) return SEQCOMP_E_UNSUPPORTED;
  // the kernels address one 256-row tile of H and all of Wt with 32-bit byte offsets
  if (4 * c * d * elt_size(in_dtype) >= (int64_t(1) << 32) || 256 * d * elt_size(in_dtype) >= (int64_t(1) << 32))
    return SEQCOMP_E_UNSUPPORTED;
  int st;
  Range out_r, scale_r;
  if ((st = check_output(out_dtype, out, out_scale, nb, c, &out_r, &scale_r))) return st;
  if (nb == 0) return SEQCOMP_OK;
  if (!H || !Wt || !Ba || !Bb || !state_in || !state_out) return SEQCOMP_E_NULL;
  if (!aligned16(H) || !aligned16(Wt) || !aligned16(Ba) || !aligned16(Bb) || !aligned16(state_in) ||
      !aligned16(state_out))
    return SEQCOMP_E_ALIGN;
  const size_t need = seqcomp_append_workspace_bytes(nb, c, out_dtype);
  Range ws_r;
  if ((st = check_workspace(workspace, workspace_bytes, need, &ws_r))) return st;
  const int es = elt_size(in_dtype);
  const size_t state_bytes = (size_t)nb * 3 * c * 4;
  Range reads[5];
  int nr = 0;
  reads[nr++] = range_of(H, (size_t)nb * 4 * d * es);
  reads[nr++] = range_of(Wt, (size_t)4 * c * d * es);
  reads[nr++] = range_of(Ba, (size_t)4 * c * 4);
  reads[nr++] = range_of(Bb, (size_t)4 * c * 4);
  // the state may be updated in place (same pointer); any other overlap is an error
  if (state_in != state_out) reads[nr++] = range_of(state_in, state_bytes);
  const Range writes[4] = {out_r, scale_r, ws_r, range_of(state_out, state_bytes)};
  if ((st = check_alias(writes, 4, reads, nr))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fp8 = out_dtype == SEQCOMP_FP8_E4M3;
  const size_t part_bytes = append_partial_region(nb, c);
  void* partial = part_bytes ? workspace : nullptr;
  void* dst = fp8 ? static_cast<char*>(workspace) + part_bytes : out;
  const int dst_dt = fp8 ? DT_F32 : out_dtype;
  hipError_t e =
      launch_csa_append(in_dtype, dst_dt, H, nb, (int)d, Wt, (int)c, Ba, Bb, state_in, state_out, dst, partial, s);
  if (e == hipSuccess && fp8)
    e = launch_quant_fp8(reinterpret_cast<const float*>(dst), nb, (int)c, static_cast<uint8_t*>(out), out_scale, s);
  return hip_status(e);
}

size_t seqcomp_rope_store_workspace_bytes(int64_t m, const int64_t* cu_seqlens_host, int64_t batch) {
  int64_t T;
  if (m < 1 || m > (int64_t(1) << 20) || check_cu(cu_seqlens_host, batch, &T) != SEQCOMP_OK) return (size_t)-1;
  if (entries_of(cu_seqlens_host, batch, m) == 0) return 0;
  return round_up((size_t)count_tiles(cu_seqlens_host, batch, m, m * kRopeTileEntries) * sizeof(TileRec), 256);
}

int seqcomp_rope_store(const void* entries, int in_dtype, int64_t c, int64_t m, const int64_t* cu_seqlens_host,
                       const int64_t* cu_seqlens_dev, int64_t batch, const int64_t* pos0_dev, int64_t rope_dims,
                       double rope_base, const int64_t* slots_dev, int64_t n_slots, uint8_t* cache_nope,
                       float* cache_scale, uint16_t* cache_rope, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!valid_in_dtype(in_dtype)) return SEQCOMP_E_DTYPE;
  if (c < 16 || c % 16 != 0 || c > (int64_t(1) << 20)) return SEQCOMP_E_UNSUPPORTED;
  if (m < 1 || m > (int64_t(1) << 20)) return SEQCOMP_E_UNSUPPORTED;
  if (rope_dims < 0 || rope_dims > c || rope_dims % 8 != 0) return SEQCOMP_E_UNSUPPORTED;
  if (!(rope_base > 0.0) || rope_base > 1e30) return SEQCOMP_E_SHAPE;   // rejects NaN too
  int64_t T = 0;
  int st = check_cu(cu_seqlens_host, batch, &T);
  if (st) return st;
  const int64_t E = entries_of(cu_seqlens_host, batch, m);
  if (n_slots < 0 || n_slots > (int64_t(1) << 40) || (!slots_dev && n_slots < E)) return SEQCOMP_E_SHAPE;
  if (E == 0) return SEQCOMP_OK;
  const int64_t cn = c - rope_dims;
  if (!entries || !cu_seqlens_dev || !cache_scale || (cn > 0 && !cache_nope) || (rope_dims > 0 && !cache_rope))
    return SEQCOMP_E_NULL;
  if (!aligned16(entries) || !aligned16(cu_seqlens_dev) || !aligned16(cache_scale) ||
      (cn > 0 && !aligned16(cache_nope)) || (rope_dims > 0 && !aligned16(cache_rope)) ||
      (pos0_dev && !aligned16(pos0_dev)) || (slots_dev && !aligned16(slots_dev)))
    return SEQCOMP_E_ALIGN;
  const size_t need = seqcomp_rope_store_workspace_bytes(m, cu_seqlens_host, batch);
  Range ws_r;
  if ((st = check_workspace(workspace, workspace_bytes, need, &ws_r))) return st;
  Range reads[4];
  int nr = 0;
  reads[nr++] = range_of(entries, (size_t)E * c * elt_size(in_dtype));
  reads[nr++] = range_of(cu_seqlens_dev, (size_t)(batch + 1) * 8);
  if (pos0_dev) reads[nr++] = range_of(pos0_dev, (size_t)batch * 8);
  if (slots_dev) reads[nr++] = range_of(slots_dev, (size_t)E * 8);
  const Range writes[4] = {cn > 0 ? range_of(cache_nope, (size_t)n_slots * cn) : Range(),
                           range_of(cache_scale, (size_t)n_slots * 4),
                           rope_dims > 0 ? range_of(cache_rope, (size_t)n_slots * rope_dims * 2) : Range(), ws_r};
  if ((st = check_alias(writes, 4, reads, nr))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TileRec* tiles = static_cast<TileRec*>(workspace);
  const int n_tiles = (int)count_tiles(cu_seqlens_host, batch, m, m * kRopeTileEntries);
  // few sequences: each workgroup looks its one tile up from the offsets, no planner launch
  const bool planned = batch > kTileLookupMaxBatch;
  hipError_t e = planned
                     ? launch_plan(cu_seqlens_dev, (int)batch, (int)m, (int)(m * kRopeTileEntries), tiles, n_tiles, s)
                     : hipSuccess;
  if (e == hipSuccess)
    e = launch_rope_store(in_dtype, entries, (int)c, (int)m, cu_seqlens_dev, (int)batch, pos0_dev, (int)rope_dims,
                          rope_base, slots_dev, n_slots, planned ? tiles : nullptr, n_tiles, cache_nope, cache_scale,
                          cache_rope, s);
  return hip_status(e);
}

size_t seqcomp_indexer_workspace_bytes(const int64_t* cu_q_host, int64_t batch) {
  int64_t T;
  if (check_cu(cu_q_host, batch, &T) != SEQCOMP_OK) return (size_t)-1;
  if (T == 0) return 0;
  return round_up((size_t)count_tiles(cu_q_host, batch, 1, kIndexerTileQueries) * sizeof(TileRec), 256);
}

int seqcomp_indexer_topk(const void* q, const float* w, const void* keys, int64_t n_heads, int64_t head_dim,
                         int in_dtype, const int64_t* cu_q_host, const int64_t* cu_q_dev,
                         const int64_t* cu_k_host, const int64_t* cu_k_dev, int64_t batch,
                         const int32_t* n_valid, int64_t k, int32_t* out_idx, float* out_score,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (in_dtype != SEQCOMP_BF16) return SEQCOMP_E_DTYPE;
  if (n_heads != kIndexerHeads || head_dim != kIndexerDim) return SEQCOMP_E_UNSUPPORTED;
  if (k < 1 || k > kIndexerMaxK) return SEQCOMP_E_UNSUPPORTED;
  int64_t T = 0, N = 0;
  int st = check_cu(cu_q_host, batch, &T);
  if (st) return st;
  if ((st = check_cu(cu_k_host, batch, &N))) return st;
  // key offsets of a sequence (and of a ragged last stage) stay below 2^31 bytes
  for (int64_t b = 0; b < batch; ++b)
    if (cu_k_host[b + 1] - cu_k_host[b] >= (int64_t(1) << 23)) return SEQCOMP_E_UNSUPPORTED;
  if (T == 0) return SEQCOMP_OK;
  if (!q || !w || !cu_q_dev || !cu_k_dev || !out_idx || (N > 0 && !keys)) return SEQCOMP_E_NULL;
  if (!aligned16(q) || !aligned16(w) || (keys && !aligned16(keys)) || !aligned16(cu_q_dev) ||
      !aligned16(cu_k_dev) || !aligned16(out_idx) || (out_score && !aligned16(out_score)) ||
      (n_valid && (reinterpret_cast<uintptr_t>(n_valid) & 3u)))
    return SEQCOMP_E_ALIGN;
  const size_t need = seqcomp_indexer_workspace_bytes(cu_q_host, batch);
  Range ws_r;
  if ((st = check_workspace(workspace, workspace_bytes, need, &ws_r))) return st;
  Range reads[6];
  int nr = 0;
  reads[nr++] = range_of(q, (size_t)T * kIndexerHeads * kIndexerDim * 2);
  reads[nr++] = range_of(w, (size_t)T * kIndexerHeads * 4);
  if (keys) reads[nr++] = range_of(keys, (size_t)N * kIndexerDim * 2);
  reads[nr++] = range_of(cu_q_dev, (size_t)(batch + 1) * 8);
  reads[nr++] = range_of(cu_k_dev, (size_t)(batch + 1) * 8);
  if (n_valid) reads[nr++] = range_of(n_valid, (size_t)T * 4);
  const Range writes[3] = {range_of(out_idx, (size_t)T * k * 4),
                           out_score ? range_of(out_score, (size_t)T * k * 4) : Range(), ws_r};
  if ((st = check_alias(writes, 3, reads, nr))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TileRec* tiles = static_cast<TileRec*>(workspace);
  const int n_tiles = (int)count_tiles(cu_q_host, batch, 1, kIndexerTileQueries);
  hipError_t e = launch_plan(cu_q_dev, (int)batch, 1, kIndexerTileQueries, tiles, n_tiles, s);
  if (e == hipSuccess)
    e = launch_indexer_topk(q, w, keys, cu_k_dev, n_valid, tiles, n_tiles, (int)k, out_idx, out_score, s);
  return hip_status(e);
}

size_t seqcomp_mqa_workspace_bytes(const int64_t* cu_q_host, int64_t batch) {
  int64_t T;
  if (check_cu(cu_q_host, batch, &T) != SEQCOMP_OK) return (size_t)-1;
  if (T == 0) return 0;
  return round_up((size_t)T * sizeof(TileRec), 256);
}

int seqcomp_shared_kv_mqa(const void* q, const void* kv, int64_t n_heads, int64_t head_dim, int in_dtype,
                          const int64_t* cu_q_host, const int64_t* cu_q_dev, const int64_t* cu_k_host,
                          const int64_t* cu_k_dev, int64_t batch, const int32_t* n_valid, const void* k_sink,
                          const void* v_sink, float scale, void* out, int out_dtype, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (in_dtype != SEQCOMP_BF16) return SEQCOMP_E_DTYPE;
  if (out_dtype != SEQCOMP_BF16 && out_dtype != SEQCOMP_F32) return SEQCOMP_E_DTYPE;
  if (n_heads != kMqaHeads || head_dim != kMqaDim) return SEQCOMP_E_UNSUPPORTED;
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return SEQCOMP_E_SHAPE;   // NaN or infinite
  int64_t T = 0, N = 0;
  int st = check_cu(cu_q_host, batch, &T);
  if (st) return st;
  if ((st = check_cu(cu_k_host, batch, &N))) return st;
  // entry offsets of a sequence stay below 2^31 bytes
  for (int64_t b = 0; b < batch; ++b)
    if (cu_k_host[b + 1] - cu_k_host[b] >= (int64_t(1) << 21)) return SEQCOMP_E_UNSUPPORTED;
  if (T > (int64_t(1) << 30)) return SEQCOMP_E_UNSUPPORTED;                               // grid of 2 T
  if (T == 0) return SEQCOMP_OK;
  if (!q || !out || !cu_q_dev || !cu_k_dev || (N > 0 && !kv) || (v_sink && !k_sink)) return SEQCOMP_E_NULL;
  if (!aligned16(q) || !aligned16(out) || (kv && !aligned16(kv)) || !aligned16(cu_q_dev) || !aligned16(cu_k_dev) ||
      (k_sink && !aligned16(k_sink)) || (v_sink && !aligned16(v_sink)) || (lse && !aligned16(lse)) ||
      (n_valid && (reinterpret_cast<uintptr_t>(n_valid) & 3u)))
    return SEQCOMP_E_ALIGN;
  const size_t need = seqcomp_mqa_workspace_bytes(cu_q_host, batch);
  Range ws_r;
  if ((st = check_workspace(workspace, workspace_bytes, need, &ws_r))) return st;
  Range reads[7];
  int nr = 0;
  reads[nr++] = range_of(q, (size_t)T * kMqaHeads * kMqaDim * 2);
  if (kv) reads[nr++] = range_of(kv, (size_t)N * kMqaDim * 2);
  reads[nr++] = range_of(cu_q_dev, (size_t)(batch + 1) * 8);
  reads[nr++] = range_of(cu_k_dev, (size_t)(batch + 1) * 8);
  if (n_valid) reads[nr++] = range_of(n_valid, (size_t)T * 4);
  if (k_sink) reads[nr++] = range_of(k_sink, kMqaDim * 2);
  if (v_sink) reads[nr++] = range_of(v_sink, kMqaDim * 2);
  const Range writes[3] = {range_of(out, (size_t)T * kMqaHeads * kMqaDim * elt_size(out_dtype)),
                           lse ? range_of(lse, (size_t)T * kMqaHeads * 4) : Range(), ws_r};
  if ((st = check_alias(writes, 3, reads, nr))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TileRec* tiles = static_cast<TileRec*>(workspace);
  hipError_t e = launch_plan(cu_q_dev, (int)batch, 1, 1, tiles, (int)T, s);
  if (e == hipSuccess)
    e = launch_mqa_sink(out_dtype == SEQCOMP_BF16 ? DT_BF16 : DT_F32, q, kv, cu_k_dev, n_valid, tiles, (int)T,
                        k_sink, v_sink, scale, out, lse, s);
  return hip_status(e);
}

}  // extern "C"
