// Lightning indexer ("Ch 04 · CSA — 长上下文的快通道", section 4): scores of
// queries against compressed indexer keys,
//
//     I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s])      (64 heads of 128 dims)
//
// and, streamed over the keys, the set of every query's k best keys.  The
// scores never reach memory: ReLU needs no normalisation over s, so each one
// is judged against a running threshold the moment it is computed.
//
// One workgroup takes 8 queries of one sequence (2 per wavefront) and sweeps
// their keys in stages of 64.  The dot products are a dense contraction: for
// a block of 32 keys a wave runs, per query, two 32-head row blocks of
// v_mfma_f32_32x32x16_bf16 over K = 128 (8 MFMAs each), with the queries'
// A fragments held in registers for the whole sweep and the key fragments
// read from LDS.  The 32x32 accumulator leaves lane l with key l % 32 and 16
// of the 64 heads (rows 8 g + 4 (l / 32) + 0..3), so the ReLU and the
// head-weighted sum are 32 fused multiply-adds per lane and query, and one
// exchange between lanes l and l ^ 32 (v_permlane32_swap) completes both
// queries' scores at once: lanes 0..31 hold query 0's, lanes 32..63 query 1's.
//
// Selection: each query owns a candidate buffer of 1536 (score, key) slots in
// LDS and a threshold tau, the k-th best score seen so far (-inf until k
// keys were kept).  A visible key whose score beats tau is appended (ballot
// + lane prefix counts; keys arrive in increasing order, so the buffer stays
// sorted by key).  When a buffer could overflow on the next block, the wave
// finds the k-th best candidate by a radix select on order-preserving 32-bit
// keys of the scores (4 passes of 8-bit histograms in LDS), keeps the k best
// in place -- a stable compaction, so ties at the threshold go to the smaller
// key index -- and raises tau to that score.  A later key with a score equal
// to tau has a larger index and so ranks below every kept one: the strict
// test "score > tau" is exact.  At the end of the sweep one more compaction
// leaves the k best, listed by increasing key index.
//
// Keys travel global -> LDS directly (buffer_load ... lds, 16 bytes a lane,
// whole 128-byte lines), through a ring of 3 stages (48 KiB), two stages
// ahead; the descriptor's range is the sequence's keys, so a ragged last
// stage reads zeros.  In LDS, 16-byte chunk c of key row r sits in slot
// c ^ (r & 15): a fragment read (16 consecutive rows, one chunk) touches 16
// distinct slots -- all 64 banks -- so it is free of bank conflicts.
#include "amdgcn.hpp"
#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kIxThreads = 256;
constexpr int kIxKeyBytes = kIndexerDim * 2;                  // one bf16 key: 256 bytes
constexpr int kIxStageKeys = 64;
constexpr int kIxStages = 3;
constexpr int kIxStageBytes = kIxStageKeys * kIxKeyBytes;     // 16 KiB
constexpr int kIxCap = 1536;                                  // candidate slots per query
constexpr int kIxCandOff = kIxStages * kIxStageBytes;         // 48 KiB of key stages
constexpr int kIxIdxOff = kIxCandOff + kIndexerTileQueries * kIxCap * 4;
constexpr int kIxHistOff = kIxIdxOff + kIndexerTileQueries * kIxCap * 4;   // + 96 KiB of candidates
constexpr int kIxLdsBytes = kIxHistOff + 4 * 256 * 4;         // + 4 KiB of histograms = 148 KiB
static_assert(kIxCap >= kIndexerMaxK + 64, "after a compaction a key block must still fit");
static_assert(kIndexerHeads == 64 && kIndexerDim == 128, "fragment layout assumes 64 heads of 128 dims");

struct IxArgs {
  const char* q;            // [T][64][128] bf16
  const float* w;           // [T][64]
  const char* keys;         // [N][128] bf16
  const int64_t* cu_k;      // [batch + 1]
  const int32_t* n_valid;   // [T] or null
  const TileRec* tiles;
  int n_tiles;
  int k;
  int32_t* out_idx;         // [T][k]
  float* out_score;         // [T][k] or null
};

// Every LDS access of this wave issued so far has completed; the compiler
// moves no memory access across this point.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Order-preserving map of a score to 32 bits: a > b as floats iff
// order_key(a) > order_key(b).  -0 is taken as +0, so the two zeros tie as
// they do as floats.  NaN never reaches it (it never beats a threshold).
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = s == 0.f ? 0u : __float_as_uint(s);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_value(uint32_t k) {
  return __uint_as_float((k >> 31) ? (k & 0x7fffffffu) : ~k);
}

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Keeps the k best of the n > k candidates (cs: scores, ci: keys, stored by
// increasing key) in place and in key order; returns the k-th best score.
// Called by the whole wave; hist is the wave's 256 counters.
__device__ __forceinline__ float compact_candidates(float* cs, int32_t* ci, int n, int k, uint32_t* hist, int lane) {
  // Radix select of the k-th largest order key, 8 bits at a time from the top:
  // `prefix` holds the bits fixed so far, `need` the rank still sought among
  // the candidates that share them.
  uint32_t prefix = 0;
  int need = k;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0u;
    wave_lds_sync();
    const uint32_t fixed = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
#pragma unroll 4
    for (int i = lane; i < n; i += 64) {
      const uint32_t u = order_key(cs[i]);
      if ((u & fixed) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    wave_lds_sync();
    uint32_t h[4], tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      h[b] = hist[lane * 4 + b];
      tot += h[b];
    }
    // candidates in the bins of higher lanes (inclusive suffix sum minus own)
    uint32_t suf = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += y;
    }
    uint32_t above = suf - tot;
    int bin = -1, rest = 0;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (bin < 0 && above < (uint32_t)need && above + h[b] >= (uint32_t)need) {
        bin = lane * 4 + b;
        rest = need - (int)above;
      }
      above += h[b];
    }
    const uint64_t found = __ballot(bin >= 0);
    const int src = __builtin_ctzll(found);
    bin = __shfl(bin, src, 64);
    rest = __shfl(rest, src, 64);
    prefix |= (uint32_t)bin << shift;
    need = rest;
  }
  // Stable in-place compaction: every candidate above the k-th, and the first
  // `need` (smallest keys) of those equal to it.  Writes land below the
  // chunk being read, and all of a chunk's reads complete before its writes.
  int kept = 0, ties = 0;
#pragma unroll 1
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    float s = 0.f;
    int32_t key = 0;
    uint32_t u = 0;
    if (i < n) {
      s = cs[i];
      key = ci[i];
      u = order_key(s);
    }
    const bool eq = i < n && u == prefix;
    const uint64_t eqm = __ballot(eq);
    const bool keep = (i < n && u > prefix) || (eq && ties + lanes_below(eqm) < need);
    const uint64_t km = __ballot(keep);
    wave_lds_sync();
    if (keep) {
      const int p = kept + lanes_below(km);
      cs[p] = s;
      ci[p] = key;
    }
    kept += __popcll(km);
    ties += __popcll(eqm);
  }
  wave_lds_sync();
  return order_key_value(prefix);
}

__global__ __launch_bounds__(kIxThreads, 1) void indexer_topk_kernel(IxArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kIxLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool upper = lane >= 32;
  const TileRec tile = a.tiles[a.n_tiles - 1 - (int)blockIdx.x];   // later (longer) tiles first
  const int seq = tile_seq(tile.flags);
  const int64_t q0 = tile.row_start;
  const int nq = tile.n_rows;
  const int64_t kbase = a.cu_k[seq];
  const int nk = (int)(a.cu_k[seq + 1] - kbase);

  // Visible keys of the tile's queries; the sweep covers the longest.
  int nv_max = 0, nv0 = 0, nv1 = 0;
#pragma unroll
  for (int j = 0; j < kIndexerTileQueries; ++j) {
    int v = 0;
    if (j < nq) v = a.n_valid ? min(max(a.n_valid[q0 + j], 0), nk) : nk;
    nv_max = max(nv_max, v);
    if (j == 2 * w) nv0 = v;
    if (j == 2 * w + 1) nv1 = v;
  }
  const int my_nv = upper ? nv1 : nv0;

  // The wave's two queries (a missing one reads the tile's first query and
  // keeps nothing): A fragments of the 4 row blocks (query j, heads
  // 32 b + l % 32) for the 8 k-steps, and the weights of the lane's 16 heads
  // per row block.
  bf16x8_t qa[4][8];
  float wv[4][16];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int j = 2 * w + (rb >> 1);
    const int64_t t = q0 + (j < nq ? j : 0);
    const char* row = a.q + ((t * kIndexerHeads + 32 * (rb & 1) + (lane & 31)) * kIxKeyBytes) + (lane >> 5) * 16;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qa[rb][kk] = __builtin_bit_cast(bf16x8_t, ld16(row + kk * 32));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 v = *reinterpret_cast<const float4*>(a.w + t * kIndexerHeads + 32 * (rb & 1) + 8 * g +
                                                        4 * (lane >> 5));
      wv[rb][4 * g + 0] = v.x;
      wv[rb][4 * g + 1] = v.y;
      wv[rb][4 * g + 2] = v.z;
      wv[rb][4 * g + 3] = v.w;
    }
  }

  float* const cand_s = reinterpret_cast<float*>(lds + kIxCandOff) + (2 * w) * kIxCap;
  int32_t* const cand_i = reinterpret_cast<int32_t*>(lds + kIxIdxOff) + (2 * w) * kIxCap;
  uint32_t* const hist = reinterpret_cast<uint32_t*>(lds + kIxHistOff) + w * 256;
  float* const my_s = cand_s + (upper ? kIxCap : 0);
  int32_t* const my_i = cand_i + (upper ? kIxCap : 0);

  // Copies of one stage: wave w fills rows 16 w .. 16 w + 15 with 4 copies of
  // 1 KiB (4 rows each); lane p writes slot p & 15 of row p >> 4 of its 4,
  // which holds chunk (p & 15) ^ (row & 15) of that key.
  const __amdgpu_buffer_rsrc_t ksrc = ranged_rsrc(a.keys + kbase * kIxKeyBytes, (uint32_t)nk * kIxKeyBytes);
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (w * 4 + i) * 4 + (lane >> 4);
    voff[i] = (uint32_t)(r * kIxKeyBytes + (((lane & 15) ^ (r & 15)) * 16));
  }
  const auto issue_stage = [&](int s) {
    char* dst = lds + (s % kIxStages) * kIxStageBytes + w * 4 * 1024;
    const uint32_t so = (uint32_t)s * kIxStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void_t*)(dst + i * 1024), 16, voff[i] + so, 0, 0, 0);
  };

  const int n_st = (nv_max + kIxStageKeys - 1) / kIxStageKeys;
  if (n_st > 0) issue_stage(0);
  if (n_st > 1) issue_stage(1);

  float tau0 = -INFINITY, tau1 = -INFINITY;
  int cnt0 = 0, cnt1 = 0;
  float tau = -INFINITY;
  const int r = lane & 31;          // key row of the lane's B fragment and score
  const int k = a.k;

#pragma unroll 1
  for (int s = 0; s < n_st; ++s) {
    if (s + 1 < n_st) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    lds_barrier();                  // stage s is in; every wave is done with stage s - 1
    if (s + 2 < n_st) issue_stage(s + 2);
    const char* st = lds + (s % kIxStages) * kIxStageBytes;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const char* kr = st + (bi * 32 + r) * kIxKeyBytes;
      f32x4_t bf[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        bf[kk] = *reinterpret_cast<const f32x4_t*>(kr + (((2 * kk + (lane >> 5)) ^ (r & 15)) * 16));
      f32x16_t acc[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][kk], __builtin_bit_cast(bf16x8_t, bf[kk]),
                                                            acc[rb], 0, 0, 0);
      float p[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s0 = fmaf(wv[2 * j][e], fmaxf(acc[2 * j][e], 0.f), s0);
          s1 = fmaf(wv[2 * j + 1][e], fmaxf(acc[2 * j + 1][e], 0.f), s1);
        }
        p[j] = s0 + s1;
      }
      // lanes < 32: query 0's halves; lanes >= 32: query 1's
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
      const float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int key = s * kIxStageKeys + bi * 32 + r;
      const bool pass = key < my_nv && score > tau;
      const uint64_t m = __ballot(pass);
      if (m) {
        const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
        const int pos = upper ? cnt1 + (int)__builtin_amdgcn_mbcnt_hi(hi, 0u)
                              : cnt0 + (int)__builtin_amdgcn_mbcnt_lo(lo, 0u);
        if (pass) {
          my_s[pos] = score;
          my_i[pos] = key;
        }
        cnt0 += __popc(lo);
        cnt1 += __popc(hi);
        wave_lds_sync();
#pragma unroll 1
        while (cnt0 > kIxCap - 32 || cnt1 > kIxCap - 32) {
          const int j = cnt0 > kIxCap - 32 ? 0 : 1;
          const float t = compact_candidates(cand_s + j * kIxCap, cand_i + j * kIxCap, j ? cnt1 : cnt0, k, hist,
                                             lane);
          if (j) {
            cnt1 = k;
            tau1 = t;
          } else {
            cnt0 = k;
            tau0 = t;
          }
        }
        tau = upper ? tau1 : tau0;
      }
    }
  }

  // Final selection and output (keys in increasing order, -1 / -inf after
  // the last selected one).
#pragma unroll 1
  for (int j = 0; j < 2; ++j) {
    const int qj = 2 * w + j;
    if (qj >= nq) break;
    int n = j ? cnt1 : cnt0;
    float* cs = cand_s + j * kIxCap;
    int32_t* ci = cand_i + j * kIxCap;
    if (n > k) {
      compact_candidates(cs, ci, n, k, hist, lane);
      n = k;
    }
    const int64_t t = q0 + qj;
    for (int i = lane; i < k; i += 64) {
      const bool have = i < n;
      a.out_idx[t * k + i] = have ? ci[i] : -1;
      if (a.out_score) a.out_score[t * k + i] = have ? cs[i] : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_indexer_topk(const void* q, const float* w, const void* keys, const int64_t* cu_k_dev,
                               const int32_t* n_valid, const TileRec* tiles, int n_tiles, int k, int32_t* out_idx,
                               float* out_score, hipStream_t stream) {
  if (n_tiles <= 0) return hipSuccess;
  IxArgs a;
  a.q = static_cast<const char*>(q);
  a.w = w;
  a.keys = static_cast<const char*>(keys);
  a.cu_k = cu_k_dev;
  a.n_valid = n_valid;
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  a.k = k;
  a.out_idx = out_idx;
  a.out_score = out_score;
  hipLaunchKernelGGL(indexer_topk_kernel, dim3(n_tiles), dim3(kIxThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace seqcomp
