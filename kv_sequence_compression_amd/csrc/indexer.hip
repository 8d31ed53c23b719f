// Lightning indexer ("Ch 04 · CSA — 长上下文的快通道", section 4): scores of
// queries against compressed indexer keys,
//
//     I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s])      (64 heads of 128 dims)
//
// and, streamed over the keys, the set of every query's k best keys.  The
// scores never reach memory: ReLU needs no normalisation over s, so each one
// is judged against a running threshold the moment it is computed.
//
// One workgroup takes 8 queries of one sequence, one per wavefront (two
// wavefronts per SIMD, so one's MFMAs run while the other forms scores), and
// sweeps their keys in stages of 64.  The dot products are a dense
// contraction: for a block of 32 keys a wave runs two 32-head row blocks of
// v_mfma_f32_32x32x16_bf16 over K = 128 (8 MFMAs each), with its query's A
// fragments held in registers for the whole sweep and the key fragments read
// from LDS.  The 32x32 accumulator leaves lane l with key l % 32 and 16 of
// the 64 heads (rows 8 g + 4 (l / 32) + 0..3 of each row block), so the ReLU
// and the head-weighted sum are 32 fused multiply-adds per lane, and one
// exchange between lanes l and l ^ 32 (v_permlane32_swap) completes the
// score.  Within a wave the MFMAs of one block are issued before the scores
// of the previous block are formed (a software pipeline over two
// accumulator sets).
//
// Selection: each query owns a candidate buffer of 1536 (score, key) slots in
// LDS and a threshold tau at or below the k-th best score seen so far (-inf
// until the first compaction).  A visible key whose score beats tau is appended (ballot
// + lane prefix counts; keys arrive in increasing order, so the buffer stays
// sorted by key).  When any buffer of the tile could overflow within the
// next stage, every wave compacts its buffer at the stage start (all at once,
// so no wave waits at the next barrier for another's compaction).  A
// compaction loads the candidates' order-preserving 32-bit keys into
// registers and radix-selects the k-th best over the bits below their common
// prefix (8-bit histograms in LDS).  Between stages one pass usually
// suffices: the wave keeps every candidate at or above the lower edge of the
// k-th best's bin (a stable compaction, at least the k best) and raises tau
// to that edge.  A later key that only equals tau ranks below the k best
// (either its score is lower or it ties with a smaller index), so the strict
// test "score > tau" loses nothing.  At the end of the sweep an exact
// selection (all passes, ties to the smaller key index) leaves the k best,
// listed by increasing key index.
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

constexpr int kIxThreads = 512;                              // 8 waves: one query each, 2 per SIMD
constexpr int kIxKeyBytes = kIndexerDim * 2;                  // one bf16 key: 256 bytes
constexpr int kIxStageKeys = 64;
constexpr int kIxStages = 3;
constexpr int kIxStageBytes = kIxStageKeys * kIxKeyBytes;     // 16 KiB
constexpr int kIxCap = 1536;                                  // candidate slots per query
constexpr int kIxCandOff = kIxStages * kIxStageBytes;         // 48 KiB of key stages
constexpr int kIxIdxOff = kIxCandOff + kIndexerTileQueries * kIxCap * 4;
constexpr int kIxHistOff = kIxIdxOff + kIndexerTileQueries * kIxCap * 4;   // + 96 KiB of candidates
constexpr int kIxFlagOff = kIxHistOff + 8 * 256 * 4;         // + 8 KiB of histograms
constexpr int kIxLdsBytes = kIxFlagOff + 16;                  // + compaction flags: ~152 KiB
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

constexpr int kIxSlotsPerLane = kIxCap / 64;                 // candidate slots a lane holds in a compaction
static_assert(kIxCap % 64 == 0, "candidate buffer in whole wave rows");

// Order key of the k-th best candidate, by radix selection on the wave's
// register copy u[] of the candidates' order keys (slot lane + 64 j; empty
// slots hold 0, below every real key).  Only the bits below the candidates'
// common prefix are searched, 8 at a time from the top: each pass counts the
// candidates that match the bits fixed so far per value of the next digit
// (histogram in LDS), and a suffix scan over the bins finds the digit of the
// k-th best.  Returns the bits fixed so far with the rest zero: after the
// last pass (`exact` set) the k-th best key itself, and `need` says how many
// candidates equal to it belong to the k best; else the lower edge of the
// k-th best's bin, with at most `limit` candidates at or above it.  EXACT
// runs every pass; otherwise passes stop once that edge keeps few enough.
template <bool EXACT>
__device__ __forceinline__ uint32_t select_kth(const uint32_t (&u)[kIxSlotsPerLane], int k, int limit,
                                               uint32_t* hist, int lane, int& need, bool& exact) {
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int j = 0; j < kIxSlotsPerLane; ++j) {
    if (u[j] != 0u) lo = min(lo, u[j]);
    hi = max(hi, u[j]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
  }
  int remaining = lo == hi ? 0 : 32 - __builtin_clz(lo ^ hi);   // low bits that differ
  uint32_t prefix = remaining == 32 ? 0u : (hi >> remaining) << remaining;
  need = k;
#pragma unroll 1
  while (remaining > 0) {
    const int width = min(8, remaining), shift = remaining - width;
    const uint32_t dmask = (1u << width) - 1u;
    *reinterpret_cast<uint4*>(hist + lane * 4) = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < kIxSlotsPerLane; ++j) {
      const bool match = u[j] != 0u && (remaining == 32 || (u[j] >> remaining) == (prefix >> remaining));
      if (match) atomicAdd(&hist[(u[j] >> shift) & dmask], 1u);
    }
    wave_lds_sync();
    const uint4 h4 = *reinterpret_cast<const uint4*>(hist + lane * 4);
    const uint32_t h[4] = {h4.x, h4.y, h4.z, h4.w};
    const uint32_t tot = h[0] + h[1] + h[2] + h[3];
    uint32_t suf = tot;                                          // inclusive suffix sum over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += y;
    }
    uint32_t above = suf - tot;                                  // candidates in higher lanes' bins
    int bin = -1, rest = 0, in_bin = 0;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (bin < 0 && above < (uint32_t)need && above + h[b] >= (uint32_t)need) {
        bin = lane * 4 + b;
        rest = need - (int)above;
        in_bin = (int)h[b];
      }
      above += h[b];
    }
    const int src = __builtin_ctzll(__ballot(bin >= 0));
    bin = __shfl(bin, src, 64);
    rest = __shfl(rest, src, 64);
    in_bin = __shfl(in_bin, src, 64);
    prefix |= (uint32_t)bin << shift;
    remaining = shift;
    // candidates kept by the bin's lower edge: the k - need above the
    // matching set, need - rest above the bin within it, and the bin
    const int at_edge = k - rest + in_bin;
    need = rest;
    if (!EXACT && at_edge <= limit) break;
  }
  exact = remaining == 0;
  return prefix;
}

// Compacts the n > k candidates (cs: scores, ci: keys, stored by increasing
// key) in place and in key order.  EXACT: keeps exactly the k best (ties to
// the smaller key) and returns the k-th best score.  Otherwise keeps at least
// the k best and at most 128 slots short of a full buffer -- every candidate
// at or above the lower edge of the k-th best's radix bin, or the exact k
// best when the passes run out -- and returns a threshold no higher than the
// k-th best (a later key must beat it to be a candidate; one equal to the
// k-th best ranks below it, having the larger index).  The number kept goes
// to `kept`.
template <bool EXACT>
__device__ __forceinline__ float compact_candidates(float* cs, int32_t* ci, int n, int k, uint32_t* hist, int lane,
                                                    int& kept) {
  uint32_t u[kIxSlotsPerLane];
  int32_t id[kIxSlotsPerLane];
#pragma unroll
  for (int j = 0; j < kIxSlotsPerLane; ++j) {
    const int i = lane + 64 * j;
    u[j] = i < n ? order_key(cs[i]) : 0u;
    id[j] = i < n ? ci[i] : 0;
  }
  int need;
  bool exact;
  const uint32_t cut = select_kth<EXACT>(u, k, kIxCap - 128, hist, lane, need, exact);
  // Stable compaction: reads are all in registers, so writes may land anywhere below.
  int out = 0, ties = 0;
#pragma unroll
  for (int j = 0; j < kIxSlotsPerLane; ++j) {
    bool keep;
    if (exact) {
      const bool eq = u[j] == cut;
      const uint64_t eqm = __ballot(eq);
      keep = u[j] > cut || (eq && ties + lanes_below(eqm) < need);
      ties += __popcll(eqm);
    } else {
      keep = u[j] >= cut && u[j] != 0u;
    }
    const uint64_t km = __ballot(keep);
    if (keep) {
      const int p = out + lanes_below(km);
      cs[p] = order_key_value(u[j]);
      ci[p] = id[j];
    }
    out += __popcll(km);
  }
  wave_lds_sync();
  kept = out;
  if (exact) return order_key_value(cut);
  return cut <= 0x007fffffu ? -INFINITY : order_key_value(cut);   // 0x007fffff: the key of -inf
}

__global__ __launch_bounds__(kIxThreads, 1) void indexer_topk_kernel(IxArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kIxLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const TileRec tile = a.tiles[a.n_tiles - 1 - (int)blockIdx.x];   // later (longer) tiles first
  const int seq = tile_seq(tile.flags);
  const int64_t q0 = tile.row_start;
  const int nq = tile.n_rows;
  const int64_t kbase = a.cu_k[seq];
  const int nk = (int)(a.cu_k[seq + 1] - kbase);

  // Visible keys of the tile's queries; the sweep covers the longest.
  int nv_max = 0, my_nv = 0;
#pragma unroll
  for (int j = 0; j < kIndexerTileQueries; ++j) {
    int v = 0;
    if (j < nq) v = a.n_valid ? min(max(a.n_valid[q0 + j], 0), nk) : nk;
    nv_max = max(nv_max, v);
    if (j == w) my_nv = v;
  }

  // The wave's query (a missing one reads the tile's first query and keeps
  // nothing): A fragments of its 2 row blocks (heads 32 b + l % 32) for the
  // 8 k-steps, and the weights of the lane's 16 heads per row block.
  bf16x8_t qa[2][8];
  float wv[2][16];
  {
    const int64_t t = q0 + (w < nq ? w : 0);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const char* row = a.q + ((t * kIndexerHeads + 32 * rb + (lane & 31)) * kIxKeyBytes) + (lane >> 5) * 16;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) qa[rb][kk] = __builtin_bit_cast(bf16x8_t, ld16(row + kk * 32));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v =
            *reinterpret_cast<const float4*>(a.w + t * kIndexerHeads + 32 * rb + 8 * g + 4 * (lane >> 5));
        wv[rb][4 * g + 0] = v.x;
        wv[rb][4 * g + 1] = v.y;
        wv[rb][4 * g + 2] = v.z;
        wv[rb][4 * g + 3] = v.w;
      }
    }
  }

  float* const cand_s = reinterpret_cast<float*>(lds + kIxCandOff) + w * kIxCap;
  int32_t* const cand_i = reinterpret_cast<int32_t*>(lds + kIxIdxOff) + w * kIxCap;
  uint32_t* const hist = reinterpret_cast<uint32_t*>(lds + kIxHistOff) + w * 256;

  // Copies of one stage: wave w fills rows 8 w .. 8 w + 7 with 2 copies of
  // 1 KiB (4 rows each); lane p writes slot p & 15 of row p >> 4 of its 4,
  // which holds chunk (p & 15) ^ (row & 15) of that key.
  const __amdgpu_buffer_rsrc_t ksrc = ranged_rsrc(a.keys + kbase * kIxKeyBytes, (uint32_t)nk * kIxKeyBytes);
  uint32_t voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (w * 2 + i) * 4 + (lane >> 4);
    voff[i] = (uint32_t)(r * kIxKeyBytes + (((lane & 15) ^ (r & 15)) * 16));
  }
  const auto issue_stage = [&](int s) {
    char* dst = lds + (s % kIxStages) * kIxStageBytes + w * 2 * 1024;
    const uint32_t so = (uint32_t)s * kIxStageBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void_t*)(dst + i * 1024), 16, voff[i] + so, 0, 0, 0);
  };

  const int n_st = (nv_max + kIxStageKeys - 1) / kIxStageKeys;
  uint8_t* const flags = reinterpret_cast<uint8_t*>(lds + kIxFlagOff);
  flags[w] = 0;
  flags[8 + w] = 0;
  if (n_st > 0) issue_stage(0);
  if (n_st > 1) issue_stage(1);

  float tau = -INFINITY;
  int cnt = 0;
  const int r = lane & 31;          // key row of the lane's B fragment and score
  const int k = a.k;

  const auto compact = [&]() { tau = compact_candidates<false>(cand_s, cand_i, cnt, k, hist, lane, cnt); };
  // B fragments of one block of 32 keys (rows 32 bi .. 32 bi + 31 of a stage).
  const auto read_block = [&](const char* st, int bi, f32x4_t (&bf)[8]) {
    const char* kr = st + (bi * 32 + r) * kIxKeyBytes;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      bf[kk] = *reinterpret_cast<const f32x4_t*>(kr + (((2 * kk + (lane >> 5)) ^ (r & 15)) * 16));
  };
  // Dot products of the query's 2 row blocks with one block of keys.
  const auto mma_block = [&](const f32x4_t (&bf)[8], f32x16_t (&acc)[2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][0], __builtin_bit_cast(bf16x8_t, bf[0]),
                                                        f32x16_t{}, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < 8; ++kk)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][kk], __builtin_bit_cast(bf16x8_t, bf[kk]),
                                                          acc[rb], 0, 0, 0);
  };
  // ReLU and head-weighted sum of a finished block: every lane ends with the
  // score of key l % 32 of the block.  ReLU is an integer max on the bit
  // pattern (negative floats are negative integers), one instruction.
  const auto block_score = [&](const f32x16_t (&acc)[2]) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0 = fmaf(wv[0][e], __int_as_float(max(__float_as_int(acc[0][e]), 0)), s0);
      s1 = fmaf(wv[1][e], __int_as_float(max(__float_as_int(acc[1][e]), 0)), s1);
    }
    const float p = s0 + s1;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    // lanes < 32: own half (rows 8 g + 0..3) + the other (rows 8 g + 4..7)
    return lane < 32 ? p + __uint_as_float(sw[1]) : __uint_as_float(sw[0]) + p;
  };
  // Appends the block's keys (lanes < 32) whose score beats the threshold.
  const auto append = [&](float score, int key0) {
    const int key = key0 + r;
    const bool pass = lane < 32 && key < my_nv && score > tau;
    const uint64_t m = __ballot(pass);
    if (m) {
      if (pass) {
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u);
        cand_s[pos] = score;
        cand_i[pos] = key;
      }
      cnt += __popcll(m);
      // Compiler ordering only: LDS operations of one wave complete in
      // order, and only this wave reads its buffer, so no wait is needed
      // (one would also stall on the key fragments already in flight).
      asm volatile("" ::: "memory");
    }
  };

  // Software pipeline over blocks: the MFMAs of a block run while the
  // previous block's scores are formed and judged.  Iteration s multiplies
  // blocks (s, 0) and (s, 1) and finishes (s - 1, 1) and (s, 0); a query
  // gains at most 64 candidates per iteration.  Compactions are taken at
  // iteration starts, by every wave at once when any query of the tile is
  // close to full, so that one wave's compaction does not hold up the others
  // at the next barrier one query at a time.
  f32x16_t acc0[2], acc1[2];
  acc1[0] = f32x16_t{};
  acc1[1] = f32x16_t{};
  int prev_key0 = 0x7fffff00;       // no previous block: no key passes
  f32x4_t bf0[8], bf1[8];
#pragma unroll 1
  for (int s = 0; s < n_st; ++s) {
    // own copies of stage s landed, own LDS writes (flags) done
    if (s + 1 < n_st) wait_vmcnt_lgkm0<2>();
    else wait_vmcnt_lgkm0<0>();
    lds_barrier();                  // stage s is in; every wave is done with stage s - 1
    if (s + 2 < n_st) issue_stage(s + 2);
    const uint32_t* fl = reinterpret_cast<const uint32_t*>(flags + 8 * (s & 1));
    if ((fl[0] | fl[1]) && cnt > k) compact();
    const char* st = lds + (s % kIxStages) * kIxStageBytes;
    read_block(st, 0, bf0);
    mma_block(bf0, acc0);
    const float sc_prev = block_score(acc1);
    read_block(st, 1, bf1);
    append(sc_prev, prev_key0);
    mma_block(bf1, acc1);
    const float sc0 = block_score(acc0);
    append(sc0, s * kIxStageKeys);
    prev_key0 = s * kIxStageKeys + 32;
    flags[8 * ((s + 1) & 1) + w] = cnt > kIxCap - 64 ? 1 : 0;
  }
  if (n_st > 0) {
    if (cnt > kIxCap - 32) compact();
    append(block_score(acc1), prev_key0);
  }

  // Final selection and output (keys in increasing order, -1 / -inf after
  // the last selected one).
  if (w < nq) {
    if (cnt > k) compact_candidates<true>(cand_s, cand_i, cnt, k, hist, lane, cnt);
    const int64_t t = q0 + w;
    for (int i = lane; i < k; i += 64) {
      const bool have = i < cnt;
      a.out_idx[t * k + i] = have ? cand_i[i] : -1;
      if (a.out_score) a.out_score[t * k + i] = have ? cand_s[i] : -INFINITY;
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
