// Dense shared-KV multi-query attention with an attention sink, over the
// compressed entries ("Ch 05 · HCA — 长上下文的全景镜": dense attention over all
// n/m' entries, and the attention sink of its section 4; "Ch 04 · CSA —
// 长上下文的快通道", section 6: the n_h = 128 heads share one KV).  For query t
// and head h, over the entries s its sequence shows it (and the sink):
//
//     alpha = Softmax(scale * q[t, h] . [k_sink, e_1, ..., e_n])
//     o[t, h] = alpha_sink * v_sink + sum_s alpha_s * e_s
//
// An entry serves as key and value; v_sink may be absent (zero).
//
// One workgroup takes 64 of a query's 128 heads (two workgroups per query):
// those heads are the rows, and all of them share each tile of 64 entries
// (64 KiB of bf16, staged global -> LDS, double-buffered).  Eight waves, two
// per SIMD, in two roles, on v_mfma_f32_32x32x16_bf16:
//  * score waves (0-3): wave w forms the 32 x 32 block S^T = E Q^T of head
//    block w & 1 and entry block w >> 1 (A = entry fragments from LDS, B =
//    the head block's query fragments, held in registers for the whole
//    sweep).  Lane l then holds head l % 32 of the block and 16 of the 32
//    entries; an exchange between lanes l and l ^ 32 gives the wave's maximum
//    per head.  The probabilities go to LDS as bf16, P[head][entry].  These
//    waves also issue the copies of the next tile;
//  * value waves (4-7): wave 4 + w accumulates O^T = E^T P^T for output
//    columns 128 w .. 128 w + 127 of the 64 heads (8 accumulators of
//    32 x 32).  The A operand needs 8 consecutive entries of one column per
//    lane: the gfx950 transposing LDS read (ds_read_b64_tr_b16) delivers them
//    from the row-major entry tile, 4 entries per read.
// The roles form a pipeline one tile deep: in step j the score waves turn
// tile j into probabilities while the value waves multiply tile j - 1 (its
// fragments read into registers during step j - 1, its probabilities in the
// other of two P buffers) and read tile j's fragments.  One workgroup
// barrier per step.  Split this way, neither role needs more than 256
// registers (queries 128 + scores; accumulators 128 + fragments), so two
// waves share each SIMD and one's MFMAs run while the other waits on LDS or
// works out exponentials.  The score waves, whose probabilities gate the next
// step, run at raised issue priority.
// The softmax of a head is taken against a fixed reference: the larger of the
// sink's logit and the first tile's maximum (over both score waves of the
// head block, exchanged through LDS).  Later tiles may exceed it by up to 64
// (log2 units), so the accumulators are never rescaled and no later tile
// needs the other wave's maximum; a tile that exceeds it by more raises the
// reference and starts the sweep again (each such restart moves past the tile
// that caused it, so there are at most as many as tiles).  Each score wave
// sums the probabilities of its own entries; the sums meet once, at the end,
// where the sink's weight joins the sum and its weight times v_sink the
// output.
//
// LDS: entry tiles 2 x 64 KiB; 16-byte chunk c of entry row r at slot
// c ^ f(r), f(r) = ((r & 3) << 2) | ((r >> 2) & 3): the score phase's reads
// (one chunk of 16 consecutive rows) and the value phase's transposing reads
// (two adjacent chunks of 4 consecutive rows) both touch distinct banks.
// P: 64 rows of 128 bytes, chunk c of head row h at slot c ^ ((h >> 1) & 7).
#include <type_traits>

#include "amdgcn.hpp"
#include "launch.hpp"

namespace seqcomp {

namespace {

constexpr int kMqThreads = 512;                              // 4 score waves + 4 value waves
constexpr int kMqTile = 64;                                   // entries per tile
constexpr int kMqRowBytes = kMqaDim * 2;                      // 1 KiB per bf16 entry
constexpr int kMqTileBytes = kMqTile * kMqRowBytes;           // 64 KiB
constexpr int kMqHeadsPerWg = 64;                             // half of a query's heads
constexpr int kMqPOff = 2 * kMqTileBytes;                     // P: 2 buffers of 64 heads x 64 entries bf16
constexpr int kMqPBytes = kMqHeadsPerWg * kMqTile * 2;        // 8 KiB
constexpr int kMqMaxOff = kMqPOff + 2 * kMqPBytes;            // per-head tile maxima, 2 halves
constexpr int kMqSumOff = kMqMaxOff + 2 * kMqHeadsPerWg * 4;  // per-head tile sums, 2 halves
constexpr int kMqFacOff = kMqSumOff + 2 * kMqHeadsPerWg * 4;  // per-head sink weights
constexpr int kMqInvOff = kMqFacOff + kMqHeadsPerWg * 4;      // per-head 1 / sum at the end
constexpr int kMqFlagOff = kMqInvOff + kMqHeadsPerWg * 4;     // restart votes: 2 tile parities x 8 bytes
constexpr int kMqLdsBytes = kMqFlagOff + 16;
static_assert(kMqLdsBytes <= 160 * 1024, "one workgroup per CU");
static_assert(kMqaHeads == 128 && kMqaDim == 512, "fragment layout assumes 128 heads of 512 dims");
constexpr float kMqHeadroom = 64.f;                           // log2 growth past the reference before a restart

struct MqArgs {
  const char* q;            // [T][128][512] bf16
  const char* kv;           // [N][512] bf16
  const int64_t* cu_k;      // [batch + 1]
  const int32_t* n_valid;   // [T] or null
  const TileRec* tiles;     // one per query; workgroups 2 t and 2 t + 1 take its two head halves
  const char* k_sink;       // [512] bf16 or null
  const char* v_sink;       // [512] bf16 or null
  float c2;                 // scale * log2(e)
  char* out;                // [T][128][512] of out_dt
  float* lse;               // [T][128] or null
};

__device__ __forceinline__ int kv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int DOUT>
__global__ __launch_bounds__(kMqThreads, 1) void mqa_sink_kernel(MqArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kMqLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wave & 3;                   // index within the wave's role
  const int h2 = lane >> 5;                 // lane half
  const TileRec tile = a.tiles[blockIdx.x >> 1];
  const int head0 = (blockIdx.x & 1) * kMqHeadsPerWg;
  const int seq = tile_seq(tile.flags);
  const int64_t t = tile.row_start;
  const int64_t kbase = a.cu_k[seq];
  const int nk = (int)(a.cu_k[seq + 1] - kbase);
  const int nv = a.n_valid ? min(max(a.n_valid[t], 0), nk) : nk;
  const int n_tiles = (nv + kMqTile - 1) / kMqTile;

  char* const P = lds + kMqPOff;
  float* const pmax = reinterpret_cast<float*>(lds + kMqMaxOff);   // [kb][64]
  float* const psm = reinterpret_cast<float*>(lds + kMqSumOff);    // [kb][64] sums at the end
  float* const sinkw = reinterpret_cast<float*>(lds + kMqFacOff);  // [64] sink weight / sum at the end
  float* const inv = reinterpret_cast<float*>(lds + kMqInvOff);    // [64]
  uint8_t* const flags = reinterpret_cast<uint8_t*>(lds + kMqFlagOff);
  const auto votes_of = [&](int j) {
    return __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(flags + 8 * (j & 1))) != 0;
  };

  // The two roles run separate code with the same sequence of workgroup
  // barriers (marked B below), so that neither role's registers are live in
  // the other's code.
  if (wave < 4) {
    // ================= score waves =================
    __builtin_amdgcn_s_setprio(1);      // their probabilities gate the next step
    // Role: head block hb (32 heads), entry block kb (32 of the tile's 64
    // entries).  Query fragments of the head block: B operand of S^T = E Q^T;
    // k-step kk covers dims 16 kk .. 16 kk + 15, lane half h2 the 8 from
    // 16 kk + 8 h2.
    const int hb_s = w & 1, kb_s = w >> 1;
    const int hl = 32 * hb_s + (lane & 31);   // head within the workgroup
    bf16x8_t qf[32];
    {
      const char* qrow = a.q + ((t * kMqaHeads + head0 + hl) * kMqRowBytes) + h2 * 16;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) qf[kk] = __builtin_bit_cast(bf16x8_t, ld16(qrow + kk * 32));
    }
    // Sink logit of head hl (log2 units; -inf without a sink).
    float s_sink = -INFINITY;
    if (a.k_sink) {
      float dot = 0.f;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) {
        const uint4 ks = ld16(a.k_sink + kk * 32 + h2 * 16);
        const uint32_t kw[4] = {ks.x, ks.y, ks.z, ks.w};
        const uint4 qv = __builtin_bit_cast(uint4, qf[kk]);
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dot = fmaf(__uint_as_float(qw[e] << 16), __uint_as_float(kw[e] << 16), dot);
          dot = fmaf(__uint_as_float(qw[e] & 0xffff0000u), __uint_as_float(kw[e] & 0xffff0000u), dot);
        }
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dot), __float_as_uint(dot), false, false);
      dot = h2 ? __uint_as_float(sw[0]) + dot : dot + __uint_as_float(sw[1]);
      s_sink = dot * a.c2;
    }
    // Softmax state of head hl, kept alike by the two score waves of its
    // head block (and both lane halves): the reference m_ref and the sum of
    // 2^(logit - m_ref) over the wave's entries.  m_ref is set at the first
    // tile, before anything is accumulated, to the largest of the sink
    // logit, that tile's maximum and the floor left by a restart; a later
    // tile may exceed it by up to the headroom (2^64 fits bf16 and, times
    // the values, fp32).  A tile that exceeds it by more ends the pass: the
    // floor rises to that tile's maximum and the sweep starts again (never in
    // practice: logits would have to grow by 44 natural units), so the
    // accumulators are never rescaled.
    float m_ref = -INFINITY, l_run = 0.f, m_floor = -INFINITY;

    // Copies of one tile: score wave w fills rows 16 w .. 16 w + 15, one 1 KiB
    // row per copy; lane p writes slot p, which holds chunk p ^ f(row) of that
    // entry.  The whole offset travels in the lane's offset register, the one
    // part of the address that the descriptor's range check covers: rows past
    // the sequence's entries then read as zeros.
    const __amdgpu_buffer_rsrc_t src = ranged_rsrc(a.kv + kbase * kMqRowBytes, (uint32_t)nk * kMqRowBytes);
    const auto issue_row = [&](int j, int i, int lane_v) {
      const int r = 16 * w + i;
      const uint32_t row_off = (uint32_t)(r * kMqRowBytes) + (uint32_t)j * kMqTileBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)(lds + (j & 1) * kMqTileBytes + r * kMqRowBytes),
                                               16, (uint32_t)((lane_v ^ kv_swz(i)) << 4) + row_off, 0, 0, 0);
    };
    const auto issue_tile = [&](int j) {
#pragma unroll
      for (int i = 0; i < 16; ++i) issue_row(j, i, lane);
    };
    // Score A fragment, k-step kk = 8 m + u: row r_s, chunk (2 kk + h2) ^ f(r_s)
    // = 16 m + ((2 u + h2) ^ f(r_s)), i.e. koff[u] + 256 m.
    const int r_s = 32 * kb_s + (lane & 31);
    uint32_t koff[8];
    {
      const int eswz = kv_swz(r_s);
#pragma unroll
      for (int u = 0; u < 8; ++u) koff[u] = (uint32_t)(r_s * kMqRowBytes + (((2 * u + h2) ^ eswz) << 4));
    }
    // Scores S^T of tile buffer E: entry fragments read kSPre k-steps ahead of
    // their MFMA, two accumulator chains (even and odd k-steps).  The copies
    // of tile j_copy go one after every second MFMA: each holds the issuing
    // wave for ~16 cycles, which the MFMAs' shadow hides (issued all at once
    // before the MFMAs, they cost 5% of the kernel's time).
    const auto score_tile = [&](const char* E, int j_copy) {
      int lane_v = lane;                  // recomputed copy offsets: kept out of registers across tiles
      asm volatile("" : "+v"(lane_v));
      constexpr int kSPre = 4;
      f32x4_t ef[kSPre];
      const auto load_s = [&](int kk) { return *reinterpret_cast<const f32x4_t*>(E + koff[kk & 7] + 256 * (kk >> 3)); };
#pragma unroll
      for (int kk = 0; kk < kSPre; ++kk) ef[kk] = load_s(kk);
      f32x16_t s2[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) {
        s2[kk & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ef[kk % kSPre]), qf[kk],
                                                             s2[kk & 1], 0, 0, 0);
        if (kk + kSPre < 32) ef[kk % kSPre] = load_s(kk + kSPre);
        if (kk & 1) issue_row(j_copy, kk >> 1, lane_v);
        __builtin_amdgcn_sched_barrier(0);   // keep this order: the scheduler would sink the reads
      }
      return s2[0] + s2[1];
    };
    // Maximum logit of head hl over the wave's 32 entries of tile j (log2
    // units).  A tile wholly inside the visible entries keeps the raw dot
    // products (the logit is folded into the exponent's fused multiply-add,
    // and the maximum logit is the larger of scale * max and scale * min, for
    // either sign of the scale); the tile that crosses the visible count turns
    // them into logits, -inf where hidden, and scales by 1 (cs).
    const auto tile_max = [&](int j, f32x16_t& s, float& cs) {
      float mt;
      if ((j + 1) * kMqTile <= nv) {
        float hi = s[0], lo = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) {
          hi = fmaxf(hi, s[e]);
          lo = fminf(lo, s[e]);
        }
        mt = fmaxf(hi * a.c2, lo * a.c2);
        cs = a.c2;
      } else {
        const int e0 = j * kMqTile + 32 * kb_s;
        mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = e0 + 8 * (e >> 2) + 4 * h2 + (e & 3);
          s[e] = key < nv ? s[e] * a.c2 : -INFINITY;
          mt = fmaxf(mt, s[e]);
        }
        cs = 1.f;
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      return fmaxf(mt, __uint_as_float(h2 ? sw[0] : sw[1]));
    };
    // Probabilities 2^(logit - m_ref) into P buffer Pb (bf16, P[head][entry],
    // 64 rows of 128 bytes, chunk c of head row h at slot c ^ ((h >> 1) & 7));
    // their sum joins l_run (both lane halves).
    const auto write_p = [&](const f32x16_t& s, float cs, char* Pb) {
      float psum = 0.f;
      char* const prow = Pb + hl * 128;
      const int pswz = (hl >> 1) & 7;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = exp2_hw(fmaf(s[4 * g + i], cs, -m_ref));
          psum += p[i];
        }
        *reinterpret_cast<uint2*>(prow + (((4 * kb_s + g) ^ pswz) << 4) + 8 * h2) =
            make_uint2(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]));
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum), false, false);
      l_run += h2 ? __uint_as_float(sw[0]) + psum : psum + __uint_as_float(sw[1]);
    };

#pragma unroll 1
    for (;;) {                            // one pass; a second only after a restart
      l_run = 0.f;
      bool again = false;
      if (n_tiles > 0) {
        issue_tile(0);
        wait_vmcnt_lgkm0<0>();            // own copies of tile 0 landed
        lds_barrier();                    // B: tile 0 in
        // tile 0: it sets the reference, from the maximum over both entry halves
        f32x16_t s = score_tile(lds, 1);  // with tile 1's copies (past the last tile: zeros or unread)
        float cs;
        const float mt0 = tile_max(0, s, cs);
        if (h2 == 0) pmax[kb_s * 64 + hl] = mt0;
        wait_lgkmcnt0();
        lds_barrier();                    // B: both halves' maxima are in
        m_ref = fmaxf(fmaxf(m_floor, s_sink), fmaxf(mt0, pmax[(kb_s ^ 1) * 64 + hl]));
        write_p(s, cs, P);
        wait_vmcnt_lgkm0<0>();            // tile 1 landed; tile 0's probabilities written
        lds_barrier();                    // B: step 1 may start
#pragma unroll 1
        for (int j = 1; j < n_tiles; ++j) {
          // with tile j + 1's copies, into the buffer of tile j - 1, which nobody reads any more
          f32x16_t s = score_tile(lds + (j & 1) * kMqTileBytes, j + 1);
          float cs;
          const float mt = tile_max(j, s, cs);
          const bool any = __ballot(mt > m_ref + kMqHeadroom) != 0;   // every lane votes, lane 0 records it
          if (lane == 0) flags[8 * (j & 1) + w] = any ? 1 : 0;
          write_p(s, cs, P + (j & 1) * kMqPBytes);
          wait_vmcnt_lgkm0<0>();          // tile j + 1 landed; probabilities and vote written
          lds_barrier();                  // B: step j + 1 may start
          // A restart ends the pass here, at the end of the step, so that the
          // loop body stays one block.
          if (votes_of(j)) {
            if (h2 == 0) pmax[kb_s * 64 + hl] = mt;
            wait_lgkmcnt0();
            lds_barrier();                // B: both halves' maxima are in
            // at least this tile's maximum from now on
            m_floor = fmaxf(m_ref, fmaxf(mt, pmax[(kb_s ^ 1) * 64 + hl]));
            again = true;
            break;
          }
        }
      }
      if (!again) break;
      wait_vmcnt<0>();                    // no copy is in flight
      lds_barrier();                      // B: the value waves have left the pass too
    }

    // ---- the normaliser of head hl: both entry halves' sums and the sink's
    // weight; its inverse and the sink's weight share go to the value waves
    if (h2 == 0) psm[kb_s * 64 + hl] = l_run;
    wait_lgkmcnt0();
    lds_barrier();                        // B: sums in
    if (kb_s == 0 && h2 == 0) {
      if (n_tiles == 0) m_ref = s_sink;   // nothing visible: the sink alone (if any)
      const float ws = a.k_sink ? exp2_hw(s_sink - m_ref) : 0.f;
      const float l = psm[hl] + psm[64 + hl] + ws;
      inv[hl] = l > 0.f ? 1.f / l : 0.f;
      sinkw[hl] = l > 0.f && a.v_sink ? ws / l : 0.f;
      if (a.lse) a.lse[t * kMqaHeads + head0 + hl] = l > 0.f ? (m_ref + __log2f(l)) * 0.6931471805599453f : -INFINITY;
    }
    wait_lgkmcnt0();
    lds_barrier();                        // B: factors in
  } else {
    // ================= value waves =================
    // Role: output columns 128 w .. 128 w + 127 of the 64 heads.  Accumulators
    // O^T[cb][hb]: column 128 w + 32 cb + (8 g + 4 h2 + i), head 32 hb + l % 32
    // (element 4 g + i).  The sink's value joins at the end, as its weight
    // times v_sink.
    f32x16_t o[4][2];
    // Per-lane offsets within a tile buffer:
    //  * value A fragment, step ks, block cb, half: row 16 ks + 8 h2 + 4 half +
    //    i16 / 4, column 128 w + 32 cb + 16 grp + 4 (i16 % 4): troff[half][cb]
    //    + 16 KiB ks (the swizzle depends on the row only through row % 16);
    //  * P fragment of step ks: head row 32 hb + l % 32, chunk (2 ks + h2) ^ ps:
    //    poff[ks] + 4 KiB hb.
    const int i16 = lane & 15, grp = (lane >> 4) & 1;
    uint32_t troff[2][4], poff[4];
    {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r = 8 * h2 + 4 * half + (i16 >> 2);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int col = 128 * w + 32 * cb + 16 * grp + 4 * (i16 & 3);
          troff[half][cb] = (uint32_t)(r * kMqRowBytes + (((col >> 3) ^ kv_swz(r)) << 4) + ((col & 7) << 1));
        }
      }
      const int ps = ((lane & 31) >> 1) & 7;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) poff[ks] = (uint32_t)((lane & 31) * 128 + (((2 * ks + h2) ^ ps) << 4));
    }
    // Transposed entry fragment (A operand of the value product) of step ks
    // (entries 16 ks ..) and column block cb of tile buffer E, 8 entries of
    // one column per lane: gfx950's transposing LDS read, 4 entries per read.
    const auto load_et_cb = [&](const char* E, int ks, int cb, bf16x8_t& f) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      v4s part[2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
        part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(E + troff[half][cb] + 16 * kMqRowBytes * ks));
      const uint2 lo = __builtin_bit_cast(uint2, part[0]), hi = __builtin_bit_cast(uint2, part[1]);
      f = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    const auto load_p = [&](const char* Pb, int ks, bf16x8_t (&f)[2]) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        f[hb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(Pb + poff[ks] + 32 * 128 * hb));
    };
    // O^T[col][head] += E^T[col][entry] P^T[entry][head] over one tile, from
    // its fragments et and probabilities in Pb; with refill, each fragment is
    // replaced by the next tile's (from E_next) as soon as its two MFMAs are
    // issued, so the transposing reads spread over the MFMAs.
    bf16x8_t et[4][4];
    const auto value_tile = [&](const char* Pb, const char* E_next, auto refill) {
      bf16x8_t bp[4][2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) load_p(Pb, ks, bp[ks]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            o[cb][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(et[ks][cb], bp[ks][hb], o[cb][hb], 0, 0, 0);
          if constexpr (decltype(refill)::value) load_et_cb(E_next, ks, cb, et[ks][cb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

#pragma unroll 1
    for (;;) {                            // one pass; a second only after a restart
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) o[cb][0] = o[cb][1] = f32x16_t{};
      bool again = false;
      if (n_tiles > 0) {
        lds_barrier();                    // B: tile 0 in
        lds_barrier();                    // B: (the score waves' maxima)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) load_et_cb(lds, ks, cb, et[ks][cb]);
        wait_lgkmcnt0();                  // tile 0's fragments read: its buffer may be refilled
        lds_barrier();                    // B: step 1 may start
#pragma unroll 1
        for (int j = 1; j < n_tiles; ++j) {
          value_tile(P + ((j - 1) & 1) * kMqPBytes, lds + (j & 1) * kMqTileBytes, std::true_type{});
          wait_lgkmcnt0();                // tile j's fragments read
          lds_barrier();                  // B: step j + 1 may start
          if (votes_of(j)) {
            lds_barrier();                // B: (the score waves' maxima)
            again = true;
            break;
          }
        }
        if (!again) value_tile(P + ((n_tiles - 1) & 1) * kMqPBytes, lds, std::false_type{});   // the last tile
      }
      if (!again) break;
      lds_barrier();                      // B: the score waves have left the pass too
    }
    lds_barrier();                        // B: sums in
    lds_barrier();                        // B: factors in

    // ---- normalise and store: o[t][head][col] = (O^T[col][head] + sink
    // weight * v_sink[col]) / sum, the sum including the sink's weight
    const uint16_t* const vs = reinterpret_cast<const uint16_t*>(a.v_sink);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hd = 32 * hb + (lane & 31);
      const float f = inv[hd], fs = sinkw[hd];
      char* orow = a.out + (t * kMqaHeads + head0 + hd) * (int64_t)kMqaDim * (DOUT == DT_BF16 ? 2 : 4);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 128 * w + 32 * cb + 8 * g + 4 * h2;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = o[cb][hb][4 * g + i] * f;
          if (vs) {
            const uint2 sv = *reinterpret_cast<const uint2*>(vs + col);
            v[0] = fmaf(fs, __uint_as_float(sv.x << 16), v[0]);
            v[1] = fmaf(fs, __uint_as_float(sv.x & 0xffff0000u), v[1]);
            v[2] = fmaf(fs, __uint_as_float(sv.y << 16), v[2]);
            v[3] = fmaf(fs, __uint_as_float(sv.y & 0xffff0000u), v[3]);
          }
          if (DOUT == DT_BF16)
            *reinterpret_cast<uint2*>(orow + col * 2) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          else
            *reinterpret_cast<float4*>(orow + col * 4) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
  }
}

}  // namespace

hipError_t launch_mqa_sink(int out_dt, const void* q, const void* kv, const int64_t* cu_k_dev, const int32_t* n_valid,
                           const TileRec* tiles, int T, const void* k_sink, const void* v_sink, float scale, void* out,
                           float* lse, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  MqArgs a;
  a.q = static_cast<const char*>(q);
  a.kv = static_cast<const char*>(kv);
  a.cu_k = cu_k_dev;
  a.n_valid = n_valid;
  a.tiles = tiles;
  a.k_sink = static_cast<const char*>(k_sink);
  a.v_sink = static_cast<const char*>(v_sink);
  a.c2 = scale * kLog2e;
  a.out = static_cast<char*>(out);
  a.lse = lse;
  if (out_dt == DT_BF16)
    hipLaunchKernelGGL(mqa_sink_kernel<DT_BF16>, dim3(2 * T), dim3(kMqThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(mqa_sink_kernel<DT_F32>, dim3(2 * T), dim3(kMqThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace seqcomp
