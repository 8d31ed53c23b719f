/*
 * seqcomp -- token-level KV sequence compressor (CSA / HCA) for AMD MI355X.
 *
 * C ABI.  Plain pointers and sizes only; device pointers are HIP device
 * memory of the current device; `stream` is a hipStream_t passed as void*
 * (NULL = the default stream).
 *
 * What is computed (sources are web pages, cited by title and equation):
 *  - projection, "序列压缩注意力" eq. attn-seqcomp-csa-proj:
 *        C^a = H W^{KV_a}, C^b = H W^{KV_b}, Z^a = H W^{Z_a}, Z^b = H W^{Z_b}
 *    (HCA: C = H W^{KV}, Z = H W^{Z});
 *  - CSA pooling, eq. attn-seqcomp-csa-softmax and eq. attn-seqcomp-csa-pool:
 *    entry i takes ONE per-channel softmax over the 2m rows
 *    [Z^a rows m i .. m(i+1)-1 (+ B^a) ; Z^b rows m(i-1) .. m i - 1 (+ B^b)]
 *    and sums the matching C^a / C^b rows weighted by it;
 *  - the entry-0 boundary, eq. attn-seqcomp-overlap-bound: the missing b rows
 *    have logit -inf and vector 0, so entry 0 is the a-stream alone;
 *  - HCA pooling, eq. attn-seqcomp-hca: a per-channel softmax over the m'
 *    rows of block i of Z + B, applied to the same rows of C; no overlap.
 * A sequence of n tokens gives floor(n/m) entries; a partial tail block is
 * dropped.  Sequences of a packed batch are independent: every sequence's
 * entry 0 takes the boundary rule, and no window crosses a sequence.
 *
 * Layouts (all row-major, element strides in elements):
 *  - H        [T x d]        rows = tokens, d contiguous.
 *  - Wt       [S*c x d]      rows = output channels ("nn.Linear" layout,
 *                            K contiguous).  CSA (S = 4): rows
 *                            [0,c) = W^{KV_a}^T, [c,2c) = W^{KV_b}^T,
 *                            [2c,3c) = W^{Z_a}^T, [3c,4c) = W^{Z_b}^T.
 *                            HCA (S = 2): [W^{KV}^T ; W^{Z}^T].
 *  - B^a, B^b [m x c] fp32;  B [m x c] fp32 (HCA).  Row r is added to the
 *                            logits of row r of a block.
 *  - pooling streams         [T x ld_in] each, channels [0, c) used.
 *  - out      [E x c]        E = sum_b floor(L_b / m), entries packed
 *                            sequence after sequence; row stride c.
 *  - out_scale [E] fp32      only for SEQCOMP_FP8_E4M3 output: entry i is
 *                            decode(out[i, :]) * out_scale[i], with
 *                            out_scale[i] = max_ch |entry_i| / 448 (1 if the
 *                            entry is all zero).
 *  - cu_seqlens [batch+1] int64: 0 = cu[0] <= cu[1] <= ... <= cu[batch];
 *    sequence b is rows [cu[b], cu[b+1]).  Both a host copy (validation,
 *    launch sizing) and a device copy (read by the kernels) are passed; they
 *    must hold the same values.
 *
 * Dtypes: inputs SEQCOMP_F32 or SEQCOMP_BF16 (all inputs of a call share
 * one dtype; biases are always fp32); outputs SEQCOMP_F32, SEQCOMP_BF16
 * (round to nearest even) or SEQCOMP_FP8_E4M3 (OCP E4M3FN, saturating,
 * round to nearest even, per-entry scale).  Accumulation is fp32.
 *
 * Alignment: every device pointer 16-byte aligned; ld_in, ld_y multiples of
 * 16 bytes; d a multiple of 64; c a multiple of 16.
 *
 * Ownership: the caller owns every buffer.  The library never allocates or
 * frees memory; scratch space comes from the caller's `workspace` (size from
 * seqcomp_workspace_bytes).  It keeps no state between calls and is safe to
 * call from several host threads on different streams, given disjoint
 * outputs and workspaces.  The one exception is
 * seqcomp_compress_fused_noalloc, which takes no workspace: it runs in a
 * 64 MiB scratch array that the library holds per device, shared by all such
 * calls on that device.
 *
 * Errors: every argument is validated on the host before any HIP call; on a
 * failed validation nothing is launched and no output is written.  A launch
 * failure returns SEQCOMP_E_HIP.  Calls are asynchronous on `stream`:
 * faults during execution surface at the caller's next synchronisation.
 * A call with zero entries returns SEQCOMP_OK and launches nothing.
 */
#ifndef SEQCOMP_H
#define SEQCOMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum seqcomp_status_code {
  SEQCOMP_OK = 0,
  SEQCOMP_E_NULL = 1,        /* a required pointer is NULL                      */
  SEQCOMP_E_SHAPE = 2,       /* a size is out of range or sizes disagree        */
  SEQCOMP_E_DTYPE = 3,       /* dtype not supported for that argument           */
  SEQCOMP_E_ALIGN = 4,       /* pointer or row stride not 16-byte aligned       */
  SEQCOMP_E_ALIAS = 5,       /* an output overlaps an input or the workspace    */
  SEQCOMP_E_WORKSPACE = 6,   /* workspace missing or smaller than required      */
  SEQCOMP_E_UNSUPPORTED = 7, /* well-formed but not supported (m, d, c)         */
  SEQCOMP_E_HIP = 8,         /* a HIP runtime call or kernel launch failed      */
  SEQCOMP_E_SEQLENS = 9,     /* cu_seqlens not 0-based / not non-decreasing / past T */
  SEQCOMP_E_SCRATCH = 10     /* the allocation-free call needs more than its 64 MiB */
};

enum seqcomp_dtype { SEQCOMP_F32 = 0, SEQCOMP_BF16 = 1, SEQCOMP_FP8_E4M3 = 2 };
enum seqcomp_mode { SEQCOMP_MODE_CSA = 0, SEQCOMP_MODE_HCA = 1 };
enum seqcomp_op { SEQCOMP_OP_POOL_CSA = 0, SEQCOMP_OP_POOL_HCA = 1, SEQCOMP_OP_FUSED = 2 };

/* Library version, major*10000 + minor*100 + patch. */
int seqcomp_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* seqcomp_status_string(int status);

/* Number of entries of a packed batch: sum_b floor((cu[b+1]-cu[b]) / m).
 * Returns -1 if cu_seqlens_host is NULL, batch < 0, m < 1 or cu is malformed. */
int64_t seqcomp_num_entries(const int64_t* cu_seqlens_host, int64_t batch, int64_t m);

/* Bytes of device workspace a call needs (0 if none).  `op` selects the
 * call: SEQCOMP_OP_POOL_CSA / SEQCOMP_OP_POOL_HCA (mode ignored) or
 * SEQCOMP_OP_FUSED with `mode`.  Returns (size_t)-1 on malformed arguments. */
size_t seqcomp_workspace_bytes(int op, int mode, int64_t m, int64_t c,
                               const int64_t* cu_seqlens_host, int64_t batch, int out_dtype);

/*
 * Projection (eq. attn-seqcomp-csa-proj): Y[T x n_out] = H[T x d] * Wt^T,
 * i.e. Y[t, j] = sum_k H[t, k] Wt[j, k].  For the compressor, n_out = S*c
 * and Wt is the stacked weight matrix above, so Y's column slabs are
 * C^a | C^b | Z^a | Z^b (HCA: C | Z) and can be passed to the pooling calls
 * with ld_in = ld_y.
 *   H, Wt: in_dtype (F32 or BF16).  Y: out_dtype (F32 or BF16), row stride ld_y >= n_out.
 *   Requires d % 64 == 0, n_out % 16 == 0.  bf16 uses the MFMA matrix cores
 *   with fp32 accumulation.  Y must not overlap H or Wt.
 */
int seqcomp_project(const void* H, int64_t T, int64_t d, int in_dtype,
                    const void* Wt, int64_t n_out,
                    void* Y, int64_t ld_y, int out_dtype, void* stream);

/*
 * CSA pooling from materialised streams (eq. attn-seqcomp-csa-softmax,
 * eq. attn-seqcomp-csa-pool, eq. attn-seqcomp-overlap-bound).
 *   Ca, Cb, Za, Zb: [T x ld_in] of in_dtype, T = cu[batch]; they may be
 *   column slices of one seqcomp_project output.  Ba, Bb: [m x c] fp32.
 *   c <= ld_in <= 2^32.  1 <= m <= 16.  out: [E x c] of out_dtype; out_scale: [E] fp32, required
 *   iff out_dtype is SEQCOMP_FP8_E4M3 (else ignored, may be NULL).
 *   workspace: seqcomp_workspace_bytes(SEQCOMP_OP_POOL_CSA, ...) bytes.
 */
int seqcomp_pool_csa(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                     int64_t ld_in, int in_dtype,
                     const float* Ba, const float* Bb, int64_t m, int64_t c,
                     const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev, int64_t batch,
                     void* out, int out_dtype, float* out_scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * HCA pooling from materialised streams (eq. attn-seqcomp-hca).
 *   C, Z: [T x ld_in] of in_dtype; B: [m x c] fp32; 1 <= m <= 256.
 *   Other arguments as seqcomp_pool_csa.
 */
int seqcomp_pool_hca(const void* C, const void* Z, int64_t ld_in, int in_dtype,
                     const float* B, int64_t m, int64_t c,
                     const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev, int64_t batch,
                     void* out, int out_dtype, float* out_scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused compressor: projection, logits + bias + boundary, per-channel
 * softmax, Hadamard-weighted sum and output encoding in one pass over H;
 * the projected streams stay on chip ("序列压缩注意力", section on the flash
 * compressor, describes the single-pass idea).
 *   mode SEQCOMP_MODE_CSA: m must be 4; Wt is [4c x d]; Ba, Bb [4 x c].
 *   mode SEQCOMP_MODE_HCA: m must be 128; Wt is [2c x d]; Ba is B [128 x c];
 *                          Bb must be NULL.
 *   H: [T x d], T = cu[batch]; d % 64 == 0; c % 16 == 0.
 *   out, out_scale, workspace as in seqcomp_pool_csa, with
 *   workspace_bytes >= seqcomp_workspace_bytes(SEQCOMP_OP_FUSED, mode, ...).
 */
int seqcomp_compress_fused(int mode, int64_t m, const void* H, int64_t d, int in_dtype,
                           const void* Wt, int64_t c, const float* Ba, const float* Bb,
                           const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev, int64_t batch,
                           void* out, int out_dtype, float* out_scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free form of seqcomp_compress_fused, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, computation and results
 * as seqcomp_compress_fused, without the workspace: the call uses a 64 MiB
 * scratch array that the library holds on each device it runs on (from the
 * first such call on that device until the process ends).  It calls no
 * allocator.
 *   A call whose workspace would exceed 64 MiB (see seqcomp_workspace_bytes
 *   with SEQCOMP_OP_FUSED) is rejected with SEQCOMP_E_SCRATCH before any
 *   launch: at c = 512 that is about 5400 tiles of 256 rows (~1.38M tokens)
 *   for CSA with bf16 or fp32 output, and about 470 tiles (~120K tokens)
 *   with fp8 output, whose fp32 staging also lives there.
 *   Every call on a device shares that device's array: calls that overlap in
 *   time on one device (two streams, two host threads) race and may produce
 *   wrong entries; serialise them.  Nothing in the array needs to start at
 *   zero (each call writes what it later reads).
 */
int seqcomp_compress_fused_noalloc(int mode, int64_t m, const void* H, int64_t d, int in_dtype,
                                   const void* Wt, int64_t c, const float* Ba, const float* Bb,
                                   const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev, int64_t batch,
                                   void* out, int out_dtype, float* out_scale, void* stream);

/*
 * CSA decode append: the compressor of eq. attn-seqcomp-csa-proj,
 * -csa-softmax and -csa-pool applied to one new block per sequence, with the
 * overlapping b-stream carried between calls as a softmax partial.  Each of
 * nb sequences has just completed a block of m = 4 tokens; entry j is that
 * block's compressed entry.  No sequence crosses a block of another.
 *   H         [4 nb x d] in_dtype: block j = rows [4j, 4j + 4) (oldest first).
 *   Wt        [4c x d], Ba, Bb [4 x c] fp32: as in seqcomp_compress_fused.
 *   state_in  [nb][3][c] fp32: for sequence j, the b-stream partial of its
 *             previous block as three planes (M, S, A) -- running maximum of
 *             log2(e) (Z^b + B^b), sum of 2^(logit - M), and that sum
 *             weighted by C^b -- exactly as this call writes it to state_out.
 *             A sequence's first block passes M = -inf, S = A = 0: its
 *             missing b rows then get weight 0 (eq. attn-seqcomp-overlap-bound).
 *             The planes are otherwise opaque to the caller.
 *   state_out [nb][3][c] fp32: block j's own b-stream partial, the state for
 *             the sequence's next append.  May be the same pointer as
 *             state_in (updated in place); must not overlap it otherwise.
 *   out       [nb x c] of out_dtype; out_scale [nb] fp32 for fp8 output.
 *   workspace seqcomp_append_workspace_bytes(nb, c, out_dtype) bytes.
 *             nb <= 2 runs one kernel with a wave per weight row and needs
 *             none.  Otherwise, when the batch's 256 x 256 tiles (64
 *             channels x 4 streams) do not fill 256 workgroups, it runs
 *             128 x 128 tiles (32 channels x 4 streams) and, if those are
 *             fewer than 256 too, splits the K loop over up to 32 workgroups
 *             per tile; their fp32 partial products take 64 KiB per tile and
 *             split (16 MiB at nb = 64, c = 512).  An fp8 output adds nb x c
 *             fp32 of staging.  0 when neither applies.
 *   Requires d % 64 == 0, c % 16 == 0.  nb == 0 returns SEQCOMP_OK.
 * Appending a sequence's blocks one call at a time gives the same entries as
 * seqcomp_compress_fused over the whole sequence (up to rounding order).
 */
int seqcomp_csa_append(const void* H, int64_t nb, int64_t d, int in_dtype, const void* Wt, int64_t c,
                       const float* Ba, const float* Bb, const float* state_in, float* state_out,
                       void* out, int out_dtype, float* out_scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of seqcomp_csa_append; (size_t)-1 on malformed arguments. */
size_t seqcomp_append_workspace_bytes(int64_t nb, int64_t c, int out_dtype);

/*
 * Partial RoPE and mixed-precision store of compressed entries into a cache
 * ("Ch 05 · HCA — 长上下文的全景镜", section on partial RoPE;
 * "混合压缩注意力双方案解析", section 3 on mixed-precision storage).
 *   entries   [E x c] of in_dtype (F32 or BF16): the packed output of a
 *             compressor call over the batch described by cu_seqlens and m
 *             (E = sum_b floor(L_b / m)).
 *   Entry e, compressing block i of sequence b, has position
 *   pos0[b] + m i + (m - 1) / 2 (the block centre; pos0_dev [batch] int64,
 *   NULL for all zero).  Its last r = rope_dims dimensions are turned in
 *   adjacent pairs: pair k (columns c - r + 2k, c - r + 2k + 1) by the angle
 *   pos * rope_base^(-2k / r); the first c - r dimensions are left as they are.
 *   Entry e goes to cache row slots_dev[e] (int64 [E]; NULL: row e); rows
 *   must be distinct; a row outside [0, n_slots) is not stored; n_slots <= 2^40.
 *   cache_nope  [n_slots x (c - r)] OCP E4M3 codes of the first c - r
 *               dimensions divided by cache_scale[row];
 *   cache_scale [n_slots] fp32: max |x| over those c - r dimensions / 448 (1 if
 *               they are all zero);
 *   cache_rope  [n_slots x r] bf16 (round to nearest even) of the rotated part.
 *   Requires c % 16 == 0, 0 <= r <= c, r % 8 == 0, rope_base > 0.
 *   workspace: seqcomp_rope_store_workspace_bytes(m, cu, batch) bytes.
 */
int seqcomp_rope_store(const void* entries, int in_dtype, int64_t c, int64_t m,
                       const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev, int64_t batch,
                       const int64_t* pos0_dev, int64_t rope_dims, double rope_base,
                       const int64_t* slots_dev, int64_t n_slots, uint8_t* cache_nope, float* cache_scale,
                       uint16_t* cache_rope, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of seqcomp_rope_store; (size_t)-1 on malformed arguments. */
size_t seqcomp_rope_store_workspace_bytes(int64_t m, const int64_t* cu_seqlens_host, int64_t batch);

/*
 * Lightning indexer ("Ch 04 · CSA — 长上下文的快通道", section 4): index
 * scores of queries against compressed indexer keys and, per query, the set
 * of its k best keys:
 *     I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s])
 * over the n_h^I = 64 indexer heads of c^I = 128 dimensions.
 *   q         [T x 64 x 128] bf16: indexer queries, packed by sequence (cu_q).
 *   w         [T x 64] fp32: head weights.
 *   keys      [N x 128] bf16: compressed indexer keys, packed by sequence
 *             (cu_k; e.g. the output of a CSA compressor with c = 128).
 *   cu_q, cu_k [batch + 1] int64, host and device copies (same values):
 *             sequence b owns queries [cu_q[b], cu_q[b+1]) and keys
 *             [cu_k[b], cu_k[b+1]); a query scores only its own sequence's keys.
 *   n_valid   [T] int32 (device) or NULL: query t sees the first n_valid[t]
 *             keys of its sequence (clamped to [0, its key count]), e.g. the
 *             entries whose blocks are complete at its position; NULL: all.
 *   k         1..1024.
 *   out_idx   [T x k] int32: the selected keys (index within the sequence),
 *             the k visible keys of largest score with ties going to the
 *             smaller index, listed by increasing index; when fewer than k
 *             keys are visible, all of them, then -1.
 *   out_score [T x k] fp32 or NULL: the selected keys' scores (-inf after the
 *             last selected key).
 * Scores are fp32 (bf16 products, fp32 accumulation); a key whose score is
 * NaN is never selected.  Requires n_heads == 64, head_dim == 128, bf16
 * inputs, and fewer than 2^23 keys per sequence.
 *   workspace: seqcomp_indexer_workspace_bytes(cu_q_host, batch) bytes.
 */
int seqcomp_indexer_topk(const void* q, const float* w, const void* keys, int64_t n_heads, int64_t head_dim,
                         int in_dtype, const int64_t* cu_q_host, const int64_t* cu_q_dev,
                         const int64_t* cu_k_host, const int64_t* cu_k_dev, int64_t batch,
                         const int32_t* n_valid, int64_t k, int32_t* out_idx, float* out_score,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of seqcomp_indexer_topk; (size_t)-1 on malformed arguments. */
size_t seqcomp_indexer_workspace_bytes(const int64_t* cu_q_host, int64_t batch);

/*
 * Dense shared-KV multi-query attention with an attention sink over
 * compressed entries ("Ch 05 · HCA — 长上下文的全景镜": dense attention over
 * every entry, and the attention sink; "Ch 04 · CSA — 长上下文的快通道",
 * section 6: all heads share one KV).  For query t and head h:
 *     alpha = Softmax(scale * q[t, h] . [k_sink, e_1, ..., e_n])
 *     out[t, h] = alpha_sink * v_sink + sum_s alpha_s * e_s
 * where e_1..e_n are the entries visible to t (each entry is key and value).
 *   q        [T x 128 x 512] bf16, packed by sequence (cu_q).
 *   kv       [N x 512] bf16 entries, packed by sequence (cu_k), e.g. the
 *            HCA compressor's output.
 *   cu_q, cu_k [batch + 1] int64, host and device copies (same values).
 *   n_valid  [T] int32 (device) or NULL: query t sees the first n_valid[t]
 *            entries of its sequence (clamped to [0, its entry count]);
 *            NULL: all.
 *   k_sink   [512] bf16 or NULL (no sink); v_sink [512] bf16 or NULL (zero
 *            value); both shared by all heads.
 *   scale    the logit scale (1/sqrt(512) in the standard form); finite.
 *   out      [T x 128 x 512] of out_dtype (SEQCOMP_BF16 or SEQCOMP_F32).
 *   lse      [T x 128] fp32 or NULL: natural log of the softmax denominator
 *            of the scaled logits (sink included); -inf when nothing is
 *            visible and there is no sink (then out is zero).
 * Products are exact bf16 x bf16 in fp32; the entries' probabilities are
 * rounded to bf16 for the value product, the sink's weight times v_sink is
 * added in fp32.  The softmax runs against a fixed per-head reference, so
 * entry and sink values must stay below 2^43 in magnitude (fp32 sums of up
 * to 2^21 terms of 2^64 times a value).  Requires n_heads == 128,
 * head_dim == 512, bf16 q / kv / sink, and fewer than 2^21 entries per
 * sequence.
 *   workspace: seqcomp_mqa_workspace_bytes(cu_q_host, batch) bytes.
 */
int seqcomp_shared_kv_mqa(const void* q, const void* kv, int64_t n_heads, int64_t head_dim, int in_dtype,
                          const int64_t* cu_q_host, const int64_t* cu_q_dev, const int64_t* cu_k_host,
                          const int64_t* cu_k_dev, int64_t batch, const int32_t* n_valid, const void* k_sink,
                          const void* v_sink, float scale, void* out, int out_dtype, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes of seqcomp_shared_kv_mqa; (size_t)-1 on malformed arguments. */
size_t seqcomp_mqa_workspace_bytes(const int64_t* cu_q_host, int64_t batch);

#ifdef __cplusplus
}
#endif

#endif /* SEQCOMP_H */
