/*
 * gptoss_attn.h -- C ABI of the GPT-OSS attention hot path on MI355X (gfx950).
 *
 * Grouped-query attention with a learned per-head sink, full-causal or
 * sliding-window masks, and YaRN-scaled RoPE on q and k; bf16 in and out,
 * fp32 accumulation.
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers unless marked "host". The library
 *     never allocates, frees or copies device memory on its own and never
 *     synchronises: the caller owns every buffer (inputs, outputs, table,
 *     workspace) and keeps it alive until the work on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues kernels on it and returns. No call clears
 *     memory with a memset, and every length and work list is read or built
 *     on the device, so the calls may be captured in a HIP graph and
 *     replayed with new buffer contents (new lengths included) as long as the
 *     host-side arguments stay the same.
 *   - bf16 means IEEE bfloat16 stored as uint16; fp32 sinks.
 *   - Strides are in ELEMENTS, not bytes; the last (head_dim) dimension must
 *     be contiguous. Outputs of gptoss_rope_qk are contiguous; the attention
 *     outputs take strides.
 *   - Host-checkable argument errors return a non-zero gptoss_status before
 *     anything is launched. A failed launch returns GPTOSS_ERR_HIP.
 *     gptoss_last_error() gives a thread-local text for the last failure.
 *     No C++ exception crosses this interface.
 *   - Device-resident integer data (cu_seqlens, cache_seqlens) cannot be
 *     checked without a synchronisation. It is trusted, and the kernels clamp
 *     every index derived from it so that bad values cannot read or write
 *     outside the buffers described by the host-side sizes.
 *
 * Supported now: head_dim == 64, num_q_heads == 8 * num_kv_heads (the GPT-OSS
 * grouping: 64 query heads over 8 KV heads). Every call that takes a table
 * rotates rotary_dim = 16, 32, 48 or 64 dims (partial rotary, rope_utils page,
 * apply_rotary_emb: the dims past rotary_dim pass through), except the
 * backward pass, the k rotation inside the prefill tile loads
 * (GPTOSS_KROT_FUSED) and the projection epilogue, which take 64 (the
 * projection also 32). Other shapes return GPTOSS_ERR_UNSUPPORTED.
 */
#ifndef GPTOSS_ATTN_H
#define GPTOSS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPTOSS_ABI_VERSION 6

typedef enum {
  GPTOSS_OK = 0,
  GPTOSS_ERR_NULL = 1,        /* a required pointer is NULL */
  GPTOSS_ERR_SHAPE = 2,       /* sizes or strides are inconsistent or out of range */
  GPTOSS_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. head_dim != 64) */
  GPTOSS_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than *_workspace_size() */
  GPTOSS_ERR_HIP = 5          /* a HIP launch or query failed; see gptoss_last_error() */
} gptoss_status;

typedef enum { GPTOSS_BSHD = 0, GPTOSS_THD = 1 } gptoss_layout;

/*
 * RoPE configuration: the RotaryEmbedding constructor on the page
 * "nemo_automodel.components.models.gpt_oss.rope_utils" (head_dim, base,
 * initial_context_length = 4096, scaling_factor = 1.0, ntk_alpha = 1.0,
 * ntk_beta = 32.0, rotary_dim = head_dim * partial_rotary_factor).
 * GPT-OSS: head_dim 64, rotary_dim 64, base 150000, scaling_factor 32.
 */
typedef struct {
  int32_t head_dim;
  int32_t rotary_dim;             /* even, 0 < rotary_dim <= head_dim */
  double base;
  double scaling_factor;          /* <= 1 means plain RoPE */
  int32_t initial_context_length;
  double ntk_alpha;               /* beta_slow of YaRN */
  double ntk_beta;                /* beta_fast of YaRN */
} gptoss_rope_config;

/*
 * Sequence description shared by gptoss_rope_qk and gptoss_attn_prefill.
 * BSHD: tensors are [batch, seqlen, heads, head_dim]; every sequence has
 *       length seqlen and token s sits at position s.
 * THD:  tensors are packed [seqlen = total tokens, heads, head_dim]; sequence n
 *       holds tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 and positions restart
 *       at 0 in every sequence. `batch` is the number of sequences and
 *       cu_seqlens a DEVICE int32 array of batch+1 entries, cu_seqlens[0] = 0,
 *       non-decreasing, cu_seqlens[batch] = seqlen. `max_seqlen` is a host-side
 *       upper bound of the sequence lengths (it sizes the grid).
 * (page "nemo_automodel.components.models.gpt_oss.rope_utils",
 *  apply_rotary_emb_qk: format "bshd" or "thd", cu_seqlens [num_sequences+1];
 *  page "nemo_automodel.components.models.gpt_oss.model", GptOssForCausalLM
 *  forward: BSHD or THD inputs.)
 */
typedef struct {
  int32_t layout;                 /* gptoss_layout */
  int32_t batch;                  /* B, or the number of packed sequences */
  int32_t seqlen;                 /* S, or the total token count T */
  int32_t max_seqlen;             /* BSHD: S; THD: >= every sequence length */
  const int32_t* cu_seqlens;      /* THD only (device); NULL for BSHD */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
} gptoss_seq_desc;

int gptoss_abi_version(void);
const char* gptoss_status_string(int status);
const char* gptoss_last_error(void);

/*
 * YaRN frequencies and concentration on the host (rope_utils page,
 * RotaryEmbedding._compute_concentration_and_inv_freq, which follows the YaRN
 * paper and works over rotary_dim; layers page, GptOssAttention.yarn_concentration).
 *   omega_out:          host double[rotary_dim / 2], nullable
 *   concentration_out:  host double, nullable
 * omega_i blends theta_i = base^(-2i/rotary_dim) and theta_i / scaling_factor
 * with a ramp linear in i between the dimensions that turn ntk_beta and
 * ntk_alpha times over initial_context_length; the concentration is
 * 0.1 ln(scaling_factor) + 1 (1 and plain RoPE when scaling_factor <= 1).
 */
gptoss_status gptoss_yarn_params(const gptoss_rope_config* cfg, double* omega_out,
                                 double* concentration_out);

/*
 * The bf16 cos/sin table (rope_utils page, RotaryEmbedding._compute_cos_sin;
 * _apply_rotary_emb_qk: cosine table concatenated with sine table, rounded
 * to the q/k dtype, concentration applied).
 *   table: device bf16 [num_positions, rotary_dim]; row p holds
 *          c*cos(p*omega_i) for i < rotary_dim/2, then c*sin(p*omega_i).
 *          Each entry is the fp64 value rounded once to bf16 (nearest-even);
 *          the angle p*omega_i is formed in fp64.
 * Errors: NULL cfg/table, num_positions < 1, bad rotary_dim.
 */
gptoss_status gptoss_rope_table_init(const gptoss_rope_config* cfg, int32_t num_positions,
                                     void* table, void* stream);

/*
 * Rotate q and k together with one shared table, out of place
 * (rope_utils page, _apply_rotary_emb_qk and apply_rotary_emb_qk).
 *   q: bf16, BSHD [B, S, Hq, D] or THD [T, Hq, D]; q_strides[3] = element
 *      strides of (batch, token, head) -- for THD q_strides[0] is ignored.
 *   k: same with Hkv heads.
 *   q_out, k_out: contiguous bf16 outputs of the same logical shapes.
 *   table: from gptoss_rope_table_init, table_rows >= max position + 1.
 * The pair (x[i], x[i + rotary_dim/2]) is multiplied as a complex number by
 * (cos_i + j sin_i) of the token's position row; each output element is the
 * exact result rounded once to bf16; dims >= rotary_dim are copied (partial
 * rotary, rope_utils page, apply_rotary_emb). rotary_dim: 16, 32, 48 or 64,
 * the table's width.
 */
gptoss_status gptoss_rope_qk(const gptoss_seq_desc* desc,
                             const void* q, const int64_t q_strides[3],
                             const void* k, const int64_t k_strides[3],
                             void* q_out, void* k_out,
                             const void* table, int32_t table_rows, int32_t rotary_dim,
                             void* stream);

/*
 * Prefill attention with sink, GQA and a causal / sliding-window mask
 * (layers page, GptOssAttention: sinks, sliding_window,
 *  softmax_scale = head_dim ** -0.5; Transformers v4.55.0 release notes,
 *  "Architecture": alternating full-context and sliding 128-token window
 *  layers, a learned per-head sink that adds a term to the softmax
 *  denominator).
 *   q, k, v: bf16 in the desc's layout (strides as in gptoss_rope_qk).
 *            With a table, q and k are the UN-rotated projections and are
 *            rotated on the fly, bit-identically to gptoss_rope_qk with the
 *            same table (rotary_dim 16, 32, 48 or 64: the table's width); with
 *            table == NULL they are taken as already rotated.
 *   sinks -INFINITY (or a shard, which has no sink term) gives the plain
 *            softmax over the visible keys for any logits: such a row's
 *            reference is its own largest score, so rows whose logits all
 *            lie far below zero do not underflow.
 *   sinks:   device fp32 [num_q_heads]; sink logit of each query head, in the
 *            units of the scaled scores (-INFINITY disables it).
 *   softmax_scale: tau; 0 selects head_dim ** -0.5 (0.125 for head_dim 64),
 *           any other value must be finite and > 0 (else GPTOSS_ERR_SHAPE).
 *   window:  0 = full causal; W > 0: key j is visible to query i iff
 *            0 <= i - j < W (W = 128 counts the query itself).
 *   out:     bf16, same layout as q, o_strides like q_strides.
 *   workspace: device scratch of at least gptoss_attn_prefill_workspace_size()
 *            bytes, 256-byte aligned; its content need not be initialised.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads). A row with no
 * visible key (only possible for empty sequences) writes nothing.
 * The token strides of k and v must be below 2^24 elements (64 rows of a key
 * tile are addressed with 32-bit byte offsets); larger ones return
 * GPTOSS_ERR_UNSUPPORTED.
 */
size_t gptoss_attn_prefill_workspace_size(const gptoss_seq_desc* desc);
gptoss_status gptoss_attn_prefill(const gptoss_seq_desc* desc,
                                  const void* q, const int64_t q_strides[3],
                                  const void* k, const int64_t k_strides[3],
                                  const void* v, const int64_t v_strides[3],
                                  const float* sinks, float softmax_scale, int32_t window,
                                  const void* table, int32_t table_rows, int32_t rotary_dim,
                                  void* out, const int64_t o_strides[3],
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptoss_attn_prefill that also writes each row's log-sum-exp, the quantity
 * the backward pass needs (its softmax normaliser, including the sink term):
 *   lse: device fp32 [tokens, num_q_heads] (tokens = batch * seqlen in (b, s)
 *        order for BSHD, the packed tokens for THD), contiguous, 16-byte
 *        aligned; lse = log(exp(sigma_h) + sum over visible j of exp(s_ij)) in
 *        natural-log units, -INFINITY for a row with no term.
 * Every other argument, the output and the errors are those of
 * gptoss_attn_prefill; lse NULL returns GPTOSS_ERR_NULL. THD tokens after the
 * last sequence are not written.
 */
gptoss_status gptoss_attn_prefill_lse(const gptoss_seq_desc* desc,
                                      const void* q, const int64_t q_strides[3],
                                      const void* k, const int64_t k_strides[3],
                                      const void* v, const int64_t v_strides[3],
                                      const float* sinks, float softmax_scale, int32_t window,
                                      const void* table, int32_t table_rows, int32_t rotary_dim,
                                      void* out, const int64_t o_strides[3], float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of gptoss_attn_prefill: the gradients of its output with
 * respect to q, k, v and the sinks. The pages define the forward (layers page,
 * GptOssAttention; Transformers v4.55.0 release notes, "Architecture") and
 * describe a training framework; the gradients are the derivatives of that
 * forward. With p_ij = exp(s_ij - lse_i), D_i = <dO_i, o_i>:
 *   dv_j = sum_i p_ij dO_i,  dS_ij = p_ij (<dO_i, v_j> - D_i),
 *   dq~_i = tau sum_j dS_ij k~_j,  dk~_j = tau sum_i dS_ij q~_i,
 *   dsigma_h = - sum_i exp(sigma_h - lse_i) D_i,
 * summed over the 8 query heads of a KV head for dk and dv. With a table, q
 * and k are the UN-rotated inputs of the forward (rotated again here exactly
 * as the forward rotates them) and dq = R^T dq~, dk = R^T dk~ (the rotation's
 * transpose with the same table; the bf16 cast of the rotated values passes
 * the gradient through).
 *   q, k, v, sinks, softmax_scale, window, table, table_rows, rotary_dim: as
 *            given to the forward call.
 *   out:     the forward's bf16 output, o_strides like q_strides.
 *   dout:    bf16 gradient of the loss with respect to out, do_strides.
 *   lse:     the forward's log-sum-exp (gptoss_attn_prefill_lse).
 *   dq, dk, dv: device bf16 outputs, contiguous in the layout of q, k, v
 *            ([B, S, H, 64] or [T, H, 64]), each element written once,
 *            rounded once from fp32 accumulation. THD tokens after the last
 *            sequence are not written.
 *   dsinks:  device fp32 [num_q_heads], overwritten (summed over all rows in a
 *            fixed order: repeated calls give identical bits).
 *   workspace: >= gptoss_attn_prefill_backward_workspace_size() bytes, 256-byte
 *            aligned: rotated q and k, per row lse (log2 units) and -D, one
 *            dsigma partial per head and 32-row query block, and the THD work
 *            lists. Its contents are dead after the call.
 * Errors as for gptoss_attn_prefill; every pointer except table is required.
 * GPTOSS_ERR_UNSUPPORTED if the rows of one sequence of q (or, with a table,
 * of the rotated q) or of dout span 2 GiB or more (the kernels address them
 * with 32-bit offsets).
 */
size_t gptoss_attn_prefill_backward_workspace_size(const gptoss_seq_desc* desc);
gptoss_status gptoss_attn_prefill_backward(const gptoss_seq_desc* desc,
                                           const void* q, const int64_t q_strides[3],
                                           const void* k, const int64_t k_strides[3],
                                           const void* v, const int64_t v_strides[3],
                                           const float* sinks, float softmax_scale, int32_t window,
                                           const void* table, int32_t table_rows, int32_t rotary_dim,
                                           const void* out, const int64_t o_strides[3],
                                           const void* dout, const int64_t do_strides[3],
                                           const float* lse, void* dq, void* dk, void* dv, float* dsinks,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptoss_attn_prefill with an explicit choice of where k is rotated when a
 * table is given (results are bit-identical either way):
 *   GPTOSS_KROT_AUTO      the library's choice (currently separate for both
 *                         layer types: measured faster on gfx950)
 *   GPTOSS_KROT_FUSED     k rotated while each tile is staged into LDS
 *   GPTOSS_KROT_SEPARATE  k rotated once into the workspace, then attended
 * Any other value returns GPTOSS_ERR_SHAPE.
 */
typedef enum { GPTOSS_KROT_AUTO = 0, GPTOSS_KROT_FUSED = 1, GPTOSS_KROT_SEPARATE = 2 } gptoss_k_rotation;
gptoss_status gptoss_attn_prefill_ex(const gptoss_seq_desc* desc,
                                     const void* q, const int64_t q_strides[3],
                                     const void* k, const int64_t k_strides[3],
                                     const void* v, const int64_t v_strides[3],
                                     const float* sinks, float softmax_scale, int32_t window,
                                     const void* table, int32_t table_rows, int32_t rotary_dim,
                                     void* out, const int64_t o_strides[3],
                                     void* workspace, size_t workspace_bytes, int32_t k_rotation,
                                     void* stream);

/*
 * Decode attention: one new query token per sequence against a KV cache
 * (the per-step attention of autoregressive generation, Transformers v4.55.0
 *  release notes, generate(); same sink / GQA / window rules as prefill).
 *   q:        bf16 [N, Hq, D], q_strides[2] = element strides of (seq, head);
 *             un-rotated if a table is given (rotated at position L_n - 1).
 *   k_cache, v_cache: bf16 [N, max_cache_len, Hkv, D]; kv_strides[3] = element
 *             strides of (seq, position, head), shared by K and V. K rows are
 *             stored already rotated at their own positions.
 *   cache_seqlens: device int32 [N]; L_n counts the cached rows INCLUDING the
 *             new token's own (already appended), 1 <= L_n <= max_cache_len.
 *             The query sits at position L_n - 1 and sees rows 0 .. L_n - 1,
 *             or the last min(L_n, W) of them on a window layer.
 *   out:      bf16 [N, Hq, D], o_strides[2].
 *   num_splits: key chunks per sequence processed in parallel and merged
 *             (0 = choose automatically: a small planning kernel reads the
 *             cache lengths and sizes the chunks for the device); results
 *             agree up to fp32 reassociation for any value.
 *   workspace: >= gptoss_attn_decode_workspace_size(...) bytes, 256-byte
 *             aligned: partial results and the chunk plan; its content need
 *             not be initialised.
 * kv_strides[1] must be >= 64 and max_cache_len * kv_strides[1] * 2 bytes below
 * 2^31 (one sequence's rows are read through a 32-bit buffer range); other
 * values return GPTOSS_ERR_UNSUPPORTED.
 */
size_t gptoss_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t max_cache_len, int32_t num_splits);
gptoss_status gptoss_attn_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim,
                                 const void* q, const int64_t q_strides[2],
                                 const void* k_cache, const void* v_cache,
                                 const int64_t kv_strides[3],
                                 const int32_t* cache_seqlens, int32_t max_cache_len,
                                 const float* sinks, float softmax_scale, int32_t window,
                                 const void* table, int32_t table_rows, int32_t rotary_dim,
                                 void* out, const int64_t o_strides[2],
                                 void* workspace, size_t workspace_bytes, int32_t num_splits,
                                 void* stream);

/*
 * One step of a context-parallel prefill: a BSHD shard of queries against a
 * shard of keys of the same sequences, without the sink (layers page,
 * GptOssAttention; rope_utils page: rotations at global positions, the
 * context-parallel arguments that split a sequence over ranks). Query s of
 * the shard sits at position q_offset + s, key j at kv_offset + j; the causal
 * / window mask and the rotations use those positions. Each row's result is
 * the attention over the shard's visible keys alone:
 *   lse = log sum_j e^{s_j} (natural log; -inf with no visible key),
 *   out = sum_j e^{s_j - lse} v_j (0 with none),
 * which gptoss_attn_merge combines across shards, adding the sink once.
 *   desc:   BSHD, seqlen = the query shard's length (THD: UNSUPPORTED).
 *   k, v:   [batch, kv_len, Hkv, 64] with k_strides / v_strides.
 *   table:  rotates q at q_offset + s and k at kv_offset + j (NULL: both
 *           pre-rotated); table_rows must cover both.
 *   out:    bf16 like q; lse: fp32 [batch * seqlen, Hq], 16-byte aligned.
 *   workspace: >= gptoss_attn_prefill_shard_workspace_size(desc, kv_len).
 * Errors as for gptoss_attn_prefill.
 */
size_t gptoss_attn_prefill_shard_workspace_size(const gptoss_seq_desc* desc, int32_t kv_len);
gptoss_status gptoss_attn_prefill_shard(const gptoss_seq_desc* desc,
                                        const void* q, const int64_t q_strides[3],
                                        const void* k, const int64_t k_strides[3],
                                        const void* v, const int64_t v_strides[3],
                                        int32_t kv_len, int32_t q_offset, int32_t kv_offset,
                                        float softmax_scale, int32_t window,
                                        const void* table, int32_t table_rows, int32_t rotary_dim,
                                        void* out, const int64_t o_strides[3], float* lse,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Merge partial attention results over disjoint sets of keys (the shards of
 * gptoss_attn_prefill_shard) and add the per-head sink once:
 *   lse = log(e^sigma_h + sum_p e^{lse_p}),  out = sum_p e^{lse_p - lse} o_p.
 *   o_parts:    bf16 [num_parts, tokens, Hq, 64], element strides part_strides
 *               {part, token, head, 1} (multiples of 8; 16-byte aligned).
 *   lse_parts:  fp32 [num_parts, tokens * Hq], contiguous (-inf: no keys).
 *   sinks:      fp32 [Hq]; NULL = no sink.
 *   out:        bf16 [tokens, Hq, 64] with o_strides {token, head} (multiples
 *               of 8; 16-byte aligned).
 *   lse_out:    optional fp32 [tokens * Hq] (NULL: not written).
 * num_parts = 0 gives out = 0 (lse_out = sigma).
 */
gptoss_status gptoss_attn_merge(int32_t num_parts, int32_t tokens, int32_t num_q_heads, int32_t head_dim,
                                const void* o_parts, const int64_t part_strides[4], const float* lse_parts,
                                const float* sinks, void* out, const int64_t o_strides[2], float* lse_out,
                                void* stream);

/* ---- KV caches of the decode loop ----
 * No page specifies a KV cache. The pages' generation loop (model.generate in
 * the Transformers v4.55.0 release notes, "Welcome GPT OSS") has every new
 * token attend to the keys and values of all earlier tokens of its sequence
 * (layers page, GptOssAttention), so a cache is where those are kept between
 * steps. A cache row holds k rotated at its own position (bf16, exactly as
 * gptoss_rope_qk rotates k) and v unchanged. Position p of sequence n lives:
 *   GPTOSS_CACHE_CONTIGUOUS  row p of sequence n:  k[n, p, g, :]
 *   GPTOSS_CACHE_PAGED       row p mod page_size of physical page
 *                            block_table[n][p / page_size]:  k[page, row, g, :]
 *   GPTOSS_CACHE_RING        slot p mod capacity of sequence n:  k[n, slot, g, :]
 *                            It keeps only the last `capacity` positions: what a
 *                            sliding-window layer whose window equals the
 *                            capacity reads (128 slots for GPT-OSS's window
 *                            layers instead of the whole context).
 * k and v caches share one layout. Element strides (head_dim contiguous):
 * CONTIGUOUS and RING {sequence, row, kv head}, PAGED {page, row, kv head}.
 */
typedef enum { GPTOSS_CACHE_CONTIGUOUS = 0, GPTOSS_CACHE_PAGED = 1, GPTOSS_CACHE_RING = 2 } gptoss_cache_kind;
typedef struct {
  int32_t kind;                 /* gptoss_cache_kind */
  int32_t capacity;             /* CONTIGUOUS: rows per sequence; RING: slots per sequence;
                                   PAGED: rows per page, a power of two >= 32 */
  int64_t strides[3];           /* element strides of k and v as above: multiples of 8, row stride >= 64 */
  const int32_t* block_table;   /* PAGED: device int32 [num_seqs, max_pages], physical page of each
                                   logical page; entries are clamped to [0, num_pages). Else NULL. */
  int32_t max_pages;            /* PAGED: block_table entries per sequence */
  int32_t num_pages;            /* PAGED: pages in the pool */
} gptoss_kv_layout;

/*
 * Store the num_new newest tokens of every sequence in a cache. cache_seqlens
 * (device int32 [num_seqs]) counts each sequence's tokens including the new
 * ones, so token t (0-based) of sequence n has position
 * p = cache_seqlens[n] - num_new + t. k is rotated at p with the table (as
 * gptoss_rope_qk rotates k: bit-identical; table NULL stores k as given) and
 * written with v at p's row. Tokens that have no row are skipped: p < 0, p at
 * or past a contiguous cache's capacity or a paged cache's
 * max_pages * page_size, and in a ring every token of the call older than the
 * last `capacity` ones (a later token of the same call takes its slot).
 *   k_new, v_new: device bf16 [num_seqs, num_new, num_kv_heads, head_dim] with
 *            element strides {sequence, token, head} in kn_strides / vn_strides.
 *   max_seqlen: host upper bound of cache_seqlens (checked against table_rows).
 * Calls that write the same row concurrently (the same position twice, or two
 * positions of a ring slot in different calls on different streams) race.
 * Errors: GPTOSS_ERR_NULL for missing pointers, GPTOSS_ERR_SHAPE for negative
 * sizes or a bad kind, GPTOSS_ERR_UNSUPPORTED for head_dim != 64, an unaligned
 * pointer or stride, a table that does not cover max_seqlen, or a paged page
 * size that is not a power of two >= 32.
 */
gptoss_status gptoss_kv_append(const gptoss_kv_layout* layout, void* k_cache, void* v_cache,
                               int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t num_new,
                               const void* k_new, const int64_t kn_strides[3],
                               const void* v_new, const int64_t vn_strides[3],
                               const int32_t* cache_seqlens, int32_t max_seqlen,
                               const void* table, int32_t table_rows, int32_t rotary_dim, void* stream);

/*
 * gptoss_attn_decode over a cache of any layout: the token at position
 * cache_seqlens[n] - 1 of every sequence attends to the positions the mask
 * allows (all earlier positions, or the last min(L, window)), each read from
 * wherever the layout keeps it. Arguments as for gptoss_attn_decode, plus:
 *   layout:     the cache layout (above); k_cache / v_cache point at row 0 of
 *               sequence 0 (CONTIGUOUS, RING) or at page 0 (PAGED).
 *   max_seqlen: host upper bound of cache_seqlens; it must not exceed a
 *               contiguous cache's capacity or a paged cache's
 *               max_pages * page_size. Device lengths above it are clamped.
 * A RING cache requires window == capacity (it holds exactly the visible
 * positions). A PAGED decode of a window layer reads from the 32-key boundary
 * at or before the window's first key; the rows in between are loaded as
 * zeros, so they need no valid contents.
 * The workspace size depends on the layout and the window.
 */
size_t gptoss_attn_decode_kv_workspace_size(const gptoss_kv_layout* layout, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t max_seqlen, int32_t window,
                                            int32_t num_splits);
gptoss_status gptoss_attn_decode_kv(const gptoss_kv_layout* layout, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    const void* q, const int64_t q_strides[2],
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* cache_seqlens, int32_t max_seqlen,
                                    const float* sinks, float softmax_scale, int32_t window,
                                    const void* table, int32_t table_rows, int32_t rotary_dim,
                                    void* out, const int64_t o_strides[2],
                                    void* workspace, size_t workspace_bytes, int32_t num_splits,
                                    void* stream);

/*
 * gptoss_attn_decode_kv without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The split partials and the split plan live
 * in a fixed scratch array the library holds on each GPU it runs on
 * (GPTOSS_DECODE_SCRATCH_BYTES, until the process ends); this call allocates
 * nothing and frees nothing. Its address is looked up on the first call on
 * each device (make one call before capturing a graph on a new device).
 * Arguments and results as for gptoss_attn_decode_kv, minus the workspace.
 * With num_splits = 0 the shortest planned split is lengthened (in steps of
 * 128 keys) when the partials of the default plan would not fit; the result
 * stays within the same tolerance, and is bit-identical to
 * gptoss_attn_decode_kv whenever the default plan fits. Calls whose partials
 * cannot fit (num_seqs * num_q_heads * splits * 264 bytes plus the plan)
 * return GPTOSS_ERR_WORKSPACE before any launch.
 * All calls of one process on one GPU share that GPU's scratch and it keeps
 * the last call's contents: calls that can run at the same time on one GPU
 * (on different streams, or from different host threads without ordering)
 * race and give undefined results; calls ordered on one stream do not.
 * Nothing in it needs to start at zero (each call writes what it reads).
 */
#define GPTOSS_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
gptoss_status gptoss_attn_decode_kv_noalloc(const gptoss_kv_layout* layout, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                            const void* q, const int64_t q_strides[2],
                                            const void* k_cache, const void* v_cache,
                                            const int32_t* cache_seqlens, int32_t max_seqlen,
                                            const float* sinks, float softmax_scale, int32_t window,
                                            const void* table, int32_t table_rows, int32_t rotary_dim,
                                            void* out, const int64_t o_strides[2], int32_t num_splits,
                                            void* stream);

/*
 * The q, k and v projections ahead of the attention with the RoPE applied to q
 * and k in the same kernel (the gpt-oss-20b module print-out: q_proj
 * 2880 -> Hq*64, k_proj and v_proj 2880 -> Hkv*64, Linear with bias; rope_utils
 * page, _apply_rotary_emb_qk). Each output is z = x W^T + b accumulated in
 * fp32 and rounded once to bf16, the projection's dtype; with a table, q and k
 * are then rotated at each token's position exactly as gptoss_rope_qk rotates
 * them, so the result equals gptoss_rope_qk applied to the table = NULL output,
 * bit for bit.
 *   desc:  token layout and positions (BSHD p = s, THD p = t - cu[n]); its
 *          num_q_heads / num_kv_heads / head_dim give the output widths.
 *   x:     device bf16 [tokens, hidden], rows x_row_stride elements apart.
 *   wq [Hq*64, hidden], wk and wv [Hkv*64, hidden]: device bf16, Linear's
 *          weight layout, rows contiguous.
 *   bq, bk, bv: device bf16 biases of the same widths; NULL = no bias.
 *   q_out [tokens, Hq, 64], k_out and v_out [tokens, Hkv, 64]: contiguous bf16.
 *   table: NULL = no rotation; else rotary_dim 64 or 32 (the dims past it
 *          pass through), table_rows >= the longest sequence.
 * hidden must be a multiple of 64 and num_kv_heads a multiple of 4 (the q, k
 * and v widths are multiples of the kernel's 256-feature tiles); other values
 * return GPTOSS_ERR_UNSUPPORTED, as do unaligned pointers or strides.
 */
gptoss_status gptoss_qkv_proj_rope(const gptoss_seq_desc* desc, const void* x, int64_t x_row_stride,
                                   int32_t hidden, const void* wq, const void* bq, const void* wk,
                                   const void* bk, const void* wv, const void* bv, const void* table,
                                   int32_t table_rows, int32_t rotary_dim, void* q_out, void* k_out,
                                   void* v_out, void* stream);

/*
 * Check of the device-resident lengths that the attention calls trust (they
 * clamp every index derived from them, so bad values give wrong results, never
 * out-of-bounds accesses). For callers and debug runs that want to know: one
 * small kernel on `stream`, no synchronisation; read `result` once the stream
 * has reached it.
 *   cu_seqlens: device int32 [batch + 1] (THD layout) or NULL to skip. Rules:
 *               cu_seqlens[0] == 0, non-decreasing, and cu_seqlens[batch] ==
 *               total_tokens when total_tokens >= 0.
 *   cache_seqlens: device int32 [num_seqs] or NULL to skip. Rule: every length
 *               in 1 .. max_cache_len (a decode query sits at position L - 1).
 *   result:     device int32 [3], written by the kernel: result[0] = OR of the
 *               gptoss_length_fault bits of the broken rules (0: all hold),
 *               result[1] = the first cu_seqlens index that breaks one (-1 if
 *               none), result[2] = the first such cache_seqlens index (-1).
 * Returns GPTOSS_ERR_NULL without result, GPTOSS_ERR_SHAPE for batch < 0 with
 * cu_seqlens or num_seqs < 0 / max_cache_len < 1 with cache_seqlens.
 */
typedef enum {
  GPTOSS_LEN_CU_START = 1,  /* cu_seqlens[0] != 0 */
  GPTOSS_LEN_CU_ORDER = 2,  /* cu_seqlens[i] < cu_seqlens[i - 1] for some i */
  GPTOSS_LEN_CU_TOTAL = 4,  /* cu_seqlens[batch] != total_tokens */
  GPTOSS_LEN_CACHE = 8      /* a cache length outside 1 .. max_cache_len */
} gptoss_length_fault;
gptoss_status gptoss_check_lengths(const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                                   const int32_t* cache_seqlens, int32_t num_seqs, int32_t max_cache_len,
                                   int32_t* result, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTOSS_ATTN_H */
