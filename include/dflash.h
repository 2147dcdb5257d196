/*
 * dflash.h - C ABI of the DFlash draft-step library for AMD Instinct MI355X (gfx950).
 *
 * One speculative step of DFlash (block-diffusion drafting with target-feature KV
 * injection) as three calls, plus set-up helpers:
 *
 *   dflash_fuse_inject_kv   fuse multi-layer target hidden states with one linear
 *                           projection and write them as K/V into every draft layer's
 *                           paged KV cache ("DFlash" wiki page, section "Conditioning on
 *                           target-model features", items 1 and 2; NVIDIA technical blog
 *                           on DFlash, section "How does DFlash speculative decoding
 *                           work?": context features go into the key-value projections of
 *                           the draft layers).
 *   dflash_draft_block      one non-causal forward pass over the block [anchor, mask x
 *                           (B - 1)], B = 16 (or 8 or 32), that drafts B - 1 tokens with the
 *                           shared LM head and argmax (wiki, "Parallel drafting with block
 *                           diffusion": one pass drafts a whole block, at a cost roughly
 *                           independent of its size; blog, same section: one forward pass
 *                           predicts a block of masked future tokens).
 *   dflash_verify_accept    greedy verification: the longest prefix of drafts that matches
 *                           the target's argmax, plus one target token (blog, same section:
 *                           the target accepts the longest valid prefix).
 *   dflash_advance          closed-loop bookkeeping between iterations: the accepted
 *                           tokens extend the context and the loop drafts again from the
 *                           target's next token (blog, same section: drafting and
 *                           verification alternate, one verification pass yielding several
 *                           tokens; wiki, "Background": the draft model proposes, the target
 *                           verifies in parallel).
 *   dflash_verify_accept_sampled
 *                           temperature-1 verification (speculative accept/reject with
 *                           residual resampling, which keeps the target's output
 *                           distribution; blog, same section; wiki, "Performance
 *                           comparison", sampling at temperature 1).
 *   dflash_prefill_input_fusion
 *                           the input-fusion variant's context prefill: the fused features
 *                           enter the drafter as its input rows and run causally through
 *                           the layers, which cache their K/V (z-lab/dflash overview page,
 *                           FAQ on KV injection versus input fusion; the variant KV
 *                           injection is compared with, whose prefill processes every
 *                           context token fully).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers unless stated otherwise; the caller owns
 *     every buffer (weights, packed weights, KV pools, tables, inputs, outputs, workspace).
 *   - Calls are asynchronous on `stream` and never synchronize the device.  The library
 *     allocates no device memory and keeps no global state.
 *   - Arguments are validated on the host before anything is launched; on a negative
 *     status nothing was enqueued.  Device-side data (token ids in [0, vocab), page ids in
 *     [0, num_pages), positions below max_pages_per_seq * page_size) is a precondition
 *     that is not checked.
 *   - Two calls that share a workspace must be ordered on one stream.
 *   - Matrices are row-major.  Linear weights use the logical [out, in] layout.
 *
 * Numerics: bf16 models keep weights, target features and the KV cache in bf16; every
 * activation (fused feature, residual stream, normed inputs, q/k/v, attention output,
 * SwiGLU product) is fp32 in memory and enters the bf16 MFMA as a hi + lo pair of bf16
 * values (the fused feature as three pieces), accumulating in fp32.  RoPE angles are
 * computed in fp64.  f32 models use fp32 everywhere.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, inconsistent shape   */
  DFLASH_ERR_UNSUPPORTED = -2,  /* a shape or dtype the kernels do not implement         */
  DFLASH_ERR_WORKSPACE = -3,    /* workspace or packed buffer smaller than required      */
  DFLASH_ERR_HIP = -4           /* a HIP launch reported an error                        */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Drafter shape.  Requirements checked by every call: block_size in {8, 16, 32},
 * page_size == 16, hidden % 64 == 0, feat_dim % 64 == 0, intermediate % 64 == 0,
 * vocab % 64 == 0, head_dim in {64, 128}, n_q_heads % n_kv_heads == 0, and a query-head
 * group G = n_q_heads / n_kv_heads in {1, 2, 4, 8} for bf16 (in {2, 4, 8}, and not 8 with
 * head_dim 128, for fp32). */
typedef struct {
  int32_t n_layers;
  int32_t hidden;         /* H */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;       /* d */
  int32_t intermediate;   /* I, SwiGLU width */
  int32_t vocab;          /* V */
  int32_t feat_dim;       /* F = (number of fused target layers) * (target hidden size) */
  int32_t block_size;     /* B = 16 (8, 32): slot 0 = last accepted token, slots 1..B-1 =
                             mask */
  int32_t page_size;      /* 16 tokens per KV page */
  int32_t mask_token_id;
  float rope_theta;
  float rms_eps;
  int32_t dtype;          /* dflash_dtype of weights, features and KV cache */
} dflash_config;

/* Logical weights for dflash_pack_weights.  Every pointer is a device pointer to a
 * row-major tensor of the model dtype.  Per-layer members point to HOST arrays of
 * n_layers device pointers.
 *   w_fuse [H, F]   lm_head [V, H]   final_norm [H]
 *   attn_norm[l] [H]   wq[l] [n_q*d, H]   wk[l], wv[l] [n_kv*d, H]   wo[l] [H, n_q*d]
 *   mlp_norm[l] [H]    w_gate[l], w_up[l] [I, H]   w_down[l] [H, I]                    */
typedef struct {
  const void* w_fuse;
  const void* lm_head;
  const void* final_norm;
  const void* const* attn_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* mlp_norm;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
} dflash_weights;

/* Paged KV cache of the draft layers (injected context only; block K/V are never
 * stored).  In the model dtype, one physical page id addressing the same page in every
 * layer:
 *   k_pool [n_layers][num_pages][n_kv_heads][page_size][head_dim]  (a page is row-major)
 *   v_pool [n_layers][num_pages][n_kv_heads][head_dim][page_size]  (a page is transposed,
 *          so the attention kernel reads 4 consecutive positions of one dim at once).
 * block_table [batch][max_pages_per_seq] maps logical page p of request b to a physical
 * page; ctx_lens [batch] is T_b, the number of context positions already injected. */
typedef struct {
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int32_t num_pages;
  int32_t max_pages_per_seq;
} dflash_kv_cache;

/* Size in bytes of the packed weight buffer for `cfg` (0 if cfg is invalid). */
size_t dflash_packed_weights_size(const dflash_config* cfg);

/* Repack the logical weights into the MFMA tile layout the kernels stream (norm gains
 * widened to fp32; Q|K|V concatenated; gate and up interleaved by 16-row tile).
 * `packed` (device, >= dflash_packed_weights_size bytes) is owned by the caller and is
 * the `packed` argument of the step calls.  Run once at load time. */
dflash_status dflash_pack_weights(const dflash_config* cfg, const dflash_weights* w,
                                  void* packed, size_t packed_bytes, hipStream_t stream);

/* Bytes of workspace the step calls need for up to `max_batch` requests and up to
 * `max_inject_rows` rows per dflash_fuse_inject_kv launch chunk (dflash_fuse_inject_kv
 * processes n_tok rows in chunks of the largest size, at most 1024 rows, whose buffers fit
 * the workspace it is given).  `max_ctx` bounds the cached context (max_pages_per_seq * 16
 * of the cache).  Returns 0 if an argument is invalid. */
size_t dflash_workspace_size(const dflash_config* cfg, int32_t max_batch,
                             int32_t max_inject_rows, int32_t max_ctx);

/* Prepare a new workspace (zeroes its 256-byte reserved head).  Must be called once after
 * the workspace is allocated; no step call needs the workspace's contents to survive
 * between calls. */
dflash_status dflash_workspace_init(void* workspace, size_t ws_bytes, hipStream_t stream);

/* Feature fusion + KV injection.
 *   feats   [n_tok, F] model dtype: concatenated target hidden states, one row per
 *           context position to inject (layer-major concatenation).
 *   seq_idx [n_tok] int32: request of each row (index into block_table).
 *   pos     [n_tok] int32: context position of each row; the row lands in page
 *           block_table[seq][pos / 16], slot pos % 16, of every layer, K rotated at pos.
 * ctx_lens is not read or changed: the caller advances it.  Rows whose positions repeat
 * are written in an unspecified order. */
dflash_status dflash_fuse_inject_kv(const dflash_config* cfg, const void* packed,
                                    const dflash_kv_cache* cache, const void* feats,
                                    const int32_t* seq_idx, const int32_t* pos, int32_t n_tok,
                                    void* workspace, size_t ws_bytes, hipStream_t stream);

/* Draft one block per request; B = cfg->block_size.
 *   embed      [V, H] model dtype: the target's embedding table (shared, not packed).
 *   anchor_ids [batch] int32: last accepted token of each request (block slot 0).
 *   draft_ids  [batch, B-1] int32 out: argmax over the vocabulary of slots 1..B-1, exact
 *              fp32 ties resolved to the lowest id.
 *   top2_gap   [batch, B-1] fp32 out, may be NULL: the largest logit of each slot minus the
 *              second largest (0 for an exact tie).  A small gap marks a near-tie, whose id
 *              can change under rounding of the logits (wiki, "Conditioning on target-model
 *              features", closing paragraph: the draft tokens come from the target's shared
 *              LM head).
 *   logits_out [batch, B-1, V] fp32 out, may be NULL: the LM-head logits of slots 1..B-1.
 * Slot j of request b sits at position ctx_lens[b] + j and attends, without a mask, to
 * the ctx_lens[b] cached context entries and the B block slots.
 * DFLASH_ERR_UNSUPPORTED if batch * max(B, 16) > 65536 or the cache's max_pages_per_seq >
 * 16384 (262144 positions per request). */
dflash_status dflash_draft_block(const dflash_config* cfg, const void* packed,
                                 const void* embed, const dflash_kv_cache* cache,
                                 const int32_t* anchor_ids, int32_t batch, int32_t* draft_ids,
                                 float* top2_gap, float* logits_out, void* workspace,
                                 size_t ws_bytes, hipStream_t stream);

/* dflash_draft_block for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the workspace replaced by a scratch array compiled into the library
 * (DFLASH_NOALLOC_SCRATCH_BYTES = 64 MiB on each device the library runs on, held until the
 * process ends; dflash_noalloc_scratch_bytes() returns the size).  The call allocates
 * nothing; the array's device address is looked up once per device, on the first call
 * with that device current.  Every call on one device shares that device's array, and no
 * call needs its previous contents: calls that overlap on one device (different streams,
 * no ordering between them) race and must not be made.  DFLASH_ERR_WORKSPACE when the draft
 * needs more scratch than the array holds (dflash_workspace_size(cfg, batch, 0,
 * max_pages_per_seq * 16) > DFLASH_NOALLOC_SCRATCH_BYTES: e.g. the Qwen3-8B shape at batch
 * 16 with a 2048-position cache fits, batch 32 does not); otherwise errors as
 * dflash_draft_block. */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
size_t dflash_noalloc_scratch_bytes(void);
dflash_status dflash_draft_block_noalloc(const dflash_config* cfg, const void* packed,
                                         const void* embed, const dflash_kv_cache* cache,
                                         const int32_t* anchor_ids, int32_t batch,
                                         int32_t* draft_ids, float* top2_gap,
                                         float* logits_out, hipStream_t stream);

/* The last stage of dflash_draft_block on its own: final RMSNorm, the shared LM head and
 * the argmax over the vocabulary.
 *   hidden     [rows, H] fp32: residual-stream rows (before the final norm).
 *   ids_out    [rows] int32 out: argmax of RMSNorm(hidden) . W_lm^T, ties -> lowest id.
 *   logits_out [rows, V] fp32 out, may be NULL.
 * `workspace`: a step workspace initialized with dflash_workspace_init and sized by
 * dflash_workspace_size for max_batch >= ceil(rows / 16); the rows are copied into the
 * fragment layout there, then the draft step's LM-head kernels run on them.
 * DFLASH_ERR_WORKSPACE if it is smaller; DFLASH_ERR_UNSUPPORTED if rows > 65536. */
dflash_status dflash_lm_head_argmax(const dflash_config* cfg, const void* packed,
                                    const float* hidden, int32_t rows, int32_t* ids_out,
                                    float* logits_out, void* workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* Greedy verification of blocks of B = block_size tokens (8, 16 or 32).
 *   draft_ids  [batch, B-1] int32: d_1..d_{B-1}.
 *   target_ids [batch, B] int32: t_0..t_{B-1}, the target's argmax after block slot j.
 *   accept_len [batch] int32 out: m + 1, m = number of leading i with d_i == t_{i-1}.
 *   bonus      [batch] int32 out: t_m.
 *   emitted    [batch, B] int32 out, may be NULL: d_1..d_m, t_m, then -1 padding.
 * DFLASH_ERR_INVALID_ARG for a null input or output, batch < 0 or another block size. */
dflash_status dflash_verify_accept(const int32_t* draft_ids, const int32_t* target_ids,
                                   int32_t batch, int32_t block_size, int32_t* accept_len,
                                   int32_t* bonus, int32_t* emitted, hipStream_t stream);

/* Closed-loop bookkeeping after dflash_verify_accept, so that a whole decoding iteration
 * (draft -> verify -> advance -> inject) runs on the stream without the host reading any
 * result.  For each request b, with T_b the context length before the call and B =
 * block_size (8, 16 or 32):
 *   inject_seq [batch * B] int32 out: b for rows b*B .. b*B+B-1;
 *   inject_pos [batch * B] int32 out: T_b + j for row b*B + j -- the positions of the
 *              block's B slots (slot 0 = the anchor at T_b), whose target hidden features
 *              the next dflash_fuse_inject_kv call writes into the cache;
 *   ctx_lens   [batch] int32 in/out: T_b -> T_b + accept_len[b] (the anchor and the
 *              accepted drafts join the context);
 *   anchor_ids [batch] int32 out: bonus[b], slot 0 of the next block.
 * accept_len, bonus [batch] int32: the outputs of dflash_verify_accept.  max_ctx: positions
 * the cache holds per request (max_pages_per_seq * 16).  Rows j >= accept_len[b] write
 * positions past the new context length: no draft reads them, and the next iteration's
 * injection (which starts at the new T_b) overwrites them first.  Precondition:
 * T_b + B <= max_ctx; positions are clamped to max_ctx - 1 so that no access leaves the
 * request's page-table row.  DFLASH_ERR_INVALID_ARG for null pointers, batch < 0, another
 * block size or max_ctx < B; batch 0 launches nothing. */
dflash_status dflash_advance(const int32_t* accept_len, const int32_t* bonus, int32_t batch,
                             int32_t block_size, int32_t max_ctx, int32_t* ctx_lens,
                             int32_t* anchor_ids, int32_t* inject_seq, int32_t* inject_pos,
                             hipStream_t stream);

/* Workspace bytes for dflash_verify_accept_sampled (0 if batch <= 0 or vocab is outside
 * 1 .. 1048576): the rows' softmax statistics and the final draw's 256-element chunk
 * sums, batch * (62 + ceil(vocab / 256)) doubles, then each drawn draft token's two
 * logits, batch * 30 floats. */
size_t dflash_verify_sampled_workspace_size(int32_t batch, int32_t vocab);

/* Temperature-1 verification (blocks of 16 tokens).
 *   draft_logits  [batch, 15, vocab] fp32, target_logits [batch, 16, vocab] fp32.
 *   u_draft, u_accept [batch, 15], u_resample [batch]: uniforms in [0, 1).
 * q_i = softmax(draft_logits[i-1]), p_i = softmax(target_logits[i-1]).
 * d_i = smallest j with cumsum(q_i)[j] > u_draft * sum(q_i); accept d_i while
 * u_accept * q_i(d_i) < p_i(d_i); at the first rejection emit the inverse-CDF sample of
 * max(0, p_i - q_i) (of p_i if that is all zero) at u_resample and stop; if all 15 are
 * accepted emit the sample of p_16 at u_resample.
 *   draft_ids [batch, 15], accept_len [batch] (number of emitted tokens, 1..16),
 *   emitted [batch, 16] (-1 padded) int32 out.
 * Weights and sums are evaluated in fp64 (exp to below 4e-10 relative), so a decision
 * differs from an exact evaluation only when u * total lies within ~1e-9 of the mass of a
 * cumulative boundary.  DFLASH_ERR_UNSUPPORTED if vocab > 1048576. */
dflash_status dflash_verify_accept_sampled(const float* draft_logits,
                                           const float* target_logits, const float* u_draft,
                                           const float* u_accept, const float* u_resample,
                                           int32_t batch, int32_t vocab, int32_t* draft_ids,
                                           int32_t* accept_len, int32_t* emitted,
                                           void* workspace, size_t ws_bytes,
                                           hipStream_t stream);

/* Bytes of workspace dflash_prefill_input_fusion needs for up to `max_tok` context rows
 * per call and a cache of `max_ctx` positions per request (max_pages_per_seq * 16).
 * Returns 0 if an argument is invalid. */
size_t dflash_prefill_workspace_size(const dflash_config* cfg, int32_t max_tok,
                                     int32_t max_ctx);

/* Context prefill of the input-fusion variant (z-lab/dflash overview page, FAQ on KV
 * injection versus input fusion), the alternative to dflash_fuse_inject_kv: instead of
 * projecting the fused feature straight into K/V, the drafter takes the fused feature
 * c_t = W_fuse . X_t as its input hidden state at context position t and runs the context
 * rows through its layers, attention being causal over the context (row t attends to
 * positions 0..t); each layer writes the K/V of the rows into its paged cache, and the
 * rows attend to those stored values (bf16 for a bf16 drafter).  The last layer's attention
 * and MLP of the context rows are not run: the draft step reads only the cached K/V, and
 * dflash_draft_block drafts over this cache unchanged.
 *   feats [n_tok, F] model dtype: concatenated target hidden states of request `seq`'s
 *         next n_tok context positions, ctx_lens[seq] .. ctx_lens[seq] + n_tok - 1 (the
 *         cache already holds positions 0 .. ctx_lens[seq] - 1 of this variant).
 *   seq   request index (row of block_table).
 * ctx_lens is read, not changed: the caller advances it.  Rows are processed in chunks of
 * 2048 positions, in order.  Precondition: ctx_lens[seq] + n_tok <= max_pages_per_seq * 16.
 * DFLASH_ERR_WORKSPACE if ws_bytes < dflash_prefill_workspace_size(cfg, n_tok, max_ctx);
 * n_tok 0 launches nothing. */
dflash_status dflash_prefill_input_fusion(const dflash_config* cfg, const void* packed,
                                          const dflash_kv_cache* cache, const void* feats,
                                          int32_t seq, int32_t n_tok, void* workspace,
                                          size_t ws_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* dflash_error_string(dflash_status status);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
