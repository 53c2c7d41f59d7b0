/*
 * wf.h — C ABI of the block-verification engine for Whisper-shaped decoders
 * on AMD Instinct MI355X (gfx950).
 *
 * The calls follow the problem as the pages state it:
 *
 *  - wf_encode_kv: the cross-attention keys and values of every decoder
 *    layer are computed from the audio memory once per request and are only
 *    read afterwards (SGLang-Omni "Whisper ASR" cookbook, section "Breakable
 *    Prefill CUDA Graph").
 *  - wf_verify_block: the anchor and its K candidates go through the target
 *    decoder in a single causally masked forward, which gives the target's
 *    next-token choice for every row of the block ("Whisper-Flash:
 *    Acoustically Conditioned Parallel Drafting for Faster Whisper
 *    Decoding", section 3.1, eq. 1). A prefill is the same call with the
 *    prompt as the block.
 *  - wf_accept: the longest prefix of candidates that matches the target's
 *    choices is accepted; the target's choice at the row after that prefix
 *    (a correction, or a bonus when every candidate matched) is emitted too
 *    (section 3.1); at temperature T > 0 candidate i is accepted with
 *    probability min(1, p/q) and a rejection draws from (p - q)+ (section
 *    3.1, appendix A.4).
 *  - wf_rollback: of the block's rows written to the cache, those of the
 *    anchor and of the a accepted candidates stay (L + 1 + a positions in
 *    all); the rest are dropped (appendix A.1).
 *
 * Conventions
 *  - Every pointer named d_* is device memory (HIP); h_* is host memory.
 *  - The caller owns all memory: weights, KV pools, page table, workspace and
 *    per-call inputs/outputs. The engine stores raw pointers and never
 *    allocates or frees device memory; keep the buffers alive until
 *    wf_destroy.
 *  - All calls except wf_create, wf_destroy and wf_device_state are
 *    asynchronous on the given stream (a hipStream_t passed as void*; NULL is
 *    the null stream) and make no host<->device copies, so a sequence of
 *    them can be captured in a HIP graph.
 *  - Host-checkable errors (null pointers, shapes, capacities) return a
 *    negative wf_status before anything is launched; wf_last_error() then
 *    returns a thread-local message. Data-dependent errors are set in a
 *    per-slot device error word (WF_DERR_* bits) and that request's work is
 *    skipped; wf_device_state copies the words to the host.
 *  - One engine is used from one host thread at a time. Nothing throws
 *    across the ABI.
 *
 * Numerics
 *  - Weights are bf16. The decoder GEMMs take fp16 activations (layer-norm,
 *    attention and GELU outputs rounded to fp16, about 2^-11 relative)
 *    against the bf16 weights converted to fp16 in registers, on fp16 MFMA
 *    with fp32 accumulation; wf_encode_kv multiplies the bf16 audio memory
 *    on bf16 MFMA.
 *  - The residual stream, layer-norm statistics, softmax and GELU are fp32.
 *  - Self-attention K/V pages and cross-attention K/V are stored in fp16;
 *    attention products run on fp16 MFMA with fp32 accumulation.
 *  - Every reduction has a fixed order that does not depend on the number
 *    of rows in the block or on the block length: a row's logits are the
 *    same bits whether it is verified alone or inside a block. No float
 *    atomics are used; repeated calls give identical bits.
 */
#ifndef WF_H
#define WF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct wf_engine wf_engine;

typedef enum {
    WF_OK = 0,
    WF_EINVAL = -1,     /* null pointer or bad scalar argument */
    WF_ESHAPE = -2,     /* unsupported model shape */
    WF_ECAPACITY = -3,  /* a buffer is too small or a count exceeds a maximum */
    WF_EHIP = -4,       /* a HIP runtime call failed */
    WF_EDEVICE = -5,    /* no usable gfx950 device */
    WF_ESTATE = -6      /* call out of order */
} wf_status;

/* Bits of the per-slot device error word. A slot with a nonzero word is
 * skipped by every later call until wf_reset clears it. */
#define WF_DERR_CONTEXT 1   /* L + n_tok > n_ctx */
#define WF_DERR_TOKEN   2   /* token id outside [0, vocab) or n_tok > T */
#define WF_DERR_STATE   4   /* verify on a slot whose last verify was not rolled back */
#define WF_DERR_ACCEPT  8   /* rollback with a > n_tok - 1, or k > budget - 1 */
#define WF_DERR_NAN     16  /* a NaN logit */
#define WF_DERR_PAGE    32  /* page-table entry outside [0, n_pages) */
#define WF_DERR_SAMPLE  64  /* sampling inputs missing or q(y) = 0 for a draft */
#define WF_DERR_TIMEOUT 128 /* the persistent pass hit its internal wait limit
                               (WF_OPT_PASS_TIMEOUT_US); that pass's outputs are
                               not valid */

/* Model and capacity description. The supported shapes have head_dim 16 or
 * 64, d_model = n_heads * head_dim with d_model a multiple of 64, d_ffn a
 * multiple of 64, n_ctx a multiple of 32 no larger than 1024 and page_size 16. */
typedef struct {
    int32_t n_layers;     /* decoder layers (32 for large-v3, 4 for turbo) */
    int32_t d_model;      /* width (1280) */
    int32_t n_heads;      /* attention heads (20) */
    int32_t head_dim;     /* 64 (16 for the tiny test model) */
    int32_t d_ffn;        /* MLP width (5120) */
    int32_t vocab;        /* vocabulary (51866); the LM head is tied to tok_emb */
    int32_t n_frames;     /* audio frames per request (1500 for a 30 s window) */
    int32_t n_ctx;        /* decoder context (448) */
    int32_t max_batch;    /* number of request slots; slot ids are [0, max_batch) */
    int32_t max_rows;     /* largest n * T of one wf_verify_block call */
    int32_t page_size;    /* tokens per KV page; must be 16 */
    int32_t n_pages;      /* physical pages in the KV pool */
    int32_t eos_id;       /* end-of-transcript token id */
    float ln_eps;         /* layer-norm epsilon (1e-5) */
    /* Parallel drafter (Whisper-Flash section 3.2, appendix A.2); 0 layers
     * disables it. Its history rows take the target's fp32 residual stream
     * as it leaves each block listed in tap_layers[0..n_taps) (zero-based,
     * before the final LN). */
    int32_t drafter_layers;   /* 0 or the number of drafter blocks (2) */
    int32_t n_taps;           /* 5 */
    int32_t tap_layers[8];    /* 1, 8, 15, 22, 29 for large-v3 */
} wf_config;

/* Per-layer weights: bf16, PyTorch Linear convention (weight [out, in],
 * row-major). Layer-norm gains/biases and all biases are bf16 vectors.
 * Self-attention has no key bias, cross-attention no key bias. */
typedef struct {
    const void *ln1_g, *ln1_b;                   /* [d] */
    const void *wq, *bq, *wk, *wv, *bv, *wo, *bo; /* [d,d] / [d] */
    const void *ln2_g, *ln2_b;
    const void *wqc, *bqc, *wkc, *wvc, *bvc, *woc, *boc;
    const void *ln3_g, *ln3_b;
    const void *w1, *b1;                          /* [d_ffn, d], [d_ffn] */
    const void *w2, *b2;                          /* [d, d_ffn], [d] */
} wf_layer_weights;

/* Drafter weights (bf16). Each drafter block has the target block's
 * tensors, including its own cross-attention K/V projections. */
typedef struct {
    const wf_layer_weights *layers; /* host array of drafter_layers entries (copied) */
    const void *w_hist;             /* [d, n_taps * d], history projection, no bias */
    const void *mask_emb;           /* [d], the learned mask vector */
    const void *lnd_g, *lnd_b;      /* the drafter's final layer norm */
} wf_drafter_weights;

typedef struct {
    const void *tok_emb;   /* [vocab, d]; also the LM head */
    const void *pos_emb;   /* [n_ctx, d] learned positions */
    const void *lnf_g, *lnf_b;
    const wf_layer_weights *layers; /* host array of n_layers entries (copied) */
    const wf_drafter_weights *drafter; /* NULL unless drafter_layers > 0 */
} wf_weights;

/* Sizes of the caller-allocated device buffers for a configuration.
 * kv_pool:  fp16 [n_layers + drafter_layers][n_pages][2][n_heads][page_size][head_dim]
 *           (the V half of a page is stored transposed, [head_dim][page_size]);
 *           the drafter's layers hold its history keys (rotated) and values.
 * xkv_pool: fp16 per slot, per layer (target layers, then drafter layers):
 *           K [n_heads][F_pad/32][32 * head_dim] then
 *           V [n_heads][F_pad/32][head_dim][32]. Each 32-frame step of K is
 *           one block in MFMA operand order: for 16-frame tile t (0, 1),
 *           dim block k (32 dims for head_dim 64, 16 for head_dim 16) and
 *           lane L = 16g + r (g = 0..3, r = 0..15), the values of frame
 *           16t + r, dims 8g..8g+7 (head_dim 16: 4g..4g+3) of block k, lanes
 *           in order. Each 32-frame step of V is transposed and contiguous;
 *           within a step, position 8g+i holds frame 4g+i for i < 4 and
 *           frame 16+4g+i-4 for i >= 4.
 *           F_pad = n_frames rounded up to 32.
 *           Must be zero-filled before the first wf_encode_kv.
 * workspace: engine-private scratch and slot state.
 * Return 0 for an invalid configuration. */
size_t wf_kv_pool_bytes(const wf_config *cfg);
size_t wf_xkv_pool_bytes(const wf_config *cfg);
size_t wf_workspace_bytes(const wf_config *cfg);

/* Create an engine on the current HIP device. d_page_table is int32
 * [max_batch][n_ctx / page_size]: slot s's logical page j lives in physical
 * page d_page_table[s][j] of kv_pool (the caller may shuffle them). The
 * workspace is zeroed here (synchronously). Fails with WF_EDEVICE when the
 * current device is not gfx950. */
wf_status wf_create(const wf_config *cfg, const wf_weights *w,
                    void *kv_pool, size_t kv_bytes,
                    void *xkv_pool, size_t xkv_bytes,
                    const int32_t *d_page_table,
                    void *workspace, size_t ws_bytes,
                    wf_engine **out);
void wf_destroy(wf_engine *e);
const char *wf_last_error(void);

/* For callers that cannot allocate device memory (harnesses that forbid
 * hipMalloc, serving loops that must not allocate): wf_create with the
 * library's own workspace instead of a caller-supplied one. The workspace is
 * a static device array of WF_STATIC_WORKSPACE_BYTES per device, resident
 * from the library's load until the process ends; this call allocates no
 * device memory (the caller still supplies the weights, both KV pools and
 * the page table). The array is cleared here (synchronously), like any
 * workspace. At most one such engine may live on a device at a time:
 * WF_ESTATE while another holds it, until wf_destroy releases it. Fails with
 * WF_ECAPACITY when wf_workspace_bytes(cfg) exceeds the array; otherwise as
 * wf_create. Calls on the engine that overlap race, as on any engine. */
#define WF_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
wf_status wf_create_static(const wf_config *cfg, const wf_weights *w,
                           void *kv_pool, size_t kv_bytes,
                           void *xkv_pool, size_t xkv_bytes,
                           const int32_t *d_page_table, wf_engine **out);

/* Set cache length 0, clear the pending-verify flag and the error word of
 * n slots. */
wf_status wf_reset(wf_engine *e, int32_t n, const int32_t *d_slots, void *stream);

/* Write-once cross K/V for n slots from the audio memory d_enc, bf16
 * [n][n_frames][d_model]:  K_c = enc Wkc^T,  V_c = enc Wvc^T + bvc,  for every
 * target layer and every drafter layer. */
wf_status wf_encode_kv(wf_engine *e, int32_t n, const int32_t *d_slots,
                       const void *d_enc, void *stream);

/* One causal pass over a block of T rows per request.
 * d_tokens int32 [n][T]: row 0 is the anchor, rows 1..n_tok-1 the
 *   candidates (for a prefill: the prompt). Rows at or beyond n_tok[b] are
 *   padding: computed but never written to the cache.
 * d_n_tok int32 [n], 0 <= n_tok <= T; 0 marks an inactive request (skipped).
 * Row i of request b sits at position L_b + i, L_b = the slot's cache length,
 *   attends to cache positions 0..L_b-1 and block rows 0..i, and its K/V are
 *   written at L_b + i when i < n_tok[b]. The slot is then pending until
 *   wf_rollback.
 * d_argmax int32 [n][T]: the target's choice for the position after each
 *   row (largest logit, lowest id on ties); -1 for skipped rows.
 * d_logits: NULL, or fp32 [n][T][vocab] logits.
 * With a drafter, the pass also projects the tapped residual streams of the
 * rows it writes into the cache and appends them to the drafter history at
 * the same positions (so the history always covers the cache length).
 * Requires n <= max_batch, n*T <= max_rows, 1 <= T <= n_ctx. */
wf_status wf_verify_block(wf_engine *e, int32_t n, const int32_t *d_slots,
                          const int32_t *d_tokens, int32_t T,
                          const int32_t *d_n_tok, int32_t *d_argmax,
                          float *d_logits, void *stream);

/* Parallel drafter pass (Whisper-Flash section 3.2, eq. 2; appendix A.2):
 * for each request the block [Emb(anchor), m, ..., m] (K mask copies) at
 * text positions L..L+K, L = the slot's cache length, goes through the
 * drafter blocks: one softmax over the history (positions < L) and the
 * block (bidirectional), RoPE (base 10000, fp32 phases) on queries and keys,
 * cross-attention to the drafter's own audio K/V, the MLP; then the
 * drafter's final LN and the shared head. Mask row i proposes the token at
 * position L+i (argmax, lowest id on ties).
 * d_anchor int32 [n]; d_block int32 [n][K+1] receives the anchor followed
 * by the K drafts, ready for wf_verify_block; d_logits: NULL or fp32
 * [n][K+1][vocab] drafter logits (row 0 is the anchor row). The slot must not be pending;
 * its length is unchanged. Within K tokens of the context end the block is
 * cut to the n_ctx - L rows that fit: drafts past them are -1 (a verify
 * must then propose at most n_ctx - L - 1 candidates). Requires
 * drafter_layers > 0, 1 <= K, n*(K+1) <= max_rows. */
wf_status wf_draft(wf_engine *e, int32_t n, const int32_t *d_slots, const int32_t *d_anchor,
                   int32_t K, int32_t *d_block, float *d_logits, void *stream);

/* Acceptance for one round, per request b with k = n_tok[b] - 1 candidates
 * and R = d_budget[b] output tokens left (k <= R - 1 is required).
 * temperature == 0: greedy — a = the longest prefix with
 *   tokens[b][i] == argmax[b][i-1] for i = 1..a; an accepted EOS stops there
 *   with no bonus; otherwise c = argmax[b][a] is emitted and is the next
 *   anchor.
 * temperature > 0: rejection sampling on fp32 softmax(logits / T) with the
 *   optional suppression mask d_suppress (uint8 [vocab], nonzero = id never
 *   emitted), draft probabilities d_q fp32 [n][T-1][vocab] (row i-1 is q_i,
 *   the distribution candidate i was drawn from) and Philox4x64-10 uniforms
 *   keyed by (seed, d_request_id[b], d_step[b], position, stream).
 * Outputs (int32 [n]): d_n_acc = a; d_next_token = c or -1 when an accepted
 *   EOS ended the request; d_n_emit = tokens emitted this round;
 *   d_done = 1 when the request ended (EOS emitted or budget used up).
 * Emitted tokens are tokens[b][1..a] followed by next_token (if >= 0). */
wf_status wf_accept(wf_engine *e, int32_t n, const int32_t *d_tokens, int32_t T,
                    const int32_t *d_n_tok, const int32_t *d_budget,
                    const int32_t *d_argmax, const float *d_logits,
                    const float *d_q, const uint8_t *d_suppress,
                    float temperature, uint64_t seed,
                    const int32_t *d_request_id, const int32_t *d_step,
                    int32_t *d_n_acc, int32_t *d_next_token,
                    int32_t *d_n_emit, int32_t *d_done, void *stream);

/* Keep L + 1 + a positions of each pending slot (d_n_acc int32 [n]); entries
 * beyond stay allocated and are masked by the length. A slot with no pending
 * verify is left unchanged. a > n_tok - 1 sets WF_DERR_ACCEPT. */
wf_status wf_rollback(wf_engine *e, int32_t n, const int32_t *d_slots,
                      const int32_t *d_n_acc, void *stream);

/* Verification-attention anchor readout ("Alignment Drift in Single-Model
 * Speculative Decoding for ASR", Verification-Attention Correction and
 * appendix D.2: the target's audio attention at one decoder layer, averaged
 * over heads, peaks at the current audio position; the scores are recomputed
 * from the key cache). With 0 <= layer < n_layers, every later verify pass
 * (wf_verify_block, wf_verify_tree) also writes into d_frame (int32, the
 * pass's [n][T] rows, at least max_rows entries; device memory the caller
 * keeps alive) the audio frame where that layer's per-head softmax over the
 * frames, averaged over heads, is largest for each row (the lowest frame
 * among equal values; -1 for rows at or beyond n_tok and skipped requests).
 * layer < 0 turns it off. */
wf_status wf_set_readout(wf_engine *e, int32_t layer, int32_t *d_frame);

/* Tree verification ("Alignment Drift in Single-Model Speculative Decoding for
 * ASR", appendix E.3: all nodes of a draft tree are checked by one target
 * forward in which each node sees only its ancestors; a tree that is a single
 * chain gives the same result as the linear block). As wf_verify_block, with
 * d_parents int32 [n][T]: parents[b][0] = -1 (node 0 is the anchor, the
 *   root) and 0 <= parents[b][i] < i for the other nodes i < n_tok[b]
 *   (entries at or beyond n_tok are ignored).
 * Node i sits at position L + depth(i), attends to cache positions 0..L-1
 * and to its ancestors and itself among the nodes, and its K/V are written
 * at cache slot L + i until wf_rollback_tree. Its argmax row is the target's
 * choice after the node's root-to-node path. A bad parent array sets
 * WF_DERR_TOKEN. Requires 1 <= T <= 64 and an engine without a drafter
 * (WF_ESTATE: the tree does not feed the drafter's history). */
wf_status wf_verify_tree(wf_engine *e, int32_t n, const int32_t *d_slots,
                         const int32_t *d_tokens, int32_t T, const int32_t *d_parents,
                         const int32_t *d_n_tok, int32_t *d_argmax, float *d_logits,
                         void *stream);

/* Greedy acceptance on a tree after wf_verify_tree. A node is accepted when
 * its parent is (the root always is), the parent is not an accepted EOS, and
 * its token equals the target's argmax at the parent. The kept path ends at
 * the deepest accepted node no deeper than R - 1 (R = d_budget[b] output
 * tokens left; the lowest node index among equally deep ones), and a is its
 * depth. Then, as in wf_accept: an accepted EOS ends the request with no
 * bonus; otherwise the argmax at that node is emitted and is the next anchor.
 * Outputs: d_path int32 [n][T], the kept nodes root first (entries past a
 * are -1), and d_n_acc, d_next_token, d_n_emit, d_done as in wf_accept.
 * Requires 1 <= T <= 64. */
wf_status wf_accept_tree(wf_engine *e, int32_t n, const int32_t *d_tokens, int32_t T,
                         const int32_t *d_parents, const int32_t *d_n_tok,
                         const int32_t *d_budget, const int32_t *d_argmax, int32_t *d_path,
                         int32_t *d_n_acc, int32_t *d_next_token, int32_t *d_n_emit,
                         int32_t *d_done, void *stream);

/* Rollback of a tree verify: in every layer the K/V of path node k (slot
 * L + path[k]) move to position L + k for k = 1..a, then the slot keeps
 * L + 1 + a positions as after wf_rollback. d_path int32 [n][T] as written by
 * wf_accept_tree. A path that is not one of this verify's nodes (path[k]
 * outside [k, n_tok)) sets WF_DERR_ACCEPT. Requires 1 <= T <= 64. */
wf_status wf_rollback_tree(wf_engine *e, int32_t n, const int32_t *d_slots, const int32_t *d_path,
                           int32_t T, const int32_t *d_n_acc, void *stream);

/* Device-resident bookkeeping of a running speculative loop (the loop of
 * Whisper-Flash section 3.1: each round verifies the anchor and its
 * candidates, emits the a accepted candidates and the next token, and the
 * next token is the next round's anchor; appendix A.1 for the output budget
 * and EOS). Keeping it on the device lets a caller capture a whole round
 * (prepare, wf_draft or a table, wf_verify_block, wf_accept, wf_rollback,
 * finish) once as a graph. Per request b (int32 [n] unless noted; the
 * caller owns the buffers):
 *   anchor   the next round's anchor token;
 *   len      the slot's cache length (as wf_rollback leaves it);
 *   emitted  tokens emitted so far, the first anchor included;
 *   done     1 once the request has ended (EOS emitted or budget used up);
 *   acc_sum, prop_sum  accepted and proposed candidates over the rounds;
 *   rounds, step       rounds the request took part in (step also keys the
 *                      sampling uniforms of wf_accept);
 *   tok_sum  tokens the rounds emitted;
 *   hist     int64 [K + 1], rounds per accepted length. */
typedef struct wf_loop_state {
    int32_t *anchor, *len, *emitted, *done;
    int32_t *acc_sum, *prop_sum, *rounds, *step, *tok_sum;
    int64_t *hist;
} wf_loop_state;

/* A round's inputs from the loop state, per request: R = n_max - emitted
 * outputs left, k = max(0, min(K, R - 1, n_ctx - len - 1)) candidates (so
 * that k <= R - 1 and the block fits the context), d_n_tok = k + 1, or 0
 * once done; d_budget = max(R, 1). With d_table (int32 [n][table_cols], the
 * candidate for each absolute position) the block d_block int32 [n][K + 1]
 * is the anchor followed by table[b][min(len + i, table_cols - 1)] for
 * i = 1..K; with d_table NULL only n_tok and the budget are written (the
 * caller fills the block, e.g. with wf_draft). Requires 0 <= K, K + 1 <=
 * n_ctx, n_max >= 1, table_cols >= 1 with a table; no state pointer NULL. */
wf_status wf_loop_prepare(wf_engine *e, int32_t n, const wf_loop_state *s, int32_t K,
                          int32_t n_max, const int32_t *d_table, int32_t table_cols,
                          int32_t *d_block, int32_t *d_n_tok, int32_t *d_budget, void *stream);

/* The state update after wf_accept and wf_rollback, per request active this
 * round (d_n_tok > 0): len += a + 1; anchor = next_token when >= 0; emitted
 * and tok_sum += n_emit; done = 1 when d_done; acc_sum += a; prop_sum +=
 * n_tok - 1; rounds and step += 1; hist[min(max(a, 0), K)] += 1 (a =
 * d_n_acc). Inactive requests are left unchanged. */
wf_status wf_loop_finish(wf_engine *e, int32_t n, const wf_loop_state *s, int32_t K,
                         const int32_t *d_n_tok, const int32_t *d_n_acc,
                         const int32_t *d_next_token, const int32_t *d_n_emit,
                         const int32_t *d_done, void *stream);

/* Shorten the cache of n slots to d_len[b] positions (0 <= d_len[b] <= the
 * current length; the slot must not be pending), e.g. to verify the same
 * block again from the same state. A bad length sets WF_DERR_STATE. */
wf_status wf_truncate(wf_engine *e, int32_t n, const int32_t *d_slots,
                      const int32_t *d_len, void *stream);

/* Synchronise the stream and copy max_batch error words and cache lengths
 * to the host (either pointer may be NULL). */
wf_status wf_device_state(wf_engine *e, int32_t *h_err, int32_t *h_len, void *stream);

/* Measurement. While timing is enabled every launch is bracketed with HIP
 * events on its stream (so calls are no longer graph-capturable).
 * wf_get_timing synchronises and returns the summed duration and the number
 * of launches of one kind since timing was last enabled. Kinds (each is one
 * kernel instantiation): 0 QKV projection + KV append, 1 self/cross output
 * projections + residual, 2 cross-attention query, 3 fc1 + GELU,
 * 4 fc2 + residual, 5 tied LM head + argmax, 6 self-attention,
 * 7 cross-attention, 8 everything else (embed, layer norms, argmax merge,
 * accept, rollback), 9 write-once cross K/V, 10 drafter pass, 11 drafter
 * history append inside the verify pass. */
wf_status wf_set_timing(wf_engine *e, int32_t enable);
wf_status wf_get_timing(wf_engine *e, int32_t kind, double *total_ms, int32_t *count);
/* Kind 12: the persistent pass kernel (below), one launch per verify pass. */

/* Execution-path options of an engine (host state, read at each call; the
 * defaults are the fastest paths measured on MI355X). None changes a result
 * beyond the summation order named here:
 *  WF_OPT_PERSISTENT (default 0): run a linear verify pass whose model has
 *    d_model 1280, d_ffn 5120 and head_dim 64, with n * T <= 1024 and
 *    T <= 64 and no anchor readout, as one persistent kernel: one workgroup
 *    per CU walks every layer's tasks and waits for the rows it reads on
 *    arrival counters. Bit-identical to the multi-kernel path. 0 runs the
 *    multi-kernel path. A pass that exceeds the kernel's internal wait limit
 *    sets WF_DERR_TIMEOUT in its requests' error words.
 *  WF_OPT_TALL_GEMM, WF_OPT_LN_FUSION (default 1): the tall-block GEMM for
 *    blocks of 97..1024 rows, the layer norm in the GEMM prologue for one
 *    row tile; 0 takes the other GEMM kernels (bit-identical).
 *  WF_OPT_XA_CHUNKS (default 0 = chosen by batch size; 4, 8, 16 or 32):
 *    frame chunks per (request, head) of cross-attention; this changes the
 *    cross-attention summation order (every choice is still independent of
 *    the block length).
 *  WF_OPT_PASS_TIMEOUT_US (default 500000): the persistent pass's wait limit
 *    in microseconds, measured per wait. Past it the pass aborts (every
 *    wait ends at once, every workgroup drains) and sets WF_DERR_TIMEOUT;
 *    a small value forces that path, for tests of the error handling.
 * Unknown options or values return WF_EINVAL. */
#define WF_OPT_PERSISTENT 1
#define WF_OPT_TALL_GEMM  2
#define WF_OPT_LN_FUSION  3
#define WF_OPT_XA_CHUNKS  4
#define WF_OPT_PASS_TIMEOUT_US 5
wf_status wf_set_option(wf_engine *e, int32_t option, int32_t value);

/* Task trace of the persistent pass: with d_trace non-NULL (device memory,
 * bytes / 32 tasks; the caller keeps it alive), every later persistent pass
 * whose task list fits writes for task t the 100 MHz device clock at its
 * start, when its inputs were ready, and at its end, and the workgroup that
 * ran it (uint64 [t][4]). NULL turns it off. wf_pass_schedule copies
 * the last pass's task list layout to h_info (int32 [20]): total tasks,
 * tasks per layer, layers, the 12 phase offsets within a layer (LN1, QKV,
 * self-attention, O, LN2, cross Q, cross-attention, O_c, LN3, fc1, fc2, end),
 * the 3 head offsets after the layers (final LN, LM head, end) and the
 * grid. */
wf_status wf_set_trace(wf_engine *e, void *d_trace, size_t bytes);
wf_status wf_pass_schedule(wf_engine *e, int32_t *h_info);


/* ------------------------------------------------------------------------
 * Audio encoder: log-mel features of a fixed window to the audio memory
 * (the encoder stage before wf_encode_kv; "Whisper-Flash ...", sections 1-2
 * and appendix A.3, Table A2, where it is a fixed cost per request; the
 * 30 s mel window of the SGLang-Omni "Whisper ASR" cookbook, "Long Audio
 * Chunking"). The pages give no layer detail; the encoder follows the
 * Whisper architecture they cite: two width-3 convolutions over time (zero
 * padding 1, the second with stride 2, each followed by exact GELU), a fixed
 * sinusoidal position table (channel j < d/2: sin(t w_j), d/2 + j:
 * cos(t w_j), w_j = 10000^(-j/(d/2-1))), n_layers pre-LN blocks of
 * bidirectional self-attention (scores / sqrt(64), biases on q, v and the
 * output projection, none on k) and a GELU MLP, then a final layer norm.
 *
 * Numerics: bf16 MFMA with fp32 accumulation; the residual stream, layer
 * norms, softmax and GELU are fp32; activations between kernels (layer-norm
 * outputs, q, k, v, attention output, MLP hidden, convolution outputs) and
 * the attention probabilities entering the PV product are bf16.
 * ------------------------------------------------------------------------ */
typedef struct wf_encoder wf_encoder;

typedef struct {
    int32_t n_layers;   /* encoder blocks (32 for large-v3 and turbo) */
    int32_t d_model;    /* width: n_heads * 64, at most 1280 */
    int32_t n_heads;    /* attention heads (head_dim must be 64) */
    int32_t head_dim;   /* 64 */
    int32_t d_ffn;      /* MLP width, a multiple of 64 (5120) */
    int32_t n_mels;     /* mel channels (128): 64, 128, 192 or 256 */
    int32_t n_frames;   /* output frames F (1500); the input has 2F frames */
    int32_t max_batch;  /* largest n of one wf_encode call */
    float ln_eps;       /* 1e-5 */
} wf_enc_config;

/* One block (bf16, PyTorch Linear convention: weight [out, in]). */
typedef struct {
    const void *ln1_g, *ln1_b;                    /* [d] */
    const void *wq, *bq, *wk, *wv, *bv, *wo, *bo; /* [d, d] / [d]; no key bias */
    const void *ln2_g, *ln2_b;
    const void *w1, *b1;                          /* [d_ffn, d], [d_ffn] */
    const void *w2, *b2;                          /* [d, d_ffn], [d] */
} wf_enc_layer_weights;

typedef struct {
    const void *conv1_w, *conv1_b;  /* [d, n_mels, 3] (PyTorch Conv1d), [d] */
    const void *conv2_w, *conv2_b;  /* [d, d, 3], [d] */
    const void *lnp_g, *lnp_b;      /* final layer norm [d] */
    const wf_enc_layer_weights *layers; /* host array of n_layers entries (copied) */
} wf_enc_weights;

/* Workspace of an encoder (activations for max_batch requests, the position
 * table and the convolution weights re-laid in window order); 0 for an
 * invalid configuration. */
size_t wf_enc_workspace_bytes(const wf_enc_config *cfg);

/* Create an encoder on the current HIP device (gfx950). The weights stay
 * the caller's and must outlive the encoder; the workspace is zeroed and
 * prepared here (synchronously). */
wf_status wf_enc_create(const wf_enc_config *cfg, const wf_enc_weights *w, void *workspace,
                        size_t ws_bytes, wf_encoder **out);
void wf_enc_destroy(wf_encoder *e);

/* d_mel: bf16 [n][n_mels][2 n_frames] (channel-major, as a feature
 * extractor produces it); d_out: bf16 [n][n_frames][d_model], the audio
 * memory that wf_encode_kv takes. 1 <= n <= max_batch. Asynchronous on the
 * stream; calls on one encoder must not overlap (they share the workspace). */
wf_status wf_encode(wf_encoder *e, int32_t n, const void *d_mel, void *d_out, void *stream);

/* Per-kind launch timing as for the engine. Kinds: 0 stem convolutions,
 * 1 QKV projection, 2 attention, 3 output projection + residual,
 * 4 fc1 + GELU, 5 fc2 + residual, 6 layer norms, 7 feature transpose. */
enum { WF_ENC_TK_STEM = 0, WF_ENC_TK_QKV = 1, WF_ENC_TK_ATTN = 2, WF_ENC_TK_OPROJ = 3,
       WF_ENC_TK_FC1 = 4, WF_ENC_TK_FC2 = 5, WF_ENC_TK_LN = 6, WF_ENC_TK_OTHER = 7,
       WF_ENC_TK_N = 8 };
wf_status wf_enc_set_timing(wf_encoder *e, int32_t enable);
wf_status wf_enc_get_timing(wf_encoder *e, int32_t kind, double *total_ms, int32_t *count);

#ifdef __cplusplus
}
#endif
#endif /* WF_H */
