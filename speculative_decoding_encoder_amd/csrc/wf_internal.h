// Kernel argument blocks and launch functions shared by the kernel files and
// the engine. Everything here is internal to libwf.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include "../../include/wf.h"

namespace wf {

// GEMM epilogues: what happens to C[m][n] = sum_k X[m][k] W[n][k].
enum Epi : int {
    EPI_QKV = 0,    // q -> fp16 buffer; k, v -> the slot's KV pages (valid rows)
    EPI_RESID = 1,  // x[m][n] += C + b[n]            (fp32 residual stream)
    EPI_F16 = 2,    // out[m][n] = fp16(C + b[n])      (cross-attention query)
    EPI_GELU = 3,   // out = fp16(GELU(C + b)), fragment-tiled (MLP hidden)
    EPI_ARGMAX = 4, // tied LM head: per 64-column tile (max, lowest argmax), logits
    EPI_XKV = 5,    // (unused: the cross K/V come from the encoder's dense GEMM)
    EPI_STORE32 = 6,// out32[m][n] = C + b_seg[n]      (drafter temporaries, history)
};

struct EpiArgs {
    const uint16_t *b0, *b1, *b2;  // bias per weight segment (bf16), may be null
    float *x;                      // EPI_RESID: x = x_in + C + b (x_in may be x)
    const float *x_in;
    float *out32;                  // EPI_STORE32 [M][N]
    uint16_t *out;                 // EPI_F16 / EPI_QKV (q) fp16 [M][N or d]; EPI_GELU fp16 tiled
    // EPI_QKV: KV append
    uint16_t *kv_layer;            // this layer's first page
    const int32_t *page_table;
    int32_t pt_stride;
    const int32_t *slots, *req_L, *req_ntok;
    int32_t T, H, hd, page_elems;
    const int32_t *row_kv;         // per row: page * 16 + offset of its position, -1: no append
    // EPI_ARGMAX
    float *logits;                 // null or [M][V]
    float *tile_max;               // [M][ld]: per row, its 64-column tiles
    int32_t *tile_idx;
    int32_t ld;
};

struct GemmArgs {
    const uint16_t *X;             // fp16, fragment-tiled (xh_index), or plain bf16 [M][K]
    const uint16_t *W0, *W1, *W2;  // weight segments, each [seg_n][K] bf16
    int32_t M, K, N, seg_n;
    int32_t S, ck;                 // K chunks (fixed per K) and k-steps per chunk
    int32_t n_tiles, m_blocks, n_groups;  // logical grid; n_groups = physical K split P
    int32_t n_wg;                  // logical workgroups (grid is padded to 8k)
    float *part;                   // subtree sums [P][M][N] when P > 1
    int32_t *cnt;                  // arrival counters [n_tiles * m_blocks]
    // layer norm in the prologue (register-tiled kernel, one row tile): X is
    // LN(lnx) computed on the fly; lnx is the fp32 residual stream [M][K]
    const float *lnx;
    const uint16_t *lng, *lnb;
    float ln_eps;
    EpiArgs e;
};

struct PrepareArgs {
    int32_t n, T, V, n_ctx, n_pages, pt_stride, page_size, max_batch;
    const int32_t *slots, *tokens, *n_tok, *page_table;
    int32_t *slot_len, *slot_pending, *slot_err;
    int32_t *req_L, *req_ntok;
    // tree verification (null for a linear block): parent of every node in,
    // its depth and ancestor-or-self bit mask out ([n][T], T <= 64)
    const int32_t *parents;
    int32_t *depth;
    uint64_t *anc;
};

struct EmbedArgs {
    int32_t M, T, d, V, n_ctx;
    const int32_t *tokens, *req_L;
    const uint16_t *tok_emb, *pos_emb;
    float *x;
    // the KV destination of every row, shared by all layers of the pass
    const int32_t *req_ntok, *slots, *page_table;
    int32_t pt_stride;
    int32_t *row_kv;               // [M]: page * 16 + offset, or -1 (padding / skipped)
    const int32_t *depth;          // tree verification: row m at position L + depth[m]
};

struct LnArgs {
    const float *x;
    int32_t M, d;
    const uint16_t *g, *b;
    float eps;
    uint16_t *out;                 // fp16 [M][d], fragment-tiled
};

struct SelfAttnArgs {
    const uint16_t *q;             // fp16 [M][d]
    const uint16_t *kv_layer;      // this layer's page base
    const int32_t *page_table, *slots, *req_L, *req_ntok;
    int32_t pt_stride, page_elems;
    int32_t n, T, H, d;
    int32_t causal;                // 1: row i sees keys <= L+i; 0: the whole block
    float scale;
    uint16_t *out;                 // fp16 [M][d], fragment-tiled
    const uint64_t *anc;           // tree verification: per row, the block keys it sees
};

// Cross-attention load ring depth (32-frame steps in flight per wave); a
// chunk's step count is a multiple of it.
constexpr int kXaRing = 2;

struct CrossAttnArgs {
    const uint16_t *q;             // fp16 [M][d]
    const uint16_t *xkv;           // pool base
    int64_t slot_stride, layer_off;
    const int32_t *slots, *req_ntok;
    int32_t n, T, H, d, F, F_pad;
    int32_t mt, G, cf, spw;        // m-tiles per request, chunk groups (of 4 chunks),
                                   // frames per chunk, 32-frame steps per chunk
                                   // (a multiple of kXaRing)
    int32_t n_items;               // n * H * mt * G workgroups
    float scale;
    float *part;                   // [item][16][hd+4] (o, m, l, spare) when G > 1
    int32_t *cnt;                  // [n*H*mt]
    uint16_t *out;                 // fp16 [M][d], fragment-tiled
};

struct LmReduceArgs {
    const float *tile_max;
    const int32_t *tile_idx;
    int32_t n_tiles, ld, M, T;     // tiles [M][ld]
    const int32_t *slots, *req_ntok;
    int32_t *slot_err;
    int32_t *argmax;
};

struct AcceptArgs {
    int32_t n, T, V, eos;
    const int32_t *tokens, *n_tok, *budget, *argmax;
    int32_t *n_acc, *next_token, *n_emit, *done;
    // sampling (temperature > 0)
    const float *logits, *q;
    const uint8_t *suppress;
    float temperature;
    uint64_t seed;
    const int32_t *request_id, *step;
    // scratch for the rows' softmax statistics, 2 floats per row [n][T]
    // (nullable: then the acceptance kernel reduces each row itself)
    float *stats;
};

struct LoopArgs {
    int32_t n, K, n_max, n_ctx, table_cols;
    wf_loop_state s;
    const int32_t *table;
    int32_t *block, *n_tok_out, *budget;
    const int32_t *n_tok, *n_acc, *next_token, *n_emit, *done;
};

struct RollbackArgs {
    int32_t n, max_batch;
    const int32_t *slots, *n_acc;
    int32_t *slot_len, *slot_pending, *slot_err;
};

// GEMM roles: each is its own kernel instantiation (and profiler symbol).
enum Role : int {
    ROLE_QKV = 0, ROLE_OPROJ = 1, ROLE_CROSS_Q = 2, ROLE_FC1 = 3, ROLE_FC2 = 4,
    ROLE_LM_HEAD = 5, ROLE_XKV = 6,   // ROLE_XKV: retired (wf_encode_kv uses launch_xkv_dense)
    ROLE_DRAFT_QKV = 7,   // drafter q, k, v (fp32 temporaries before RoPE)
    ROLE_HIST = 8,        // history projection of the tapped streams
    ROLE_HIST_KV = 9,     // drafter k, v of history rows
};

struct TapArgs {
    const float *x;
    int32_t M, d, j, n_taps;
    uint16_t *out;                 // fp16 [M][n_taps*d], fragment-tiled
};

struct RopeArgs {
    const float *tmp;              // [M][ncols] fp32 projections
    int32_t ncols, q_off, k_off, v_off;   // column offsets; q_off < 0: no query
    int32_t M, T, H, hd, d;
    const int32_t *slots, *req_L, *req_ntok, *page_table;
    int32_t pt_stride, page_elems;
    uint16_t *kv_layer;            // drafter layer's first page
    uint16_t *q_out;               // fp16 [M][d] rotated queries
};

struct PrepareDraftArgs {
    int32_t n, K, V, n_ctx, n_pages, pt_stride, max_batch;
    const int32_t *slots, *anchor, *page_table;
    int32_t *slot_len, *slot_pending, *slot_err;
    int32_t *req_L, *req_ntok;
};

struct EmbedDraftArgs {
    int32_t M, T, d, V;
    const int32_t *anchor;
    const uint16_t *tok_emb, *mask;
    float *x;
};

// Verification-attention anchor readout at one decoder layer: the layer's
// cross-attention scores recomputed from the cross K cache, per head the
// softmax over frames, summed over heads, and the peak frame per row.
struct ReadoutArgs {
    const uint16_t *q;             // the layer's cross queries, fp16 [M][d]
    const uint16_t *xkv;           // write-once pool
    int64_t slot_stride, layer_off;
    const int32_t *slots, *req_ntok;
    int32_t n, T, H, hd, d, F, F_pad, max_batch, nc;   // nc: 128-frame chunks
    float sl2e;                    // scale * log2(e)
    float2 *ml;                    // [M][H]: row max and sum of 2^((s - max) sl2e)
    float2 *part;                  // [M][nc]: (peak value, frame) per chunk
    int32_t *frame;                // [M] out: peak frame, -1 for skipped rows
};
hipError_t launch_readout(const ReadoutArgs &a, int mt, hipStream_t st);

// Greedy acceptance on a token tree, one thread per request.
struct TreeAcceptArgs {
    int32_t n, T, eos;
    const int32_t *tokens, *parents, *n_tok, *budget, *argmax;
    int32_t *path, *n_acc, *next_token, *n_emit, *done;
};

// Move the K/V of each pending slot's accepted tree path (cache slot
// L + path[k]) to position L + k, every layer.
struct CompactArgs {
    int32_t n, T, n_layers, H, hd, max_batch, pt_stride, page_elems;
    size_t layer_elems;
    const int32_t *slots, *path, *n_acc, *slot_len, *slot_pending, *page_table;
    int32_t *slot_err;
    uint16_t *kv;
};

// ---------------------------------------------------------------------------
// Persistent pass kernel (k_pass.hip): one launch runs every decoder layer of
// a linear verify pass, the final layer norm, the tied LM head and the per-row
// argmax. Its workgroups (one per CU) walk a fixed task list; a task waits
// for the 16-row tiles it reads through per-(layer, phase, tile) arrival
// counters, so phases overlap wherever their rows allow.

// Decoder weights of one layer (bf16, the layout of wf_layer_weights).
struct LayerW {
    const uint16_t *ln1_g, *ln1_b, *wq, *bq, *wk, *wv, *bv, *wo, *bo;
    const uint16_t *ln2_g, *ln2_b, *wqc, *bqc, *wkc, *wvc, *bvc, *woc, *boc;
    const uint16_t *ln3_g, *ln3_b, *w1, *b1, *w2, *b2;
};

// Phases of one layer, in task-list order, then the head's two phases.
enum PassPhase : int {
    PH_LN1 = 0, PH_QKV, PH_SA, PH_O, PH_LN2, PH_CQ, PH_XA, PH_OC, PH_LN3, PH_FC1, PH_FC2,
    PH_PER_LAYER,                  // 11
    PH_LNF = PH_PER_LAYER, PH_LMH, // head phases (after the last layer)
};
// GEMM phases' tilings, in this order in PassArgs::g
enum PassGemm : int { PG_QKV = 0, PG_O, PG_CQ, PG_OC, PG_FC1, PG_FC2, PG_LMH, PG_N };

struct PassGemmCfg {
    int32_t n_tiles, m_blocks, n_groups;   // column tiles, row blocks, K groups
    int32_t n_tasks;                       // ceil8(n_tiles) * m_blocks * n_groups
};

constexpr int kPassMaxRows = 1024;         // M <= 1024: at most 64 row tiles

struct PassArgs {
    int32_t n, T, M, RT, mt;               // requests, block, rows, row tiles, tiles per request
    int32_t max_batch;                     // slot ids are [0, max_batch)
    int32_t n_layers, d, H, hd, F, V;      // F: MLP width
    float ln_eps, scale;
    const LayerW *lw;                      // [n_layers], device
    const uint16_t *tok_emb, *lnf_g, *lnf_b;
    // per-request state of the pass
    const int32_t *slots, *req_L, *req_ntok, *row_kv, *page_table;
    int32_t *slot_err;
    int32_t pt_stride, page_elems;
    uint16_t *kv;                          // KV pool; layer l at kv + l * kv_layer_elems
    int64_t kv_layer_elems;
    const uint16_t *xkv;
    int64_t xkv_slot_elems, xkv_layer_elems;
    int32_t n_frames, F_pad, xa_G, xa_cf, xa_spw;
    // activations, each written once per launch (see k_pass.hip)
    float *xv;                             // residual versions [3 n_layers + 1][M][d]
    uint16_t *lnv;                         // layer-norm outputs [3 n_layers + 1][Mp][d] (tiled)
    uint16_t *qv, *cqv;                    // self / cross queries [n_layers][M][d]
    uint16_t *sav, *xav;                   // attention outputs [n_layers][Mp][d] (tiled)
    uint16_t *hsv;                         // MLP hidden [n_layers][Mp][F] (tiled)
    int64_t x_stride, act_stride, q_stride, hs_stride;
    float *part;                           // GEMM K-group sums
    int32_t *gcnt;                         // and their arrival counters
    float *xapart;                         // cross-attention chunk-group partials
    int32_t *xacnt;
    // head
    float *logits;                         // nullable [M][V]
    float *tile_max;
    int32_t *tile_idx;
    int32_t ld, n_vtiles;
    int32_t *argmax;                       // [M]
    // drafter history taps (n_taps = 0: none)
    uint16_t *taps;
    int32_t n_taps, tap_layers[8];
    // schedule
    int32_t *cnt;                          // [(n_layers * PH_PER_LAYER + 2) * RT] arrival counters
    int32_t *abort_flag;
    int32_t ph_off[PH_PER_LAYER + 1];      // task offsets of the phases within a layer
    int32_t per_layer, head_off[3], total;
    PassGemmCfg g[PG_N];
    int32_t sa_items, xa_items;            // per layer
    int64_t timeout_ticks;                 // wait limit, 100 MHz clock
    uint64_t *trace;                       // nullable: per task (start, end) clock
};

hipError_t launch_pass(const PassArgs &a, int mb_class, int grid, hipStream_t st);
hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t st);
// Size class of the pass kernel's GEMM tiles for a block of M rows, and
// per class and projection (PassGemm) the rows and columns of a task and
// the number of K groups.
int pass_class_of_rows(int M);
void pass_tiling(int cl, int pg, int &bm, int &bn, int &groups);

hipError_t launch_accept_tree(const TreeAcceptArgs &a, hipStream_t st);
hipError_t launch_compact(const CompactArgs &a, hipStream_t st);
hipError_t launch_tap(const TapArgs &a, hipStream_t st);
hipError_t launch_rope_append(const RopeArgs &a, hipStream_t st);
hipError_t launch_prepare_draft(const PrepareDraftArgs &a, hipStream_t st);
hipError_t launch_embed_draft(const EmbedDraftArgs &a, hipStream_t st);
hipError_t launch_draft_out(const int32_t *anchor, const int32_t *argmax, const int32_t *req_ntok,
                            int n, int K, int32_t *block, hipStream_t st);
hipError_t launch_gemm(int role, const GemmArgs &a, int mb, hipStream_t st);
// dense bf16 MFMA GEMM of the audio encoder with the cross K/V pool epilogue
// (encoder.hip); K a multiple of 32, H * hd the model width
hipError_t launch_xkv_dense(const uint16_t *enc, int M, int K, const uint16_t *wk,
                            const uint16_t *wv, const uint16_t *bv, uint16_t *xkv,
                            long long slot_stride, long long layer_off, const int32_t *slots,
                            int F, int F_pad, int H, int hd, int max_batch, hipStream_t st);
// register-tiled variant for short blocks: (mb, nb) in {1x1, 1x2, 1x4, 2x2,
// 2x4, 4x2, 4x4} (the LM head: nb = 4, mb up to 6); built for the chunk lengths
// gemm_rk_built accepts, one wave per chunk of the workgroup's K group
hipError_t launch_gemm_rk(int role, const GemmArgs &a, int mb, int nb, hipStream_t st);
bool gemm_rk_built(int role, int ck);
// tall-block kernel for verify passes of many requests: 16 mb x 64 tiles
// (mb 6 or 8), four waves sharing the activations through LDS, the whole of
// K per workgroup (QKV and fc1; K = 1280)
hipError_t launch_gemm_tl(int role, const GemmArgs &a, int mb, hipStream_t st);
bool gemm_tl_built(int role, int S, int ck);
hipError_t launch_prepare(const PrepareArgs &a, hipStream_t st);
hipError_t launch_embed(const EmbedArgs &a, hipStream_t st);
hipError_t launch_layernorm(const LnArgs &a, hipStream_t st);
hipError_t launch_self_attn(const SelfAttnArgs &a, int hd, int mt, hipStream_t st);
hipError_t launch_cross_attn(const CrossAttnArgs &a, int hd, hipStream_t st);
hipError_t launch_lm_reduce(const LmReduceArgs &a, hipStream_t st);
hipError_t launch_accept(const AcceptArgs &a, hipStream_t st);
hipError_t launch_loop_prepare(const LoopArgs &a, hipStream_t st);
hipError_t launch_loop_finish(const LoopArgs &a, hipStream_t st);
hipError_t launch_accept_sample(const AcceptArgs &a, hipStream_t st);
size_t sample_scratch_floats(int n, int T);   // floats of AcceptArgs::stats the split draw uses
hipError_t launch_rollback(const RollbackArgs &a, hipStream_t st);
hipError_t launch_truncate(const RollbackArgs &a, hipStream_t st);  // n_acc = new lengths
hipError_t launch_reset(int32_t n, int32_t max_batch, const int32_t *slots, int32_t *len,
                        int32_t *pending, int32_t *err, hipStream_t st);

}  // namespace wf
