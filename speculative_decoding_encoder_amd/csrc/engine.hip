// Host side of libwf.so: argument checks, workspace layout, and the launch
// plan of one verify pass (embed, then per layer LN1 -> QKV + KV append ->
// self-attention -> O + residual -> LN2 -> cross Q -> cross-attention ->
// O_c + residual -> LN3 -> fc1 + GELU -> fc2 + residual, then the final LN,
// the tied LM head with its argmax, and the per-row argmax merge).
#include "../../include/wf.h"
#include "wf_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace wf;

namespace {

thread_local char g_err[512] = "";

wf_status fail(wf_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// K chunking of the GEMMs: a function of K only (see k_gemm.hip).
void gemm_chunks(int K, int &ck, int &S) {
    const int ks = K / 32;
    S = (ks % 8 == 0) ? 8 : 2;
    ck = ks / S;
}
constexpr int kSplitRowsCap = 128;   // GEMM K-split scratch sized for this many rows x 8

// Cross-attention chunking: up to 32 chunks per (request, head) -- enough
// waves to cover the GPU when the batch is small -- of spw 32-frame steps
// each (a multiple of the load ring depth), then the fewest chunks (a
// multiple of 4, one per wave of a group) that still cover the frames at that
// length. Depends on the number of requests only, never on the block length,
// so a row's bits do not depend on its block. want_chunks (4, 8, 16 or 32;
// wf_set_option WF_OPT_XA_CHUNKS) fixes the first choice instead.
void cross_chunks(int n, int H, int F, int want_chunks, int &cf, int &G, int &spw) {
    const int steps = cdiv(F, 32);
    const int want = cdiv(2048, n * H);
    int C = want >= 32 ? 32 : (want >= 16 ? 16 : (want >= 8 ? 8 : 4));
    if (want_chunks == 4 || want_chunks == 8 || want_chunks == 16 || want_chunks == 32)
        C = want_chunks;
    spw = cdiv(cdiv(steps, C), kXaRing) * kXaRing;
    C = cdiv(cdiv(steps, spw), 4) * 4;
    cf = spw * 32;
    G = C / 4;
}

int all_layers(const wf_config *c) { return c->n_layers + c->drafter_layers; }

struct Layout {
    size_t x, xs, hs, q, tdepth, tanc, rdml, rdpart, part, gcnt, xapart, xacnt, lmmax, lmidx, reqL, reqN, len, pend, err;
    size_t taps, dam, rowkv;
    // persistent pass (absent when pass_rows == 0): per-layer activations,
    // written once per launch, the arrival counters and the weight table
    size_t pxv, plnv, pqv, pcqv, psav, pxav, phsv, pcnt, plw;
    int pass_rows;                 // rows (multiple of 16) the pass buffers hold
    size_t total;
    size_t part_bytes, xapart_bytes;
    int n_vtiles;
};

// The persistent pass covers the Whisper large-v3 / turbo decoder width
// (its GEMM chunking and layer-norm registers are built for d = 1280, MLP
// 5120, head_dim 64) and blocks of up to 1024 rows.
bool pass_shape_ok(const wf_config *c) {
    return c->d_model == 1280 && c->d_ffn == 5120 && c->head_dim == 64;
}
int pass_rows_of(const wf_config *c) {
    if (!pass_shape_ok(c)) return 0;
    return std::min((c->max_rows + 15) / 16 * 16, kPassMaxRows);
}

bool config_ok(const wf_config *c, std::string *why) {
    auto bad = [&](const char *m) { if (why) *why = m; return false; };
    if (!c) return bad("null config");
    if (c->n_layers < 1) return bad("n_layers < 1");
    if (c->head_dim != 16 && c->head_dim != 64) return bad("head_dim must be 16 or 64");
    if (c->n_heads < 1 || c->d_model != c->n_heads * c->head_dim) return bad("d_model != n_heads*head_dim");
    if (c->d_model % 64) return bad("d_model must be a multiple of 64");
    if (c->d_ffn < 64 || c->d_ffn % 64) return bad("d_ffn must be a positive multiple of 64");
    if (c->vocab < 2) return bad("vocab < 2");
    if (c->n_frames < 1) return bad("n_frames < 1");
    if (c->n_ctx < 32 || c->n_ctx % 32 || c->n_ctx > 1024)
        return bad("n_ctx must be a multiple of 32 in [32, 1024]");
    if (c->page_size != 16) return bad("page_size must be 16");
    if (c->max_batch < 1 || c->max_rows < 1) return bad("max_batch and max_rows must be >= 1");
    if (c->n_pages < 1) return bad("n_pages < 1");
    if (c->eos_id < 0 || c->eos_id >= c->vocab) return bad("eos_id outside the vocabulary");
    if (!(c->ln_eps > 0.f)) return bad("ln_eps must be > 0");
    if (c->drafter_layers < 0 || c->drafter_layers > 8) return bad("drafter_layers outside [0, 8]");
    if (c->drafter_layers > 0) {
        if (c->n_taps < 1 || c->n_taps > 8) return bad("n_taps outside [1, 8]");
        for (int j = 0; j < c->n_taps; ++j)
            if (c->tap_layers[j] < 0 || c->tap_layers[j] >= c->n_layers)
                return bad("tap layer outside the decoder");
    }
    return true;
}

Layout layout_of(const wf_config *c) {
    Layout L{};
    const size_t M = (size_t)c->max_rows, d = c->d_model, f = c->d_ffn;
    const int H = c->n_heads, hd = c->head_dim;
    L.n_vtiles = cdiv(c->vocab, 64);
    // K-split subtree sums: up to 8 groups of kSplitRowsCap rows of the widest projection
    size_t part = (size_t)8 * kSplitRowsCap * std::max(3 * d, f) * 4;
    L.part_bytes = part;
    // cross-attention merge partials: 4 chunk groups per (request, head) at
    // the largest batch for verify blocks of one row tile (small batches take
    // up to 8 groups in the same bytes); blocks that would not fit take fewer
    // groups
    const size_t xap = std::max((size_t)c->max_batch * H * 4 * 16 * (hd + 4) * 4, (size_t)8 << 20);
    L.xapart_bytes = xap;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
    L.x = take(M * d * 4);
    const size_t Mp = (M + 15) / 16 * 16;   // fp16 activation buffers hold whole 16-row tiles
    L.xs = take(Mp * d * 2);
    // the MLP hidden layer (fp16), or the drafter's fp32 projections [M][3d]
    L.hs = take(Mp * std::max(f * 2, 3 * d * 4));
    L.q = take(M * d * 2);
    L.tdepth = take(M * 4);   // tree verification: node depths
    L.tanc = take(M * 8);     // and ancestor masks
    // anchor readout: per row and head (max, sum), per row and 128-frame chunk a peak
    L.rdml = take(M * H * 8);
    L.rdpart = take(M * (size_t)cdiv(c->n_frames, 128) * 8);
    L.part = take(part);
    L.gcnt = take((size_t)cdiv(std::max(3 * (int)d, (int)f), 16) * (cdiv((int)M, 16) + 1) * 4);
    L.xapart = take(xap);
    L.xacnt = take((size_t)c->max_batch * H * (c->n_ctx / 16 + 1) * 4);
    L.lmmax = take((size_t)L.n_vtiles * M * 4);
    L.lmidx = take((size_t)L.n_vtiles * M * 4);
    L.reqL = take((size_t)c->max_batch * 4);
    L.reqN = take((size_t)c->max_batch * 4);
    L.len = take((size_t)c->max_batch * 4);
    L.pend = take((size_t)c->max_batch * 4);
    L.err = take((size_t)c->max_batch * 4);
    L.taps = take(c->drafter_layers > 0 ? Mp * (size_t)c->n_taps * d * 2 : 0);
    L.dam = take(M * 4);
    L.rowkv = take(M * 4);
    L.pass_rows = pass_rows_of(c);
    if (L.pass_rows > 0) {
        const size_t Pm = (size_t)L.pass_rows, NL = (size_t)c->n_layers;
        L.pxv = take((3 * NL + 1) * Pm * d * 4);
        L.plnv = take((3 * NL + 1) * Pm * d * 2);
        L.pqv = take(NL * Pm * d * 2);
        L.pcqv = take(NL * Pm * d * 2);
        L.psav = take(NL * Pm * d * 2);
        L.pxav = take(NL * Pm * d * 2);
        L.phsv = take(NL * Pm * f * 2);
        // counters [(NL * phases + 2) * 64 tiles], then the abort flag
        L.pcnt = take(((NL * PH_PER_LAYER + 2) * 64 + 64) * 4);
        L.plw = take(NL * sizeof(LayerW));
    }
    L.total = o;
    return L;
}

int f_pad_of(const wf_config *c) { return cdiv(c->n_frames, 32) * 32; }

enum TimingKind {
    TK_QKV = 0, TK_OPROJ = 1, TK_QC = 2, TK_FC1 = 3, TK_FC2 = 4, TK_LMHEAD = 5,
    TK_SELF = 6, TK_CROSS = 7, TK_OTHER = 8, TK_XKV = 9, TK_DRAFT = 10, TK_HIST = 11,
    TK_PASS = 12, TK_N = 13
};

}  // namespace

struct wf_engine {
    wf_config c;
    Layout lay;
    int static_dev = -1;                    // device whose static workspace it holds, or -1
    int F_pad, pt_stride, page_elems;
    const uint16_t *tok_emb, *pos_emb, *lnf_g, *lnf_b;
    std::vector<LayerW> layers;
    std::vector<LayerW> dlayers;            // drafter blocks
    const uint16_t *w_hist, *mask_emb, *lnd_g, *lnd_b;
    uint16_t *taps;                         // fp16 [max_rows][n_taps*d], fragment-tiled
    int32_t *dam;                           // drafter argmax [max_rows]
    uint16_t *kv, *xkv;
    size_t kv_layer_elems, xkv_slot_elems, xkv_layer_elems;
    const int32_t *pt;
    char *ws;
    float *x;
    uint16_t *xs, *hs, *q;
    int32_t *tdepth;                         // tree verification: per row, its node's depth
    uint64_t *tanc;                          // and ancestor-or-self mask
    float2 *rdml, *rdpart;                   // anchor readout scratch
    int readout_layer = -1;                  // wf_set_readout: layer, or -1
    int32_t *readout_frame = nullptr;        // and its output [rows]
    float *part;
    int32_t *gcnt;
    float *xapart;
    int32_t *xacnt;
    float *lmmax;
    int32_t *lmidx;
    int32_t *reqL, *reqN, *len, *pend, *err;
    int32_t *rowkv;                          // per verify row: KV page * 16 + offset, or -1
    bool ln_fusion = true;                   // wf_set_option(WF_OPT_LN_FUSION)
    bool tall_gemm = true;                   // wf_set_option(WF_OPT_TALL_GEMM)
    bool persistent = false;                 // wf_set_option(WF_OPT_PERSISTENT)
    int n_cu = 0;                            // compute units: the pass kernel's grid
    int xa_chunks = 0;                       // wf_set_option(WF_OPT_XA_CHUNKS); 0: by batch
    int64_t pass_timeout_ticks = 50000000;   // wf_set_option(WF_OPT_PASS_TIMEOUT_US): 0.5 s
    // persistent pass buffers (see Layout)
    float *pxv = nullptr;
    uint16_t *plnv = nullptr, *pqv = nullptr, *pcqv = nullptr, *psav = nullptr, *pxav = nullptr,
             *phsv = nullptr;
    int32_t *pcnt = nullptr;
    LayerW *plw = nullptr;
    uint64_t *trace = nullptr;               // wf_set_trace: per task (start, end)
    size_t trace_tasks = 0;
    int last_pass_tasks = 0;
    int32_t last_sched[20] = {};             // total, per_layer, n_layers, ph_off[12], head_off[3]
    // optional per-kernel timing with HIP events
    bool timing = false;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_used = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> spans[TK_N];
};

namespace {

hipEvent_t next_event(wf_engine *e) {
    if (e->ev_used == e->ev_pool.size()) {
        // no system-scope fence at the timestamps: the events only bracket
        // kernels on this stream, and the fence would add to every interval
        hipEvent_t ev;
        if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        e->ev_pool.push_back(ev);
    }
    return e->ev_pool[e->ev_used++];
}

// Launch wrapper that optionally brackets the launch with events.
template <typename F>
wf_status timed(wf_engine *e, int kind, hipStream_t st, F &&launch) {
    hipEvent_t a = nullptr, b = nullptr;
    if (e->timing) {
        a = next_event(e);
        b = next_event(e);
        if (a) (void)hipEventRecord(a, st);
    }
    hipError_t err = launch();
    if (err != hipSuccess) return fail(WF_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    if (e->timing && a && b) {
        (void)hipEventRecord(b, st);
        e->spans[kind].push_back({a, b});
    }
    return WF_OK;
}

wf_status run_ln(wf_engine *e, int M, const uint16_t *g, const uint16_t *b, hipStream_t st) {
    LnArgs a{e->x, M, e->c.d_model, g, b, e->c.ln_eps, e->xs};
    return timed(e, TK_OTHER, st, [&] { return launch_layernorm(a, st); });
}

#define WF_TRY_(expr)                     \
    do {                                  \
        wf_status _s = (expr);            \
        if (_s != WF_OK) return _s;       \
    } while (0)

// Rows up to which the verify-pass GEMMs use the register-tiled kernel.
constexpr int kRegTiledMaxRows = 1024;
// Row range in which QKV and fc1 use the tall-block kernel (on MI355X, QKV
// at 288 rows: 31 us against 40; at 864 rows 49 against 54 in isolation).
constexpr int kTallMinRows = 97, kTallMaxRows = 1024;

// X W^T with role's epilogue. With lng/lnb the input is LN(x) of the
// residual stream: fused into the GEMM's prologue for one row tile, else the
// layer-norm kernel writes X (= xs) first.
wf_status run_gemm(wf_engine *e, int kind, int role, const uint16_t *X, int M,
                   int K, const uint16_t *W0, const uint16_t *W1, const uint16_t *W2, int seg_n,
                   int N, const EpiArgs &ea, hipStream_t st, const uint16_t *lng = nullptr,
                   const uint16_t *lnb = nullptr) {
    GemmArgs a{};
    a.X = X;
    a.W0 = W0;
    a.W1 = W1 ? W1 : W0;
    a.W2 = W2 ? W2 : W0;
    a.M = M;
    a.K = K;
    a.N = N;
    a.seg_n = seg_n;
    int ck, S;
    gemm_chunks(K, ck, S);
    a.S = S;
    a.ck = ck;
    a.part = e->part;
    a.cnt = e->gcnt;
    a.e = ea;
    const bool split_k_ok = role != ROLE_LM_HEAD && role != ROLE_XKV;
    const int mt_need = cdiv(M, 16);
    const bool rk = M <= kRegTiledMaxRows && gemm_rk_built(role, ck);
    // the prologue holds a row in registers: K <= 16 * 8 * LN_GPL. Not for
    // the LM head: its 811 column tiles would each recompute the statistics.
    const bool fuse_ln = lng && rk && mt_need <= 1 && e->ln_fusion && K <= 1280 &&
                         role != ROLE_LM_HEAD;
    if (lng && !fuse_ln) WF_TRY_(run_ln(e, M, lng, lnb, st));
    if (fuse_ln) {
        a.lnx = e->x;
        a.lng = lng;
        a.lnb = lnb;
        a.ln_eps = e->c.ln_eps;
    }
    if (e->tall_gemm && M >= kTallMinRows && M <= kTallMaxRows && gemm_tl_built(role, S, ck) &&
        !fuse_ln) {
        // tall blocks (tens of requests), 64-column tiles (from a sweep on
        // MI355X): the wide projections (QKV, fc1, the LM head, the
        // drafter's QKV and history K/V) 96 or 128 rows over the whole of K,
        // or 64 rows at two workgroups per CU when that gives more than 512
        // tiles; the d-wide ones (O, O_c, cross Q) 96 rows from 576 rows on
        // (below, the register-tiled kernel's 64 x 32 tiles win); fc2 (K =
        // 5120) 96 rows in 4 K groups
        int mbt = 6, P = 1;
        bool take = true;
        if (role == ROLE_QKV || role == ROLE_FC1 || role == ROLE_LM_HEAD ||
            role == ROLE_DRAFT_QKV || role == ROLE_HIST_KV) {
            // 96 or 128 rows: the fewer rounds of 256 workgroups times the
            // rows per workgroup (measured: 864 x 3840 128 rows 31.9 vs 39.5 us,
            // 864 x 5120 96 rows 43.2 vs 45.3 us); 64 rows two per CU
            // (measured: the LM head 288 x 51866 122 vs 155 us, 864 x 51866
            // 312 vs 417 us, 864 x 3840 30.7 us, 864 x 5120 38.4 vs 42.6 us;
            // at 288 x 3840 17.9 against 15.7 us with 96 rows)
            const int c6 = cdiv(cdiv(N, 64) * cdiv(M, 96), 256) * 6;
            const int c8 = cdiv(cdiv(N, 64) * cdiv(M, 128), 256) * 8;
            mbt = c8 < c6 ? 8 : 6;
            if (cdiv(N, 64) * cdiv(M, 64) > 512) mbt = 4;
        }
        else if (role == ROLE_OPROJ || role == ROLE_CROSS_Q) take = M >= 576;
        else P = 4;
        a.n_tiles = cdiv(N, 64);
        a.m_blocks = cdiv(M, 16 * mbt);
        a.n_groups = P;
        a.n_wg = a.n_tiles * a.m_blocks * P;
        // K-group sums: per (tile, K group) 4 waves x mb tiles of 1 KB
        if (P > 1 && (size_t)a.n_tiles * a.m_blocks * P * 4 * mbt * 1024 > e->lay.part_bytes)
            take = false;
        if (take) return timed(e, kind, st, [&] { return launch_gemm_tl(role, a, mbt, st); });
    }
    if (rk) {
        // Register-tiled kernel (tiles from a sweep on MI355X). One row tile:
        // 16 columns per workgroup and a 2-way K split (a weight-streaming
        // GEMV, latency-bound); the LM head 64 columns. Taller blocks: 32 x 64
        // tiles (the LM head 64 x 64: it reads the activations once per
        // column tile), and a K split only while the grid is small.
        int mb, nb, P = 1;
        // K-group sums go to scratch in the MFMA lane layout: whole tiles
        auto fits = [&](int P_) {
            return (size_t)P_ * cdiv(N, 16 * nb) * cdiv(M, 16 * mb) * (16 * mb) * (16 * nb) * 4 <=
                   e->lay.part_bytes;
        };
        if (mt_need <= 1) {
            // with the layer-norm prologue every workgroup recomputes the row
            // statistics: wide projections take 64-column tiles. K groups
            // (from sweeps at 9 rows on MI355X, weights from HBM): O and O_c
            // run unsplit (4.9 against 5.4 us in 2 groups), fc2 (K = 5120) in
            // 4 (7.9 against 8.2 in 2 and 10.7 unsplit), the layer-norm
            // consumers below 128 tiles in 2 (cross-Q unsplit: 9.1 against
            // 8.1 us in the pass)
            mb = 1;
            nb = (role == ROLE_LM_HEAD || (fuse_ln && N >= 4096)) ? 4 : 1;
            if (split_k_ok && S >= 2) {
                if (K >= 4096 && S >= 4 && fits(4)) P = 4;
                else if (fuse_ln && cdiv(N, 16 * nb) < 128 && fits(2)) P = 2;
            }
        } else if (mt_need <= 8) {
            // a few requests (2 to 8 row tiles): one-row-tile blocks of 16
            // columns up to 3 row tiles, then 32 x 32 tiles in 2 K groups
            // (from a sweep of verify steps at 18 / 36 / 72 rows on MI355X:
            // 2.42 / 2.60 / 3.17 ms against 3.47 / 3.26 / 3.61 with the taller
            // tiles below)
            mb = mt_need <= 3 ? 1 : 2;
            nb = role == ROLE_LM_HEAD ? 4 : (mt_need <= 3 ? 1 : 2);
            if (split_k_ok && mt_need > 3 && fits(2)) P = 2;
        } else {
            // the LM head reads the activations once per 64-column tile:
            // 96-row blocks from 6 row tiles on (1.2x faster at 288 rows);
            // the d-wide projections (O, O_c, cross Q, fc2) take 64 x 32
            // tiles from 8 row tiles on (1.15-1.3x at 288 rows)
            mb = role != ROLE_LM_HEAD || mt_need <= 2 ? 2 : (mt_need >= 6 ? 6 : 4);
            nb = 4;
            if (role != ROLE_LM_HEAD && mt_need >= 8 && N <= 2048) {
                mb = 4;
                nb = 2;
            }
            if (split_k_ok) {
                while (P < S && cdiv(N, 16 * nb) * cdiv(M, 16 * mb) * P < 128 && fits(2 * P))
                    P *= 2;
            }
        }
        a.n_tiles = cdiv(N, 16 * nb);
        a.m_blocks = cdiv(M, 16 * mb);
        a.n_groups = P;
        a.n_wg = a.n_tiles * a.m_blocks * a.n_groups;
        return timed(e, kind, st, [&] { return launch_gemm_rk(role, a, mb, nb, st); });
    }
    a.n_tiles = cdiv(N, 64);
    // LDS-staged kernel for tall blocks (prefill, the cross K/V): row blocks
    // of up to 32 rows, the tallest that still gives about 256 workgroups; the
    // row blocks of one weight tile share it through L2.
    int mb = 2;
    while (mb > 1 && a.n_tiles * cdiv(M, 16 * mb) < 256) mb >>= 1;
    while (mb > 1 && (mb >> 1) >= mt_need) mb >>= 1;
    a.m_blocks = cdiv(M, 16 * mb);
    a.n_groups = 1;
    a.n_wg = a.n_tiles * a.m_blocks;
    return timed(e, kind, st, [&] { return launch_gemm(role, a, mb, st); });
}

#define WF_TRY(expr)                      \
    do {                                  \
        wf_status _s = (expr);            \
        if (_s != WF_OK) return _s;       \
    } while (0)

}  // namespace

// Error message setter shared with the encoder's host code.
namespace wf {
wf_status set_error(wf_status s, const char *msg) { return fail(s, "%s", msg); }
}  // namespace wf

// The workspace of engines made by wf_create_static: one array per device,
// resident from the code object's load until the process ends. In host code
// the name is only a stand-in; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[WF_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void *g_static_ptr[kMaxDevices];      // per device: the address of scratch there
bool g_static_held[kMaxDevices];      // per device: an engine owns the array
}  // namespace

extern "C" {

size_t wf_kv_pool_bytes(const wf_config *c) {
    if (!config_ok(c, nullptr)) return 0;
    return (size_t)all_layers(c) * c->n_pages * 2 * c->n_heads * c->page_size * c->head_dim * 2;
}

size_t wf_xkv_pool_bytes(const wf_config *c) {
    if (!config_ok(c, nullptr)) return 0;
    return (size_t)c->max_batch * all_layers(c) * 2 * c->n_heads * f_pad_of(c) * c->head_dim * 2;
}

size_t wf_workspace_bytes(const wf_config *c) {
    if (!config_ok(c, nullptr)) return 0;
    return layout_of(c).total;
}

const char *wf_last_error(void) { return g_err; }

wf_status wf_create(const wf_config *cfg, const wf_weights *w, void *kv_pool, size_t kv_bytes,
                    void *xkv_pool, size_t xkv_bytes, const int32_t *d_page_table,
                    void *workspace, size_t ws_bytes, wf_engine **out) {
    if (!out) return fail(WF_EINVAL, "out is null");
    *out = nullptr;
    std::string why;
    if (!config_ok(cfg, &why)) return fail(WF_ESHAPE, "bad config: %s", why.c_str());
    if (!w || !w->tok_emb || !w->pos_emb || !w->lnf_g || !w->lnf_b || !w->layers)
        return fail(WF_EINVAL, "null weight pointer");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const wf_layer_weights &L = w->layers[l];
        const void *ps[] = {L.ln1_g, L.ln1_b, L.wq, L.bq, L.wk, L.wv, L.bv, L.wo, L.bo,
                            L.ln2_g, L.ln2_b, L.wqc, L.bqc, L.wkc, L.wvc, L.bvc, L.woc, L.boc,
                            L.ln3_g, L.ln3_b, L.w1, L.b1, L.w2, L.b2};
        for (const void *p : ps)
            if (!p) return fail(WF_EINVAL, "null weight pointer in layer %d", l);
    }
    if (cfg->drafter_layers > 0) {
        const wf_drafter_weights *dw = w->drafter;
        if (!dw || !dw->layers || !dw->w_hist || !dw->mask_emb || !dw->lnd_g || !dw->lnd_b)
            return fail(WF_EINVAL, "null drafter weight pointer");
        for (int l = 0; l < cfg->drafter_layers; ++l) {
            const wf_layer_weights &L = dw->layers[l];
            const void *ps[] = {L.ln1_g, L.ln1_b, L.wq, L.bq, L.wk, L.wv, L.bv, L.wo, L.bo,
                                L.ln2_g, L.ln2_b, L.wqc, L.bqc, L.wkc, L.wvc, L.bvc, L.woc, L.boc,
                                L.ln3_g, L.ln3_b, L.w1, L.b1, L.w2, L.b2};
            for (const void *p : ps)
                if (!p) return fail(WF_EINVAL, "null weight pointer in drafter layer %d", l);
        }
    }
    if (!kv_pool || !xkv_pool || !d_page_table || !workspace)
        return fail(WF_EINVAL, "null pool, page table or workspace");
    if (kv_bytes < wf_kv_pool_bytes(cfg)) return fail(WF_ECAPACITY, "kv_pool too small");
    if (xkv_bytes < wf_xkv_pool_bytes(cfg)) return fail(WF_ECAPACITY, "xkv_pool too small");
    if (ws_bytes < wf_workspace_bytes(cfg)) return fail(WF_ECAPACITY, "workspace too small");

    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(WF_EDEVICE, "no HIP device");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(WF_EDEVICE, "device is %s, not gfx950", prop.gcnArchName);

    wf_engine *e = new wf_engine();
    e->c = *cfg;
    e->lay = layout_of(cfg);
    e->n_cu = prop.multiProcessorCount;
    e->F_pad = f_pad_of(cfg);
    e->pt_stride = cfg->n_ctx / cfg->page_size;
    e->page_elems = 2 * cfg->n_heads * cfg->page_size * cfg->head_dim;
    e->tok_emb = (const uint16_t *)w->tok_emb;
    e->pos_emb = (const uint16_t *)w->pos_emb;
    e->lnf_g = (const uint16_t *)w->lnf_g;
    e->lnf_b = (const uint16_t *)w->lnf_b;
    auto conv = [](const wf_layer_weights &s) {
        return LayerW{(const uint16_t *)s.ln1_g, (const uint16_t *)s.ln1_b, (const uint16_t *)s.wq,
                   (const uint16_t *)s.bq,    (const uint16_t *)s.wk,    (const uint16_t *)s.wv,
                   (const uint16_t *)s.bv,    (const uint16_t *)s.wo,    (const uint16_t *)s.bo,
                   (const uint16_t *)s.ln2_g, (const uint16_t *)s.ln2_b, (const uint16_t *)s.wqc,
                   (const uint16_t *)s.bqc,   (const uint16_t *)s.wkc,   (const uint16_t *)s.wvc,
                   (const uint16_t *)s.bvc,   (const uint16_t *)s.woc,   (const uint16_t *)s.boc,
                   (const uint16_t *)s.ln3_g, (const uint16_t *)s.ln3_b, (const uint16_t *)s.w1,
                   (const uint16_t *)s.b1,    (const uint16_t *)s.w2,    (const uint16_t *)s.b2};
    };
    e->layers.resize(cfg->n_layers);
    for (int l = 0; l < cfg->n_layers; ++l) e->layers[l] = conv(w->layers[l]);
    e->w_hist = e->mask_emb = e->lnd_g = e->lnd_b = nullptr;
    if (cfg->drafter_layers > 0) {
        const wf_drafter_weights *dw = w->drafter;
        e->dlayers.resize(cfg->drafter_layers);
        for (int l = 0; l < cfg->drafter_layers; ++l) e->dlayers[l] = conv(dw->layers[l]);
        e->w_hist = (const uint16_t *)dw->w_hist;
        e->mask_emb = (const uint16_t *)dw->mask_emb;
        e->lnd_g = (const uint16_t *)dw->lnd_g;
        e->lnd_b = (const uint16_t *)dw->lnd_b;
    }
    e->kv = (uint16_t *)kv_pool;
    e->xkv = (uint16_t *)xkv_pool;
    e->kv_layer_elems = (size_t)cfg->n_pages * e->page_elems;
    e->xkv_layer_elems = (size_t)2 * cfg->n_heads * e->F_pad * cfg->head_dim;
    e->xkv_slot_elems = (size_t)all_layers(cfg) * e->xkv_layer_elems;
    e->pt = d_page_table;
    char *ws = (char *)workspace;
    const Layout &L = e->lay;
    e->ws = ws;
    e->x = (float *)(ws + L.x);
    e->xs = (uint16_t *)(ws + L.xs);
    e->hs = (uint16_t *)(ws + L.hs);
    e->q = (uint16_t *)(ws + L.q);
    e->tdepth = (int32_t *)(ws + L.tdepth);
    e->tanc = (uint64_t *)(ws + L.tanc);
    e->rdml = (float2 *)(ws + L.rdml);
    e->rdpart = (float2 *)(ws + L.rdpart);
    e->part = (float *)(ws + L.part);
    e->gcnt = (int32_t *)(ws + L.gcnt);
    e->xapart = (float *)(ws + L.xapart);
    e->xacnt = (int32_t *)(ws + L.xacnt);
    e->lmmax = (float *)(ws + L.lmmax);
    e->lmidx = (int32_t *)(ws + L.lmidx);
    e->reqL = (int32_t *)(ws + L.reqL);
    e->reqN = (int32_t *)(ws + L.reqN);
    e->len = (int32_t *)(ws + L.len);
    e->pend = (int32_t *)(ws + L.pend);
    e->err = (int32_t *)(ws + L.err);
    e->rowkv = (int32_t *)(ws + L.rowkv);
    e->taps = (uint16_t *)(ws + L.taps);
    e->dam = (int32_t *)(ws + L.dam);
    if (L.pass_rows > 0) {
        e->pxv = (float *)(ws + L.pxv);
        e->plnv = (uint16_t *)(ws + L.plnv);
        e->pqv = (uint16_t *)(ws + L.pqv);
        e->pcqv = (uint16_t *)(ws + L.pcqv);
        e->psav = (uint16_t *)(ws + L.psav);
        e->pxav = (uint16_t *)(ws + L.pxav);
        e->phsv = (uint16_t *)(ws + L.phsv);
        e->pcnt = (int32_t *)(ws + L.pcnt);
        e->plw = (LayerW *)(ws + L.plw);
    }
    if (hipMemset(workspace, 0, L.total) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        delete e;
        return fail(WF_EHIP, "clearing the workspace failed");
    }
    if (L.pass_rows > 0 &&
        (hipMemcpy(e->plw, e->layers.data(), e->layers.size() * sizeof(LayerW),
                   hipMemcpyHostToDevice) != hipSuccess ||
         hipDeviceSynchronize() != hipSuccess)) {
        delete e;
        return fail(WF_EHIP, "copying the layer weight table failed");
    }
    *out = e;
    return WF_OK;
}

void wf_destroy(wf_engine *e) {
    if (!e) return;
    for (hipEvent_t ev : e->ev_pool) hipEventDestroy(ev);
    if (e->static_dev >= 0) {
        std::lock_guard<std::mutex> g(g_static_mu);
        g_static_held[e->static_dev] = false;
    }
    delete e;
}

wf_status wf_create_static(const wf_config *cfg, const wf_weights *w, void *kv_pool,
                           size_t kv_bytes, void *xkv_pool, size_t xkv_bytes,
                           const int32_t *d_page_table, wf_engine **out) {
    if (!out) return fail(WF_EINVAL, "out is null");
    *out = nullptr;
    std::string why;
    if (!config_ok(cfg, &why)) return fail(WF_ESHAPE, "bad config: %s", why.c_str());
    const size_t need = wf_workspace_bytes(cfg);
    if (need > WF_STATIC_WORKSPACE_BYTES)
        return fail(WF_ECAPACITY,
                    "this configuration needs a %zu-byte workspace; the static one holds %zu "
                    "(lower max_rows or max_batch, or use wf_create)",
                    need, (size_t)WF_STATIC_WORKSPACE_BYTES);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(WF_EDEVICE, "no HIP device");
    if (dev < 0 || dev >= kMaxDevices) return fail(WF_EDEVICE, "device %d out of range", dev);
    std::lock_guard<std::mutex> g(g_static_mu);
    if (g_static_held[dev])
        return fail(WF_ESTATE, "an engine on device %d already holds the static workspace", dev);
    if (!g_static_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (r != hipSuccess || !ptr)
            return fail(WF_EHIP, "hipGetSymbolAddress of the static workspace failed: %s",
                        hipGetErrorString(r));
        g_static_ptr[dev] = ptr;
    }
    // wf_create checks everything else and clears the array before use
    const wf_status st = wf_create(cfg, w, kv_pool, kv_bytes, xkv_pool, xkv_bytes, d_page_table,
                                   g_static_ptr[dev], WF_STATIC_WORKSPACE_BYTES, out);
    if (st != WF_OK) return st;
    (*out)->static_dev = dev;
    g_static_held[dev] = true;
    return WF_OK;
}

wf_status wf_reset(wf_engine *e, int32_t n, const int32_t *d_slots, void *stream) {
    if (!e || !d_slots) return fail(WF_EINVAL, "null argument");
    if (n < 1 || n > e->c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    hipStream_t st = (hipStream_t)stream;
    return timed(e, TK_OTHER, st,
                 [&] {
                     return launch_reset(n, e->c.max_batch, d_slots, e->len, e->pend, e->err, st);
                 });
}

wf_status wf_encode_kv(wf_engine *e, int32_t n, const int32_t *d_slots, const void *d_enc,
                       void *stream) {
    if (!e || !d_slots || !d_enc) return fail(WF_EINVAL, "null argument");
    if (n < 1 || n > e->c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    const wf_config &c = e->c;
    const long long M = (long long)n * c.n_frames;
    if (M > 0x7fffffffLL / 2) return fail(WF_ECAPACITY, "too many frames");
    hipStream_t st = (hipStream_t)stream;
    for (int l = 0; l < all_layers(&c); ++l) {
        const LayerW &w = l < c.n_layers ? e->layers[l] : e->dlayers[l - c.n_layers];
        WF_TRY(timed(e, TK_XKV, st, [&] {
            return launch_xkv_dense((const uint16_t *)d_enc, (int)M, c.d_model, w.wkc, w.wvc, w.bvc,
                                    e->xkv, (long long)e->xkv_slot_elems,
                                    (long long)l * (long long)e->xkv_layer_elems, d_slots,
                                    c.n_frames, e->F_pad, c.n_heads, c.head_dim, c.max_batch, st);
        }));
    }
    return WF_OK;
}

namespace {

// Frame chunking of the cross-attention for n requests and mt row tiles.
void cross_plan(const wf_engine *e, int n, int mt, int &cf, int &G, int &spw) {
    const wf_config &c = e->c;
    const int H = c.n_heads, hd = c.head_dim;
    cross_chunks(n, H, c.n_frames, e->xa_chunks, cf, G, spw);
    const size_t rowbytes = (size_t)16 * (hd + 4) * 4;
    while (G > 1 && (size_t)n * H * mt * G * rowbytes > e->lay.xapart_bytes) {
        // long prefill blocks: fewer, longer chunks so the group partials fit
        G >>= 1;
        spw = cdiv(cdiv(cdiv(c.n_frames, 32), 4 * G), kXaRing) * kXaRing;
        cf = spw * 32;
    }
}

struct Pass {
    int n, T, M, mt, cf, G, spw;
    const int32_t *slots;
    int kind;   // -1: per-kernel kinds; else every launch is timed under this kind
};

int K_(const Pass &p, int k) { return p.kind < 0 ? k : p.kind; }

// Self-attention output projection, cross-attention sublayer and MLP sublayer
// of one block (target layer or drafter layer); xkv_layer indexes the
// write-once pool.
wf_status run_out_cross_mlp(wf_engine *e, const LayerW &w, int xkv_layer, const Pass &p,
                            hipStream_t st) {
    const wf_config &c = e->c;
    const int M = p.M, d = c.d_model, H = c.n_heads, hd = c.head_dim;
    EpiArgs ra{};
    ra.b0 = w.bo;
    ra.x = e->x;
    ra.x_in = e->x;
    WF_TRY(run_gemm(e, K_(p, TK_OPROJ), ROLE_OPROJ, e->xs, M, d, w.wo, nullptr, nullptr, d, d, ra,
                    st));
    EpiArgs fa{};
    fa.b0 = w.bqc;
    fa.out = e->q;
    WF_TRY(run_gemm(e, K_(p, TK_QC), ROLE_CROSS_Q, e->xs, M, d, w.wqc, nullptr, nullptr, d, d, fa,
                    st, w.ln2_g, w.ln2_b));
    CrossAttnArgs ca{};
    ca.q = e->q;
    ca.xkv = e->xkv;
    ca.slot_stride = (int64_t)e->xkv_slot_elems;
    ca.layer_off = (int64_t)xkv_layer * e->xkv_layer_elems;
    ca.slots = p.slots;
    ca.req_ntok = e->reqN;
    ca.n = p.n;
    ca.T = p.T;
    ca.H = H;
    ca.d = d;
    ca.F = c.n_frames;
    ca.F_pad = e->F_pad;
    ca.mt = p.mt;
    ca.G = p.G;
    ca.cf = p.cf;
    ca.spw = p.spw;
    ca.n_items = p.n * H * p.mt * p.G;
    ca.scale = 1.0f / std::sqrt((float)hd);
    ca.part = e->xapart;
    ca.cnt = e->xacnt;
    ca.out = e->xs;
    WF_TRY(timed(e, K_(p, TK_CROSS), st, [&] { return launch_cross_attn(ca, hd, st); }));
    EpiArgs oa{};
    oa.b0 = w.boc;
    oa.x = e->x;
    oa.x_in = e->x;
    WF_TRY(run_gemm(e, K_(p, TK_OPROJ), ROLE_OPROJ, e->xs, M, d, w.woc, nullptr, nullptr, d, d, oa,
                    st));
    EpiArgs ga{};
    ga.b0 = w.b1;
    ga.out = e->hs;
    WF_TRY(run_gemm(e, K_(p, TK_FC1), ROLE_FC1, e->xs, M, d, w.w1, nullptr, nullptr, c.d_ffn,
                    c.d_ffn, ga, st, w.ln3_g, w.ln3_b));
    EpiArgs f2{};
    f2.b0 = w.b2;
    f2.x = e->x;
    f2.x_in = e->x;
    WF_TRY(run_gemm(e, K_(p, TK_FC2), ROLE_FC2, e->hs, M, c.d_ffn, w.w2, nullptr, nullptr, d, d, f2,
                    st));
    return WF_OK;
}

// Final layer norm, tied LM head with its argmax epilogue, per-row merge.
wf_status run_head(wf_engine *e, const uint16_t *g, const uint16_t *b, const Pass &p,
                   float *d_logits, int32_t *d_argmax, hipStream_t st) {
    const wf_config &c = e->c;
    EpiArgs la{};
    la.logits = d_logits;
    la.tile_max = e->lmmax;
    la.tile_idx = e->lmidx;
    la.ld = e->lay.n_vtiles;
    WF_TRY(run_gemm(e, K_(p, TK_LMHEAD), ROLE_LM_HEAD, e->xs, p.M, c.d_model, e->tok_emb, nullptr,
                    nullptr, c.vocab, c.vocab, la, st, g, b));
    LmReduceArgs lr{e->lmmax, e->lmidx, e->lay.n_vtiles, e->lay.n_vtiles, p.M, p.T, p.slots, e->reqN,
                    e->err, d_argmax};
    return timed(e, K_(p, TK_OTHER), st, [&] { return launch_lm_reduce(lr, st); });
}

// RoPE of the drafter's projections in the fp32 temporary and append of
// keys/values at positions L+i (rows i < req_ntok) of drafter layer dl.
wf_status run_rope_append(wf_engine *e, int dl, const Pass &p, int ncols, int q_off, int k_off,
                          int v_off, int kind, hipStream_t st) {
    const wf_config &c = e->c;
    RopeArgs ra{};
    ra.tmp = reinterpret_cast<const float *>(e->hs);
    ra.ncols = ncols;
    ra.q_off = q_off;
    ra.k_off = k_off;
    ra.v_off = v_off;
    ra.M = p.M;
    ra.T = p.T;
    ra.H = c.n_heads;
    ra.hd = c.head_dim;
    ra.d = c.d_model;
    ra.slots = p.slots;
    ra.req_L = e->reqL;
    ra.req_ntok = e->reqN;
    ra.page_table = e->pt;
    ra.pt_stride = e->pt_stride;
    ra.page_elems = e->page_elems;
    ra.kv_layer = e->kv + (size_t)(c.n_layers + dl) * e->kv_layer_elems;
    ra.q_out = e->q;
    return timed(e, kind, st, [&] { return launch_rope_append(ra, st); });
}

int grid_of(const wf_engine *e) { return e->n_cu > 0 ? e->n_cu : 256; }

// Drafter history of the rows just written to the cache: h = W_h taps (into
// the residual buffer, free after the head), then per drafter layer
// k = RoPE(W_k LN1(h)), v = W_v LN1(h) + b_v into its pages.
wf_status run_history(wf_engine *e, const Pass &p, hipStream_t st) {
    const wf_config &c = e->c;
    if (c.drafter_layers <= 0) return WF_OK;
    const int M = p.M, d = c.d_model;
    EpiArgs ha{};
    ha.out32 = e->x;
    WF_TRY(run_gemm(e, TK_HIST, ROLE_HIST, e->taps, M, c.n_taps * d, e->w_hist, nullptr,
                    nullptr, d, d, ha, st));
    for (int dl = 0; dl < c.drafter_layers; ++dl) {
        const LayerW &w = e->dlayers[dl];
        EpiArgs ka{};
        ka.b1 = w.bv;
        ka.out32 = reinterpret_cast<float *>(e->hs);
        WF_TRY(run_gemm(e, TK_HIST, ROLE_HIST_KV, e->xs, M, d, w.wk, w.wv, nullptr, d, 2 * d, ka,
                        st, w.ln1_g, w.ln1_b));
        WF_TRY(run_rope_append(e, dl, p, 2 * d, -1, 0, d, TK_HIST, st));
    }
    return WF_OK;
}

// The persistent pass (k_pass.hip): every layer, the final layer norm and the
// LM head with its argmax in one launch after prepare and embed. Returns
// WF_ESTATE when this pass cannot take it (the caller then runs the
// multi-kernel path).
wf_status run_pass(wf_engine *e, const Pass &p, const int32_t *d_tokens, const int32_t *d_n_tok,
                   int32_t *d_argmax, float *d_logits, hipStream_t st) {
    const wf_config &c = e->c;
    const int n = p.n, T = p.T, M = p.M, d = c.d_model, H = c.n_heads, NL = c.n_layers;
    const int cl = pass_class_of_rows(M);
    PassArgs a{};
    a.n = n;
    a.T = T;
    a.M = M;
    a.RT = cdiv(M, 16);
    a.mt = p.mt;
    a.max_batch = c.max_batch;
    a.n_layers = NL;
    a.d = d;
    a.H = H;
    a.hd = c.head_dim;
    a.F = c.d_ffn;
    a.V = c.vocab;
    a.ln_eps = c.ln_eps;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    // tilings: column tiles, row blocks and K groups of every projection
    const int Ns[PG_N] = {3 * d, d, d, d, c.d_ffn, d, c.vocab};
    for (int g = 0; g < PG_N; ++g) {
        int bm = 0, bn = 0, P = 0;
        pass_tiling(cl, g, bm, bn, P);
        if (bm == 0) return WF_ESTATE;
        PassGemmCfg &t = a.g[g];
        t.n_tiles = cdiv(Ns[g], bn);
        t.m_blocks = cdiv(M, bm);
        t.n_groups = P;
        t.n_tasks = cdiv(t.n_tiles, 8) * 8 * t.m_blocks * P;
        if (g == PG_LMH && bn != 64) return WF_ESTATE;
        if (P > 1) {
            // K-group sums: per (tile, row block) P groups of whole MFMA tiles
            const size_t bytes = (size_t)t.n_tiles * t.m_blocks * P * bm * bn * 4;
            if (bytes > e->lay.part_bytes) return WF_ESTATE;
        }
    }
    WF_TRY(timed(e, TK_OTHER, st, [&] {
        PrepareArgs pa{n, T, c.vocab, c.n_ctx, c.n_pages, e->pt_stride, c.page_size, c.max_batch,
                       p.slots, d_tokens, d_n_tok, e->pt, e->len, e->pend, e->err, e->reqL,
                       e->reqN, nullptr, e->tdepth, e->tanc};
        return launch_prepare(pa, st);
    }));
    const int n_cnt = (NL * PH_PER_LAYER + 2) * 64 + 64;
    WF_TRY(timed(e, TK_OTHER, st, [&] { return launch_fill_i32(e->pcnt, n_cnt, 0, st); }));
    const size_t Pm = (size_t)e->lay.pass_rows;
    WF_TRY(timed(e, TK_OTHER, st, [&] {
        EmbedArgs ema{M,        T,      d,       c.vocab, c.n_ctx, d_tokens, e->reqL,
                      e->tok_emb, e->pos_emb, e->pxv, e->reqN, p.slots, e->pt, e->pt_stride,
                      e->rowkv, nullptr};
        return launch_embed(ema, st);
    }));
    a.lw = e->plw;
    a.tok_emb = e->tok_emb;
    a.lnf_g = e->lnf_g;
    a.lnf_b = e->lnf_b;
    a.slots = p.slots;
    a.req_L = e->reqL;
    a.req_ntok = e->reqN;
    a.row_kv = e->rowkv;
    a.page_table = e->pt;
    a.slot_err = e->err;
    a.pt_stride = e->pt_stride;
    a.page_elems = e->page_elems;
    a.kv = e->kv;
    a.kv_layer_elems = (int64_t)e->kv_layer_elems;
    a.xkv = e->xkv;
    a.xkv_slot_elems = (int64_t)e->xkv_slot_elems;
    a.xkv_layer_elems = (int64_t)e->xkv_layer_elems;
    a.n_frames = c.n_frames;
    a.F_pad = e->F_pad;
    a.xa_G = p.G;
    a.xa_cf = p.cf;
    a.xa_spw = p.spw;
    a.xv = e->pxv;
    a.lnv = e->plnv;
    a.qv = e->pqv;
    a.cqv = e->pcqv;
    a.sav = e->psav;
    a.xav = e->pxav;
    a.hsv = e->phsv;
    a.x_stride = (int64_t)(Pm * d);
    a.act_stride = (int64_t)(Pm * d);
    a.q_stride = (int64_t)(Pm * d);
    a.hs_stride = (int64_t)(Pm * c.d_ffn);
    a.part = e->part;
    a.gcnt = e->gcnt;
    a.xapart = e->xapart;
    a.xacnt = e->xacnt;
    a.logits = d_logits;
    a.tile_max = e->lmmax;
    a.tile_idx = e->lmidx;
    a.ld = e->lay.n_vtiles;
    a.n_vtiles = e->lay.n_vtiles;
    a.argmax = d_argmax;
    a.taps = e->taps;
    a.n_taps = c.drafter_layers > 0 ? c.n_taps : 0;
    for (int j = 0; j < 8; ++j) a.tap_layers[j] = c.tap_layers[j];
    a.cnt = e->pcnt;
    a.abort_flag = e->pcnt + (NL * PH_PER_LAYER + 2) * 64;
    const int n_ln = cdiv(a.RT, 2);
    a.sa_items = n * H * p.mt;
    a.xa_items = n * H * p.mt * p.G;
    const int per[PH_PER_LAYER] = {n_ln,
                                   a.g[PG_QKV].n_tasks,
                                   cdiv(a.sa_items, 2),
                                   a.g[PG_O].n_tasks,
                                   n_ln,
                                   a.g[PG_CQ].n_tasks,
                                   cdiv(a.xa_items, 2),
                                   a.g[PG_OC].n_tasks,
                                   n_ln,
                                   a.g[PG_FC1].n_tasks,
                                   a.g[PG_FC2].n_tasks};
    int off = 0;
    for (int k = 0; k < PH_PER_LAYER; ++k) {
        a.ph_off[k] = off;
        off += per[k];
    }
    a.ph_off[PH_PER_LAYER] = off;
    a.per_layer = off;
    a.head_off[0] = 0;
    a.head_off[1] = n_ln;
    a.head_off[2] = n_ln + a.g[PG_LMH].n_tasks;
    a.total = NL * a.per_layer + a.head_off[2];
    a.timeout_ticks = e->pass_timeout_ticks;   // 100 MHz clock; a pass takes milliseconds
    a.trace = (e->trace && (size_t)a.total <= e->trace_tasks) ? e->trace : nullptr;
    e->last_pass_tasks = a.total;
    e->last_sched[0] = a.total;
    e->last_sched[1] = a.per_layer;
    e->last_sched[2] = NL;
    for (int k = 0; k <= PH_PER_LAYER; ++k) e->last_sched[3 + k] = a.ph_off[k];
    for (int k = 0; k < 3; ++k) e->last_sched[15 + k] = a.head_off[k];
    e->last_sched[18] = grid_of(e);
    const int grid = grid_of(e);
    WF_TRY(timed(e, TK_PASS, st, [&] { return launch_pass(a, cl, grid, st); }));
    return run_history(e, p, st);
}

}  // namespace

// One verify pass; d_parents (nullable) makes the block a token tree.
static wf_status verify_pass(wf_engine *e, int32_t n, const int32_t *d_slots,
                             const int32_t *d_tokens, int32_t T, const int32_t *d_parents,
                             const int32_t *d_n_tok, int32_t *d_argmax, float *d_logits,
                             void *stream) {
    if (!e || !d_slots || !d_tokens || !d_n_tok || !d_argmax)
        return fail(WF_EINVAL, "null argument");
    const wf_config &c = e->c;
    if (n < 1 || n > c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    if (T < 1 || T > c.n_ctx) return fail(WF_EINVAL, "T outside [1, n_ctx]");
    if ((long long)n * T > c.max_rows) return fail(WF_ECAPACITY, "n*T exceeds max_rows");
    hipStream_t st = (hipStream_t)stream;
    const int M = n * T, d = c.d_model, H = c.n_heads, hd = c.head_dim;
    Pass p{n, T, M, cdiv(T, 16), 0, 0, 0, d_slots, -1};
    cross_plan(e, n, p.mt, p.cf, p.G, p.spw);

    if (e->persistent && e->lay.pass_rows > 0 && !d_parents && e->readout_layer < 0 && T <= 64 &&
        M <= e->lay.pass_rows) {
        const wf_status s = run_pass(e, p, d_tokens, d_n_tok, d_argmax, d_logits, st);
        if (s != WF_ESTATE) return s;   // WF_ESTATE: this shape takes the multi-kernel path
    }

    PrepareArgs pa{n, T, c.vocab, c.n_ctx, c.n_pages, e->pt_stride, c.page_size, c.max_batch,
                   d_slots, d_tokens, d_n_tok, e->pt, e->len, e->pend, e->err, e->reqL, e->reqN,
                   d_parents, e->tdepth, e->tanc};
    WF_TRY(timed(e, TK_OTHER, st, [&] { return launch_prepare(pa, st); }));
    EmbedArgs ema{M,      T,      d,        c.vocab,         c.n_ctx, d_tokens, e->reqL,
                  e->tok_emb, e->pos_emb, e->x, e->reqN, d_slots, e->pt, e->pt_stride, e->rowkv,
                  d_parents ? e->tdepth : nullptr};
    WF_TRY(timed(e, TK_OTHER, st, [&] { return launch_embed(ema, st); }));

    for (int l = 0; l < c.n_layers; ++l) {
        const LayerW &w = e->layers[l];
        uint16_t *kvl = e->kv + (size_t)l * e->kv_layer_elems;
        // self-attention sublayer: QKV with the K/V append, causal attention
        EpiArgs qa{};
        qa.b0 = w.bq;
        qa.b2 = w.bv;
        qa.out = e->q;
        qa.kv_layer = kvl;
        qa.page_table = e->pt;
        qa.pt_stride = e->pt_stride;
        qa.slots = d_slots;
        qa.req_L = e->reqL;
        qa.req_ntok = e->reqN;
        qa.T = T;
        qa.H = H;
        qa.hd = hd;
        qa.page_elems = e->page_elems;
        qa.row_kv = e->rowkv;
        WF_TRY(run_gemm(e, TK_QKV, ROLE_QKV, e->xs, M, d, w.wq, w.wk, w.wv, d, 3 * d, qa, st,
                        w.ln1_g, w.ln1_b));
        SelfAttnArgs sa{e->q, kvl, e->pt, d_slots, e->reqL, e->reqN, e->pt_stride,
                        e->page_elems, n, T, H, d, 1, 1.0f / std::sqrt((float)hd), e->xs,
                        d_parents ? e->tanc : nullptr};
        WF_TRY(timed(e, TK_SELF, st, [&] { return launch_self_attn(sa, hd, p.mt, st); }));
        WF_TRY(run_out_cross_mlp(e, w, l, p, st));
        if (l == e->readout_layer) {
            // the layer's cross queries are still in q
            ReadoutArgs ra{e->q, e->xkv, (int64_t)e->xkv_slot_elems,
                           (int64_t)(l * e->xkv_layer_elems), d_slots, e->reqN, n, T, H, hd, d,
                           c.n_frames, e->F_pad, c.max_batch, cdiv(c.n_frames, 128),
                           1.4426950408889634f / std::sqrt((float)hd), e->rdml, e->rdpart,
                           e->readout_frame};
            WF_TRY(timed(e, TK_OTHER, st, [&] { return launch_readout(ra, p.mt, st); }));
        }
        // history taps for the drafter (residual stream after this block)
        for (int j = 0; j < (c.drafter_layers > 0 ? c.n_taps : 0); ++j) {
            if (c.tap_layers[j] != l) continue;
            TapArgs ta{e->x, M, d, j, c.n_taps, e->taps};
            WF_TRY(timed(e, TK_HIST, st, [&] { return launch_tap(ta, st); }));
        }
    }
    WF_TRY(run_head(e, e->lnf_g, e->lnf_b, p, d_logits, d_argmax, st));
    return run_history(e, p, st);
}

wf_status wf_verify_block(wf_engine *e, int32_t n, const int32_t *d_slots,
                          const int32_t *d_tokens, int32_t T, const int32_t *d_n_tok,
                          int32_t *d_argmax, float *d_logits, void *stream) {
    return verify_pass(e, n, d_slots, d_tokens, T, nullptr, d_n_tok, d_argmax, d_logits, stream);
}

wf_status wf_set_readout(wf_engine *e, int32_t layer, int32_t *d_frame) {
    if (!e) return fail(WF_EINVAL, "null engine");
    if (layer >= e->c.n_layers) return fail(WF_EINVAL, "layer outside the decoder");
    if (layer >= 0 && !d_frame) return fail(WF_EINVAL, "null output");
    e->readout_layer = layer < 0 ? -1 : layer;
    e->readout_frame = layer < 0 ? nullptr : d_frame;
    return WF_OK;
}

wf_status wf_verify_tree(wf_engine *e, int32_t n, const int32_t *d_slots,
                         const int32_t *d_tokens, int32_t T, const int32_t *d_parents,
                         const int32_t *d_n_tok, int32_t *d_argmax, float *d_logits,
                         void *stream) {
    if (!e || !d_parents) return fail(WF_EINVAL, "null argument");
    if (T < 1 || T > 64) return fail(WF_EINVAL, "a tree has 1 to 64 nodes");
    if (e->c.drafter_layers > 0)
        return fail(WF_ESTATE, "tree verification does not feed the drafter's history");
    return verify_pass(e, n, d_slots, d_tokens, T, d_parents, d_n_tok, d_argmax, d_logits,
                       stream);
}

wf_status wf_accept_tree(wf_engine *e, int32_t n, const int32_t *d_tokens, int32_t T,
                         const int32_t *d_parents, const int32_t *d_n_tok,
                         const int32_t *d_budget, const int32_t *d_argmax, int32_t *d_path,
                         int32_t *d_n_acc, int32_t *d_next_token, int32_t *d_n_emit,
                         int32_t *d_done, void *stream) {
    if (!e || !d_tokens || !d_parents || !d_n_tok || !d_budget || !d_argmax || !d_path ||
        !d_n_acc || !d_next_token || !d_n_emit || !d_done)
        return fail(WF_EINVAL, "null argument");
    if (n < 1 || n > e->c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    if (T < 1 || T > 64) return fail(WF_EINVAL, "a tree has 1 to 64 nodes");
    TreeAcceptArgs a{n, T, e->c.eos_id, d_tokens, d_parents, d_n_tok, d_budget, d_argmax,
                     d_path, d_n_acc, d_next_token, d_n_emit, d_done};
    hipStream_t st = (hipStream_t)stream;
    return timed(e, TK_OTHER, st, [&] { return launch_accept_tree(a, st); });
}

wf_status wf_rollback_tree(wf_engine *e, int32_t n, const int32_t *d_slots, const int32_t *d_path,
                           int32_t T, const int32_t *d_n_acc, void *stream) {
    if (!e || !d_slots || !d_path || !d_n_acc) return fail(WF_EINVAL, "null argument");
    if (n < 1 || n > e->c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    if (T < 1 || T > 64) return fail(WF_EINVAL, "a tree has 1 to 64 nodes");
    const wf_config &c = e->c;
    CompactArgs ca{n, T, c.n_layers, c.n_heads, c.head_dim, c.max_batch, e->pt_stride,
                   e->page_elems, e->kv_layer_elems, d_slots, d_path, d_n_acc, e->len, e->pend,
                   e->pt, e->err, e->kv};
    hipStream_t st = (hipStream_t)stream;
    WF_TRY(timed(e, TK_OTHER, st, [&] { return launch_compact(ca, st); }));
    RollbackArgs ra{n, c.max_batch, d_slots, d_n_acc, e->len, e->pend, e->err};
    return timed(e, TK_OTHER, st, [&] { return launch_rollback(ra, st); });
}

wf_status wf_draft(wf_engine *e, int32_t n, const int32_t *d_slots, const int32_t *d_anchor,
                   int32_t K, int32_t *d_block, float *d_logits, void *stream) {
    if (!e || !d_slots || !d_anchor || !d_block) return fail(WF_EINVAL, "null argument");
    const wf_config &c = e->c;
    if (c.drafter_layers < 1) return fail(WF_ESTATE, "the engine has no drafter");
    if (n < 1 || n > c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    if (K < 1 || K + 1 > c.n_ctx) return fail(WF_EINVAL, "K outside [1, n_ctx - 1]");
    const int T = K + 1;
    if ((long long)n * T > c.max_rows) return fail(WF_ECAPACITY, "n*(K+1) exceeds max_rows");
    hipStream_t st = (hipStream_t)stream;
    const int M = n * T, d = c.d_model, H = c.n_heads, hd = c.head_dim;
    Pass p{n, T, M, cdiv(T, 16), 0, 0, 0, d_slots, TK_DRAFT};
    cross_plan(e, n, p.mt, p.cf, p.G, p.spw);

    PrepareDraftArgs pa{n, K, c.vocab, c.n_ctx, c.n_pages, e->pt_stride, c.max_batch, d_slots,
                        d_anchor, e->pt, e->len, e->pend, e->err, e->reqL, e->reqN};
    WF_TRY(timed(e, TK_DRAFT, st, [&] { return launch_prepare_draft(pa, st); }));
    EmbedDraftArgs ea{M, T, d, c.vocab, d_anchor, e->tok_emb, e->mask_emb, e->x};
    WF_TRY(timed(e, TK_DRAFT, st, [&] { return launch_embed_draft(ea, st); }));
    for (int dl = 0; dl < c.drafter_layers; ++dl) {
        const LayerW &w = e->dlayers[dl];
        EpiArgs qa{};
        qa.b0 = w.bq;
        qa.b2 = w.bv;
        qa.out32 = reinterpret_cast<float *>(e->hs);
        WF_TRY(run_gemm(e, TK_DRAFT, ROLE_DRAFT_QKV, e->xs, M, d, w.wq, w.wk, w.wv, d, 3 * d, qa,
                        st, w.ln1_g, w.ln1_b));
        WF_TRY(run_rope_append(e, dl, p, 3 * d, 0, d, 2 * d, TK_DRAFT, st));
        uint16_t *kvl = e->kv + (size_t)(c.n_layers + dl) * e->kv_layer_elems;
        SelfAttnArgs sa{e->q, kvl, e->pt, d_slots, e->reqL, e->reqN, e->pt_stride,
                        e->page_elems, n, T, H, d, 0, 1.0f / std::sqrt((float)hd), e->xs};
        WF_TRY(timed(e, TK_DRAFT, st, [&] { return launch_self_attn(sa, hd, p.mt, st); }));
        WF_TRY(run_out_cross_mlp(e, w, c.n_layers + dl, p, st));
    }
    WF_TRY(run_head(e, e->lnd_g, e->lnd_b, p, d_logits, e->dam, st));
    return timed(e, TK_DRAFT, st, [&] {
        return launch_draft_out(d_anchor, e->dam, e->reqN, n, K, d_block, st);
    });
}

wf_status wf_accept(wf_engine *e, int32_t n, const int32_t *d_tokens, int32_t T,
                    const int32_t *d_n_tok, const int32_t *d_budget, const int32_t *d_argmax,
                    const float *d_logits, const float *d_q, const uint8_t *d_suppress,
                    float temperature, uint64_t seed, const int32_t *d_request_id,
                    const int32_t *d_step, int32_t *d_n_acc, int32_t *d_next_token,
                    int32_t *d_n_emit, int32_t *d_done, void *stream) {
    if (!e || !d_tokens || !d_n_tok || !d_budget || !d_n_acc || !d_next_token || !d_n_emit ||
        !d_done)
        return fail(WF_EINVAL, "null argument");
    if (n < 1 || n > e->c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    if (T < 1 || T > e->c.n_ctx) return fail(WF_EINVAL, "T outside [1, n_ctx]");
    if (!(temperature >= 0.f) || std::isinf(temperature))
        return fail(WF_EINVAL, "temperature must be finite and >= 0");
    if (temperature == 0.f && !d_argmax) return fail(WF_EINVAL, "greedy accept needs d_argmax");
    if (temperature > 0.f && (!d_logits || (T > 1 && !d_q) || !d_request_id || !d_step))
        return fail(WF_EINVAL, "sampling needs logits, q (when T > 1), request ids and steps");
    AcceptArgs a{};
    a.n = n;
    a.T = T;
    a.V = e->c.vocab;
    a.eos = e->c.eos_id;
    a.tokens = d_tokens;
    a.n_tok = d_n_tok;
    a.budget = d_budget;
    a.argmax = d_argmax;
    a.n_acc = d_n_acc;
    a.next_token = d_next_token;
    a.n_emit = d_n_emit;
    a.done = d_done;
    a.logits = d_logits;
    a.q = d_q;
    a.suppress = d_suppress;
    a.temperature = temperature;
    a.seed = seed;
    a.request_id = d_request_id;
    a.step = d_step;
    // the LM head's per-tile maxima are consumed by then: their buffer holds
    // the rows' softmax statistics when it is large enough
    if (temperature > 0.f &&
        sample_scratch_floats(n, T) <= (size_t)e->lay.n_vtiles * e->c.max_rows)
        a.stats = e->lmmax;
    hipStream_t st = (hipStream_t)stream;
    return timed(e, TK_OTHER, st, [&] { return launch_accept(a, st); });
}

wf_status wf_rollback(wf_engine *e, int32_t n, const int32_t *d_slots, const int32_t *d_n_acc,
                      void *stream) {
    if (!e || !d_slots || !d_n_acc) return fail(WF_EINVAL, "null argument");
    if (n < 1 || n > e->c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    RollbackArgs a{n, e->c.max_batch, d_slots, d_n_acc, e->len, e->pend, e->err};
    hipStream_t st = (hipStream_t)stream;
    return timed(e, TK_OTHER, st, [&] { return launch_rollback(a, st); });
}

wf_status wf_truncate(wf_engine *e, int32_t n, const int32_t *d_slots, const int32_t *d_len,
                      void *stream) {
    if (!e || !d_slots || !d_len) return fail(WF_EINVAL, "null argument");
    if (n < 1 || n > e->c.max_batch) return fail(WF_ECAPACITY, "n outside [1, max_batch]");
    RollbackArgs a{n, e->c.max_batch, d_slots, d_len, e->len, e->pend, e->err};
    hipStream_t st = (hipStream_t)stream;
    return timed(e, TK_OTHER, st, [&] { return launch_truncate(a, st); });
}

static bool loop_state_ok(const wf_loop_state *s) {
    return s && s->anchor && s->len && s->emitted && s->done && s->acc_sum && s->prop_sum &&
           s->rounds && s->step && s->tok_sum && s->hist;
}

wf_status wf_loop_prepare(wf_engine *e, int32_t n, const wf_loop_state *s, int32_t K,
                          int32_t n_max, const int32_t *d_table, int32_t table_cols,
                          int32_t *d_block, int32_t *d_n_tok, int32_t *d_budget, void *stream) {
    if (!e || !loop_state_ok(s) || !d_n_tok || !d_budget || (d_table && !d_block))
        return fail(WF_EINVAL, "null argument");
    if (n < 1) return fail(WF_EINVAL, "n < 1");
    if (K < 0 || K + 1 > e->c.n_ctx) return fail(WF_EINVAL, "K outside [0, n_ctx - 1]");
    if (n_max < 1) return fail(WF_EINVAL, "n_max < 1");
    if (d_table && table_cols < 1) return fail(WF_EINVAL, "table_cols < 1");
    LoopArgs a{};
    a.n = n;
    a.K = K;
    a.n_max = n_max;
    a.n_ctx = e->c.n_ctx;
    a.table_cols = table_cols;
    a.s = *s;
    a.table = d_table;
    a.block = d_block;
    a.n_tok_out = d_n_tok;
    a.budget = d_budget;
    hipStream_t st = (hipStream_t)stream;
    return timed(e, TK_OTHER, st, [&] { return launch_loop_prepare(a, st); });
}

wf_status wf_loop_finish(wf_engine *e, int32_t n, const wf_loop_state *s, int32_t K,
                         const int32_t *d_n_tok, const int32_t *d_n_acc,
                         const int32_t *d_next_token, const int32_t *d_n_emit,
                         const int32_t *d_done, void *stream) {
    if (!e || !loop_state_ok(s) || !d_n_tok || !d_n_acc || !d_next_token || !d_n_emit || !d_done)
        return fail(WF_EINVAL, "null argument");
    if (n < 1) return fail(WF_EINVAL, "n < 1");
    if (K < 0) return fail(WF_EINVAL, "K < 0");
    LoopArgs a{};
    a.n = n;
    a.K = K;
    a.s = *s;
    a.n_tok = d_n_tok;
    a.n_acc = d_n_acc;
    a.next_token = d_next_token;
    a.n_emit = d_n_emit;
    a.done = d_done;
    hipStream_t st = (hipStream_t)stream;
    return timed(e, TK_OTHER, st, [&] { return launch_loop_finish(a, st); });
}

wf_status wf_device_state(wf_engine *e, int32_t *h_err, int32_t *h_len, void *stream) {
    if (!e) return fail(WF_EINVAL, "null engine");
    hipStream_t st = (hipStream_t)stream;
    if (hipStreamSynchronize(st) != hipSuccess) return fail(WF_EHIP, "stream synchronize failed");
    const size_t bytes = (size_t)e->c.max_batch * 4;
    if (h_err && hipMemcpy(h_err, e->err, bytes, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(WF_EHIP, "copy of error words failed");
    if (h_len && hipMemcpy(h_len, e->len, bytes, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(WF_EHIP, "copy of lengths failed");
    return WF_OK;
}

wf_status wf_set_option(wf_engine *e, int32_t option, int32_t value) {
    if (!e) return fail(WF_EINVAL, "null engine");
    switch (option) {
        case WF_OPT_PERSISTENT: e->persistent = value != 0; return WF_OK;
        case WF_OPT_TALL_GEMM: e->tall_gemm = value != 0; return WF_OK;
        case WF_OPT_LN_FUSION: e->ln_fusion = value != 0; return WF_OK;
        case WF_OPT_XA_CHUNKS:
            if (value != 0 && value != 4 && value != 8 && value != 16 && value != 32)
                return fail(WF_EINVAL, "WF_OPT_XA_CHUNKS takes 0, 4, 8, 16 or 32");
            e->xa_chunks = value;
            return WF_OK;
        case WF_OPT_PASS_TIMEOUT_US:
            if (value < 0) return fail(WF_EINVAL, "WF_OPT_PASS_TIMEOUT_US must be >= 0");
            e->pass_timeout_ticks = (int64_t)value * 100;
            return WF_OK;
    }
    return fail(WF_EINVAL, "unknown option %d", option);
}

wf_status wf_set_trace(wf_engine *e, void *d_trace, size_t bytes) {
    if (!e) return fail(WF_EINVAL, "null engine");
    e->trace = d_trace ? (uint64_t *)d_trace : nullptr;
    e->trace_tasks = d_trace ? bytes / 32 : 0;
    return WF_OK;
}

wf_status wf_pass_schedule(wf_engine *e, int32_t *h_info) {
    if (!e || !h_info) return fail(WF_EINVAL, "null argument");
    for (int k = 0; k < 20; ++k) h_info[k] = e->last_sched[k];
    return WF_OK;
}

wf_status wf_set_timing(wf_engine *e, int32_t enable) {
    if (!e) return fail(WF_EINVAL, "null engine");
    e->timing = enable != 0;
    for (auto &v : e->spans) v.clear();
    e->ev_used = 0;
    return WF_OK;
}

wf_status wf_get_timing(wf_engine *e, int32_t kind, double *total_ms, int32_t *count) {
    if (!e || !total_ms || !count) return fail(WF_EINVAL, "null argument");
    if (kind < 0 || kind >= TK_N) return fail(WF_EINVAL, "unknown timing kind");
    double tot = 0;
    for (auto &p : e->spans[kind]) {
        if (hipEventSynchronize(p.second) != hipSuccess)
            return fail(WF_EHIP, "event synchronize failed");
        float ms = 0;
        if (hipEventElapsedTime(&ms, p.first, p.second) != hipSuccess)
            return fail(WF_EHIP, "elapsed time failed");
        tot += ms;
    }
    *total_ms = tot;
    *count = (int32_t)e->spans[kind].size();
    return WF_OK;
}

}  // extern "C"
