// Persistent verify pass: one launch runs every decoder layer of a linear
// block, the final layer norm and the tied LM head with the per-row argmax.
//
// A layer is eleven dependent steps (three layer norms, six projections,
// self- and cross-attention), each moving a few MB at tens of requests. As
// separate launches every step pays dispatch, a cold load pipeline and a
// drain. Here one workgroup of eight waves per CU walks a fixed task list:
// task t goes to workgroup t mod G, tasks in the list order layer by layer
// and phase by phase. A task waits only for the 16-row tiles it reads, on
// per-(layer, phase, tile) arrival counters that the producing tasks bump
// after their stores are published (agent-scope release); the projections
// issue their weight loads before that wait. Different row tiles, and so
// different requests, move through the phases independently.
//
// Every wait depends only on tasks earlier in the list, so with all G
// workgroups resident the earliest unfinished task can always run. The
// waits are bounded by a clock limit: past it the pass sets an abort flag
// that ends every other wait at once, marks its requests' error words and
// drains.
//
// Memory: every activation a task reads was written by other workgroups in
// this launch, and each buffer is written once per launch (per layer and
// phase its own buffer, see PassArgs), so a workgroup never holds a stale
// copy of a line in its caches: plain loads read the producers' data once
// their counter is seen. Scratch that is reused within the launch (K-group
// sums, cross-attention chunk-group partials, their counters) moves through
// device-coherent accesses, as in the standalone kernels.
//
// Arithmetic is that of the standalone kernels (the same GEMM chunk order,
// layer-norm, attention and argmax code), so the pass gives the same bits as
// the multi-kernel path.
#include "attn_items.h"
#include "gemm_task.h"
#include "../../include/wf.h"

namespace wf {
namespace {

constexpr int kThreads = 512;
constexpr int kHd = 64;

// The pass arguments are read through a pointer into the kernel-argument
// segment (address space 4: scalar loads) that each task launders, so the
// compiler loads the fields a task uses inside that task instead of keeping
// every field of the block live across the whole task loop.
using PA = const __attribute__((address_space(4))) PassArgs &;
// The kernel hands its argument-segment address to the task functions (the
// segment pointer builtin is only defined in the kernel itself); a task
// moves it back to scalar registers, where the field loads are scalar.
__device__ __forceinline__ PA pass_args(uint64_t kp) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)kp);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(kp >> 32));
    const __attribute__((address_space(4))) char *p =
        (const __attribute__((address_space(4))) char *)(((uint64_t)hi << 32) | lo);
    asm volatile("" : "+s"(p));
    return *(const __attribute__((address_space(4))) PassArgs *)p;
}

__device__ __forceinline__ int ld_acq(const int *p) {
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ long long clock100() {
    return (long long)__builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ int *slot_cnt(PA a, int l, int ph) {
    return a.cnt + ((size_t)l * PH_PER_LAYER + ph) * a.RT;
}
__device__ __forceinline__ int *head_cnt(PA a, int k) {
    return a.cnt + ((size_t)a.n_layers * PH_PER_LAYER + k) * a.RT;
}

// Number of (request, 16-row tile) attention items whose rows meet row tile r.
__device__ __forceinline__ int items_over_tile(PA a, int r) {
    const int r0 = 16 * r, r1 = min(16 * r + 16, a.M);
    int c = 0;
    for (int b = r0 / a.T; b <= (r1 - 1) / a.T && b < a.n; ++b)
        for (int mt = 0; mt < a.mt; ++mt) {
            const int s = b * a.T + 16 * mt, e = b * a.T + min(16 * mt + 16, a.T);
            if (max(s, r0) < min(e, r1)) ++c;
        }
    return c;
}

// Wait-limit exceeded: end every other wait and mark every request.
__device__ __forceinline__ void pass_abort(PA a) {
    __hip_atomic_store(a.abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int lane = threadIdx.x & 63;
    for (int b = lane; b < a.n; b += 64) {
        const int s = a.slots[b];
        if (s >= 0 && s < a.max_batch) atomicOr(&a.slot_err[s], WF_DERR_TIMEOUT);
    }
}

// Time the current task's inputs became ready (trace only).
__shared__ long long g_t_ready;

// The calling wave polls the counters of row tiles [r0, r1) (at most 64)
// until each reaches c (per_item: c times the attention items over the
// tile). One wave per item polls and the workgroup then meets at a barrier:
// hundreds of waves spinning on the same counter lines would hold up the
// producers' own increments to them. The poll interval grows from ~50 ns
// to ~0.5 us while the inputs are far from ready.
__device__ __forceinline__ void poll_tiles(PA a, const int *cnt, int r0, int r1, int c,
                                           bool per_item) {
    const int lane = threadIdx.x & 63;
    const int r = r0 + lane;
    const bool mine = r < r1;
    const int want = mine ? (per_item ? c * items_over_tile(a, r) : c) : 0;
    const long long t0 = clock100();
    for (int it = 0;; ++it) {
        const int v = mine ? ld_acq(cnt + r) : 0;
        if (__all(v >= want)) break;
        if (ld_acq(a.abort_flag)) break;
        if (clock100() - t0 > a.timeout_ticks) {
            pass_abort(a);
            break;
        }
        if (it < 16) __builtin_amdgcn_s_sleep(2);
        else if (it < 64) __builtin_amdgcn_s_sleep(8);
        else __builtin_amdgcn_s_sleep(20);
    }
    if (a.trace && lane == 0) g_t_ready = clock100();
}
// The whole workgroup waits: wave 0 polls, then the barrier.
__device__ __forceinline__ void wait_tiles(PA a, const int *cnt, int r0, int r1, int c,
                                           bool per_item) {
    if ((threadIdx.x >> 6) == 0) poll_tiles(a, cnt, r0, r1, c, per_item);
    __syncthreads();
}

// Every wave: its stores are complete; then the workgroup meets.
__device__ __forceinline__ void stores_done() {
    wait_vmem();
    __syncthreads();
}
// One wave publishes the workgroup's stores (agent-scope release) and bumps
// the counters of row tiles [r0, r1); lane i gets the old value of tile
// r0 + i (or -1).
__device__ __forceinline__ int publish_tiles(int *cnt, int r0, int r1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int lane = threadIdx.x & 63;
    int old = -1;
    if (r0 + lane < r1)
        old = __hip_atomic_fetch_add(cnt + r0 + lane, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    return old;
}

// GEMM tilings per size class: (row tiles, 16-column tiles per wave, column
// slices). Class 0: one row tile (a request or two); class 1: up to six;
// class 2: more (tens of requests). The tiles keep every task body within
// the 256 registers a wave has at two waves per SIMD.
template <int CL, int PG>
struct Tile {
    static constexpr bool DW = PG == PG_O || PG == PG_CQ || PG == PG_OC;   // d-wide output
    static constexpr int MB = CL == 0 ? 1 : CL == 1 ? 2 : PG == PG_FC2 ? 6 : 3;
    static constexpr int NB = PG == PG_LMH ? 4 : PG == PG_FC2 ? 1 : CL == 0 ? 1
                            : DW ? (CL == 1 ? 1 : 2) : (CL == 1 ? 2 : 4);
    static constexpr int WN = PG == PG_FC2 ? 4 : 1;
    static constexpr int NT = MB * NB;
    // loads in flight per wave: the whole 5-k-step chunk of the d-deep
    // projections (issued at once, the weights before the input wait), a
    // 5-deep ring over fc2's 20-k-step chunks
    static constexpr int D = PG == PG_FC2 ? 3 : PG == PG_LMH ? 3 : (CL == 2 && !DW) ? 4 : 5;
};

template <int CL, int PG>
constexpr int tile_lds() {
    return GemmTaskShape<Tile<CL, PG>::MB, Tile<CL, PG>::NB, Tile<CL, PG>::WN>::LDS_BYTES;
}
constexpr int cmax(int x, int y) { return x > y ? x : y; }
// attention: two items, each two (o, m, l) row buffers, and a flag
constexpr int kAttnLds = 2 * 2 * 16 * (kHd + 4) * 4 + 16;
template <int CL>
constexpr int pass_lds() {
    return cmax(cmax(cmax(tile_lds<CL, PG_QKV>(), tile_lds<CL, PG_O>()),
                     cmax(tile_lds<CL, PG_FC1>(), tile_lds<CL, PG_FC2>())),
                cmax(tile_lds<CL, PG_LMH>(), kAttnLds));
}

__device__ __forceinline__ GemmArgs gemm_args(PA a, int pg, const uint16_t *X,
                                              int K, int N, const uint16_t *W0,
                                              const uint16_t *W1, const uint16_t *W2,
                                              int seg_n) {
    GemmArgs g{};
    g.X = X;
    g.W0 = W0;
    g.W1 = W1 ? W1 : W0;
    g.W2 = W2 ? W2 : W0;
    g.M = a.M;
    g.K = K;
    g.N = N;
    g.seg_n = seg_n;
    g.S = 8;
    g.ck = K >> 8;
    g.n_tiles = a.g[pg].n_tiles;
    g.m_blocks = a.g[pg].m_blocks;
    g.n_groups = a.g[pg].n_groups;
    g.part = a.part;
    g.cnt = a.gcnt;
    return g;
}

// One projection task: wait for the input rows, run the tile, publish.
template <int CL, int PG, int EPI, int CK>
__device__ __forceinline__ void proj_task(PA a, const GemmArgs &g, int lid, const int *need,
                          int need_c, bool need_items, int *mine, char *smem) {
    using Tl = Tile<CL, PG>;
    int ntile, mblock, grp;
    if (!gemm_task_coords(g, lid, ntile, mblock, grp)) return;
    const int r0 = mblock * Tl::MB, r1 = min(r0 + Tl::MB, a.RT);
    auto wait = [&] { wait_tiles(a, need, r0, r1, need_c, need_items); };
    if (!gemm_task<EPI, Tl::MB, Tl::NB, Tl::WN, CK, Tl::D>(g, ntile, mblock, grp, smem, wait))
        return;
    stores_done();
    if ((threadIdx.x >> 6) == 0) publish_tiles(mine, r0, r1);
}

// Layer norm of 32 rows (two row tiles): which 0..2 the layer's LN1..LN3,
// 3 the final one. Also writes a drafter history tap of the residual stream
// it reads when that stream is the output of a tapped block.
__device__ __forceinline__ void ln_task(PA a, int l, int which, int j) {
    const int NL = a.n_layers;
    const int r0 = 2 * j, r1 = min(2 * j + 2, a.RT);
    const int *need = nullptr;
    int need_c = 0;
    if (which == 0 && l > 0) { need = slot_cnt(a, l - 1, PH_FC2); need_c = a.g[PG_FC2].n_tiles; }
    if (which == 1) { need = slot_cnt(a, l, PH_O); need_c = a.g[PG_O].n_tiles; }
    if (which == 2) { need = slot_cnt(a, l, PH_OC); need_c = a.g[PG_OC].n_tiles; }
    if (which == 3) { need = slot_cnt(a, NL - 1, PH_FC2); need_c = a.g[PG_FC2].n_tiles; }
    if (need) wait_tiles(a, need, r0, r1, need_c, false);
    const int ver = which == 3 ? 3 * NL : 3 * l + which;
    const float *x = a.xv + (size_t)ver * a.x_stride;
    uint16_t *out = a.lnv + (size_t)ver * a.act_stride;
    const LayerW &w = a.lw[which == 3 ? 0 : l];
    const uint16_t *gg_p = which == 0 ? w.ln1_g : which == 1 ? w.ln2_g : which == 2 ? w.ln3_g : a.lnf_g;
    const uint16_t *bb_p = which == 0 ? w.ln1_b : which == 1 ? w.ln2_b : which == 2 ? w.ln3_b : a.lnf_b;
    // the tapped block whose output this stream is (LN1 of layer l reads the
    // output of block l - 1, the final norm that of the last block)
    int tap = -1;
    if (a.n_taps > 0 && (which == 0 || which == 3)) {
        const int blk = which == 0 ? l - 1 : NL - 1;
        for (int k = 0; k < a.n_taps; ++k)
            if (a.tap_layers[k] == blk) tap = k;
    }
    const int m = 32 * j + (threadIdx.x >> 4), r16 = threadIdx.x & 15;
    const int d = a.d;
    if (m < a.M) {
        LnRow row;
        ln_load16(x + (size_t)m * d, d, r16, row);
        const int last = (d >> 3) - 1;
        // gains and biases in two halves: the first with the row, the second
        // once the first half's outputs are out (register budget)
        constexpr int H1 = LN_GPL / 2;
        u32x4 gg[H1], bb[H1];
#pragma unroll
        for (int i = 0; i < H1; ++i) {
            const int kg = min(r16 + 16 * i, last);
            gg[i] = ld16(gg_p + kg * 8);
            bb[i] = ld16(bb_p + kg * 8);
        }
        float mean, rstd;
        ln_reduce16(row, d, r16, a.ln_eps, mean, rstd);
#pragma unroll
        for (int i = 0; i < LN_GPL; ++i) {
            const int kg = r16 + 16 * i;
            if (i == H1) {
#pragma unroll
                for (int q = 0; q < H1; ++q) {
                    const int kq = min(r16 + 16 * (H1 + q), last);
                    gg[q] = ld16(gg_p + kq * 8);
                    bb[q] = ld16(bb_p + kq * 8);
                }
            }
            if (kg > last) break;
            *reinterpret_cast<u32x4 *>(out + xh_index(m, kg * 8, d)) =
                ln_h8(row.v[2 * i], row.v[2 * i + 1], gg[i % H1], bb[i % H1], mean, rstd);
            if (tap >= 0) {
                const float4 x0 = row.v[2 * i], x1 = row.v[2 * i + 1];
                const u32x4 v = {pack_h2(x0.x, x0.y), pack_h2(x0.z, x0.w), pack_h2(x1.x, x1.y),
                                 pack_h2(x1.z, x1.w)};
                *reinterpret_cast<u32x4 *>(
                    a.taps + xh_index(m, tap * d + kg * 8, a.n_taps * d)) = v;
            }
        }
    }
    stores_done();
    if ((threadIdx.x >> 6) == 0)
        publish_tiles(which == 3 ? head_cnt(a, 0) : slot_cnt(a, l, which == 0 ? PH_LN1 : which == 1 ? PH_LN2 : PH_LN3), r0, r1);
}

// Rows [s, e) of an attention item -> its row tiles [p0, p1).
__device__ __forceinline__ void item_tiles(PA a, int b, int mtile, int &p0, int &p1) {
    const int s = b * a.T + 16 * mtile, e = b * a.T + min(16 * mtile + 16, a.T);
    p0 = s >> 4;
    p1 = ((e - 1) >> 4) + 1;
}

// Two self-attention items (request, head, 16-row tile) per task, four waves each.
__device__ __forceinline__ void sa_task(PA a, int l, int j, char *smem) {
    const int wave = threadIdx.x >> 6, half = wave >> 2, w4 = wave & 3;
    const int item = 2 * j + half;
    const bool valid = item < a.sa_items;
    const int bh = valid ? item / a.mt : 0, mtile = valid ? item - bh * a.mt : 0;
    const int b = bh / a.H;
    if (valid && w4 == 0) {
        // the request's K/V rows and its queries
        const int r0 = (b * a.T) >> 4, r1 = ((b * a.T + a.T - 1) >> 4) + 1;
        poll_tiles(a, slot_cnt(a, l, PH_QKV), r0, r1, a.g[PG_QKV].n_tiles, false);
    }
    __syncthreads();
    SelfAttnArgs s{};
    s.q = a.qv + (size_t)l * a.q_stride;
    s.kv_layer = a.kv + (size_t)l * a.kv_layer_elems;
    s.page_table = a.page_table;
    s.slots = a.slots;
    s.req_L = a.req_L;
    s.req_ntok = a.req_ntok;
    s.pt_stride = a.pt_stride;
    s.page_elems = a.page_elems;
    s.n = a.n;
    s.T = a.T;
    s.H = a.H;
    s.d = a.d;
    s.causal = 1;
    s.scale = a.scale;
    s.out = a.sav + (size_t)l * a.act_stride;
    s.anc = nullptr;
    auto mbuf = reinterpret_cast<float (*)[16 * (kHd + 4)]>(smem + half * 2 * 16 * (kHd + 4) * 4);
    self_attn_item<kHd, false>(s, bh, mtile, valid, w4, mbuf);
    stores_done();
    if (w4 == 0 && valid) {
        int p0, p1;
        item_tiles(a, b, mtile, p0, p1);
        publish_tiles(slot_cnt(a, l, PH_SA), p0, p1);
    }
}

template <int SPW>
__device__ __forceinline__ bool xa_item(const CrossAttnArgs &c, int item, bool valid, int w4, char *smem,
                        int half) {
    auto mbuf = reinterpret_cast<float (*)[16 * (kHd + 4)]>(smem + half * 2 * 16 * (kHd + 4) * 4);
    int *last = reinterpret_cast<int *>(smem + 2 * 2 * 16 * (kHd + 4) * 4) + half;
    return cross_attn_item<kHd, SPW>(c, item, valid, w4, mbuf, last);
}

// Two cross-attention items (request, head, 16-row tile, chunk group) per task.
template <int CL>
__device__ __forceinline__ void xa_task(PA a, int l, int j, char *smem) {
    const int wave = threadIdx.x >> 6, half = wave >> 2, w4 = wave & 3;
    const int item = 2 * j + half;
    const bool valid = item < a.xa_items;
    const int bhm = valid ? item / a.xa_G : 0;
    const int mtile = bhm % a.mt, b = (bhm / a.mt) / a.H;
    int p0 = 0, p1 = 0;
    if (valid) item_tiles(a, b, mtile, p0, p1);
    if (valid && w4 == 0) poll_tiles(a, slot_cnt(a, l, PH_CQ), p0, p1, a.g[PG_CQ].n_tiles, false);
    __syncthreads();
    CrossAttnArgs c{};
    c.q = a.cqv + (size_t)l * a.q_stride;
    c.xkv = a.xkv;
    c.slot_stride = a.xkv_slot_elems;
    c.layer_off = (int64_t)l * a.xkv_layer_elems;
    c.slots = a.slots;
    c.req_ntok = a.req_ntok;
    c.n = a.n;
    c.T = a.T;
    c.H = a.H;
    c.d = a.d;
    c.F = a.n_frames;
    c.F_pad = a.F_pad;
    c.mt = a.mt;
    c.G = a.xa_G;
    c.cf = a.xa_cf;
    c.spw = a.xa_spw;
    c.n_items = a.xa_items;
    c.scale = a.scale;
    c.part = a.xapart;
    c.cnt = a.xacnt;
    c.out = a.xav + (size_t)l * a.act_stride;
    // straight-line chunk loops for the chunk lengths of the class's batches
    // (one request: 2 steps; 2..10: 2, 4 or 6; more: 6 or 12), else the loop
    bool rep;
    if (CL == 0 && a.xa_spw == 2) rep = xa_item<2>(c, item, valid, w4, smem, half);
    else if (CL == 1 && a.xa_spw == 4) rep = xa_item<4>(c, item, valid, w4, smem, half);
    else if (CL >= 1 && a.xa_spw == 6) rep = xa_item<6>(c, item, valid, w4, smem, half);
    else if (CL == 2 && a.xa_spw == 12) rep = xa_item<12>(c, item, valid, w4, smem, half);
    else rep = xa_item<0>(c, item, valid, w4, smem, half);
    stores_done();
    if (w4 == 0 && rep) publish_tiles(slot_cnt(a, l, PH_XA), p0, p1);
}

// Per row of row tile r: merge the LM head's per-64-column (max, lowest
// index) in any order (the merge is order-free), -1 for rows past a
// request's n_tok, NaN flags the slot. 32 threads per row.
__device__ __forceinline__ void lm_reduce_tile(PA a, int r) {
    const int tid = threadIdx.x, l32 = tid & 31;
    const int m = 16 * r + (tid >> 5);
    float v = -INFINITY;
    int idx = 0x7fffffff, nan = 0;
    if (m < a.M) {
        const float *tm = a.tile_max + (size_t)m * a.ld;
        const int32_t *tx = a.tile_idx + (size_t)m * a.ld;
        for (int t = l32; t < a.n_vtiles; t += 32) {
            const int ti = tx[t];
            const float tv = tm[t];
            if (ti < 0) nan = 1;
            else argmax_merge(v, idx, tv, ti);
        }
    }
    argmax16(v, idx, nan);
    {
        float va, vb;
        int ia, ib, na, nb;
        rows16_pair(v, va, vb);
        rows16_pair(idx, ia, ib);
        rows16_pair(nan, na, nb);
        v = va;
        idx = ia;
        argmax_merge(v, idx, vb, ib);
        nan = na | nb;
    }
    if (l32 == 0 && m < a.M) {
        const int b = m / a.T, i = m - (m / a.T) * a.T;
        int out = idx;
        if (i >= a.req_ntok[b]) out = -1;
        else if (nan) {
            atomicOr(&a.slot_err[a.slots[b]], WF_DERR_NAN);
            out = -1;
        }
        a.argmax[m] = out;
    }
}

template <int CL>
__device__ __forceinline__ void lmh_task(PA a, int lid, char *smem) {
    using Tl = Tile<CL, PG_LMH>;
    const int NL = a.n_layers;
    GemmArgs g = gemm_args(a, PG_LMH, a.lnv + (size_t)(3 * NL) * a.act_stride, a.d, a.V,
                           a.tok_emb, nullptr, nullptr, a.V);
    g.e.logits = a.logits;
    g.e.tile_max = a.tile_max;
    g.e.tile_idx = a.tile_idx;
    g.e.ld = a.ld;
    int ntile, mblock, grp;
    if (!gemm_task_coords(g, lid, ntile, mblock, grp)) return;
    const int r0 = mblock * Tl::MB, r1 = min(r0 + Tl::MB, a.RT);
    auto wait = [&] { wait_tiles(a, head_cnt(a, 0), r0, r1, 1, false); };
    gemm_task<EPI_ARGMAX, Tl::MB, Tl::NB, Tl::WN, 5, Tl::D>(g, ntile, mblock, grp, smem, wait);
    stores_done();
    int *mask = reinterpret_cast<int *>(smem);
    if ((threadIdx.x >> 6) == 0) {
        const int old = publish_tiles(head_cnt(a, 1), r0, r1);
        // the last task of a row tile merges its rows
        const unsigned long long done = __ballot(old == a.g[PG_LMH].n_tiles - 1);
        if ((threadIdx.x & 63) == 0) *mask = (int)(done & 0xffffffffull);
    }
    __syncthreads();
    const int mk = *mask;
    for (int k = 0; k < r1 - r0; ++k)
        if ((mk >> k) & 1) lm_reduce_tile(a, r0 + k);
}

// Task entry points: separate functions (not inlined), so that each task
// body gets its own register allocation and the kernel needs only the
// largest of them.
#define WF_TASK __device__ __attribute__((noinline))
WF_TASK void task_ln(uint64_t kp, int l, int which, int j) { ln_task(pass_args(kp), l, which, j); }
WF_TASK void task_sa(uint64_t kp, int l, int j, char *smem) { sa_task(pass_args(kp), l, j, smem); }
template <int CL>
WF_TASK void task_xa(uint64_t kp, int l, int j, char *smem) { xa_task<CL>(pass_args(kp), l, j, smem); }
template <int CL>
WF_TASK void task_lmh(uint64_t kp, int j, char *smem) { lmh_task<CL>(pass_args(kp), j, smem); }
template <int CL> WF_TASK void task_qkv(uint64_t kp, int l, int j, char *smem);
template <int CL> WF_TASK void task_o(uint64_t kp, int l, int j, char *smem);
template <int CL> WF_TASK void task_cq(uint64_t kp, int l, int j, char *smem);
template <int CL> WF_TASK void task_oc(uint64_t kp, int l, int j, char *smem);
template <int CL> WF_TASK void task_fc1(uint64_t kp, int l, int j, char *smem);
template <int CL> WF_TASK void task_fc2(uint64_t kp, int l, int j, char *smem);

template <int CL>
__device__ __forceinline__ void run_task(PA a, uint64_t kp, int t, char *smem) {
    const int NL = a.n_layers;
    if (t >= NL * a.per_layer) {
        const int r = t - NL * a.per_layer;
        if (r < a.head_off[1]) task_ln(kp, NL - 1, 3, r);
        else task_lmh<CL>(kp, r - a.head_off[1], smem);
        return;
    }
    const int l = t / a.per_layer;
    const int r = t - l * a.per_layer;
    int ph = 0;
#pragma unroll
    for (int k = 1; k < PH_PER_LAYER; ++k)
        if (r >= a.ph_off[k]) ph = k;
    const int j = r - a.ph_off[ph];
    switch (ph) {
        case PH_LN1: task_ln(kp, l, 0, j); break;
        case PH_LN2: task_ln(kp, l, 1, j); break;
        case PH_LN3: task_ln(kp, l, 2, j); break;
        case PH_SA: task_sa(kp, l, j, smem); break;
        case PH_XA: task_xa<CL>(kp, l, j, smem); break;
        case PH_QKV: task_qkv<CL>(kp, l, j, smem); break;
        case PH_O: task_o<CL>(kp, l, j, smem); break;
        case PH_CQ: task_cq<CL>(kp, l, j, smem); break;
        case PH_OC: task_oc<CL>(kp, l, j, smem); break;
        case PH_FC1: task_fc1<CL>(kp, l, j, smem); break;
        case PH_FC2: task_fc2<CL>(kp, l, j, smem); break;
        default: break;
    }
}

template <int CL>
WF_TASK void task_qkv(uint64_t kp, int l, int j, char *smem) {
    PA a = pass_args(kp);
    const LayerW &w = a.lw[l];
    const int d = a.d;
    const size_t act = (size_t)l * a.act_stride;
    (void)act;
    GemmArgs g = gemm_args(a, PG_QKV, a.lnv + (size_t)(3 * l) * a.act_stride, d, 3 * d,
                           w.wq, w.wk, w.wv, d);
    g.e.b0 = w.bq;
    g.e.b2 = w.bv;
    g.e.out = a.qv + (size_t)l * a.q_stride;
    g.e.kv_layer = a.kv + (size_t)l * a.kv_layer_elems;
    g.e.page_table = a.page_table;
    g.e.pt_stride = a.pt_stride;
    g.e.slots = a.slots;
    g.e.req_L = a.req_L;
    g.e.req_ntok = a.req_ntok;
    g.e.T = a.T;
    g.e.H = a.H;
    g.e.hd = a.hd;
    g.e.page_elems = a.page_elems;
    g.e.row_kv = a.row_kv;
    proj_task<CL, PG_QKV, EPI_QKV, 5>(a, g, j, slot_cnt(a, l, PH_LN1), 1, false,
                                      slot_cnt(a, l, PH_QKV), smem);
}

template <int CL>
WF_TASK void task_o(uint64_t kp, int l, int j, char *smem) {
    PA a = pass_args(kp);
    const LayerW &w = a.lw[l];
    const int d = a.d;
    const size_t act = (size_t)l * a.act_stride;
    (void)act;
    GemmArgs g = gemm_args(a, PG_O, a.sav + act, d, d, w.wo, nullptr, nullptr, d);
    g.e.b0 = w.bo;
    g.e.x_in = a.xv + (size_t)(3 * l) * a.x_stride;
    g.e.x = a.xv + (size_t)(3 * l + 1) * a.x_stride;
    proj_task<CL, PG_O, EPI_RESID, 5>(a, g, j, slot_cnt(a, l, PH_SA), a.H, true,
                                      slot_cnt(a, l, PH_O), smem);
}

template <int CL>
WF_TASK void task_cq(uint64_t kp, int l, int j, char *smem) {
    PA a = pass_args(kp);
    const LayerW &w = a.lw[l];
    const int d = a.d;
    const size_t act = (size_t)l * a.act_stride;
    (void)act;
    GemmArgs g = gemm_args(a, PG_CQ, a.lnv + (size_t)(3 * l + 1) * a.act_stride, d, d,
                           w.wqc, nullptr, nullptr, d);
    g.e.b0 = w.bqc;
    g.e.out = a.cqv + (size_t)l * a.q_stride;
    proj_task<CL, PG_CQ, EPI_F16, 5>(a, g, j, slot_cnt(a, l, PH_LN2), 1, false,
                                     slot_cnt(a, l, PH_CQ), smem);
}

template <int CL>
WF_TASK void task_oc(uint64_t kp, int l, int j, char *smem) {
    PA a = pass_args(kp);
    const LayerW &w = a.lw[l];
    const int d = a.d;
    const size_t act = (size_t)l * a.act_stride;
    (void)act;
    GemmArgs g = gemm_args(a, PG_OC, a.xav + act, d, d, w.woc, nullptr, nullptr, d);
    g.e.b0 = w.boc;
    g.e.x_in = a.xv + (size_t)(3 * l + 1) * a.x_stride;
    g.e.x = a.xv + (size_t)(3 * l + 2) * a.x_stride;
    proj_task<CL, PG_OC, EPI_RESID, 5>(a, g, j, slot_cnt(a, l, PH_XA), a.H, true,
                                       slot_cnt(a, l, PH_OC), smem);
}

template <int CL>
WF_TASK void task_fc1(uint64_t kp, int l, int j, char *smem) {
    PA a = pass_args(kp);
    const LayerW &w = a.lw[l];
    const int d = a.d;
    const size_t act = (size_t)l * a.act_stride;
    (void)act;
    GemmArgs g = gemm_args(a, PG_FC1, a.lnv + (size_t)(3 * l + 2) * a.act_stride, d, a.F,
                           w.w1, nullptr, nullptr, a.F);
    g.e.b0 = w.b1;
    g.e.out = a.hsv + (size_t)l * a.hs_stride;
    proj_task<CL, PG_FC1, EPI_GELU, 5>(a, g, j, slot_cnt(a, l, PH_LN3), 1, false,
                                       slot_cnt(a, l, PH_FC1), smem);
}

template <int CL>
WF_TASK void task_fc2(uint64_t kp, int l, int j, char *smem) {
    PA a = pass_args(kp);
    const LayerW &w = a.lw[l];
    const int d = a.d;
    const size_t act = (size_t)l * a.act_stride;
    (void)act;
    GemmArgs g = gemm_args(a, PG_FC2, a.hsv + (size_t)l * a.hs_stride, a.F, d, w.w2,
                           nullptr, nullptr, d);
    g.e.b0 = w.b2;
    g.e.x_in = a.xv + (size_t)(3 * l + 2) * a.x_stride;
    g.e.x = a.xv + (size_t)(3 * l + 3) * a.x_stride;
    proj_task<CL, PG_FC2, EPI_RESID, 20>(a, g, j, slot_cnt(a, l, PH_FC1),
                                         a.g[PG_FC1].n_tiles, false,
                                         slot_cnt(a, l, PH_FC2), smem);
}

template <int CL>
__global__ __launch_bounds__(kThreads) void pass_kernel(PassArgs args) {
    // at least 82 KB: one workgroup per CU whatever the class's tiles need
    __shared__ __attribute__((aligned(16))) char smem[cmax(pass_lds<CL>(), 82 * 1024)];
    const int total = args.total;
    const uint64_t kp = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        PA a = pass_args(kp);
        const long long t0 = a.trace ? clock100() : 0;
        if (a.trace && threadIdx.x == 0) g_t_ready = t0;
        run_task<CL>(a, kp, t, smem);
        __syncthreads();   // the task's LDS is free for the next one
        if (a.trace && threadIdx.x == 0) {
            a.trace[4 * (size_t)t] = (uint64_t)t0;
            a.trace[4 * (size_t)t + 1] = (uint64_t)g_t_ready;
            a.trace[4 * (size_t)t + 2] = (uint64_t)clock100();
            a.trace[4 * (size_t)t + 3] = (uint64_t)blockIdx.x;
        }
    }
}

__global__ void fill_i32_kernel(int32_t *p, int n, int32_t v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace

int pass_class_of_rows(int M) { return M <= 16 ? 0 : (M <= 96 ? 1 : 2); }

// Host side of the class tilings: rows and columns per task and K groups.
void pass_tiling(int cl, int pg, int &bm, int &bn, int &groups) {
    auto set = [&](int mb, int nb, int wn) {
        bm = 16 * mb;
        bn = 16 * nb * wn;
        groups = 8 / (8 / wn);
    };
#define WF_PT(C, P)                                                                   \
    if (cl == C && pg == P) {                                                         \
        set(Tile<C, P>::MB, Tile<C, P>::NB, Tile<C, P>::WN);                          \
        return;                                                                       \
    }
#define WF_PT_ALL(C) WF_PT(C, PG_QKV) WF_PT(C, PG_O) WF_PT(C, PG_CQ) WF_PT(C, PG_OC) \
                     WF_PT(C, PG_FC1) WF_PT(C, PG_FC2) WF_PT(C, PG_LMH)
    WF_PT_ALL(0)
    WF_PT_ALL(1)
    WF_PT_ALL(2)
#undef WF_PT_ALL
#undef WF_PT
    bm = bn = groups = 0;
}

hipError_t launch_pass(const PassArgs &a, int cl, int grid, hipStream_t st) {
    if (a.RT > 64 || a.hd != kHd || a.d > 16 * 8 * LN_GPL) return hipErrorInvalidValue;
    switch (cl) {
        case 0: hipLaunchKernelGGL(pass_kernel<0>, dim3(grid), dim3(kThreads), 0, st, a); break;
        case 1: hipLaunchKernelGGL(pass_kernel<1>, dim3(grid), dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(pass_kernel<2>, dim3(grid), dim3(kThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

}  // namespace wf
