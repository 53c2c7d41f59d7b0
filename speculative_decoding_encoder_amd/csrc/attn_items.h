// Attention kernels on fp16 MFMA (16x16x32, fp32 accumulate).
//
// Both kernels process a 16-row tile of one request's queries for one head
// and walk the keys in 32-key steps with an online softmax (running max m,
// running sum l, rescaled output o). Step boundaries are absolute key
// indices, so a row's result does not depend on how many other rows share
// its tile: a block of K+1 rows and K+1 single-row passes give the same bits.
//
// Both compute the transposed products, so that a lane owns one query row and
// the probabilities never leave its registers:
//  S^T = K Q^T : A = 16 keys x 32 dims, B = Q^T; lane (g, r16) gets row r16's
//                scores for keys 4g..4g+3 of each 16-key tile.
//  O^T += V^T P^T : A = V^T (16 dims x 32 keys), B = P^T, which is those 8
//                probabilities packed as they are (keys 4g..4g+3 of each
//                tile). Lane (g, r16) accumulates row r16, dims 4g..4g+3 of
//                each 16-dim tile.
// Row max and sum take a local pass over 8 values and two lane exchanges.
//
// Self-attention reads the paged cache: a page holds 16 positions; K is
// [head][16][hd] and V is stored transposed, [head][hd][16], so that a V^T
// operand is two 8-byte loads (positions 4g..4g+3 of the step's two pages).
// Tree verification ("Alignment Drift ...", App. E.3) replaces the in-block
// causal mask with each node's ancestors (and itself): node i's K/V sit at
// cache slot L+i, and row i sees block key L+j only where bit j of its
// ancestor mask is set (node 0, the root, at L is everyone's ancestor).
// Row i of the block (position L+i) sees the cached prefix and the block rows
// up to itself, keys 0..L+i: the anchor and the candidates go through the
// target in one causal pass (Whisper-Flash section 3.1).
//
// Cross-attention reads the write-once pool: K steps in MFMA operand order
// and V [head][F_pad / 32][hd][32], the transposed V of each 32-frame step one
// contiguous block with its frames in the order of the score tiles (block
// position 8g + j holds frame 4g + j for j < 4, frame 16 + 4g + j - 4
// otherwise), so that every operand load reads consecutive addresses.
//
// A workgroup is four waves. In self-attention they split the 32-key steps
// of one (request, head, 16-row tile) by absolute step index (wave w takes
// steps w, w+4, ...); in cross-attention each wave takes one chunk of frames
// and a workgroup four consecutive chunks. The waves' (m, l, o) partials
// meet in LDS as ((w0+w1)+(w2+w3)); cross-attention workgroups of one tile
// meet the same way through device-coherent scratch (the last to arrive
// merges). A partial that saw only masked keys has m = -inf and weight 0, so
// steps or chunks a row cannot see leave its bits unchanged.
#pragma once
#include "wf_device.h"
#include "wf_internal.h"
namespace wf {

template <int HD>
struct QFrag {
    u32x4 a[2];   // HD = 64: dims 8g..8g+7 and 32+8g..32+8g+7
    u32x2 h;      // HD = 16: dims 4g..4g+3
};

template <int HD>
__device__ __forceinline__ QFrag<HD> load_q(const uint16_t *qrow, bool ok, int g) {
    QFrag<HD> f;
    if constexpr (HD == 64) {
        f.a[0] = ok ? ld16(qrow + 8 * g) : u32x4{0u, 0u, 0u, 0u};
        f.a[1] = ok ? ld16(qrow + 32 + 8 * g) : u32x4{0u, 0u, 0u, 0u};
    } else {
        f.h = ok ? ld8(qrow + 4 * g) : u32x2{0u, 0u};
    }
    return f;
}

// element (row, c) of a fragment-tiled fp16 activation buffer of width K
__device__ __forceinline__ void store_act(uint16_t *out, int row, int c, int K, float v) {
    out[xh_index(row, c, K)] = f2h_bits(v);
}

// K and V^T fragments of one 32-key step.
template <int HD>
struct KVStep {
    u32x4 k[2][2];     // HD = 64: [16-key tile][dim half]
    u32x2 k16[2];      // HD = 16
    u32x4 v[HD / 16];  // V^T: 16 dims x 8 keys per lane
};

// ---------------------------------------------------------------------------
// Transposed online softmax (cross-attention): the running state of query row
// r16, its output for dims dt * 16 + 4g + r.
template <int NDT>
struct SmRow {
    float m, l;
    f32x4 o[NDT];
    __device__ __forceinline__ void init() {
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
};

// One 32-key step (keys key0 .. key0 + 31). Scores stay unscaled: the
// running max m is in raw score units and every weight is
// 2^((s - m) * sl2e), sl2e = scale * log2(e). MASK (a step some row cannot
// see whole): keys >= live_to (this lane's row) get weight 0 and keys >=
// vlive_to (past the data) a zero V operand; other steps skip the masking
// and the -inf guards (their scores are finite). TREE (tree verification):
// block keys tree_L + j also need bit j of the row's ancestor mask anc.
template <int HD, bool MASK, bool TREE = false>
__device__ __forceinline__ void attend_step_t(const QFrag<HD> &q, const KVStep<HD> &f, int key0,
                                              int live_to, int vlive_to, float sl2e,
                                              SmRow<HD / 16> &st, int g, uint64_t anc = ~0ull,
                                              int tree_L = 0) {
    constexpr int NDT = HD / 16;
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (HD == 64) {
            s[t] = mfma_f16_k32(f.k[t][0], q.a[0], s[t]);
            s[t] = mfma_f16_k32(f.k[t][1], q.a[1], s[t]);
        } else {
            s[t] = mfma_f16_k16(f.k16[t], q.h, s[t]);
        }
        if constexpr (MASK) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * t + 4 * g + r;
                bool dead = key >= live_to;
                if constexpr (TREE) {
                    const int j = key - tree_L;
                    dead = dead || (j >= 0 && j < 64 && !((anc >> j) & 1ull));
                }
                if (dead) s[t][r] = -INFINITY;
            }
        }
    }
    float tm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    {
        float a, b;
        rows16_pair(tm, a, b);
        halves32_pair(fmaxf(a, b), a, b);
        tm = fmaxf(a, b);
    }
    const float mnew = fmaxf(st.m, tm);
    const float ms = mnew * sl2e;
    // unmasked steps: mnew is finite, and st.m = -inf (first step) gives 0
    const float alpha = (MASK && mnew == -INFINITY) ? 0.f
                                                    : __builtin_amdgcn_exp2f(__fmaf_rn(st.m, sl2e, -ms));
    float p[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            p[t][r] = (MASK && s[t][r] == -INFINITY) ? 0.f
                                                      : __builtin_amdgcn_exp2f(__fmaf_rn(s[t][r], sl2e, -ms));
    float ls = ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
               ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
    {
        float a, b;                           // the four lanes of a row agree
        rows16_pair(ls, a, b);
        halves32_pair(a + b, a, b);
        ls = a + b;
    }
    st.l = alpha * st.l + ls;
    st.m = mnew;
    const u32x4 pb = {pack_h2(p[0][0], p[0][1]), pack_h2(p[0][2], p[0][3]),
                      pack_h2(p[1][0], p[1][1]), pack_h2(p[1][2], p[1][3])};
    u32x4 vm = {~0u, ~0u, ~0u, ~0u};
    if constexpr (MASK) {
        // block positions 8g + 2w, 8g + 2w + 1 of dead frames: zero operand
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int fr = key0 + (w < 2 ? 4 * g + 2 * w : 16 + 4 * g + 2 * (w - 2));
            vm[w] = (fr < vlive_to ? 0x0000ffffu : 0u) | (fr + 1 < vlive_to ? 0xffff0000u : 0u);
        }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        st.o[dt] *= alpha;
        st.o[dt] = mfma_f16_k32(MASK ? (f.v[dt] & vm) : f.v[dt], pb, st.o[dt]);
    }
}

// Partial (o, m, l) of 16 rows in LDS, rows of HD + 4 floats.
template <int HD, int NDT>
__device__ __forceinline__ void put_row(float *buf, const SmRow<NDT> &s, int g, int r16) {
    constexpr int PW = HD + 4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(&buf[r16 * PW + dt * 16 + 4 * g]) = s.o[dt];
    if (g == 0) {
        buf[r16 * PW + HD] = s.m;
        buf[r16 * PW + HD + 1] = s.l;
    }
}
// s = s (+) partial in buf: rescale both to the larger running max.
template <int HD, int NDT>
__device__ __forceinline__ void merge_row(SmRow<NDT> &s, const float *buf, float sl2e, int g,
                                          int r16) {
    constexpr int PW = HD + 4;
    const float mb = buf[r16 * PW + HD], lb = buf[r16 * PW + HD + 1];
    const float M = fmaxf(s.m, mb);
    const float wa = (s.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((s.m - M) * sl2e);
    const float wb = (mb == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mb - M) * sl2e);
    s.l = s.l * wa + lb * wb;
    s.m = M;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        s.o[dt] = s.o[dt] * wa + *reinterpret_cast<const f32x4 *>(&buf[r16 * PW + dt * 16 + 4 * g]) * wb;
}
// ((w0+w1)+(w2+w3)) over the four waves; the result lands in wave 0.
template <int HD, int NDT>
__device__ __forceinline__ void merge_waves_t(SmRow<NDT> &s, float (*mbuf)[16 * (HD + 4)],
                                              float sl2e, int wave, int g, int r16) {
    if (wave & 1) put_row<HD>(mbuf[wave >> 1], s, g, r16);
    __syncthreads();
    if (!(wave & 1)) merge_row<HD>(s, mbuf[wave >> 1], sl2e, g, r16);
    __syncthreads();
    if (wave == 2) put_row<HD>(mbuf[0], s, g, r16);
    __syncthreads();
    if (wave == 0) merge_row<HD>(s, mbuf[0], sl2e, g, r16);
}


// ---------------------------------------------------------------------------
// Self-attention over the paged KV cache, causal inside the block (or over
// the whole block, causal = 0): one item (request, head, 16-row tile) on the
// four waves w4 = 0..3 of a wave group. A workgroup may run another item on
// its other waves, so every call runs the same three workgroup barriers (the
// wave merge) whatever the item; valid = false runs the barriers only.
template <int HD, bool TREE>
__device__ __forceinline__ void self_attn_item(const SelfAttnArgs &a, int bh, int mtile,
                                               bool valid, int w4,
                                               float (*mbuf)[16 * (HD + 4)]) {
    constexpr int NDT = HD / 16;
    const int lane = threadIdx.x & 63, t4 = w4 * 64 + lane;
    const int r16 = lane & 15, g = lane >> 4;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int row0 = mtile * 16;
    const int ntok = valid ? a.req_ntok[b] : 0;
    const bool live = valid && ntok > 0 && row0 < ntok;
    if (valid && !live) {
        // skipped request or a tile of padding rows: zeros
        for (int idx = t4; idx < 16 * HD; idx += 256) {
            const int rr = idx / HD, c = idx - rr * HD;
            const int row = row0 + rr;
            if (row < a.T) store_act(a.out, b * a.T + row, h * HD + c, a.d, 0.f);
        }
    }
    SmRow<NDT> st;
    st.init();
    const float sl2e = a.scale * 1.4426950408889634f;
    const int qrow = row0 + r16;
    // the request's length and slot and this tile's queries go out together
    // with n_tok (in bounds for any request of the batch), so the chain to
    // the first K/V load is the page table only
    const int L = a.req_L[b];
    const int slot = a.slots[b];
    const QFrag<HD> q = load_q<HD>(a.q + (size_t)(b * a.T + qrow) * a.d + h * HD, qrow < a.T, g);
    if (live) {
        // last key any row of this tile may see (the whole block when not causal)
        const int kmax = a.causal ? L + min(row0 + 15, ntok - 1) : L + ntok - 1;
        // this lane's row r16 sees keys <= lim; keys below mask_from every row sees
        const int lim = a.causal ? L + min(row0 + r16, ntok - 1) : kmax;
        // tree verification: a row sees its ancestors among block keys L + 1 ..
        // (key L, the root, is every row's ancestor)
        const int mask_from = TREE ? L + 1 : (a.causal ? L + min(row0, ntok - 1) : kmax) + 1;
        const int last_page = kmax >> 4;   // pages past this one were never validated
        // the request's page ids, one per lane (at most 64 pages)
        const int32_t *pt = a.page_table + (size_t)slot * a.pt_stride;
        const int ptl = lane <= last_page ? pt[lane] : 0;
        const uint64_t anc = TREE ? a.anc[(size_t)b * a.T + min(qrow, a.T - 1)] : ~0ull;

        const uint16_t *kvl = a.kv_layer;
        const size_t vt_off = (size_t)a.H * 16 * HD;
        // step j: keys 32j .. 32j+31 on pages 2j, 2j+1. K tile t as the A
        // operand of S^T = K Q^T; V^T as the A operand of O^T += V^T P^T,
        // positions 4g..4g+3 of each page (the order the score tiles leave P in)
        auto load = [&](int j, KVStep<HD> &f) {
            int page[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                page[t] = __shfl(ptl, min(2 * j + t, last_page));
                const uint16_t *krow =
                    kvl + (size_t)page[t] * a.page_elems + ((size_t)h * 16 + r16) * HD;
                if constexpr (HD == 64) {
                    f.k[t][0] = ld16(krow + 8 * g);
                    f.k[t][1] = ld16(krow + 32 + 8 * g);
                } else {
                    f.k16[t] = ld8(krow + 4 * g);
                }
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const size_t dim_off = vt_off + ((size_t)h * HD + dt * 16 + r16) * 16 + 4 * g;
                const u32x2 lo = ld8(kvl + (size_t)page[0] * a.page_elems + dim_off);
                const u32x2 hi = ld8(kvl + (size_t)page[1] * a.page_elems + dim_off);
                f.v[dt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        };
        const int nsteps = (kmax >> 5) + 1;             // absolute 32-key steps
        KVStep<HD> cur, nxt;
        if (w4 < nsteps) load(w4, cur);
        for (int j = w4; j < nsteps; j += 4) {
            load(min(j + 4, nsteps - 1), nxt);        // unconditional: exact wait counts
            const int key0 = 32 * j;
            if (key0 + 32 > mask_from)
                attend_step_t<HD, true, TREE>(q, cur, key0, lim + 1, kmax + 1, sl2e, st, g, anc,
                                              L);
            else attend_step_t<HD, false>(q, cur, key0, lim + 1, kmax + 1, sl2e, st, g);
            cur = nxt;
        }
    }
    merge_waves_t<HD>(st, mbuf, sl2e, w4, g, r16);
    if (live && w4 == 0 && qrow < a.T) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_act(a.out, b * a.T + qrow, h * HD + dt * 16 + 4 * g + r, a.d,
                          st.o[dt][r] / st.l);
    }
}

// ---------------------------------------------------------------------------
// Cross-attention over the write-once pool: one item (request, head, 16-row
// tile, chunk group) on the four waves w4 = 0..3 of a wave group; wave w4
// takes chunk 4 * group + w4 of cf frames (spw 32-frame steps, a multiple of
// the load ring depth kXaRing). Every call runs the same workgroup barriers
// whatever the item (three for the wave merge, one more when there are
// chunk groups); valid = false runs the barriers only. Returns true for
// exactly one item of each (request, head, tile) once its output is final:
// with one group, that item; with several, the last group to arrive, which
// merges them; for a skipped request, group 0.
// SPW > 0: the chunk length is a compile-time a.spw and the step loop is
// straight-line code (the compiler's wait counts then keep kXaRing - 1
// steps in flight; across a loop back-edge it waits for the whole ring).
template <int HD, int SPW>
__device__ __forceinline__ bool cross_attn_item(const CrossAttnArgs &a, int item, bool valid,
                                                int w4, float (*mbuf)[16 * (HD + 4)],
                                                int *last) {
    constexpr int NDT = HD / 16;
    const int lane = threadIdx.x & 63, t4 = w4 * 64 + lane;
    const int r16 = lane & 15, g = lane >> 4;
    const int grp = item % a.G;
    const int bhm = item / a.G;               // (b * H + h) * mt + mtile
    const int mtile = bhm % a.mt;
    const int bh = bhm / a.mt;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int ntok = valid ? a.req_ntok[b] : 0;
    const bool live = valid && ntok > 0;
    const int row0 = mtile * 16;
    const int qrow = row0 + r16;
    const float sl2e = a.scale * 1.4426950408889634f;

    SmRow<NDT> st;
    st.init();
    // the slot and this tile's queries go out together with n_tok (in bounds
    // for any request of the batch)
    const int slot = a.slots[b];
    const QFrag<HD> q = load_q<HD>(a.q + (size_t)(b * a.T + qrow) * a.d + h * HD, qrow < a.T, g);
    if (live) {
        const uint16_t *base = a.xkv + (size_t)slot * a.slot_stride + a.layer_off;
        const uint16_t *kh = base + (size_t)h * a.F_pad * HD;
        const uint16_t *vh = base + (size_t)a.H * a.F_pad * HD + (size_t)h * a.F_pad * HD;

        const int c0 = (grp * 4 + w4) * a.cf;          // first frame of this wave's chunk
        const int c1 = min(c0 + a.cf, a.F);            // end of its live frames
        const int last_fb = a.F_pad - 32;              // loads stay inside this head's frames
        auto load = [&](int s, KVStep<HD> &f) {
            const int fb = min(c0 + 32 * s, last_fb);
            const uint16_t *kstep = kh + (size_t)(fb >> 5) * 32 * HD;   // fragment-order K block
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if constexpr (HD == 64) {
                    f.k[t][0] = ld16_nt(kstep + (t * 2 + 0) * 512 + lane * 8);
                    f.k[t][1] = ld16_nt(kstep + (t * 2 + 1) * 512 + lane * 8);
                } else {
                    f.k16[t] = ld8_nt(kstep + t * 256 + lane * 4);
                }
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                f.v[dt] = ld16_nt(vh + ((size_t)(fb >> 5) * HD + dt * 16 + r16) * 32 + 8 * g);
        };
        KVStep<HD> f[kXaRing];
#pragma unroll
        for (int i = 0; i < kXaRing; ++i) load(i, f[i]);
        // the refill is unconditional (past the chunk: its last step again, an
        // L2 hit) and pinned after the step
        auto two = [&](int s0) {
#pragma unroll
            for (int i = 0; i < kXaRing; ++i) {
                const int key0 = c0 + 32 * (s0 + i);
                if (key0 + 32 > c1) attend_step_t<HD, true>(q, f[i], key0, c1, c1, sl2e, st, g);
                else attend_step_t<HD, false>(q, f[i], key0, c1, c1, sl2e, st, g);
                __builtin_amdgcn_sched_barrier(0);
                load(min(s0 + i + kXaRing, a.spw - 1), f[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if constexpr (SPW > 0) {
#pragma unroll
            for (int s0 = 0; s0 < SPW; s0 += kXaRing) two(s0);
        } else {
            for (int s0 = 0; s0 < a.spw; s0 += kXaRing) two(s0);
        }
    }
    merge_waves_t<HD>(st, mbuf, sl2e, w4, g, r16);

    if (a.G == 1) {
        if (live && w4 == 0 && qrow < a.T) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    store_act(a.out, b * a.T + qrow, h * HD + dt * 16 + 4 * g + r, a.d,
                              st.o[dt][r] / st.l);
        }
        return valid;
    }
    // publish this group's (o, m, l) rows; the last group to arrive merges
    constexpr int GPW = HD + 4;                   // o[HD], m, l, 2 spare: 16-byte rows
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (size_t)(item - grp) * 16 * GPW, 0, 0x7fffffff, 0x00020000);
    if (live && w4 == 0) {
        const int gb = grp * 16 * GPW * 4;        // this group's bytes
        if (g == 0)
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{__float_as_uint(st.m), __float_as_uint(st.l)}, rs,
                gb + (r16 * GPW + HD) * 4, 0, CPOL_SC1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, st.o[dt]), rs,
                                                   gb + (r16 * GPW + dt * 16 + 4 * g) * 4, 0,
                                                   CPOL_SC1);
        wait_vmem();
        int prev = 0;
        if (lane == 0) prev = arrive(&a.cnt[bhm]);
        prev = __shfl(prev, 0);
        if (lane == 0) *last = (prev == a.G - 1);
    }
    __syncthreads();
    if (!live) return valid && grp == 0;
    if (!*last) return false;
    if (t4 == 0) rearm(&a.cnt[bhm]);
    // thread: row rr, HD/16 consecutive dims; every group's (m, l) and o
    // values load at once. Per row: M = max_g m_g, w_g = exp(m_g - M), and
    // L = sum_g l_g w_g, o = sum_g o_g w_g in the pairwise tree over 8
    // groups (missing groups add zero).
    constexpr int DPT = HD / 16;
    const int rr = t4 >> 4, d0 = (t4 & 15) * DPT;
    u32x2 ml[8];
    float ov[8][DPT];
#pragma unroll
    for (int q2 = 0; q2 < 8; ++q2) {
        if (q2 < a.G) {
            const int gb = (q2 * 16 * GPW + rr * GPW) * 4;
            ml[q2] = __builtin_amdgcn_raw_buffer_load_b64(rs, gb + HD * 4, 0, CPOL_SC1);
            if constexpr (DPT == 4) {
                const u32x4 v =
                    __builtin_amdgcn_raw_buffer_load_b128(rs, gb + d0 * 4, 0, CPOL_SC1);
#pragma unroll
                for (int k = 0; k < 4; ++k) ov[q2][k] = __uint_as_float(v[k]);
            } else {
#pragma unroll
                for (int k = 0; k < DPT; ++k)
                    ov[q2][k] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(rs, gb + (d0 + k) * 4, 0, CPOL_SC1));
            }
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int q2 = 0; q2 < 8; ++q2)
        if (q2 < a.G) M = fmaxf(M, __uint_as_float(ml[q2][0]));
    float lw[8], ow[8][DPT];
#pragma unroll
    for (int q2 = 0; q2 < 8; ++q2) {
        float w = 0.f;
        if (q2 < a.G) {
            const float mg = __uint_as_float(ml[q2][0]);
            w = (mg == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mg - M) * sl2e);
        }
        lw[q2] = q2 < a.G ? __uint_as_float(ml[q2][1]) * w : 0.f;
#pragma unroll
        for (int k = 0; k < DPT; ++k) ow[q2][k] = q2 < a.G ? ov[q2][k] * w : 0.f;
    }
    auto tree8 = [](const float (&v)[8]) {
        return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    };
    const float L = tree8(lw);
    const int row = row0 + rr;
    if (row < a.T) {
#pragma unroll
        for (int k = 0; k < DPT; ++k) {
            const float t[8] = {ow[0][k], ow[1][k], ow[2][k], ow[3][k],
                                ow[4][k], ow[5][k], ow[6][k], ow[7][k]};
            store_act(a.out, b * a.T + row, h * HD + d0 + k, a.d, tree8(t) / L);
        }
    }
    return true;
}

}  // namespace wf
