// Attention kernels on fp16 MFMA (16x16x32, fp32 accumulate).
//
// Both kernels process a 16-row tile of one request's queries for one head
// and walk the keys in 32-key steps with an online softmax (running max m,
// running sum l, rescaled output o). Step boundaries are absolute key
// indices, so a row's result does not depend on how many other rows share
// its tile: a block of K+1 rows and K+1 single-row passes give the same bits.
//
//  S = Q K^T : A = Q rows (16 x 32 dims per MFMA), B = 16 keys.
//  O += P V  : A = P (16 rows x 32 keys, fp16, staged through LDS to change
//              from the C layout to the A layout), B = V^T (16 dims x 32 keys).
//
// Self-attention reads the paged cache: a page holds 16 positions; K is
// [head][16][hd] and V is stored transposed, [head][hd][16], so that both
// MFMA B operands are contiguous 16-byte loads. Row i of the block (position
// L+i) sees keys 0..L+i ("one causal target pass over the anchor and the
// candidates", Whisper-Flash section 3.1).
//
// Cross-attention reads the write-once pool (K [head][F_pad][hd], V^T
// [head][hd][F_pad]); the frames are split into chunks handled by separate
// waves, whose (m, l, o) partials are merged in chunk order by the last wave
// to finish.
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

// 16x16 score tile: rows of Q against the 16 keys whose rows start at krow
// (this lane's key row; lane r16 loads key r16).
template <int HD>
__device__ __forceinline__ f32x4 qk_tile(const QFrag<HD> &q, const uint16_t *krow, int g) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (HD == 64) {
        s = mfma_f16_k32(q.a[0], ld16(krow + 8 * g), s);
        s = mfma_f16_k32(q.a[1], ld16(krow + 32 + 8 * g), s);
    } else {
        s = mfma_f16_k16(q.h, ld8(krow + 4 * g), s);
    }
    return s;
}

// Online-softmax update for the 4 rows a lane holds (C layout rows 4g+r)
// given two 16-key score tiles already scaled and masked (-inf = masked).
// Writes the fp16 probabilities into this wave's LDS tile P[16][32].
template <int NDT>
__device__ __forceinline__ void softmax_step(f32x4 &s0, f32x4 &s1, float (&mrun)[4],
                                             float (&lrun)[4], f32x4 (&o)[NDT],
                                             uint16_t *P, int g, int r16) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float tm = max16(fmaxf(s0[r], s1[r]));
        const float mnew = fmaxf(mrun[r], tm);
        const float alpha = (mnew == -INFINITY) ? 0.f : __expf(mrun[r] - mnew);
        const float p0 = (s0[r] == -INFINITY) ? 0.f : __expf(s0[r] - mnew);
        const float p1 = (s1[r] == -INFINITY) ? 0.f : __expf(s1[r] - mnew);
        lrun[r] = alpha * lrun[r] + sum16(p0 + p1);
        mrun[r] = mnew;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt][r] *= alpha;
        const int row = 4 * g + r;
        P[row * 32 + r16] = f2h_bits(p0);
        P[row * 32 + 16 + r16] = f2h_bits(p1);
    }
}

__device__ __forceinline__ void store_split(uint16_t *out, size_t row_off, int c, float v) {
    uint16_t hi, lo;
    split_bf16(v, hi, lo);
    const size_t base = row_off + (size_t)(c >> 3) * 16 + (c & 7);
    out[base] = hi;
    out[base + 8] = lo;
}

// ---------------------------------------------------------------------------
// Self-attention over the paged KV cache, causal inside the block.
// grid = (n * H, ceil(T / 16)), block = one wave.
template <int HD>
__global__ __launch_bounds__(64) void self_attn_kernel(SelfAttnArgs a) {
    constexpr int NDT = HD / 16;
    __shared__ __attribute__((aligned(16))) uint16_t P[16 * 32];
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    const int b = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
    const int row0 = blockIdx.y * 16;
    const int ntok = a.req_ntok[b];
    const size_t ld_out = (size_t)2 * a.d;

    if (ntok == 0 || row0 >= ntok) {
        // skipped request or a tile of padding rows: zeros
        for (int idx = lane; idx < 16 * HD; idx += 64) {
            const int rr = idx / HD, c = idx - rr * HD;
            const int row = row0 + rr;
            if (row < a.T) store_split(a.out, (size_t)(b * a.T + row) * ld_out, h * HD + c, 0.f);
        }
        return;
    }
    const int L = a.req_L[b];
    const int32_t *pt = a.page_table + (size_t)a.slots[b] * a.pt_stride;
    const int qrow = row0 + r16;
    const QFrag<HD> q = load_q<HD>(a.q + (size_t)(b * a.T + qrow) * a.d + h * HD, qrow < a.T, g);

    // last key any row of this tile may see (the whole block when not causal)
    const int kmax = a.causal ? L + min(row0 + 15, ntok - 1) : L + ntok - 1;
    int lim[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lim[r] = a.causal ? L + min(row0 + 4 * g + r, ntok - 1) : kmax;

    float mrun[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float lrun[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t *kvl = a.kv_layer;
    const size_t vt_off = (size_t)a.H * 16 * HD;
    const int last_page = kmax >> 4;   // pages past this one were never validated

    for (int kb = 0; kb <= kmax; kb += 32) {
        f32x4 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int lp = (kb >> 4) + t;
            if (lp <= last_page) {
                const int page = pt[lp];
                const uint16_t *krow =
                    kvl + (size_t)page * a.page_elems + ((size_t)h * 16 + r16) * HD;
                s[t] = qk_tile<HD>(q, krow, g);
            } else {
                s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kb + 16 * t + r16;
                s[t][r] = (key <= lim[r]) ? s[t][r] * a.scale : -INFINITY;
            }
        }
        softmax_step<NDT>(s[0], s[1], mrun, lrun, o, P, g, r16);
        __syncthreads();
        const u32x4 pa = *reinterpret_cast<const u32x4 *>(&P[r16 * 32 + 8 * g]);
        const int vkey = kb + 8 * g;                 // this lane's 8 keys
        const bool vlive = (vkey >> 4) <= last_page;
        const int vpage = vlive ? pt[vkey >> 4] : 0;
        const bool tail = (vkey + 8 > kmax + 1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const uint16_t *vp = kvl + (size_t)vpage * a.page_elems + vt_off +
                                 ((size_t)h * HD + dt * 16 + r16) * 16 + (vkey & 15);
            u32x4 vb = vlive ? ld16(vp) : u32x4{0u, 0u, 0u, 0u};
            if (tail) {   // keys past the last live one: zero the operand
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k0 = vkey + 2 * j;
                    uint32_t w = vb[j];
                    if (k0 > kmax) w &= 0xffff0000u;
                    if (k0 + 1 > kmax) w &= 0x0000ffffu;
                    vb[j] = w;
                }
            }
            o[dt] = mfma_f16_k32(pa, vb, o[dt]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + 4 * g + r;
            if (row < a.T)
                store_split(a.out, (size_t)(b * a.T + row) * ld_out, h * HD + dt * 16 + r16,
                            o[dt][r] / lrun[r]);
        }
}

// ---------------------------------------------------------------------------
// Cross-attention over the write-once audio K/V. One wave (one workgroup)
// per item (request, head, m-tile, frame chunk).
template <int HD>
__global__ __launch_bounds__(64) void cross_attn_kernel(CrossAttnArgs a) {
    constexpr int NDT = HD / 16;
    constexpr int PW = HD + 2;   // partial row: m, l, o[HD]
    __shared__ __attribute__((aligned(16))) uint16_t P[16 * 32];
    const int lane = threadIdx.x;
    const int r16 = lane & 15, g = lane >> 4;
    const int item = blockIdx.x;
    const int ch = item % a.nch;
    const int bhm = item / a.nch;            // (b * H + h) * mt + mtile
    const int mtile = bhm % a.mt;
    const int bh = bhm / a.mt;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int ntok = a.req_ntok[b];
    if (ntok == 0) return;                   // every chunk of this request skips
    const int row0 = mtile * 16;
    const size_t ld_out = (size_t)2 * a.d;

    const uint16_t *base = a.xkv + (size_t)a.slots[b] * a.slot_stride + a.layer_off;
    const uint16_t *kh = base + (size_t)h * a.F_pad * HD;
    const uint16_t *vh = base + (size_t)a.H * a.F_pad * HD + (size_t)h * HD * a.F_pad;

    const int qrow = row0 + r16;
    const QFrag<HD> q = load_q<HD>(a.q + (size_t)(b * a.T + qrow) * a.d + h * HD, qrow < a.T, g);

    float mrun[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float lrun[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int f0 = ch * a.cf;
    const int f1 = min(f0 + a.cf, a.F);
    // K/V fragments of one 32-frame step; the next step is loaded while the
    // current one is computed
    struct KV {
        u32x4 k[2][2];     // [16-frame tile][dim half] (HD = 64)
        u32x2 k16[2];      // HD = 16
        u32x4 v[NDT];
    };
    auto load_kv = [&](int fb, KV &f) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint16_t *krow = kh + (size_t)(fb + 16 * t + r16) * HD;
            if constexpr (HD == 64) {
                f.k[t][0] = ld16(krow + 8 * g);
                f.k[t][1] = ld16(krow + 32 + 8 * g);
            } else {
                f.k16[t] = ld8(krow + 4 * g);
            }
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            f.v[dt] = ld16(vh + (size_t)(dt * 16 + r16) * a.F_pad + fb + 8 * g);
    };
    KV cur, nxt;
    load_kv(f0, cur);
    for (int fb = f0; fb < f1; fb += 32) {
        if (fb + 32 < f1) load_kv(fb + 32, nxt);
        f32x4 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (HD == 64) {
                s[t] = mfma_f16_k32(q.a[0], cur.k[t][0], s[t]);
                s[t] = mfma_f16_k32(q.a[1], cur.k[t][1], s[t]);
            } else {
                s[t] = mfma_f16_k16(q.h, cur.k16[t], s[t]);
            }
            const bool ok = fb + 16 * t + r16 < f1;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[t][r] = ok ? s[t][r] * a.scale : -INFINITY;
        }
        softmax_step<NDT>(s[0], s[1], mrun, lrun, o, P, g, r16);
        __syncthreads();
        const u32x4 pa = *reinterpret_cast<const u32x4 *>(&P[r16 * 32 + 8 * g]);
        const int vf = fb + 8 * g;
        const bool tail = vf + 8 > f1;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            u32x4 vb = cur.v[dt];
            if (tail) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k0 = vf + 2 * j;
                    uint32_t w = vb[j];
                    if (k0 >= f1) w &= 0xffff0000u;
                    if (k0 + 1 >= f1) w &= 0x0000ffffu;
                    vb[j] = w;
                }
            }
            o[dt] = mfma_f16_k32(pa, vb, o[dt]);
        }
        __syncthreads();
        cur = nxt;
    }

    if (a.nch == 1) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + 4 * g + r;
                if (row < a.T)
                    store_split(a.out, (size_t)(b * a.T + row) * ld_out, h * HD + dt * 16 + r16,
                                o[dt][r] / lrun[r]);
            }
        return;
    }
    // publish (m, l, o) for this chunk
    float *pp = a.part + (size_t)item * 16 * PW;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (r16 == 0) {
            store_coherent(pp + row * PW + 0, mrun[r]);
            store_coherent(pp + row * PW + 1, lrun[r]);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) store_coherent(pp + row * PW + 2 + dt * 16 + r16, o[dt][r]);
    }
    wait_vmem();
    int prev = 0;
    if (lane == 0) prev = arrive(&a.cnt[bhm]);
    prev = __shfl(prev, 0);
    if (prev != a.nch - 1) return;
    if (lane == 0) rearm(&a.cnt[bhm]);
    // merge chunks in order. Per row r: M = max_c m_c, w_c = exp(m_c - M),
    // L = sum_c l_c w_c; then o = sum_c o_c w_c / L.
    __shared__ float wts[16][17];
    const float *pb = a.part + (size_t)(item - ch) * 16 * PW;
    if (lane < 16) {
        const int rr = lane;
        float mx = -INFINITY;
        for (int c = 0; c < a.nch; ++c) mx = fmaxf(mx, load_coherent(pb + (size_t)c * 16 * PW + rr * PW));
        float l = 0.f;
        for (int c = 0; c < a.nch; ++c) {
            const float *pc = pb + (size_t)c * 16 * PW + rr * PW;
            const float w = __expf(load_coherent(pc) - mx);
            l += load_coherent(pc + 1) * w;
            wts[rr][c] = w;
        }
        wts[rr][16] = l;
    }
    __syncthreads();
    for (int idx = lane; idx < 16 * HD; idx += 64) {
        const int rr = idx / HD, dim = idx - rr * HD;
        const int row = row0 + rr;
        if (row >= a.T) continue;
        float acc = 0.f;
        for (int c = 0; c < a.nch; ++c)
            acc += load_coherent(pb + (size_t)c * 16 * PW + rr * PW + 2 + dim) * wts[rr][c];
        store_split(a.out, (size_t)(b * a.T + row) * ld_out, h * HD + dim, acc / wts[rr][16]);
    }
}

hipError_t launch_self_attn(const SelfAttnArgs &a, int hd, int mt, hipStream_t st) {
    dim3 grid(a.n * a.H, mt);
    if (hd == 64) hipLaunchKernelGGL(self_attn_kernel<64>, grid, dim3(64), 0, st, a);
    else if (hd == 16) hipLaunchKernelGGL(self_attn_kernel<16>, grid, dim3(64), 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_cross_attn(const CrossAttnArgs &a, int hd, hipStream_t st) {
    dim3 grid(a.n_items);
    if (hd == 64) hipLaunchKernelGGL(cross_attn_kernel<64>, grid, dim3(64), 0, st, a);
    else if (hd == 16) hipLaunchKernelGGL(cross_attn_kernel<16>, grid, dim3(64), 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wf
