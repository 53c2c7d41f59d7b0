// Attention kernels on fp16 MFMA: the standalone self- and cross-attention
// launches of the verify pass (one item per workgroup of four waves; the
// item bodies and the shared arithmetic are in attn_items.h) and the anchor
// readout.
#include "attn_items.h"

namespace wf {

// Self-attention: grid = (n * H, ceil(T / 16)), 256 threads.
template <int HD, bool TREE>
__global__ __launch_bounds__(256) void self_attn_kernel(SelfAttnArgs a) {
    __shared__ __attribute__((aligned(16))) float mbuf[2][16 * (HD + 4)];
    self_attn_item<HD, TREE>(a, blockIdx.x, blockIdx.y, true, threadIdx.x >> 6, mbuf);
}

// Cross-attention: one workgroup per (request, head, 16-row tile, chunk
// group). Three workgroups fit a CU, so a batch of 32 requests (640
// workgroups) runs in one round.
template <int HD, int SPW>
__global__ __launch_bounds__(256, 3) void cross_attn_kernel(CrossAttnArgs a) {
    __shared__ __attribute__((aligned(16))) float mbuf[2][16 * (HD + 4)];
    __shared__ int last;
    cross_attn_item<HD, SPW>(a, blockIdx.x, true, threadIdx.x >> 6, mbuf, &last);
}

// Anchor readout ("Alignment Drift ...", Verification-Attention Correction
// and App. D.2): at one decoder layer, the cross-attention probabilities of
// every verify row, averaged over heads, and their peak frame. The scores
// are recomputed from the cross K cache with the attention kernels'
// transposed product (S^T = K Q^T on fp16 MFMA: lane (g, r16) gets row r16's
// scores for frames 4g..4g+3 of each 16-frame tile of a 32-frame step).
// Three kernels, every reduction in a fixed order:
//  1. per (request, head, 16-row tile): each row's max m and sum l of
//     2^((s - m) scale log2 e) over the frames; wave w takes steps w, w+4, ...
//     (online per lane), the row's 4 lanes meet by lane swaps, the 4 waves in
//     order through LDS;
//  2. per (request, 16-row tile, 128 frames): wave w takes step 4 chunk + w
//     and sums over the heads (in order) 2^((s - m) scale log2 e) / l; each
//     row's largest (lowest frame among equals) over the lane's 8 frames, the
//     row's 4 lanes, then the 4 waves in order;
//  3. per row: the chunks' peaks merged in chunk order.
template <int HD>
__device__ __forceinline__ void readout_scores(const uint16_t *kh, int fb, const QFrag<HD> &q,
                                               int lane, f32x4 (&s)[2]) {
    const uint16_t *kstep = kh + (size_t)(fb >> 5) * 32 * HD;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (HD == 64) {
            s[t] = mfma_f16_k32(ld16(kstep + (t * 2 + 0) * 512 + lane * 8), q.a[0], s[t]);
            s[t] = mfma_f16_k32(ld16(kstep + (t * 2 + 1) * 512 + lane * 8), q.a[1], s[t]);
        } else {
            s[t] = mfma_f16_k16(ld8(kstep + t * 256 + lane * 4), q.h, s[t]);
        }
    }
}
// (m, l) += (m2, l2); the same bits on both sides of a lane swap
__device__ __forceinline__ void ml_merge(float &m, float &l, float m2, float l2, float sl2e) {
    if (m2 == -INFINITY) return;                  // the other side saw no frame
    if (m == -INFINITY) { m = m2; l = l2; return; }
    const float mm = fmaxf(m, m2);
    l = l * __builtin_amdgcn_exp2f((m - mm) * sl2e) + l2 * __builtin_amdgcn_exp2f((m2 - mm) * sl2e);
    m = mm;
}

template <int HD>
__global__ __launch_bounds__(256) void readout_stats_kernel(ReadoutArgs a) {
    __shared__ float2 sw[4][16];
    const int b = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
    const int row0 = blockIdx.y * 16;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int slot = a.slots[b];
    if (a.req_ntok[b] == 0 || row0 >= a.req_ntok[b] || slot < 0 || slot >= a.max_batch) return;
    const int qrow = row0 + r16;
    const QFrag<HD> q = load_q<HD>(a.q + (size_t)(b * a.T + qrow) * a.d + h * HD, qrow < a.T, g);
    const uint16_t *kh = a.xkv + (size_t)slot * a.slot_stride + a.layer_off + (size_t)h * a.F_pad * HD;
    float m = -INFINITY, l = 0.f;
    const int nsteps = (a.F + 31) >> 5;
    for (int j = wave; j < nsteps; j += 4) {
        f32x4 s[2];
        readout_scores<HD>(kh, 32 * j, q, lane, s);
        float v[8], tm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int f = 32 * j + 16 * t + 4 * g + r;
                v[4 * t + r] = f < a.F ? s[t][r] : -INFINITY;
                tm = fmaxf(tm, v[4 * t + r]);
            }
        if (tm == -INFINITY) continue;
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ls += __builtin_amdgcn_exp2f((v[i] - tm) * a.sl2e);
        ml_merge(m, l, tm, ls, a.sl2e);
    }
    // the row's four lanes (g = 0..3): lane swaps across 16-lane rows
    {
        float ma, mb, la, lb;
        rows16_pair(m, ma, mb);
        rows16_pair(l, la, lb);
        ml_merge(ma, la, mb, lb, a.sl2e);
        halves32_pair(ma, m, mb);
        halves32_pair(la, l, lb);
        ml_merge(m, l, mb, lb, a.sl2e);
    }
    if (g == 0) sw[wave][r16] = make_float2(m, l);
    __syncthreads();
    if (tid < 16 && row0 + tid < a.T) {
        float mi = sw[0][tid].x, li = sw[0][tid].y;
        for (int w = 1; w < 4; ++w) ml_merge(mi, li, sw[w][tid].x, sw[w][tid].y, a.sl2e);
        a.ml[(size_t)(b * a.T + row0 + tid) * a.H + h] = make_float2(mi, li);
    }
}

template <int HD>
__global__ __launch_bounds__(256) void readout_peak_kernel(ReadoutArgs a) {
    __shared__ float sv[4][16];
    __shared__ int si[4][16];
    const int b = blockIdx.x / a.nc, chunk = blockIdx.x - (blockIdx.x / a.nc) * a.nc;
    const int row0 = blockIdx.y * 16;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int slot = a.slots[b];
    if (a.req_ntok[b] == 0 || row0 >= a.req_ntok[b] || slot < 0 || slot >= a.max_batch) return;
    const int qrow = row0 + r16;
    const size_t qoff = (size_t)(b * a.T + min(qrow, a.T - 1));
    const int fb = min(32 * (4 * chunk + wave), ((a.F + 31) >> 5) * 32 - 32);
    const bool step_live = 32 * (4 * chunk + wave) < a.F;
    const uint16_t *kb = a.xkv + (size_t)slot * a.slot_stride + a.layer_off;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = 0.f;
    for (int h = 0; h < a.H; ++h) {
        const QFrag<HD> q = load_q<HD>(a.q + qoff * a.d + h * HD, qrow < a.T, g);
        const float2 ml = a.ml[qoff * a.H + h];
        f32x4 s[2];
        readout_scores<HD>(kb + (size_t)h * a.F_pad * HD, fb, q, lane, s);
        const float il = 1.0f / ml.y;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[4 * t + r] = __fmaf_rn(__builtin_amdgcn_exp2f((s[t][r] - ml.x) * a.sl2e), il,
                                         p[4 * t + r]);
    }
    // this lane's 8 frames, then the row's 4 lanes, then the waves
    float v = -INFINITY;
    int idx = 0x7fffffff;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int f = fb + 16 * t + 4 * g + r;
            if (step_live && f < a.F) argmax_merge(v, idx, p[4 * t + r], f);
        }
    {
        float va, vb;
        int ia, ib;
        rows16_pair(v, va, vb);
        rows16_pair(idx, ia, ib);
        argmax_merge(va, ia, vb, ib);
        halves32_pair(va, v, vb);
        halves32_pair(ia, idx, ib);
        argmax_merge(v, idx, vb, ib);
    }
    if (g == 0) {
        sv[wave][r16] = v;
        si[wave][r16] = idx;
    }
    __syncthreads();
    if (tid < 16 && row0 + tid < a.T) {
        float bv = sv[0][tid];
        int bi = si[0][tid];
        for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, sv[w][tid], si[w][tid]);
        a.part[(size_t)(b * a.T + row0 + tid) * a.nc + chunk] = make_float2(bv, __int_as_float(bi));
    }
}

__global__ void readout_merge_kernel(ReadoutArgs a) {
    const int m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= a.n * a.T) return;
    const int b = m / a.T, i = m - (m / a.T) * a.T;
    const int slot = a.slots[b];
    int out = -1;
    if (i < a.req_ntok[b] && slot >= 0 && slot < a.max_batch) {
        float v = -INFINITY;
        int idx = 0x7fffffff;
        for (int c = 0; c < a.nc; ++c) {
            const float2 pv = a.part[(size_t)m * a.nc + c];
            argmax_merge(v, idx, pv.x, __float_as_int(pv.y));
        }
        out = idx < a.F ? idx : -1;
    }
    a.frame[m] = out;
}

hipError_t launch_readout(const ReadoutArgs &a, int mt, hipStream_t st) {
    if ((a.hd != 64 && a.hd != 16) || a.nc != (a.F + 127) / 128) return hipErrorInvalidValue;
    if (a.hd == 64) {
        hipLaunchKernelGGL(readout_stats_kernel<64>, dim3(a.n * a.H, mt), dim3(256), 0, st, a);
        hipLaunchKernelGGL(readout_peak_kernel<64>, dim3(a.n * a.nc, mt), dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL(readout_stats_kernel<16>, dim3(a.n * a.H, mt), dim3(256), 0, st, a);
        hipLaunchKernelGGL(readout_peak_kernel<16>, dim3(a.n * a.nc, mt), dim3(256), 0, st, a);
    }
    hipLaunchKernelGGL(readout_merge_kernel, dim3((a.n * a.T + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_self_attn(const SelfAttnArgs &a, int hd, int mt, hipStream_t st) {
    dim3 grid(a.n * a.H, mt);
    if (a.anc) {
        if (hd == 64) hipLaunchKernelGGL((self_attn_kernel<64, true>), grid, dim3(256), 0, st, a);
        else if (hd == 16) hipLaunchKernelGGL((self_attn_kernel<16, true>), grid, dim3(256), 0, st, a);
        else return hipErrorInvalidValue;
    } else {
        if (hd == 64) hipLaunchKernelGGL((self_attn_kernel<64, false>), grid, dim3(256), 0, st, a);
        else if (hd == 16) hipLaunchKernelGGL((self_attn_kernel<16, false>), grid, dim3(256), 0, st, a);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_cross_attn(const CrossAttnArgs &a, int hd, hipStream_t st) {
    if (a.G < 1 || a.G > 8) return hipErrorInvalidValue;   // the merge holds 8 groups
    dim3 grid(a.n_items);
    if (hd == 64) {
        // the chunk lengths of 1500 frames: batches of 32 and more (12
        // steps), small batches (2), a few in between (4, 6)
        if (a.spw == 12) hipLaunchKernelGGL((cross_attn_kernel<64, 12>), grid, dim3(256), 0, st, a);
        else if (a.spw == 6) hipLaunchKernelGGL((cross_attn_kernel<64, 6>), grid, dim3(256), 0, st, a);
        else if (a.spw == 4) hipLaunchKernelGGL((cross_attn_kernel<64, 4>), grid, dim3(256), 0, st, a);
        else if (a.spw == 2) hipLaunchKernelGGL((cross_attn_kernel<64, 2>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((cross_attn_kernel<64, 0>), grid, dim3(256), 0, st, a);
    } else if (hd == 16) {
        hipLaunchKernelGGL((cross_attn_kernel<16, 0>), grid, dim3(256), 0, st, a);
    }
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wf
