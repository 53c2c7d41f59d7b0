// Kernels of the parallel drafter (Whisper-Flash section 3.2, eq. 2, and
// appendix A.2) around the shared GEMM / attention kernels:
//  * tap_kernel: the target's residual stream after a tapped block, written
//    as one column block of the fp16 history operand [M][n_taps*d];
//  * rope_append_kernel: rotary embedding (base 10000, fp32 phases, explicit
//    text positions; dimension i pairs with i + hd/2) of queries and keys,
//    and the append of keys and values into the drafter's KV pages;
//  * prepare_draft_kernel / embed_draft_kernel: per-request validation and
//    the block [Emb(anchor), m, ..., m];
//  * draft_out_kernel: the anchor followed by the drafts (argmax of mask rows).
#include "wf_device.h"
#include "wf_internal.h"
#include "../../include/wf.h"

namespace wf {

__global__ __launch_bounds__(256) void tap_kernel(TapArgs a) {
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= a.M) return;
    const float *x = a.x + (size_t)m * a.d;
    const size_t width = (size_t)a.n_taps * a.d;
    for (int kg = lane; kg < a.d / 8; kg += 64) {
        u32x4 v;
        for (int j = 0; j < 4; ++j) v[j] = pack_h2(x[kg * 8 + 2 * j], x[kg * 8 + 2 * j + 1]);
        *reinterpret_cast<u32x4 *>(a.out + xh_index(m, a.j * a.d + kg * 8, (int)width)) = v;
    }
}

// One thread per (row, head, pair i < hd/2).
__global__ __launch_bounds__(256) void rope_append_kernel(RopeArgs a) {
    const int half = a.hd >> 1;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)a.M * a.H * half;
    if (idx >= total) return;
    const int i = (int)(idx % half);
    const int h = (int)((idx / half) % a.H);
    const int m = (int)(idx / ((long)half * a.H));
    const int b = m / a.T, r = m - (m / a.T) * a.T;
    if (r >= a.req_ntok[b]) return;
    const int pos = a.req_L[b] + r;
    const float inv = powf(10000.0f, -(2.0f * (float)i) / (float)a.hd);
    const float ang = (float)pos * inv;
    const float c = cosf(ang), s = sinf(ang);
    const float *row = a.tmp + (size_t)m * a.ncols;
    const int c0 = h * a.hd + i, c1 = c0 + half;
    if (a.q_off >= 0) {
        const float qa = row[a.q_off + c0], qb = row[a.q_off + c1];
        a.q_out[(size_t)m * a.d + c0] = f2h_bits(qa * c - qb * s);
        a.q_out[(size_t)m * a.d + c1] = f2h_bits(qa * s + qb * c);
    }
    const float ka = row[a.k_off + c0], kb = row[a.k_off + c1];
    const int page = a.page_table[(size_t)a.slots[b] * a.pt_stride + (pos >> 4)];
    const int off = pos & 15;
    uint16_t *pg = a.kv_layer + (size_t)page * a.page_elems;
    pg[((size_t)h * 16 + off) * a.hd + i] = f2h_bits(ka * c - kb * s);
    pg[((size_t)h * 16 + off) * a.hd + i + half] = f2h_bits(ka * s + kb * c);
    uint16_t *vt = pg + (size_t)a.H * 16 * a.hd;
    vt[((size_t)h * a.hd + i) * 16 + off] = f2h_bits(row[a.v_off + c0]);
    vt[((size_t)h * a.hd + i + half) * 16 + off] = f2h_bits(row[a.v_off + c1]);
}

// One thread per request. The block occupies positions L..L+K of the slot's
// drafter pages (transiently: the next verify overwrites them).
__global__ void prepare_draft_kernel(PrepareDraftArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const int slot = a.slots[b];
    a.req_L[b] = 0;
    a.req_ntok[b] = 0;
    if (slot < 0 || slot >= a.max_batch) return;
    const int L = a.slot_len[slot];
    int code = 0;
    if (a.slot_err[slot] != 0) return;
    const int anc = a.anchor[b];
    if (anc < 0 || anc >= a.V) code |= WF_DERR_TOKEN;
    if (a.slot_pending[slot] != 0) code |= WF_DERR_STATE;
    // near the end of the context the block keeps the rows that fit (the
    // drafts past them come out as -1); a full cache drafts nothing
    const int nt = min(a.K + 1, a.n_ctx - L);
    if (nt <= 0) return;
    if (code == 0) {
        for (int j = 0; j <= (L + nt - 1) / 16; ++j) {
            const int p = a.page_table[(size_t)slot * a.pt_stride + j];
            if (p < 0 || p >= a.n_pages) code |= WF_DERR_PAGE;
        }
    }
    if (code) {
        atomicOr(&a.slot_err[slot], code);
        return;
    }
    a.req_L[b] = L;
    a.req_ntok[b] = nt;
}

__global__ __launch_bounds__(256) void embed_draft_kernel(EmbedDraftArgs a) {
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= a.M) return;
    const int b = m / a.T, i = m - (m / a.T) * a.T;
    int anc = a.anchor[b];
    anc = anc < 0 ? 0 : (anc >= a.V ? a.V - 1 : anc);
    const uint16_t *src = i == 0 ? a.tok_emb + (size_t)anc * a.d : a.mask;
    float *x = a.x + (size_t)m * a.d;
    for (int c = lane; c < a.d; c += 64) x[c] = bf2f(src[c]);
}

__global__ void draft_out_kernel(const int32_t *anchor, const int32_t *argmax,
                                 const int32_t *req_ntok, int n, int K, int32_t *block) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * (K + 1)) return;
    const int b = idx / (K + 1), i = idx - (idx / (K + 1)) * (K + 1);
    if (req_ntok[b] == 0) block[idx] = i == 0 ? anchor[b] : -1;
    else block[idx] = i == 0 ? anchor[b] : (i < req_ntok[b] ? argmax[idx] : -1);
}

hipError_t launch_tap(const TapArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(tap_kernel, dim3((a.M + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_rope_append(const RopeArgs &a, hipStream_t st) {
    const long total = (long)a.M * a.H * (a.hd / 2);
    hipLaunchKernelGGL(rope_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, a);
    return hipGetLastError();
}
hipError_t launch_prepare_draft(const PrepareDraftArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(prepare_draft_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_embed_draft(const EmbedDraftArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(embed_draft_kernel, dim3((a.M + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_draft_out(const int32_t *anchor, const int32_t *argmax, const int32_t *req_ntok,
                            int n, int K, int32_t *block, hipStream_t st) {
    hipLaunchKernelGGL(draft_out_kernel, dim3((n * (K + 1) + 255) / 256), dim3(256), 0, st, anchor,
                       argmax, req_ntok, n, K, block);
    return hipGetLastError();
}

}  // namespace wf
