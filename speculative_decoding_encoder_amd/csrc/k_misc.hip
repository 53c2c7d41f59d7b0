// Small kernels around the verify pass: per-request validation and slot
// state, token + position embedding, layer norm into split-bf16, the final
// argmax reduction of the tied LM head, greedy acceptance and rollback.
#include "wf_device.h"
#include "wf_internal.h"
#include "../../include/wf.h"

namespace wf {

// One thread per request: validate the block, mark the slot pending and
// record (L, n_tok) for the rest of the pass. A request that fails is
// skipped (n_tok = 0) and its slot's error word gets the reason.
__global__ void prepare_kernel(PrepareArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const int slot = a.slots[b];
    const int nt = a.n_tok[b];
    if (slot < 0 || slot >= a.max_batch) {   // no slot to report to: skip
        a.req_L[b] = 0;
        a.req_ntok[b] = 0;
        return;
    }
    const int L = a.slot_len[slot];
    int code = 0;
    if (a.slot_err[slot] != 0) code = -1;   // already failed: skip quietly
    if (nt < 0 || nt > a.T) code |= WF_DERR_TOKEN;
    if (code == 0 && nt > 0) {
        if (L + nt > a.n_ctx) code |= WF_DERR_CONTEXT;
        for (int i = 0; i < nt; ++i) {
            const int t = a.tokens[(size_t)b * a.T + i];
            if (t < 0 || t >= a.V) code |= WF_DERR_TOKEN;
        }
        if (code == 0) {
            const int last = (L + nt - 1) / a.page_size;
            for (int j = 0; j <= last; ++j) {
                const int p = a.page_table[(size_t)slot * a.pt_stride + j];
                if (p < 0 || p >= a.n_pages) code |= WF_DERR_PAGE;
            }
        }
        if (code == 0 && atomicCAS(&a.slot_pending[slot], 0, nt) != 0) code |= WF_DERR_STATE;
    }
    if (code > 0) atomicOr(&a.slot_err[slot], code);
    a.req_L[b] = L;
    a.req_ntok[b] = code == 0 ? nt : 0;
}

// x[m] = tok_emb[token] + pos_emb[L + i]  (fp32). One wave per row; tokens
// and positions are clamped so that padding rows stay in bounds.
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= a.M) return;
    const int b = m / a.T, i = m - (m / a.T) * a.T;
    int tok = a.tokens[m];
    tok = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);
    int pos = a.req_L[b] + i;
    pos = pos >= a.n_ctx ? a.n_ctx - 1 : pos;
    const uint16_t *e = a.tok_emb + (size_t)tok * a.d;
    const uint16_t *p = a.pos_emb + (size_t)pos * a.d;
    float *x = a.x + (size_t)m * a.d;
    for (int c = lane; c < a.d; c += 64) x[c] = bf2f(e[c]) + bf2f(p[c]);
}

// Layer norm of fp32 rows into the split-bf16 operand layout
// [M][d/8][hi 8 | lo 8]. Mean and variance in fp32, two passes, fixed
// reduction order. One wave per row; a lane owns groups of 8 columns.
__global__ __launch_bounds__(256) void layernorm_kernel(LnArgs a) {
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= a.M) return;
    const float *x = a.x + (size_t)m * a.d;
    const int ng = a.d >> 3;
    float s = 0.f;
    for (int kg = lane; kg < ng; kg += 64) {
        const float4 v0 = *reinterpret_cast<const float4 *>(x + kg * 8);
        const float4 v1 = *reinterpret_cast<const float4 *>(x + kg * 8 + 4);
        s += ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w));
    }
    const float mean = wave_sum(s) / (float)a.d;
    float q = 0.f;
    for (int kg = lane; kg < ng; kg += 64) {
        for (int j = 0; j < 8; ++j) {
            const float t = x[kg * 8 + j] - mean;
            q += t * t;
        }
    }
    const float var = wave_sum(q) / (float)a.d;
    const float rstd = 1.0f / sqrtf(var + a.eps);
    uint16_t *out = a.out + (size_t)m * 2 * a.d;
    for (int kg = lane; kg < ng; kg += 64) {
        uint16_t hi[8], lo[8];
        for (int j = 0; j < 8; ++j) {
            const int c = kg * 8 + j;
            const float y = (x[c] - mean) * rstd * bf2f(a.g[c]) + bf2f(a.b[c]);
            split_bf16(y, hi[j], lo[j]);
        }
        u32x4 vh, vl;
        for (int j = 0; j < 4; ++j) {
            vh[j] = (uint32_t)hi[2 * j] | ((uint32_t)hi[2 * j + 1] << 16);
            vl[j] = (uint32_t)lo[2 * j] | ((uint32_t)lo[2 * j + 1] << 16);
        }
        *reinterpret_cast<u32x4 *>(out + kg * 16) = vh;
        *reinterpret_cast<u32x4 *>(out + kg * 16 + 8) = vl;
    }
}

// Per row: merge the LM head's per-tile (max, lowest argmax) in a fixed
// order. -1 for rows of skipped requests and for padding rows; a NaN logit
// flags the slot.
__global__ __launch_bounds__(256) void lm_reduce_kernel(LmReduceArgs a) {
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= a.M) return;
    float v = -INFINITY;
    int idx = 0x7fffffff;
    int nan = 0;
    for (int t = lane; t < a.n_tiles; t += 64) {
        const int ti = a.tile_idx[(size_t)t * a.ld + m];
        if (ti < 0) { nan = 1; continue; }
        argmax_merge(v, idx, a.tile_max[(size_t)t * a.ld + m], ti);
    }
    wave_argmax(v, idx);
    for (int o = 1; o < 64; o <<= 1) nan |= __shfl_xor(nan, o);
    if (lane == 0) {
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

// Greedy acceptance, one thread per request (Whisper-Flash section 3.1 and
// appendix A.1): longest agreeing prefix, EOS without bonus, budget.
__device__ void accept_greedy_one(const AcceptArgs &a, int b) {
    const int nt = a.n_tok[b];
    int n_acc = 0, next = -1, n_emit = 0, done = 0;
    if (nt > 0) {
        const int k = nt - 1;
        const int R = a.budget[b];
        const int32_t *tok = a.tokens + (size_t)b * a.T;
        const int32_t *am = a.argmax + (size_t)b * a.T;
        if (R < 1 || k > R - 1 || nt > a.T) {
            n_acc = -1; done = 1;                 // rejected by rollback
        } else {
            int acc = 0;
            bool eos_stop = false;
            while (acc < k && tok[acc + 1] == am[acc] && am[acc] >= 0) {
                ++acc;
                if (tok[acc] == a.eos) { eos_stop = true; break; }
            }
            n_acc = acc;
            if (eos_stop) {
                n_emit = acc; done = 1;
            } else if (am[acc] < 0) {
                n_acc = -1; done = 1;             // the target row failed
            } else {
                next = am[acc];
                n_emit = acc + 1;
                done = (next == a.eos) || (acc + 1 >= R);
            }
        }
    }
    a.n_acc[b] = n_acc;
    a.next_token[b] = next;
    a.n_emit[b] = n_emit;
    a.done[b] = done;
}

__global__ void accept_greedy_kernel(AcceptArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < a.n) accept_greedy_one(a, b);
}

// Keep L + 1 + a positions (appendix A.1) and clear the pending flag.
__global__ void rollback_kernel(RollbackArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const int slot = a.slots[b];
    if (slot < 0 || slot >= a.max_batch) return;
    const int p = a.slot_pending[slot];
    if (p == 0) return;
    const int acc = a.n_acc[b];
    if (acc < 0 || acc > p - 1) {
        atomicOr(&a.slot_err[slot], WF_DERR_ACCEPT);
    } else {
        a.slot_len[slot] += 1 + acc;
    }
    a.slot_pending[slot] = 0;
}

// Shorten a slot's cache to a given length (never lengthen it).
__global__ void truncate_kernel(RollbackArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const int slot = a.slots[b];
    if (slot < 0 || slot >= a.max_batch) return;
    const int nl = a.n_acc[b];
    if (a.slot_pending[slot] != 0 || nl < 0 || nl > a.slot_len[slot]) {
        atomicOr(&a.slot_err[slot], WF_DERR_STATE);
        return;
    }
    a.slot_len[slot] = nl;
}

__global__ void reset_kernel(int32_t n, int32_t max_batch, const int32_t *slots, int32_t *len,
                             int32_t *pending, int32_t *err) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n) return;
    const int s = slots[b];
    if (s < 0 || s >= max_batch) return;
    len[s] = 0;
    pending[s] = 0;
    err[s] = 0;
}

hipError_t launch_prepare(const PrepareArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(prepare_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_embed(const EmbedArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(embed_kernel, dim3((a.M + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_layernorm(const LnArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(layernorm_kernel, dim3((a.M + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_lm_reduce(const LmReduceArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(lm_reduce_kernel, dim3((a.M + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_accept(const AcceptArgs &a, hipStream_t st) {
    if (a.temperature > 0.f) return launch_accept_sample(a, st);
    hipLaunchKernelGGL(accept_greedy_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_rollback(const RollbackArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(rollback_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_truncate(const RollbackArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(truncate_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_reset(int32_t n, int32_t max_batch, const int32_t *slots, int32_t *len,
                        int32_t *pending, int32_t *err, hipStream_t st) {
    hipLaunchKernelGGL(reset_kernel, dim3((n + 63) / 64), dim3(64), 0, st, n, max_batch, slots,
                       len, pending, err);
    return hipGetLastError();
}

}  // namespace wf
