// Small kernels around the verify pass: per-request validation and slot
// state, token + position embedding, layer norm into fp16 activations, the final
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
    if (a.parents) {
        // tree: node 0 is the root, parents[i] < i; depth and the
        // ancestor-or-self mask of every node (padding rows and skipped
        // requests: the root's)
        const int32_t *par = a.parents + (size_t)b * a.T;
        int32_t *dep = a.depth + (size_t)b * a.T;
        uint64_t *anc = a.anc + (size_t)b * a.T;
        const bool live = code == 0 && nt > 0;
        if (live && par[0] != -1) code |= WF_DERR_TOKEN;
        dep[0] = 0;
        anc[0] = 1ull;
        for (int i = 1; i < a.T; ++i) {
            const int p = (live && i < nt) ? par[i] : 0;
            if (p < 0 || p >= i) code |= WF_DERR_TOKEN;
            const bool ok = live && i < nt && p >= 0 && p < i;
            dep[i] = ok ? dep[p] + 1 : 0;
            anc[i] = ok ? (anc[p] | (1ull << i)) : 1ull;
        }
    }
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

// x[m] = tok_emb[token] + pos_emb[L + i]  (fp32). One thread per 8 columns
// of a row; tokens and positions are clamped so that padding rows stay in
// bounds.
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
    const int ng = a.d >> 3;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)a.M * ng) return;
    const int m = (int)(idx / ng), kg = (int)(idx - (long)m * ng);
    const int b = m / a.T, i = m - (m / a.T) * a.T;
    int tok = a.tokens[m];
    tok = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);
    int pos = a.req_L[b] + (a.depth ? a.depth[m] : i);
    pos = pos >= a.n_ctx ? a.n_ctx - 1 : (pos < 0 ? 0 : pos);
    const u32x4 e = ld16(a.tok_emb + (size_t)tok * a.d + kg * 8);
    const u32x4 p = ld16(a.pos_emb + (size_t)pos * a.d + kg * 8);
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf2f((uint16_t)(e[j] & 0xffffu)) + bf2f((uint16_t)(p[j] & 0xffffu));
        v[2 * j + 1] = bf2f((uint16_t)(e[j] >> 16)) + bf2f((uint16_t)(p[j] >> 16));
    }
    float *x = a.x + (size_t)m * a.d + kg * 8;
    *reinterpret_cast<float4 *>(x) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(x + 4) = make_float4(v[4], v[5], v[6], v[7]);
    if (kg == 0) {
        // position L + i of a row that is appended (i < n_tok; the prepare
        // step has checked its page), else -1
        int rk = -1;
        if (i < a.req_ntok[b]) {
            const int p = a.req_L[b] + i;
            rk = a.page_table[(size_t)a.slots[b] * a.pt_stride + (p >> 4)] * 16 + (p & 15);
        }
        a.row_kv[m] = rk;
    }
}

// Layer norm of the fp32 residual stream into fragment-tiled fp16
// activations (ln_load16 / ln_reduce16 / ln_apply): 16 lanes per row, 4 rows
// per workgroup.
__global__ __launch_bounds__(64) void layernorm_kernel(LnArgs a) {
    const int m = blockIdx.x * 4 + (threadIdx.x >> 4);
    const int r16 = threadIdx.x & 15;
    if (m >= a.M) return;
    const float *x = a.x + (size_t)m * a.d;
    LnRow row;
    ln_load16(x, a.d, r16, row);
    // gains and biases go out with the row (clamped, unconditional), so the
    // kernel waits for memory once
    const int last = (a.d >> 3) - 1;
    u32x4 gg[LN_GPL], bb[LN_GPL];
#pragma unroll
    for (int i = 0; i < LN_GPL; ++i) {
        const int kg = min(r16 + 16 * i, last);
        gg[i] = ld16(a.g + kg * 8);
        bb[i] = ld16(a.b + kg * 8);
    }
    float mean, rstd;
    ln_reduce16(row, a.d, r16, a.eps, mean, rstd);
#pragma unroll
    for (int i = 0; i < LN_GPL; ++i) {
        const int kg = r16 + 16 * i;
        if (kg > last) break;
        *reinterpret_cast<u32x4 *>(a.out + xh_index(m, kg * 8, a.d)) =
            ln_h8(row.v[2 * i], row.v[2 * i + 1], gg[i], bb[i], mean, rstd);
    }
}

// Per row: merge the LM head's per-tile (max, lowest argmax) in a fixed
// order. -1 for rows of skipped requests and for padding rows; a NaN logit
// flags the slot.
// One workgroup per row; the row's tiles are contiguous ([M][ld]).
__global__ __launch_bounds__(256) void lm_reduce_kernel(LmReduceArgs a) {
    __shared__ float sv[4];
    __shared__ int si[4], sn[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float v = -INFINITY;
    int idx = 0x7fffffff;
    int nan = 0;
    const float *tm = a.tile_max + (size_t)m * a.ld;
    const int32_t *tx = a.tile_idx + (size_t)m * a.ld;
#pragma unroll 4
    for (int t = tid; t < a.n_tiles; t += 256) {
        const int ti = tx[t];
        const float tv = tm[t];
        if (ti < 0) nan = 1;
        else argmax_merge(v, idx, tv, ti);
    }
    wave_argmax(v, idx);
    nan = wave_or(nan);
    if (lane == 0) {
        sv[wave] = v;
        si[wave] = idx;
        sn[wave] = nan;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < 4; ++w) {
            argmax_merge(v, idx, sv[w], si[w]);
            nan |= sn[w];
        }
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
// Running-loop bookkeeping, one thread per request (the arithmetic is
// integer: the same results in any order).
__global__ void loop_prepare_kernel(LoopArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const int R = a.n_max - a.s.emitted[b];
    const int L = a.s.len[b];
    const int k = max(0, min(min(a.K, R - 1), a.n_ctx - L - 1));
    a.n_tok_out[b] = a.s.done[b] > 0 ? 0 : k + 1;
    a.budget[b] = max(R, 1);
    if (a.table) {
        const int T = a.K + 1;
        int32_t *blk = a.block + (size_t)b * T;
        const int32_t *tab = a.table + (size_t)b * a.table_cols;
        blk[0] = a.s.anchor[b];
        for (int i = 1; i < T; ++i) blk[i] = tab[min(max(L + i, 0), a.table_cols - 1)];
    }
}

__global__ void loop_finish_kernel(LoopArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const int nt = a.n_tok[b];
    if (nt <= 0) return;
    const int acc = a.n_acc[b], nxt = a.next_token[b], ne = a.n_emit[b];
    a.s.len[b] += acc + 1;
    if (nxt >= 0) a.s.anchor[b] = nxt;
    a.s.emitted[b] += ne;
    a.s.tok_sum[b] += ne;
    if (a.done[b] > 0) a.s.done[b] = 1;
    a.s.acc_sum[b] += acc;
    a.s.prop_sum[b] += nt - 1;
    a.s.rounds[b] += 1;
    a.s.step[b] += 1;
    atomicAdd(reinterpret_cast<unsigned long long *>(a.s.hist) + min(max(acc, 0), a.K), 1ull);
}

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

// Greedy acceptance on a token tree ("Alignment Drift ...", App. E.3), one
// thread per request: a node is accepted when its parent is (the root
// always is), the parent is not an accepted EOS and its token is the
// target's choice at the parent; the kept path ends at the deepest accepted
// node no deeper than R - 1 (the lowest index among equally deep ones).
// Then as in the linear round: accepting EOS finishes the request with no
// bonus, else the target's choice there is emitted and is the next anchor.
// The parents were validated by the verify pass; a request whose rows
// failed (argmax -1 on the path) is rejected (n_acc = -1).
__global__ void accept_tree_kernel(TreeAcceptArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const int nt = a.n_tok[b];
    int32_t *path = a.path + (size_t)b * a.T;
    for (int i = 0; i < a.T; ++i) path[i] = -1;
    int n_acc = 0, next = -1, n_emit = 0, done = 0;
    const int R = a.budget[b];
    if (nt > 0 && nt <= a.T && nt <= 64 && R >= 1) {
        const int32_t *tok = a.tokens + (size_t)b * a.T;
        const int32_t *par = a.parents + (size_t)b * a.T;
        const int32_t *am = a.argmax + (size_t)b * a.T;
        uint64_t acc = 1ull;                      // bit i: node i accepted
        int depth[64];
        depth[0] = 0;
        int best = 0;
        for (int i = 1; i < nt; ++i) {
            const int p = par[i];
            depth[i] = 0;
            if (p < 0 || p >= i) continue;        // invalid: never accepted
            depth[i] = depth[p] + 1;
            const bool ok = ((acc >> p) & 1ull) && !(p > 0 && tok[p] == a.eos) &&
                            am[p] >= 0 && tok[i] == am[p];
            if (ok) {
                acc |= 1ull << i;
                if (depth[i] <= R - 1 && depth[i] > depth[best]) best = i;
            }
        }
        n_acc = depth[best];
        for (int i = best, k = n_acc; k >= 0; i = par[i], --k) path[k] = i;
        if (n_acc > 0 && tok[best] == a.eos) {
            n_emit = n_acc;
            done = 1;
        } else if (am[best] < 0) {
            n_acc = -1;                           // the target row failed
            done = 1;
        } else {
            next = am[best];
            n_emit = n_acc + 1;
            done = (next == a.eos) || (n_acc + 1 >= R);
        }
    } else if (nt > 0) {
        n_acc = -1;
        done = 1;
    }
    a.n_acc[b] = n_acc;
    a.next_token[b] = next;
    a.n_emit[b] = n_emit;
    a.done[b] = done;
}

// Rollback of a tree verify, first half: in every layer, the K and V of the
// accepted path's node at depth k (cache slot L + path[k], k = 1..a) move to
// position L + k. One workgroup per (request, layer); each thread owns some
// (head, dimension) elements and copies them in depth order. A source slot
// L + path[k] (path[k] >= k) is only ever a destination L + k' for k' >
// path[k] >= k, which the same thread writes later, so no copy reads a
// moved value. The slot's length is then updated by the linear rollback.
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
    const int b = blockIdx.x / a.n_layers, l = blockIdx.x - b * a.n_layers;
    const int slot = a.slots[b];
    if (slot < 0 || slot >= a.max_batch) return;
    const int p = a.slot_pending[slot];
    const int acc = a.n_acc[b];
    if (p == 0 || acc < 1 || acc > p - 1 || acc > 63) return;   // rollback checks the rest
    const int32_t *path = a.path + (size_t)b * a.T;
    for (int k = 1; k <= acc; ++k) {
        const int s = path[k];
        if (s < k || s >= p) {                    // not a path of this verify
            if (threadIdx.x == 0 && l == 0) atomicOr(&a.slot_err[slot], WF_DERR_ACCEPT);
            return;
        }
    }
    const int L = a.slot_len[slot];
    const int32_t *pt = a.page_table + (size_t)slot * a.pt_stride;
    uint16_t *kvl = a.kv + (size_t)l * a.layer_elems;
    const size_t v_off = (size_t)a.H * 16 * a.hd;
    for (int e = threadIdx.x; e < a.H * a.hd; e += blockDim.x) {
        const int h = e / a.hd, dim = e - h * a.hd;
        for (int k = 1; k <= acc; ++k) {
            const int src = L + path[k], dst = L + k;
            uint16_t *ps = kvl + (size_t)pt[src >> 4] * a.page_elems;
            uint16_t *pd = kvl + (size_t)pt[dst >> 4] * a.page_elems;
            pd[((size_t)h * 16 + (dst & 15)) * a.hd + dim] = ps[((size_t)h * 16 + (src & 15)) * a.hd + dim];
            pd[v_off + ((size_t)h * a.hd + dim) * 16 + (dst & 15)] =
                ps[v_off + ((size_t)h * a.hd + dim) * 16 + (src & 15)];
        }
    }
}

hipError_t launch_accept_tree(const TreeAcceptArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(accept_tree_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_compact(const CompactArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(compact_kernel, dim3(a.n * a.n_layers), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_prepare(const PrepareArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(prepare_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_embed(const EmbedArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)(((long)a.M * (a.d >> 3) + 255) / 256)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_layernorm(const LnArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(layernorm_kernel, dim3((a.M + 3) / 4), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_lm_reduce(const LmReduceArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(lm_reduce_kernel, dim3(a.M), dim3(256), 0, st, a);
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
hipError_t launch_loop_prepare(const LoopArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(loop_prepare_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_loop_finish(const LoopArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(loop_finish_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
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
