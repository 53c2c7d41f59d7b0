// Pieces shared by the two GEMM kernels: the epilogues applied to
// C[m][n] = sum_k X[m][k] W[n][k] and the fixed-order combine of K-split
// subtree sums.
#pragma once
#include "wf_device.h"
#include "wf_internal.h"

namespace wf {

__device__ __forceinline__ float gelu_erf(float t) {
    return 0.5f * t * (1.0f + erff(t * 0.70710678118654752f));
}

__device__ __forceinline__ float bias_at(const uint16_t *b, int c) {
    return b ? bf2f(b[c]) : 0.0f;
}

// Per-element epilogue for the elementwise modes.
template <int EPI>
__device__ __forceinline__ void epi_elem(const GemmArgs &a, int m, int n, float v) {
    const EpiArgs &e = a.e;
    if constexpr (EPI == EPI_RESID) {
        float t = v + bias_at(e.b0, n);
        e.x[(size_t)m * a.N + n] += t;
    } else if constexpr (EPI == EPI_F16) {
        e.out[(size_t)m * a.N + n] = f2h_bits(v + bias_at(e.b0, n));
    } else if constexpr (EPI == EPI_GELU) {
        e.out[xh_index(m, n, a.N)] = f2h_bits(gelu_erf(v + bias_at(e.b0, n)));
    } else if constexpr (EPI == EPI_QKV) {
        const int d = a.seg_n;
        const int seg = n / d;
        const int c = n - seg * d;
        if (seg == 0) {
            e.out[(size_t)m * d + c] = f2h_bits(v + bias_at(e.b0, c));
            return;
        }
        const int b = m / e.T;
        const int i = m - b * e.T;
        if (i >= e.req_ntok[b]) return;       // padding row or skipped request
        const int pos = e.req_L[b] + i;
        const int page = e.page_table[(size_t)e.slots[b] * e.pt_stride + (pos >> 4)];
        const int off = pos & 15;
        const int h = c / e.hd, dim = c - (c / e.hd) * e.hd;
        uint16_t *pg = e.kv_layer + (size_t)page * e.page_elems;
        if (seg == 1) {
            pg[((size_t)h * 16 + off) * e.hd + dim] = f2h_bits(v);
        } else {
            pg[(size_t)e.H * 16 * e.hd + ((size_t)h * e.hd + dim) * 16 + off] =
                f2h_bits(v + bias_at(e.b2, c));
        }
    } else if constexpr (EPI == EPI_STORE32) {
        const int seg = n / a.seg_n;
        const uint16_t *bb = seg == 0 ? e.b0 : (seg == 1 ? e.b1 : e.b2);
        e.out32[(size_t)m * a.N + n] = v + bias_at(bb, n - seg * a.seg_n);
    } else if constexpr (EPI == EPI_XKV) {
        const int d = a.seg_n;
        const int seg = n / d;
        const int c = n - seg * d;
        const int b = m / e.F;
        const int f = m - b * e.F;
        const int h = c / e.hd, dim = c - (c / e.hd) * e.hd;
        const int slot = e.slots[b];
        if (slot < 0 || slot >= e.max_batch) return;
        uint16_t *base = e.xkv + (size_t)slot * e.xkv_slot_stride + e.xkv_layer_off;
        if (seg == 0) {
            base[((size_t)h * e.F_pad + f) * e.hd + dim] = f2h_bits(v);
        } else {
            // V: per head, 32-frame steps of [hd][32 frames] (one contiguous
            // block per step, in the order the attention kernel reads it)
            base[(size_t)e.H * e.F_pad * e.hd + (size_t)h * e.F_pad * e.hd +
                 ((size_t)(f >> 5) * e.hd + dim) * 32 + (f & 31)] = f2h_bits(v + bias_at(e.b1, c));
        }
    }
}

// Combine P subtree sums with the pairwise tree (P in {2, 4, 8}).
__device__ __forceinline__ float tree_combine(const float *part, size_t stride, int P) {
    float v[8];
    for (int s = 0; s < P; ++s) v[s] = load_coherent(part + (size_t)s * stride);
    if (P == 2) return v[0] + v[1];
    if (P == 4) return (v[0] + v[1]) + (v[2] + v[3]);
    return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

__host__ __device__ constexpr int epi_of(int role) {
    return role == ROLE_QKV ? EPI_QKV
         : role == ROLE_CROSS_Q ? EPI_F16
         : role == ROLE_FC1 ? EPI_GELU
         : role == ROLE_LM_HEAD ? EPI_ARGMAX
         : role == ROLE_XKV ? EPI_XKV
         : (role == ROLE_DRAFT_QKV || role == ROLE_HIST || role == ROLE_HIST_KV) ? EPI_STORE32
         : EPI_RESID;
}

}  // namespace wf
