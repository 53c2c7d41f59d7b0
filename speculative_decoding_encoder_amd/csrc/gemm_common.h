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

// Epilogues of the elementwise modes, split so that a lane pays for the
// column-dependent part (segment, head, bias) once, issues the loads of all
// its rows together (residual values, KV destinations), and then stores.
// Every path computes an element the same way: epi_elem is the same three
// steps for one element.
struct EpiCol {
    float bias;                    // the column's bias (0 without one)
    int seg, c;                    // weight segment and column within it
    int kcol, vcol;                // EPI_QKV: the column's place in a K / V page
};

template <int EPI>
__device__ __forceinline__ EpiCol epi_col(const GemmArgs &a, int n) {
    const EpiArgs &e = a.e;
    EpiCol k{};
    n = min(n, a.N - 1);                        // columns past N are never stored
    if constexpr (EPI == EPI_QKV || EPI == EPI_STORE32) {
        k.seg = n / a.seg_n;
        k.c = n - k.seg * a.seg_n;
    } else {
        k.c = n;
    }
    if constexpr (EPI == EPI_QKV) {
        const int h = k.c / e.hd, dim = k.c - h * e.hd;
        k.kcol = h * 16 * e.hd + dim;                       // K page: [H][16][hd]
        k.vcol = e.H * 16 * e.hd + (h * e.hd + dim) * 16;   // V page: [H][hd][16]
        k.bias = k.seg == 0 ? bias_at(e.b0, k.c) : (k.seg == 2 ? bias_at(e.b2, k.c) : 0.0f);
    } else if constexpr (EPI == EPI_STORE32) {
        const uint16_t *bb = k.seg == 0 ? e.b0 : (k.seg == 1 ? e.b1 : e.b2);
        k.bias = bias_at(bb, k.c);
    } else {
        k.bias = bias_at(e.b0, n);
    }
    return k;
}

// The per-row input of element (m, n), as raw bits: the residual value
// (EPI_RESID) or the row's KV destination (EPI_QKV). The row is clamped, so
// the load is unconditional.
template <int EPI>
__device__ __forceinline__ uint32_t epi_load(const GemmArgs &a, int m, int n) {
    m = min(m, a.M - 1);
    if constexpr (EPI == EPI_RESID)
        return __float_as_uint(a.e.x_in[(size_t)m * a.N + min(n, a.N - 1)]);
    else if constexpr (EPI == EPI_QKV)
        return (uint32_t)a.e.row_kv[m];
    else
        return 0u;
}

template <int EPI>
__device__ __forceinline__ void epi_store(const GemmArgs &a, const EpiCol &k, int m, int n,
                                          uint32_t in, float v) {
    const EpiArgs &e = a.e;
    if constexpr (EPI == EPI_RESID) {
        const float t = v + k.bias;
        e.x[(size_t)m * a.N + n] = __uint_as_float(in) + t;
    } else if constexpr (EPI == EPI_F16) {
        e.out[(size_t)m * a.N + n] = f2h_bits(v + k.bias);
    } else if constexpr (EPI == EPI_GELU) {
        e.out[xh_index(m, n, a.N)] = f2h_bits(gelu_erf(v + k.bias));
    } else if constexpr (EPI == EPI_QKV) {
        if (k.seg == 0) {
            e.out[(size_t)m * a.seg_n + k.c] = f2h_bits(v + k.bias);
            return;
        }
        const int rk = (int)in;
        if (rk < 0) return;                   // padding row or skipped request
        uint16_t *pg = e.kv_layer + (size_t)(rk >> 4) * e.page_elems;
        if (k.seg == 1) pg[k.kcol + (rk & 15) * e.hd] = f2h_bits(v);
        else pg[k.vcol + (rk & 15)] = f2h_bits(v + k.bias);
    } else if constexpr (EPI == EPI_STORE32) {
        e.out32[(size_t)m * a.N + n] = v + k.bias;
    }
}

template <int EPI>
__device__ __forceinline__ void epi_elem(const GemmArgs &a, int m, int n, float v) {
    const EpiCol k = epi_col<EPI>(a, n);
    epi_store<EPI>(a, k, m, n, epi_load<EPI>(a, m, n), v);
}

// The epilogue of the MT x 4 rows a lane holds in one column (the MFMA
// output layout: rows m0[t] .. m0[t] + 3 of tile t): the loads of all rows
// first, then the stores of the rows and columns in range.
template <int EPI, int MT>
__device__ __forceinline__ void epi_column(const GemmArgs &a, const int (&m0)[MT], int n,
                                           const f32x4 (&v)[MT]) {
    const EpiCol k = epi_col<EPI>(a, n);
    uint32_t in[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) in[t][r] = epi_load<EPI>(a, m0[t] + r, n);
    if (n >= a.N) return;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (m0[t] + r < a.M) epi_store<EPI>(a, k, m0[t] + r, n, in[t][r], v[t][r]);
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
         : (role == ROLE_DRAFT_QKV || role == ROLE_HIST || role == ROLE_HIST_KV) ? EPI_STORE32
         : EPI_RESID;
}

}  // namespace wf
