// Skinny bf16 GEMM for the decoder projections, the tied LM head and the
// write-once cross K/V:  C[m][n] = sum_k X[m][k] * W[n][k].
//
// Design for gfx950 (wave64, 16x16x32 bf16 MFMA):
//  * A workgroup is 4 waves; each wave owns 16 weight rows (output columns)
//    and a block of up to 4 16-row M tiles. A lane loads its 16-byte weight
//    fragments straight from HBM into registers (one pass over the weights
//    per M block) and its activation fragments from L1/L2.
//  * The activation operand is split-bf16: X = hi + lo, two MFMAs per k-step
//    with the same weight fragment, so activations carry ~16 mantissa bits
//    while weights stay bf16.
//  * K is cut into S chunks of CK k-steps that depend only on K. A chunk's
//    partial sum always starts from zero and the partials are added in chunk
//    order. A workgroup either owns one chunk (split mode: partials go to
//    scratch and the last workgroup to arrive adds them up and runs the
//    epilogue) or all chunks (full mode). Both give the same bits, and no
//    result depends on M: a row's output is identical whether it is verified
//    alone or inside a block.
//  * Logical workgroups are remapped so that those sharing a weight tile (the
//    M blocks or K chunks of one N tile) are consecutive on one XCD and hit
//    the same L2.
#include "wf_device.h"
#include "wf_internal.h"

namespace wf {

static constexpr int MB = 4;  // 16-row M tiles per workgroup

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
        float t = gelu_erf(v + bias_at(e.b0, n));
        uint16_t hi, lo;
        split_bf16(t, hi, lo);
        size_t base = (size_t)m * (2 * a.N) + (size_t)(n >> 3) * 16 + (n & 7);
        e.out[base] = hi;
        e.out[base + 8] = lo;
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
            base[(size_t)e.H * e.F_pad * e.hd + ((size_t)h * e.hd + dim) * e.F_pad + f] =
                f2h_bits(v + bias_at(e.b1, c));
        }
    }
}

template <int EPI, int CK, bool XS>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    // XCD-aware remap: hardware workgroup w runs on XCD w % 8; logical ids
    // that are consecutive within one XCD share an N tile.
    const int per = gridDim.x >> 3;
    const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lid >= a.n_wg) return;
    const int ntile = lid / (a.m_blocks * a.n_groups);
    const int rem = lid - ntile * (a.m_blocks * a.n_groups);
    const int mblock = rem / a.n_groups;
    const int grp = rem - mblock * a.n_groups;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;

    const int n_lane = ntile * 64 + wave * 16 + r16;  // weight row this lane streams
    const bool wok = n_lane < a.N;
    const uint16_t *wrow = a.W0;
    if (wok) {
        const int seg = n_lane / a.seg_n;
        const uint16_t *wb = seg == 0 ? a.W0 : (seg == 1 ? a.W1 : a.W2);
        wrow = wb + (size_t)(n_lane - seg * a.seg_n) * a.K;
    }
    const int s_lo = a.split ? grp : 0;
    const int s_hi = a.split ? grp + 1 : a.S;
    const int m_base = mblock * MB * 16;

    f32x4 total[MB];
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) total[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = s_lo; s < s_hi; ++s) {
        const int k0 = s * CK * 32;
        u32x4 wf[CK];
#pragma unroll
        for (int kk = 0; kk < CK; ++kk)
            wf[kk] = wok ? ld16(wrow + k0 + kk * 32 + 8 * g) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            const int mrow0 = m_base + mt * 16;
            if (mrow0 < a.M) {
                const int m = mrow0 + r16;
                const bool mok = m < a.M;
                if constexpr (XS) {
                    const uint16_t *xr = a.X + (size_t)m * (2 * a.K);
                    u32x4 xh[CK], xl[CK];
#pragma unroll
                    for (int kk = 0; kk < CK; ++kk) {
                        const uint16_t *p = xr + (size_t)(((k0 + kk * 32) >> 3) + g) * 16;
                        xh[kk] = mok ? ld16(p) : u32x4{0u, 0u, 0u, 0u};
                        xl[kk] = mok ? ld16(p + 8) : u32x4{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (int kk = 0; kk < CK; ++kk) {
                        c = mfma_bf16_k32(xh[kk], wf[kk], c);
                        c = mfma_bf16_k32(xl[kk], wf[kk], c);
                    }
                } else {
                    const uint16_t *xr = a.X + (size_t)m * a.K;
                    u32x4 xh[CK];
#pragma unroll
                    for (int kk = 0; kk < CK; ++kk)
                        xh[kk] = mok ? ld16(xr + k0 + kk * 32 + 8 * g) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int kk = 0; kk < CK; ++kk) c = mfma_bf16_k32(xh[kk], wf[kk], c);
                }
            }
            if (s == s_lo) total[mt] = c;
            else total[mt] += c;
        }
    }

    const int n_out = ntile * 64 + wave * 16 + r16;   // C column held by this lane

    if constexpr (EPI == EPI_ARGMAX) {
        __shared__ float smax[4][MB * 16];
        __shared__ int sidx[4][MB * 16];
        __shared__ int snan[4][MB * 16];
        const EpiArgs &e = a.e;
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mt * 16 + 4 * g + r;
                const int m = m_base + row;
                const float v = total[mt][r];
                const bool ok = n_out < a.N;
                if (e.logits && ok && m < a.M) e.logits[(size_t)m * a.N + n_out] = v;
                const bool isn = ok && (v != v);
                float bv = (ok && !isn) ? v : -INFINITY;
                int bi = ok ? n_out : 0x7fffffff;
                int nn = isn ? 1 : 0;
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    float v2 = __shfl_xor(bv, o);
                    int i2 = __shfl_xor(bi, o);
                    argmax_merge(bv, bi, v2, i2);
                    nn |= __shfl_xor(nn, o);
                }
                if (r16 == 0) {
                    smax[wave][row] = bv;
                    sidx[wave][row] = bi;
                    snan[wave][row] = nn;
                }
            }
        }
        __syncthreads();
        if (tid < MB * 16) {
            const int m = m_base + tid;
            if (m < a.M) {
                float bv = smax[0][tid];
                int bi = sidx[0][tid];
                int nn = snan[0][tid];
                for (int w = 1; w < 4; ++w) {
                    argmax_merge(bv, bi, smax[w][tid], sidx[w][tid]);
                    nn |= snan[w][tid];
                }
                e.tile_max[(size_t)ntile * e.ld + m] = bv;
                e.tile_idx[(size_t)ntile * e.ld + m] = nn ? -1 : bi;
            }
        }
        return;
    } else {
        if (!a.split) {
#pragma unroll
            for (int mt = 0; mt < MB; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m_base + mt * 16 + 4 * g + r;
                    if (m < a.M && n_out < a.N) epi_elem<EPI>(a, m, n_out, total[mt][r]);
                }
            return;
        }
        // split mode: publish this chunk's partial, the last arriver reduces.
#pragma unroll
        for (int mt = 0; mt < MB; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m_base + mt * 16 + 4 * g + r;
                if (m < a.M && n_out < a.N)
                    a.part[((size_t)s_lo * a.M + m) * a.N + n_out] = total[mt][r];
            }
        __shared__ int last;
        fence_release();
        __syncthreads();
        if (tid == 0) {
            const int prev = atomicAdd(&a.cnt[ntile], 1);
            last = (prev == a.S - 1);
        }
        __syncthreads();
        if (!last) return;
        fence_acquire();
        if (tid == 0) a.cnt[ntile] = 0;   // ready for the next launch
        const int rows = min(MB * 16, a.M - m_base);
        for (int idx = tid; idx < rows * 64; idx += 256) {
            const int rr = idx >> 6, cc = idx & 63;
            const int m = m_base + rr, n = ntile * 64 + cc;
            if (n >= a.N) continue;
            float v = a.part[(size_t)m * a.N + n];
            for (int s = 1; s < a.S; ++s) v += a.part[((size_t)s * a.M + m) * a.N + n];
            epi_elem<EPI>(a, m, n, v);
        }
    }
}

template <int EPI, int CK, bool XS>
static hipError_t launch_one(const GemmArgs &a, hipStream_t st) {
    const int grid = ((a.n_wg + 7) / 8) * 8;
    hipLaunchKernelGGL((gemm_kernel<EPI, CK, XS>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int EPI, bool XS>
static hipError_t launch_ck(const GemmArgs &a, int ck, hipStream_t st) {
    switch (ck) {
        case 2: return launch_one<EPI, 2, XS>(a, st);
        case 4: return launch_one<EPI, 4, XS>(a, st);
        case 8: return launch_one<EPI, 8, XS>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(int epi, const GemmArgs &a, int ck, bool xsplit, hipStream_t st) {
    if (!xsplit) {
        if (epi != EPI_XKV) return hipErrorInvalidValue;
        return launch_ck<EPI_XKV, false>(a, ck, st);
    }
    switch (epi) {
        case EPI_QKV: return launch_ck<EPI_QKV, true>(a, ck, st);
        case EPI_RESID: return launch_ck<EPI_RESID, true>(a, ck, st);
        case EPI_F16: return launch_ck<EPI_F16, true>(a, ck, st);
        case EPI_GELU: return launch_ck<EPI_GELU, true>(a, ck, st);
        case EPI_ARGMAX: return launch_ck<EPI_ARGMAX, true>(a, ck, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace wf
