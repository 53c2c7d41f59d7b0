// LDS-staged GEMM for tall blocks (long prefill blocks) and the write-once
// cross K/V: C[m][n] = sum_k X[m][k] * W[n][k].
//
// Design for gfx950 (wave64, 16x16x32 bf16 MFMA, fp32 accumulate):
//  * A workgroup is 4 waves and owns 64 output columns (16 per wave) of a
//    block of BM = 16 * MB rows. Each wave streams its 16 weight rows from
//    HBM straight into registers through a 3-deep prefetch ring (one pass
//    over the weights per row block); the activation slice of each 32-deep
//    k-step is staged once per workgroup in LDS (double-buffered) and read
//    by all four waves.
//  * The activation operand is fp16 (fragment-tiled); the bf16 weights are
//    converted to fp16 in registers for the fp16 MFMA. The cross K/V
//    projection multiplies the bf16 audio memory with the bf16 weights as
//    they are (bf16 MFMA).
//  * K is cut into S = 8 chunks (2 when K = 64). A chunk's partial sum
//    starts from zero, and the partials are combined by a fixed pairwise tree
//    ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)). A workgroup owns S/P consecutive
//    chunks (P = 1, 2, 4 or S) and reduces them with the same tree; when
//    P > 1 the subtree sums go to scratch and the last workgroup of the tile
//    to arrive combines them and runs the epilogue. Every P gives the same
//    bits, and nothing depends on M: a row's output is identical whether it
//    is verified alone or inside a block.
//  * Split partials cross workgroups (and XCDs) with device-coherent stores
//    and loads (agent-scope relaxed atomics), completed with a vector-memory
//    wait before the arrival counter is bumped, instead of a full L2
//    write-back fence.
//  * Logical workgroups are remapped so that those sharing a weight tile (the
//    row blocks and K groups of one N tile) are consecutive on one XCD.
#include "gemm_common.h"

namespace wf {

template <int MB>
__device__ __forceinline__ void acc_zero(f32x4 (&c)[MB]) {
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) c[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
}
template <int MB>
__device__ __forceinline__ void acc_add(f32x4 (&dst)[MB], const f32x4 (&src)[MB]) {
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) dst[mt] = dst[mt] + src[mt];
}

// Pairwise-tree accumulation of consecutive chunk partials. After chunk j
// (0-based within the group) the partial p is merged with the stack as a
// binary counter: ((p0+p1)+(p2+p3))+... with the left operand always the
// older sum.
template <int MB>
struct Tree {
    f32x4 l0[MB], l1[MB], l2[MB];
    __device__ __forceinline__ void push(int j, f32x4 (&p)[MB]) {
        if ((j & 1) == 0) {
            if (j == 0) { for (int mt = 0; mt < MB; ++mt) l0[mt] = p[mt]; }
            else if (j == 2 || j == 6) { for (int mt = 0; mt < MB; ++mt) l1[mt] = p[mt]; }
            else { for (int mt = 0; mt < MB; ++mt) l2[mt] = p[mt]; }   // j == 4
            return;
        }
        // odd j: combine with the pending left sibling(s)
        if (j == 1) { for (int mt = 0; mt < MB; ++mt) l0[mt] = l0[mt] + p[mt]; }
        else if (j == 3) {
            for (int mt = 0; mt < MB; ++mt) l1[mt] = l1[mt] + p[mt];
            for (int mt = 0; mt < MB; ++mt) l0[mt] = l0[mt] + l1[mt];
        } else if (j == 5) { for (int mt = 0; mt < MB; ++mt) l2[mt] = l2[mt] + p[mt]; }
        else {   // j == 7
            for (int mt = 0; mt < MB; ++mt) l1[mt] = l1[mt] + p[mt];
            for (int mt = 0; mt < MB; ++mt) l2[mt] = l2[mt] + l1[mt];
            for (int mt = 0; mt < MB; ++mt) l0[mt] = l0[mt] + l2[mt];
        }
    }
};

template <int ROLE, int MB, int KS>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    constexpr int EPI = epi_of(ROLE);
    constexpr bool XH = ROLE != ROLE_XKV;   // fp16 activations (the audio memory is bf16)
    constexpr int BM = MB * 16;
    constexpr int XROW = 40;                      // uint16 per row per k-step (padded: no
                                                  // bank conflicts across 16 rows)
    constexpr int XPARTS = 4;                     // 16-byte parts per row per k-step
    constexpr int NPARTS = BM * KS * XPARTS;      // 16-byte parts per stage
    constexpr int XV = (NPARTS + 255) / 256;      // parts per thread
    // stage layout in LDS: [k-step][row][XROW]
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][KS * BM * XROW];

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
    const int m_base = mblock * BM;
    const int rows = min(BM, a.M - m_base);

    const int n_lane = ntile * 64 + wave * 16 + r16;  // weight row this lane streams
    const bool wok = n_lane < a.N;
    const uint16_t *wrow = a.W0;
    if (wok) {
        const int seg = n_lane / a.seg_n;
        const uint16_t *wb = seg == 0 ? a.W0 : (seg == 1 ? a.W1 : a.W2);
        wrow = wb + (size_t)(n_lane - seg * a.seg_n) * a.K + 8 * g;
    }
    const int cpg = a.S / a.n_groups;               // chunks per group
    const int ck = a.ck;                            // k-steps per chunk (multiple of KS)
    const int t0 = grp * cpg * ck;                  // first k-step of this group
    const int nstages = cpg * ck / KS;
    const int spc = ck / KS;                        // stages per chunk

    // activation stage (KS k-steps of this block's rows): global -> registers
    // one stage ahead -> LDS
    u32x4 xr[XV];
    auto load_x = [&](int st) {
        const int tb = t0 + st * KS;
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int idx = tid + v * 256;
            xr[v] = u32x4{0u, 0u, 0u, 0u};
            if (idx < NPARTS) {
                const int kk = idx / (BM * XPARTS);
                const int r2 = idx - kk * (BM * XPARTS);
                const int rr = r2 / XPARTS, part = r2 - (r2 / XPARTS) * XPARTS;
                const int k0 = (tb + kk) * 32;
                if (rr < rows) {
                    if constexpr (XH)   // fragment-tiled X
                        xr[v] = ld16(a.X + xh_index(m_base + rr, k0 + 8 * part, a.K));
                    else
                        xr[v] = ld16(a.X + (size_t)(m_base + rr) * a.K + k0 + part * 8);
                }
            }
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int idx = tid + v * 256;
            if (idx < NPARTS) {
                const int kr = idx / XPARTS, part = idx - (idx / XPARTS) * XPARTS;
                *reinterpret_cast<u32x4 *>(&xs[buf][kr * XROW + part * 8]) = xr[v];
            }
        }
    };
    // weight fragments of one stage
    struct WS { u32x4 f[KS]; };
    auto load_w = [&](int st, WS &w) {
        const int tb = t0 + st * KS;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            w.f[kk] = wok ? ld16(wrow + (tb + kk) * 32) : u32x4{0u, 0u, 0u, 0u};
    };

    Tree<MB> tree;
    f32x4 c[MB];
    acc_zero(c);
    WS wa, wb, wc;                        // stages s, s+1, s+2
    load_w(0, wa);
    if (nstages > 1) load_w(1, wb);
    load_x(0);
    store_x(0);
    if (nstages > 1) load_x(1);
    __syncthreads();
    const int mt_live = (rows + 15) >> 4;
    for (int s = 0; s < nstages; ++s) {
        const int buf = s & 1;
        if (s + 1 < nstages) store_x(buf ^ 1);     // stage s+1 into the other buffer
        if (s + 2 < nstages) {
            load_x(s + 2);
            load_w(s + 2, wc);
        }
        const uint16_t *xb = xs[buf];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const u32x4 wcur = XH ? bf16x8_to_f16x8(wa.f[kk]) : wa.f[kk];
#pragma unroll
            for (int mt = 0; mt < MB; ++mt) {
                if (mt < mt_live) {
                    const uint16_t *xrow = xb + (kk * BM + mt * 16 + r16) * XROW;
                    const u32x4 xf = *reinterpret_cast<const u32x4 *>(xrow + g * 8);
                    if constexpr (XH) c[mt] = mfma_f16_k32(xf, wcur, c[mt]);
                    else c[mt] = mfma_bf16_k32(xf, wcur, c[mt]);
                }
            }
        }
        if ((s + 1) % spc == 0) {          // end of a chunk
            tree.push(s / spc, c);
            acc_zero(c);
        }
        wa = wb;
        wb = wc;
        __syncthreads();
    }
    f32x4 (&total)[MB] = tree.l0;

    const int n_out = ntile * 64 + wave * 16 + r16;   // C column held by this lane

    if constexpr (EPI == EPI_ARGMAX) {
        __shared__ float smax[4][BM];
        __shared__ int sidx[4][BM];
        __shared__ int snan[4][BM];
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
                argmax16(bv, bi, nn);
                if (r16 == 0) {
                    smax[wave][row] = bv;
                    sidx[wave][row] = bi;
                    snan[wave][row] = nn;
                }
            }
        }
        __syncthreads();
        if (tid < BM) {
            const int m = m_base + tid;
            if (m < a.M) {
                float bv = smax[0][tid];
                int bi = sidx[0][tid];
                int nn = snan[0][tid];
                for (int w = 1; w < 4; ++w) {
                    argmax_merge(bv, bi, smax[w][tid], sidx[w][tid]);
                    nn |= snan[w][tid];
                }
                e.tile_max[(size_t)m * e.ld + ntile] = bv;
                e.tile_idx[(size_t)m * e.ld + ntile] = nn ? -1 : bi;
            }
        }
        return;
    } else {
        if (a.n_groups == 1) {
            int m0[MB];
#pragma unroll
            for (int mt = 0; mt < MB; ++mt) m0[mt] = m_base + mt * 16 + 4 * g;
            epi_column<EPI, MB>(a, m0, n_out, total);
            return;
        }
        // publish this group's subtree sum; the last arriver combines
        const size_t stride = (size_t)a.M * a.N;
#pragma unroll
        for (int mt = 0; mt < MB; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m_base + mt * 16 + 4 * g + r;
                if (m < a.M && n_out < a.N)
                    store_coherent(a.part + (size_t)grp * stride + (size_t)m * a.N + n_out,
                                   total[mt][r]);
            }
        wait_vmem();
        __shared__ int last;
        __syncthreads();
        const int cidx = ntile * a.m_blocks + mblock;
        if (tid == 0) last = (arrive(&a.cnt[cidx]) == a.n_groups - 1);
        __syncthreads();
        if (!last) return;
        if (tid == 0) rearm(&a.cnt[cidx]);
        for (int idx = tid; idx < rows * 64; idx += 256) {
            const int rr = idx >> 6, cc = idx & 63;
            const int m = m_base + rr, n = ntile * 64 + cc;
            if (n >= a.N) continue;
            epi_elem<EPI>(a, m, n, tree_combine(a.part + (size_t)m * a.N + n, stride,
                                                a.n_groups));
        }
    }
}

template <int ROLE, int MB, int KS>
static hipError_t launch_one(const GemmArgs &a, hipStream_t st) {
    const int grid = ((a.n_wg + 7) / 8) * 8;
    hipLaunchKernelGGL((gemm_kernel<ROLE, MB, KS>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

// stage depth: 5 k-steps when the chunk allows it, else 1
template <int ROLE>
static hipError_t launch_mb(const GemmArgs &a, int mb, hipStream_t st) {
    const bool k5 = a.ck % 5 == 0;
    switch (mb) {
        case 1: return k5 ? launch_one<ROLE, 1, 5>(a, st) : launch_one<ROLE, 1, 1>(a, st);
        case 2: return k5 ? launch_one<ROLE, 2, 5>(a, st) : launch_one<ROLE, 2, 1>(a, st);
        case 4: return k5 ? launch_one<ROLE, 4, 5>(a, st) : launch_one<ROLE, 4, 1>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_rk_a(int role, const GemmArgs &a, int mb, int nb, hipStream_t st);
hipError_t launch_gemm_rk_b(int role, const GemmArgs &a, int mb, int nb, hipStream_t st);
hipError_t launch_gemm_rk_c(int role, const GemmArgs &a, int mb, int nb, hipStream_t st);

hipError_t launch_gemm_tl_a(int role, const GemmArgs &a, int mb, hipStream_t st);
hipError_t launch_gemm_tl_b(int role, const GemmArgs &a, int mb, hipStream_t st);
hipError_t launch_gemm_tl_c(int role, const GemmArgs &a, int mb, hipStream_t st);

hipError_t launch_gemm_tl(int role, const GemmArgs &a, int mb, hipStream_t st) {
    switch (role) {
        case ROLE_QKV: case ROLE_OPROJ: case ROLE_CROSS_Q: return launch_gemm_tl_a(role, a, mb, st);
        case ROLE_FC1: case ROLE_FC2: return launch_gemm_tl_b(role, a, mb, st);
        case ROLE_LM_HEAD: case ROLE_DRAFT_QKV: case ROLE_HIST_KV:
            return launch_gemm_tl_c(role, a, mb, st);
    }
    return hipErrorInvalidValue;
}

bool gemm_tl_built(int role, int S, int ck) {
    if (S != 8) return false;
    if (role == ROLE_QKV || role == ROLE_FC1 || role == ROLE_OPROJ || role == ROLE_CROSS_Q ||
        role == ROLE_LM_HEAD || role == ROLE_DRAFT_QKV || role == ROLE_HIST_KV)
        return ck == 5;
    return role == ROLE_FC2 && ck == 20;
}

hipError_t launch_gemm_rk(int role, const GemmArgs &a, int mb, int nb, hipStream_t st) {
    switch (role) {
        case ROLE_QKV: case ROLE_OPROJ: case ROLE_CROSS_Q:
            return launch_gemm_rk_a(role, a, mb, nb, st);
        case ROLE_FC1: case ROLE_FC2:
            return launch_gemm_rk_b(role, a, mb, nb, st);
        case ROLE_LM_HEAD: case ROLE_DRAFT_QKV: case ROLE_HIST: case ROLE_HIST_KV:
            return launch_gemm_rk_c(role, a, mb, nb, st);
    }
    return hipErrorInvalidValue;
}

bool gemm_rk_built(int role, int ck) {
    if (role == ROLE_XKV) return false;
    if (role == ROLE_FC2) return ck == 1 || ck == 20;
    if (role == ROLE_HIST) return ck == 5 || ck == 25;
    return ck == 1 || ck == 5;
}

hipError_t launch_gemm(int role, const GemmArgs &a, int mb, hipStream_t st) {
    switch (role) {
        case ROLE_QKV: return launch_mb<ROLE_QKV>(a, mb, st);
        case ROLE_OPROJ: return launch_mb<ROLE_OPROJ>(a, mb, st);
        case ROLE_CROSS_Q: return launch_mb<ROLE_CROSS_Q>(a, mb, st);
        case ROLE_FC1: return launch_mb<ROLE_FC1>(a, mb, st);
        case ROLE_FC2: return launch_mb<ROLE_FC2>(a, mb, st);
        case ROLE_LM_HEAD: return launch_mb<ROLE_LM_HEAD>(a, mb, st);
        case ROLE_DRAFT_QKV: return launch_mb<ROLE_DRAFT_QKV>(a, mb, st);
        case ROLE_HIST: return launch_mb<ROLE_HIST>(a, mb, st);
        case ROLE_HIST_KV: return launch_mb<ROLE_HIST_KV>(a, mb, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace wf
