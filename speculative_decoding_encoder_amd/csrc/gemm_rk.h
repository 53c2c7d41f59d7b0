// Register-tiled GEMM for short row blocks (the verify pass, M = B(K+1)):
// C[m][n] = sum_k X[m][k] W[n][k]; fp16 activations against the bf16 weights
// converted to fp16 in registers (fp16 MFMA 16x16x32), fp32 accumulate. The
// cross K/V projection takes the bf16 audio memory as is (bf16 MFMA).
//
//  * A workgroup owns a BM x BN output tile (BM = 16 MB, BN = 16 NB) and the
//    S/P consecutive K chunks of its K group; it has one wave per chunk.
//  * A wave keeps all MB x NB MFMA tiles of its chunk in registers, so one
//    activation fragment feeds NB MFMAs and one weight fragment (converted
//    once) feeds MB. Both operands go from global memory
//    straight into a D-deep register ring; the chunk's CK k-steps are fully
//    unrolled, so every ring slot is a fixed register set. Each weight
//    fragment is loaded by exactly one wave per row block.
//  * The chunk's k-steps run in order from zero; the
//    waves' chunk sums meet in LDS in the pairwise tree
//    ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)), and K groups (P > 1) in the same
//    tree through scratch. That is also the order of the LDS-staged kernel,
//    so a row gets the same bits from either kernel whatever M, the tile
//    shape or P.
//  * LNX (one row tile): the activations are LN(x) of the fp32 residual
//    stream, normalised while the fragments are loaded; the row statistics
//    come from the same code as the standalone layer-norm kernel, so the
//    fragments carry the bits it would have written.
#pragma once
#include "gemm_common.h"

namespace wf {

template <int ROLE, int MB, int NB, int CK, bool LNX>
__global__ __launch_bounds__(512) void gemm_rk_kernel(GemmArgs a) {
    static_assert(!LNX || MB == 1, "the layer-norm prologue covers one row tile");
    constexpr int EPI = epi_of(ROLE);
    constexpr bool XH = ROLE != ROLE_XKV;          // fp16 fragment-tiled activations
    constexpr int NT = MB * NB;
    constexpr int NX = MB;                         // activation fragments per k-step
    // ring of ~144 VGPRs (~96 for the largest tile over long chunks: no spills)
    constexpr int D0 = (NT >= 16 && CK > 5 ? 24 : 36) / (NX + NB);
    constexpr int D1 = D0 < 1 ? 1 : D0;
    constexpr int D2 = D1 > CK ? CK : D1;
    constexpr int D = LNX && D2 > 3 ? 3 : D2;       // LNX also holds a row of x
    constexpr int XSTEP = XH ? 512 : 32;           // uint16 per k-step (fragment-tiled X: one
                                                   // 1 KB block per 16-row tile)
    constexpr int BM = 16 * MB, BN = 16 * NB;
    __shared__ f32x4 red[2][NT][64];

    const int per = gridDim.x >> 3;
    const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lid >= a.n_wg) return;
    const int ntile = lid / (a.m_blocks * a.n_groups);
    const int rem = lid - ntile * (a.m_blocks * a.n_groups);
    const int mblock = rem / a.n_groups;
    const int grp = rem - mblock * a.n_groups;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int W = a.S / a.n_groups;                // waves = chunks of this K group
    const int m_base = mblock * BM, n_base = ntile * BN;
    const int ts = (grp * W + wave) * CK;          // first k-step of this wave's chunk

    // Rows past M and columns past N load a clamped (valid) row instead:
    // their results are never stored, and unconditional loads keep the
    // compiler's wait counts exact, so the ring really overlaps.
    const uint16_t *xp[MB];
    const float *lxp = nullptr;
    if constexpr (LNX) {
        const int m = min(m_base + r16, a.M - 1);
        lxp = a.lnx + (size_t)m * a.K + (size_t)ts * 32 + g * 8;
    } else {
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) {
            if constexpr (XH) {
                // rows of the last tile past M are read, never stored; tiles
                // past the last one repeat it
                const int tile = min((m_base >> 4) + mt, (a.M - 1) >> 4);
                xp[mt] = a.X + ((size_t)tile * (a.K >> 5) + ts) * 512 + (g * 16 + r16) * 8;
            } else {
                const int m = min(m_base + mt * 16 + r16, a.M - 1);
                xp[mt] = a.X + (size_t)m * a.K + g * 8 + (size_t)ts * 32;
            }
        }
    }
    const uint16_t *wp[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
        const int n = min(n_base + nt * 16 + r16, a.N - 1);
        const int seg = n / a.seg_n;
        const uint16_t *wb = seg == 0 ? a.W0 : (seg == 1 ? a.W1 : a.W2);
        wp[nt] = wb + (size_t)(n - seg * a.seg_n) * a.K + g * 8 + (size_t)ts * 32;
    }
    struct Fr {
        u32x4 x[NX];
        float4 lx0, lx1;     // LNX: raw x of the fragment's 8 columns
        u32x4 lg, lb;        // LNX: their gains and biases
        u32x4 w[NB];
    };
    auto load = [&](Fr &fr, int s) {
        if constexpr (LNX) {
            fr.lx0 = *reinterpret_cast<const float4 *>(lxp + s * 32);
            fr.lx1 = *reinterpret_cast<const float4 *>(lxp + s * 32 + 4);
            const int k0 = (ts + s) * 32 + g * 8;
            fr.lg = ld16(a.lng + k0);
            fr.lb = ld16(a.lnb + k0);
        } else {
#pragma unroll
            for (int mt = 0; mt < MB; ++mt) fr.x[mt] = ld16(xp[mt] + s * XSTEP);
        }
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) fr.w[nt] = ld16(wp[nt] + s * 32);
    };

    // LNX: row 4w+g of x goes out first (16 lanes per row), then the ring;
    // its statistics are reduced from registers while the ring is in
    // flight. With fewer than four waves, later rows (4w+g + 4W i) follow.
    LnRow lrow;
    const int ln_rows = min(16, a.M - m_base);
    if constexpr (LNX) {
        // unconditional (rows past the block repeat its last row), so that
        // the statistics wait for these loads only
        ln_load16(a.lnx + (size_t)(m_base + min(4 * wave + g, ln_rows - 1)) * a.K, a.K, r16,
                  lrow);
    }
    // sched_barrier(0) pins the issue order (the scheduler would otherwise
    // sink the ring's loads next to their MFMAs to save registers)
    Fr f[D];
#pragma unroll
    for (int i = 0; i < D; ++i) load(f[i], i);
    __builtin_amdgcn_sched_barrier(0);
    float ln_mean = 0.f, ln_rstd = 0.f;
    if constexpr (LNX) {
        __shared__ float lnst[16][2];
        {
            const int r = 4 * wave + g;
            float mean, rstd;
            ln_reduce16(lrow, a.K, r16, a.ln_eps, mean, rstd);
            if (r16 == 0 && r < ln_rows) {
                lnst[r][0] = mean;
                lnst[r][1] = rstd;
            }
        }
        for (int r = 4 * wave + g + 4 * W; r < ln_rows; r += 4 * W) {   // fewer than 4 waves
            ln_load16(a.lnx + (size_t)(m_base + r) * a.K, a.K, r16, lrow);
            float mean, rstd;
            ln_reduce16(lrow, a.K, r16, a.ln_eps, mean, rstd);
            if (r16 == 0) {
                lnst[r][0] = mean;
                lnst[r][1] = rstd;
            }
        }
        // LDS-only barrier: the ring's loads stay in flight
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        const int rr = min(r16, ln_rows - 1);
        ln_mean = lnst[rr][0];
        ln_rstd = lnst[rr][1];
    }
    f32x4 c[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < CK; ++s) {
        Fr &cur = f[s % D];
        if constexpr (LNX) cur.x[0] = ln_h8(cur.lx0, cur.lx1, cur.lg, cur.lb, ln_mean, ln_rstd);
        if constexpr (XH) {
            u32x4 wh[NB];
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) wh[nt] = bf16x8_to_f16x8(cur.w[nt]);
#pragma unroll
            for (int mt = 0; mt < MB; ++mt)
#pragma unroll
                for (int nt = 0; nt < NB; ++nt)
                    c[mt * NB + nt] = mfma_f16_k32(cur.x[mt], wh[nt], c[mt * NB + nt]);
        } else {
#pragma unroll
            for (int mt = 0; mt < MB; ++mt)
#pragma unroll
                for (int nt = 0; nt < NB; ++nt)
                    c[mt * NB + nt] = mfma_bf16_k32(cur.x[mt], cur.w[nt], c[mt * NB + nt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (s + D < CK) load(cur, s + D);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Pairwise tree over the waves: at stride st, wave r (a multiple of 2st)
    // adds wave r+st; pairs go through LDS two at a time.
    for (int st = 1; st < W; st <<= 1) {
        const int pairs = W / (2 * st);
        for (int p0 = 0; p0 < pairs; p0 += 2) {
            const int p = wave / (2 * st);              // this wave's pair
            const bool in_batch = p >= p0 && p < p0 + 2;
            const int pos = wave - p * 2 * st;          // 0: receiver, st: sender
            if (in_batch && pos == st) {
#pragma unroll
                for (int j = 0; j < NT; ++j) red[p - p0][j][lane] = c[j];
            }
            __syncthreads();
            if (in_batch && pos == 0) {
#pragma unroll
                for (int j = 0; j < NT; ++j) c[j] = c[j] + red[p - p0][j][lane];
            }
            __syncthreads();
        }
    }
    // wave 0 holds the workgroup's sum; share it
    if (wave == 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j) red[0][j][lane] = c[j];
    }
    __syncthreads();

    if constexpr (EPI == EPI_ARGMAX) {
        // per row: (max, lowest index) over this workgroup's BN columns
        const EpiArgs &e = a.e;
        for (int mt = wave; mt < MB; mt += W) {
            f32x4 v[NB];
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) v[nt] = red[0][mt * NB + nt][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m_base + mt * 16 + 4 * g + r;
                float bv = -INFINITY;
                int bi = 0x7fffffff, nn = 0;
#pragma unroll
                for (int nt = 0; nt < NB; ++nt) {
                    const int n = n_base + nt * 16 + r16;
                    if (n >= a.N) continue;
                    const float x = v[nt][r];
                    if (e.logits && m < a.M) e.logits[(size_t)m * a.N + n] = x;
                    if (x != x) nn = 1;
                    else argmax_merge(bv, bi, x, n);
                }
                argmax16(bv, bi, nn);
                if (r16 == 0 && m < a.M) {
                    e.tile_max[(size_t)m * e.ld + ntile] = bv;
                    e.tile_idx[(size_t)m * e.ld + ntile] = nn ? -1 : bi;
                }
            }
        }
        return;
    } else {
        if (a.n_groups == 1) {
            for (int j = wave; j < NT; j += W) {
                const int mt = j / NB, nt = j - (j / NB) * NB;
                const f32x4 v[1] = {red[0][j][lane]};
                const int m0[1] = {m_base + mt * 16 + 4 * g};
                epi_column<EPI, 1>(a, m0, n_base + nt * 16 + r16, v);
            }
            return;
        }
        // K groups: each publishes its sum in the MFMA lane layout (16 bytes
        // per lane and tile, device-coherent); the last group to arrive loads
        // them all and combines each tile in the pairwise tree.
        const int P = a.n_groups;
        const int cidx = ntile * a.m_blocks + mblock;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            a.part + (size_t)cidx * P * NT * 256, 0, 0x7fffffff, 0x00020000);
        for (int j = wave; j < NT; j += W)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, red[0][j][lane]), rs,
                                                   (grp * NT + j) * 1024 + lane * 16, 0, CPOL_SC1);
        wait_vmem();
        __shared__ int last;
        __syncthreads();
        if (tid == 0) last = (arrive(&a.cnt[cidx]) == P - 1);
        __syncthreads();
        if (!last) return;
        if (tid == 0) rearm(&a.cnt[cidx]);
        for (int j = wave; j < NT; j += W) {
            f32x4 v[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < P)
                    v[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rs, (s * NT + j) * 1024 + lane * 16, 0, CPOL_SC1));
            f32x4 t[1];
            if (P == 2) t[0] = v[0] + v[1];
            else if (P == 4) t[0] = (v[0] + v[1]) + (v[2] + v[3]);
            else t[0] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
            const int m0[1] = {m_base + (j / NB) * 16 + 4 * g};
            epi_column<EPI, 1>(a, m0, n_base + (j % NB) * 16 + r16, t);
        }
    }
}

template <int ROLE, int MB, int NB, int CK, bool LNX>
hipError_t launch_rk(const GemmArgs &a, hipStream_t st) {
    const int grid = ((a.n_wg + 7) / 8) * 8;
    const int waves = a.S / a.n_groups;
    hipLaunchKernelGGL((gemm_rk_kernel<ROLE, MB, NB, CK, LNX>), dim3(grid), dim3(64 * waves), 0, st,
                       a);
    return hipGetLastError();
}

// chunk lengths (k-steps) each role is built for: K = d_model gives 1 (width
// 64) or 5 (width 1280); fc2 (K = d_ffn) 1 or 20; the history projection
// (K = 5 d_model) 5 or 25
template <int ROLE>
constexpr bool rk_ck_built(int ck) {
    return ROLE == ROLE_FC2 ? (ck == 1 || ck == 20)
         : ROLE == ROLE_HIST ? (ck == 5 || ck == 25)
         : (ck == 1 || ck == 5);
}
// roles whose input is a layer norm of the residual stream
template <int ROLE>
constexpr bool rk_has_ln() {
    return ROLE == ROLE_QKV || ROLE == ROLE_CROSS_Q || ROLE == ROLE_FC1 || ROLE == ROLE_LM_HEAD ||
           ROLE == ROLE_DRAFT_QKV || ROLE == ROLE_HIST_KV;
}

template <int ROLE, int MB, int NB, bool LNX>
hipError_t launch_rk_ck(const GemmArgs &a, hipStream_t st) {
    switch (a.ck) {
        case 1: if constexpr (rk_ck_built<ROLE>(1)) return launch_rk<ROLE, MB, NB, 1, LNX>(a, st); break;
        case 5: if constexpr (rk_ck_built<ROLE>(5)) return launch_rk<ROLE, MB, NB, 5, LNX>(a, st); break;
        case 20: if constexpr (rk_ck_built<ROLE>(20)) return launch_rk<ROLE, MB, NB, 20, LNX>(a, st); break;
        case 25: if constexpr (rk_ck_built<ROLE>(25)) return launch_rk<ROLE, MB, NB, 25, LNX>(a, st); break;
    }
    return hipErrorInvalidValue;
}

template <int ROLE>
hipError_t launch_rk_role(const GemmArgs &a, int mb, int nb, hipStream_t st) {
    if (a.lnx) {
        // layer-norm prologue: one row tile, 16 or 64 columns (the LM head 64)
        if constexpr (rk_has_ln<ROLE>()) {
            if (mb == 1 && nb == 4) return launch_rk_ck<ROLE, 1, 4, true>(a, st);
            if constexpr (ROLE != ROLE_LM_HEAD)
                if (mb == 1 && nb == 1) return launch_rk_ck<ROLE, 1, 1, true>(a, st);
        }
        return hipErrorInvalidValue;
    }
    if constexpr (ROLE == ROLE_LM_HEAD) {
        switch (mb) {
            case 1: return launch_rk_ck<ROLE, 1, 4, false>(a, st);
            case 2: return launch_rk_ck<ROLE, 2, 4, false>(a, st);
            case 4: return launch_rk_ck<ROLE, 4, 4, false>(a, st);
            case 6: return launch_rk_ck<ROLE, 6, 4, false>(a, st);
        }
        return hipErrorInvalidValue;
    } else {
        switch (mb * 8 + nb) {
            case 1 * 8 + 1: return launch_rk_ck<ROLE, 1, 1, false>(a, st);
            case 1 * 8 + 2: return launch_rk_ck<ROLE, 1, 2, false>(a, st);
            case 1 * 8 + 4: return launch_rk_ck<ROLE, 1, 4, false>(a, st);
            case 2 * 8 + 2: return launch_rk_ck<ROLE, 2, 2, false>(a, st);
            case 2 * 8 + 4: return launch_rk_ck<ROLE, 2, 4, false>(a, st);
            case 4 * 8 + 2: return launch_rk_ck<ROLE, 4, 2, false>(a, st);
            case 4 * 8 + 4: return launch_rk_ck<ROLE, 4, 4, false>(a, st);
        }
        return hipErrorInvalidValue;
    }
}

}  // namespace wf
