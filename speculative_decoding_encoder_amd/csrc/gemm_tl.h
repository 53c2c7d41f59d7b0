// Tall-block GEMM for verify passes of many requests (M = B(K+1) in the
// hundreds): C[m][n] = sum_k X[m][k] W[n][k], fp16 X (fragment-tiled), bf16 W
// converted to fp16 in registers, fp16 MFMA 16x16x32, fp32 accumulate.
//
//  * A workgroup is four waves, one per SIMD, and owns a BM x BN tile
//    (BM = 16 MB rows, BN = 64 NW columns). Every wave covers all BM rows
//    and its own 16 NW columns, so a wave keeps MB x NW accumulator tiles and
//    one weight fragment feeds MB MFMAs, one activation fragment NW.
//  * The activations of a k-step (MB fragments of 1 KB, already in MFMA
//    lane order) are fetched once per workgroup into a register ring D
//    k-steps ahead and copied into a ring of five LDS buffers three k-steps
//    ahead; all four waves read them from there, the next k-step's
//    fragments while the current k-step's MFMAs run, and meet at a barrier
//    after every second k-step. Weight fragments go
//    from global memory straight into each wave's registers through the
//    same ring; each weight element is loaded by exactly one wave per row
//    block.
//  * The workgroup walks the CPG consecutive K chunks of its K group in
//    order. Per accumulator the k-steps run in order from zero per chunk;
//    chunk sums meet in the pairwise tree
//    ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)), K groups (P = S / CPG > 1) in the
//    same tree through scratch. That is the order of the register-tiled and
//    LDS-staged kernels, so a row's bits do not depend on the kernel, the
//    tile shape, P or M.
#pragma once
#include "gemm_common.h"

namespace wf {

// Pairwise-tree accumulation of consecutive chunk sums: after chunk j the
// partial p merges with the pending left siblings like a binary counter,
// ((p0+p1)+(p2+p3))+..., the older sum always on the left. l0 ends as the
// total of the (power-of-two) run of chunks.
template <int NT>
struct ChunkStack {
    f32x4 l0[NT], l1[NT], l2[NT];
    __device__ __forceinline__ void push(int j, const f32x4 (&p)[NT]) {
        if ((j & 1) == 0) {
            if (j == 0) {
#pragma unroll
                for (int t = 0; t < NT; ++t) l0[t] = p[t];
            } else if (j == 2 || j == 6) {
#pragma unroll
                for (int t = 0; t < NT; ++t) l1[t] = p[t];
            } else {   // j == 4
#pragma unroll
                for (int t = 0; t < NT; ++t) l2[t] = p[t];
            }
            return;
        }
        if (j == 1) {
#pragma unroll
            for (int t = 0; t < NT; ++t) l0[t] = l0[t] + p[t];
        } else if (j == 3) {
#pragma unroll
            for (int t = 0; t < NT; ++t) l0[t] = l0[t] + (l1[t] + p[t]);
        } else if (j == 5) {
#pragma unroll
            for (int t = 0; t < NT; ++t) l2[t] = l2[t] + p[t];
        } else {   // j == 7
#pragma unroll
            for (int t = 0; t < NT; ++t) l0[t] = l0[t] + (l2[t] + (l1[t] + p[t]));
        }
    }
};

// OCC: workgroups per CU the registers are budgeted for. Two co-resident
// workgroups hide each other's barrier and load waits; it pays once a launch
// has more than a CU's worth of tiles per CU.
template <int ROLE, int MB, int NW, int CPG, int CK, int D = 5, int OCC = 1>
__global__ __launch_bounds__(256, OCC) void gemm_tl_kernel(GemmArgs a) {
    constexpr int EPI = epi_of(ROLE);
    constexpr int NT = MB * NW;                    // accumulator tiles per wave
    // D: ring depth (k-steps ahead); the k-step loop is unrolled by L, a
    // multiple of D and of 2 (the fragment double buffer)
    constexpr int L = D % 2 == 0 ? D : 2 * D;
    static_assert((CPG * CK) % L == 0, "the K group is a whole number of unrolled turns");
    constexpr int XF = MB;                         // activation fragments per k-step
    constexpr int XL = (XF * 64 + 255) / 256;      // 16-byte activation loads per thread
    constexpr int BM = 16 * MB, BN = 64 * NW;
    constexpr int P = 8 / CPG;                     // K groups (the K chunks are 8)
    __shared__ __attribute__((aligned(16))) uint16_t xs[5][XF * 512];

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
    const int n_wave = ntile * BN + wave * 16 * NW;   // first column of this wave
    const int ts = grp * CPG * CK;                    // first k-step of this K group
    constexpr int NSTEPS = CPG * CK;
    const int KS = a.K >> 5;

    // activation piece q of a stage: fragment (row tile) f = q / 64, 16 bytes
    // of lane q % 64; k-step t of it sits at (tile * KS + t) * 512. Tiles
    // past the last repeat it; pieces past the stage (q >= XF * 64) load a
    // valid address and are not staged.
    const uint16_t *xsrc[XL];
#pragma unroll
    for (int v = 0; v < XL; ++v) {
        const int q = tid + v * 256;
        const int f = min(q >> 6, XF - 1);
        const int tile = min((m_base >> 4) + f, (a.M - 1) >> 4);
        xsrc[v] = a.X + ((size_t)tile * KS + ts) * 512 + (q & 63) * 8;
    }
    const uint16_t *wp[NW];
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
        const int n = min(n_wave + nt * 16 + r16, a.N - 1);   // clamped: never stored
        const int seg = n / a.seg_n;
        const uint16_t *wb = seg == 0 ? a.W0 : (seg == 1 ? a.W1 : a.W2);
        wp[nt] = wb + (size_t)(n - seg * a.seg_n) * a.K + g * 8 + (size_t)ts * 32;
    }
    struct Slot { u32x4 x[XL]; u32x4 w[NW]; };
    auto load_x = [&](Slot &r, int s) {                 // s: k-step within the group
        const int t = min(s, NSTEPS - 1);               // past the end: a valid repeat
#pragma unroll
        for (int v = 0; v < XL; ++v) r.x[v] = ld16(xsrc[v] + (size_t)t * 512);
    };
    auto load_w = [&](Slot &r, int s) {
        const int t = min(s, NSTEPS - 1);
#pragma unroll
        for (int nt = 0; nt < NW; ++nt) r.w[nt] = ld16(wp[nt] + (size_t)t * 32);
    };
    auto stage = [&](const Slot &r, int buf) {
#pragma unroll
        for (int v = 0; v < XL; ++v)
            if (XL * 256 == XF * 64 || tid + v * 256 < XF * 64)
                *reinterpret_cast<u32x4 *>(&xs[buf][(tid + v * 256) * 8]) = r.x[v];
    };
    auto read_frags = [&](u32x4 (&xf)[XF], int buf) {
#pragma unroll
        for (int f = 0; f < XF; ++f)
            xf[f] = *reinterpret_cast<const u32x4 *>(&xs[buf][f * 512 + lane * 8]);
    };

    // Entering k-step s: ring slot t % D holds the weights of k-step t for
    // t in [s, s + D) and the activations of k-step t for t in [s + 3,
    // s + 3 + D) (D >= 4); LDS buffer t % 5 holds the activations of k-step
    // t for t in [s + 1, s + 3) and xc those of k-step s. Each k-step stages
    // k-step s + 3 and reads the fragments of k-step s + 1 while its MFMAs
    // run; odd k-steps end with a barrier. That is enough: the fragments of
    // k-step t are read at k-step t - 1, two or more k-steps after they were
    // staged (at t - 3), with a barrier after t - 3 or t - 2; and buffer
    // t % 5 is staged again at k-step t + 2, after the barrier that follows
    // t - 1 or t.
    Slot ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        load_x(ring[i], i);
        load_w(ring[i], i);
    }
    static_assert(D >= 4, "the ring holds the activations three k-steps ahead");
    stage(ring[0], 0);
    stage(ring[1], 1);
    stage(ring[2], 2);
    load_x(ring[0], D);
    load_x(ring[1], D + 1);
    load_x(ring[2], D + 2);
    __syncthreads();
    u32x4 xa[XF], xb[XF];
    read_frags(xa, 0);

    ChunkStack<NT> tree;
    f32x4 c[NT];
    auto step = [&](int s, Slot &cur, Slot &two, u32x4 (&xc)[XF], u32x4 (&xn)[XF]) {
        if (s % CK == 0) {
#pragma unroll
            for (int j = 0; j < NT; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // sched_barrier(0) pins the phase order (the scheduler would
        // otherwise sink the fragment reads next to their MFMAs a step later)
        stage(two, (s + 3) % 5);
        load_x(two, s + 3 + D);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(xn, (s + 1) % 5);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 wh[NW];
#pragma unroll
        for (int nt = 0; nt < NW; ++nt) wh[nt] = bf16x8_to_f16x8(cur.w[nt]);
#pragma unroll
        for (int mt = 0; mt < MB; ++mt)
#pragma unroll
            for (int nt = 0; nt < NW; ++nt)
                c[mt * NW + nt] = mfma_f16_k32(xc[mt], wh[nt], c[mt * NW + nt]);
        __builtin_amdgcn_sched_barrier(0);
        load_w(cur, s + D);
        if ((s + 1) % CK == 0) tree.push(s / CK, c);
        if (s & 1) __syncthreads();
    };
    for (int ss = 0; ss < NSTEPS / L; ++ss) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int s = ss * L + i;
            if (i % 2 == 0) step(s, ring[i % D], ring[(i + 3) % D], xa, xb);
            else step(s, ring[i % D], ring[(i + 3) % D], xb, xa);
        }
    }
    f32x4 (&total)[NT] = tree.l0;

    if constexpr (P > 1) {
        // K groups: each publishes its sum in the MFMA lane layout (16 bytes
        // per lane and tile, device-coherent); the last group to arrive
        // combines the others with its own registers in the pairwise tree.
        const int cidx = ntile * a.m_blocks + mblock;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            a.part + (size_t)cidx * P * 4 * NT * 256, 0, 0x7fffffff, 0x00020000);
        const int lane_off = lane * 16 + wave * NT * 1024;
#pragma unroll
        for (int j = 0; j < NT; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, total[j]), rs,
                                                   lane_off + (grp * 4 * NT + j) * 1024, 0, CPOL_SC1);
        wait_vmem();
        __shared__ int last;
        __syncthreads();
        if (tid == 0) last = (arrive(&a.cnt[cidx]) == P - 1);
        __syncthreads();
        if (!last) return;
        if (tid == 0) rearm(&a.cnt[cidx]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 v[P];
#pragma unroll
            for (int s = 0; s < P; ++s)
                v[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rs, lane_off + (s * 4 * NT + j) * 1024, 0, CPOL_SC1));
#pragma unroll
            for (int s = 0; s < P; ++s)
                if (s == grp) v[s] = total[j];
            if constexpr (P == 2) total[j] = v[0] + v[1];
            else if constexpr (P == 4) total[j] = (v[0] + v[1]) + (v[2] + v[3]);
            else total[j] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        }
    }

    if constexpr (EPI == EPI_ARGMAX) {
        // per row and 64-column tile: (max, lowest index), NaN flagged. The
        // workgroup's BM x 64 scores go to LDS; two threads per row scan 32
        // columns each in column order and merge.
        static_assert(NW == 1, "one 64-column tile per workgroup");
        __shared__ float sv[BM][65];
        const EpiArgs &e = a.e;
        const int n = n_wave + r16;
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mt * 16 + 4 * g + r;
                const float x = total[mt][r];
                sv[row][wave * 16 + r16] = x;
                if (e.logits && m_base + row < a.M && n < a.N) e.logits[(size_t)(m_base + row) * a.N + n] = x;
            }
        }
        __syncthreads();
        if (tid < 2 * BM) {                       // whole waves: BM is a multiple of 32
            const int row = tid >> 1, half = tid & 1;
            float bv = -INFINITY;
            int bi = 0x7fffffff, nn = 0;
            for (int c = 0; c < 32; ++c) {
                const int col = ntile * 64 + half * 32 + c;
                if (col >= a.N) break;
                const float x = sv[row][half * 32 + c];
                if (x != x) nn = 1;
                else argmax_merge(bv, bi, x, col);
            }
            argmax_bfly16<0>(bv, bi);                 // the lane pair (xor 1)
            nn |= bfly16<0>(nn);
            const int m = m_base + row;
            if (half == 0 && m < a.M) {
                e.tile_max[(size_t)m * e.ld + ntile] = bv;
                e.tile_idx[(size_t)m * e.ld + ntile] = nn ? -1 : bi;
            }
        }
    } else {
        int m0[MB];
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) m0[mt] = m_base + mt * 16 + 4 * g;
#pragma unroll
        for (int nt = 0; nt < NW; ++nt) {
            f32x4 v[MB];
#pragma unroll
            for (int mt = 0; mt < MB; ++mt) v[mt] = total[mt * NW + nt];
            epi_column<EPI, MB>(a, m0, n_wave + nt * 16 + r16, v);
        }
    }
}

// The verify-pass instances. K = 1280 (5 k-steps per chunk): 96 x 64 tiles
// (mb 6) or 128 x 64 (mb 8) over the whole of K, and for the wide
// projections with many tiles 64 x 64 (mb 4) at two workgroups per CU. K =
// 5120 (fc2, 20 k-steps per chunk): 96 x 64 tiles in 4 K groups of 2
// chunks, two workgroups per CU.
template <int ROLE>
constexpr bool tl_has_mb4() {
    return ROLE == ROLE_QKV || ROLE == ROLE_FC1 || ROLE == ROLE_LM_HEAD || ROLE == ROLE_DRAFT_QKV ||
           ROLE == ROLE_HIST_KV;
}

template <int ROLE>
hipError_t launch_tl(const GemmArgs &a, int mb, hipStream_t st) {
    if (a.S != 8) return hipErrorInvalidValue;
    const int grid = ((a.n_wg + 7) / 8) * 8;
    if (a.ck == 5 && a.n_groups == 1 && mb == 6)
        hipLaunchKernelGGL((gemm_tl_kernel<ROLE, 6, 1, 8, 5>), dim3(grid), dim3(256), 0, st, a);
    else if (a.ck == 5 && a.n_groups == 1 && mb == 8)
        hipLaunchKernelGGL((gemm_tl_kernel<ROLE, 8, 1, 8, 5>), dim3(grid), dim3(256), 0, st, a);
    else if (a.ck == 20 && a.n_groups == 4 && mb == 6)
        hipLaunchKernelGGL((gemm_tl_kernel<ROLE, 6, 1, 2, 20, 4, 2>), dim3(grid), dim3(256), 0, st, a);
    else if constexpr (tl_has_mb4<ROLE>()) {
        if (a.ck == 5 && a.n_groups == 1 && mb == 4)
            hipLaunchKernelGGL((gemm_tl_kernel<ROLE, 4, 1, 8, 5, 5, 2>), dim3(grid), dim3(256), 0, st,
                               a);
        else
            return hipErrorInvalidValue;
    } else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wf
