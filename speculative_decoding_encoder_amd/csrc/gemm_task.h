// GEMM task of the persistent pass kernel: one BM x BN output tile of
// C[m][n] = sum_k X[m][k] W[n][k] over the K chunks of one K group, computed
// by a workgroup of eight waves. fp16 fragment-tiled activations against the
// bf16 weights converted to fp16 in registers (fp16 MFMA 16x16x32), fp32
// accumulate.
//
//  * The eight waves form WC chunk lanes x WN column slices. Wave (cw, sl)
//    runs K chunk grp * WC + cw (its CK k-steps, in order, from zero) for the
//    BM rows and its slice of NB 16-column tiles, with both operands streamed
//    from global memory straight into a D-deep register ring.
//  * The weights do not depend on the previous phase, so the ring's weight
//    loads go out before the task waits for its inputs; the activation loads
//    follow the wait.
//  * The WC chunk sums of a slice meet in LDS in the pairwise tree, K groups
//    (P = S / WC > 1) in the same tree through device-coherent scratch (the
//    last group to arrive combines). With S = 8 chunks the order is
//    ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)) per output element, the order of
//    every other GEMM kernel of the engine: a row's bits do not depend on
//    the kernel, the tile, the K split or M.
#pragma once
#include "gemm_common.h"

namespace wf {

template <int MB, int NB, int WN>
struct GemmTaskShape {
    static constexpr int WC = 8 / WN;             // chunk lanes (one chunk per wave)
    static constexpr int NT = MB * NB;            // accumulator tiles per wave
    static constexpr int BM = 16 * MB, BN = 16 * NB * WN;
    // combine buffer: at the first tree level WC / 2 senders per slice, one
    // 1 KB block per tile; the argmax epilogue's score tile
    static constexpr int RED_BYTES = (WC / 2 > 0 ? WC / 2 : 1) * WN * NT * 1024;
    static constexpr int SV_BYTES = BM * (BN + 1) * 4;
    static constexpr int LDS_BYTES = (RED_BYTES > SV_BYTES ? RED_BYTES : SV_BYTES) + 16;
};

// Logical task lid of a GEMM phase -> (column tile, row block, K group).
// Tasks that share a column tile (the weight tile) are 8 apart, so that a
// launch whose workgroups sit on the XCDs round-robin puts them on one XCD
// and its L2 serves the weights to every row block. n_ct8 is the number of
// column tiles rounded up to a multiple of 8; lids of padding columns
// return false.
__device__ __forceinline__ bool gemm_task_coords(const GemmArgs &a, int lid, int &ntile,
                                                 int &mblock, int &grp) {
    const int per8 = a.m_blocks * a.n_groups;     // tasks per column tile
    const int hi = lid / (8 * per8);
    const int r = lid - hi * 8 * per8;
    const int k = r >> 3;                         // (mblock, grp) within the column tile
    ntile = hi * 8 + (r & 7);
    mblock = k / a.n_groups;
    grp = k - mblock * a.n_groups;
    return ntile < a.n_tiles;
}

// Returns true when this workgroup applied the epilogue (always with P = 1;
// with K groups, the last group of the tile to arrive). smem holds
// GemmTaskShape::LDS_BYTES.
template <int EPI, int MB, int NB, int WN, int CK, int D, typename Wait>
__device__ __forceinline__ bool gemm_task(const GemmArgs &a, int ntile, int mblock, int grp,
                                          char *smem, Wait &&wait) {
    using S = GemmTaskShape<MB, NB, WN>;
    constexpr int WC = S::WC, NT = S::NT, BM = S::BM, BN = S::BN;
    constexpr int DD = D > CK ? CK : D;
    // K groups: S / WC with S = 8 chunks (the caller's n_groups agrees)
    constexpr int P = WN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int cw = wave / WN, sl = wave - (wave / WN) * WN;
    const int m_base = mblock * BM;
    const int n_sl = ntile * BN + sl * NB * 16;   // first column of this wave's slice
    const int ts = (grp * WC + cw) * CK;          // first k-step of this wave's chunk
    const int KS = a.K >> 5;

    const uint16_t *xp[MB];
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) {
        // rows past M are read (never stored); tiles past the last repeat it
        const int tile = min((m_base >> 4) + mt, (a.M - 1) >> 4);
        xp[mt] = a.X + ((size_t)tile * KS + ts) * 512 + lane * 8;
    }
    const uint16_t *wp[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
        const int n = min(n_sl + nt * 16 + r16, a.N - 1);   // clamped: never stored
        const int seg = n / a.seg_n;
        const uint16_t *wb = seg == 0 ? a.W0 : (seg == 1 ? a.W1 : a.W2);
        wp[nt] = wb + (size_t)(n - seg * a.seg_n) * a.K + g * 8 + (size_t)ts * 32;
    }
    struct Fr {
        u32x4 x[MB];
        u32x4 w[NB];
    };
    Fr f[DD];
#pragma unroll
    for (int i = 0; i < DD; ++i)
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) f[i].w[nt] = ld16(wp[nt] + i * 32);
    wait();
#pragma unroll
    for (int i = 0; i < DD; ++i)
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) f[i].x[mt] = ld16(xp[mt] + i * 512);
    __builtin_amdgcn_sched_barrier(0);

    f32x4 c[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < CK; ++s) {
        Fr &cur = f[s % DD];
        u32x4 wh[NB];
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) wh[nt] = bf16x8_to_f16x8(cur.w[nt]);
#pragma unroll
        for (int mt = 0; mt < MB; ++mt)
#pragma unroll
            for (int nt = 0; nt < NB; ++nt)
                c[mt * NB + nt] = mfma_f16_k32(cur.x[mt], wh[nt], c[mt * NB + nt]);
        __builtin_amdgcn_sched_barrier(0);
        if (s + DD < CK) {
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) cur.w[nt] = ld16(wp[nt] + (s + DD) * 32);
#pragma unroll
            for (int mt = 0; mt < MB; ++mt) cur.x[mt] = ld16(xp[mt] + (s + DD) * 512);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // pairwise tree over the chunk lanes of each slice: at stride st, lane
    // cw (a multiple of 2 st) adds lane cw + st, the older sum on the left
    f32x4 *red = reinterpret_cast<f32x4 *>(smem);
#pragma unroll
    for (int st = 1; st < WC; st <<= 1) {
        const int pos = cw % (2 * st);
        const int slot = (cw / (2 * st)) * WN + sl;
        if (pos == st) {
#pragma unroll
            for (int j = 0; j < NT; ++j) red[(slot * NT + j) * 64 + lane] = c[j];
        }
        __syncthreads();
        if (pos == 0) {
#pragma unroll
            for (int j = 0; j < NT; ++j) c[j] = c[j] + red[(slot * NT + j) * 64 + lane];
        }
        __syncthreads();
    }

    int *flag = reinterpret_cast<int *>(smem + S::LDS_BYTES - 16);
    if constexpr (P > 1) {
        // K groups: the cw = 0 waves publish their slice's sum in the MFMA
        // lane layout (16 bytes per lane and tile, device-coherent); the
        // last group to arrive combines every group's tiles in the tree
        const int cidx = ntile * a.m_blocks + mblock;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            a.part + (size_t)cidx * P * WN * NT * 256, 0, 0x7fffffff, 0x00020000);
        if (cw == 0) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c[j]), rs,
                                                       ((grp * WN + sl) * NT + j) * 1024 + lane * 16,
                                                       0, CPOL_SC1);
        }
        wait_vmem();
        __syncthreads();
        if (tid == 0) *flag = (arrive(&a.cnt[cidx]) == P - 1);
        __syncthreads();
        if (!*flag) return false;
        if (tid == 0) rearm(&a.cnt[cidx]);
        if (cw == 0) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                f32x4 v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (q < P)
                        v[q] = q == grp ? c[j]
                                        : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs, ((q * WN + sl) * NT + j) * 1024 + lane * 16, 0,
                                              CPOL_SC1));
                if constexpr (P == 2) c[j] = v[0] + v[1];
                else if constexpr (P == 4) c[j] = (v[0] + v[1]) + (v[2] + v[3]);
                else c[j] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
            }
        }
    }

    if constexpr (EPI == EPI_ARGMAX) {
        // per row and 64-column tile: (max, lowest index), NaN flagged. The
        // tile's scores go to LDS; two threads per row scan 32 columns each
        // in column order and merge.
        static_assert(BN == 64, "one 64-column tile per task");
        float *sv = reinterpret_cast<float *>(smem);
        const EpiArgs &e = a.e;
        if (cw == 0) {
#pragma unroll
            for (int mt = 0; mt < MB; ++mt)
#pragma unroll
                for (int nt = 0; nt < NB; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = mt * 16 + 4 * g + r;
                        const int col = sl * NB * 16 + nt * 16 + r16;
                        const float x = c[mt * NB + nt][r];
                        sv[row * (BN + 1) + col] = x;
                        const int n = ntile * BN + col;
                        if (e.logits && m_base + row < a.M && n < a.N)
                            e.logits[(size_t)(m_base + row) * a.N + n] = x;
                    }
        }
        __syncthreads();
        for (int q = tid; q < 2 * BM; q += 512) {
            const int row = q >> 1, half = q & 1;
            float bv = -INFINITY;
            int bi = 0x7fffffff, nn = 0;
            for (int cc = 0; cc < 32; ++cc) {
                const int col = ntile * 64 + half * 32 + cc;
                if (col >= a.N) break;
                const float x = sv[row * (BN + 1) + half * 32 + cc];
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
    } else if constexpr (WC == 1) {
        int m0[MB];
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) m0[mt] = m_base + mt * 16 + 4 * g;
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) {
            f32x4 v[MB];
#pragma unroll
            for (int mt = 0; mt < MB; ++mt) v[mt] = c[mt * NB + nt];
            epi_column<EPI, MB>(a, m0, n_sl + nt * 16 + r16, v);
        }
    } else {
        // the sums sit in the cw = 0 waves: through LDS, every wave takes a
        // share of the (slice, column tile) pairs, all MB rows each
        if (cw == 0) {
#pragma unroll
            for (int j = 0; j < NT; ++j) red[(sl * NT + j) * 64 + lane] = c[j];
        }
        __syncthreads();
        int m0[MB];
#pragma unroll
        for (int mt = 0; mt < MB; ++mt) m0[mt] = m_base + mt * 16 + 4 * g;
        for (int q = wave; q < WN * NB; q += 8) {
            const int qs = q / NB, nt = q - (q / NB) * NB;
            f32x4 v[MB];
#pragma unroll
            for (int mt = 0; mt < MB; ++mt) v[mt] = red[(qs * NT + mt * NB + nt) * 64 + lane];
            epi_column<EPI, MB>(a, m0, ntile * BN + qs * NB * 16 + nt * 16 + r16, v);
        }
    }
    return true;
}

}  // namespace wf
