// Audio encoder forward on gfx950: a fixed window of log-mel features to the
// audio memory that wf_encode_kv projects (the encoder stage of
// "Whisper-Flash ...", §1-2 and App. A.3 Table A2; the 30 s mel window of the
// SGLang-Omni "Whisper ASR" cookbook, "Long Audio Chunking").
//
//   melT    = features transposed to time-major rows, one zero row each side
//   g1      = GELU(conv3(melT) + b1)            GEMM, K = 3 n_mels (3 taps)
//   x       = GELU(conv3_s2(g1) + b2) + pos     GEMM, K = 3 d, A rows 2 apart
//   per block: LN1 -> QKV GEMM (q, k, v^T per head) -> attention (all frames)
//              -> O GEMM + residual -> LN2 -> fc1 GEMM + GELU -> fc2 + residual
//   out     = LN_post(x)                        bf16 [n][F][d]
//
// Unlike the decoder pass this work is MFMA-bound (a 30 s window is about
// 2.3 TFLOP through 32 blocks), so the kernels are dense-contraction designs:
//
//  * GEMM: C = A W^T, bf16 x bf16 -> fp32 (16x16x32 MFMA). A workgroup of 4
//    waves owns a 128 x 256 tile (each wave 64 x 128: 4 x 8 accumulator
//    tiles); both operands go through double-buffered LDS in 32-deep k-steps
//    (the 16-byte chunks of a row XOR-swizzled: conflict-free fragment
//    reads), the global loads of a k-step issued two k-steps ahead (K % 64
//    == 0). Grids of two or more rounds take 256 x 256 tiles on eight waves
//    whose operands are copied straight into LDS, two 64-deep stages. The MFMA
//    computes C^T so a lane holds one output row and four consecutive
//    columns (8- or 16-byte epilogue stores). Row tiles are grouped by 8 per
//    column walk and workgroups are dealt to the 8 XCDs in consecutive
//    runs, so the tiles that share operands meet in one L2.
//    A row m of the A operand is A + (m / rpr) * sreq + (m % rpr) * srow: a
//    plain matrix (rpr = M), or a width-3 convolution read in place from
//    time-major rows with zero borders (K = 3 C_in consecutive elements,
//    srow = C_in for stride 1, 2 C_in for stride 2).
//  * Attention: one workgroup per (request, head, 256 queries), each wave 64
//    queries; 64-key steps of K ([key][dim]) and V^T ([dim][key]) through
//    double-buffered LDS. S^T = K Q^T and O^T += V^T P^T keep a query per
//    lane, so P stays in registers as the B operand (bf16) and only the
//    running max crosses lanes (two exchanges) per step; the row sums come
//    from the MFMA too (a tile of ones times P^T).
#include "../../include/wf.h"
#include "wf_device.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace wf {
wf_status set_error(wf_status s, const char *msg);   // engine.hip (wf_last_error)
}

namespace wf {
namespace enc {

enum { EE_CONV1 = 0, EE_CONV2 = 1, EE_QKV = 2, EE_RESID = 3, EE_GELU = 4, EE_XKV = 5 };

struct GemmArgs {
    const uint16_t *A;                 // bf16; row m at A + (m / rpr) * sreq + (m % rpr) * srow
    int rpr;
    long long sreq;
    int srow;
    const uint16_t *W0, *W1, *W2;      // bf16 [N][K], in segments of seg_n rows
    const uint16_t *b0, *b1, *b2;      // per-segment biases (nullable)
    int M, N, K, seg_n;
    int n_m, n_n, n_wg;                // row tiles, column tiles, workgroups
    float *x;                          // EE_RESID, EE_CONV2: fp32 [M][N]
    const float *pos;                  // EE_CONV2: fp32 [F][N]
    uint16_t *out;                     // EE_GELU: bf16 [M][N]; EE_CONV1: padded rows
    int F, Tm;                         // frames and feature frames per request
    uint16_t *q, *k, *vt;              // EE_QKV
    int H, Fq;                         // heads; frames padded to the query tile
    // EE_XKV: a decoder layer's cross K (segment 0) and V (segment 1, bias b1)
    // into the write-once pool, fp16, in its per-head layouts
    uint16_t *xkv;
    long long slot_stride, layer_off;
    const int32_t *slots;
    int F_pad, hd, max_batch;
};

constexpr int GBK = 32, GROW = 32;   // k-step depth; LDS row: the k-step's 32 elements
// The four 16-byte chunks of LDS row r are stored XOR-swizzled: chunk c at
// c ^ ((r >> 1) & 3). Eight lanes reading one chunk of eight consecutive
// rows (a fragment read) then hit eight different 16-byte bank groups, and
// so do eight lanes writing two whole rows.
__host__ __device__ constexpr int swz(int r, int c) { return r * GROW + ((c ^ ((r >> 1) & 3)) << 3); }

__device__ __forceinline__ float gelu(float t) {
    return 0.5f * t * (1.0f + erff(t * 0.70710678118654752f));
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two floats to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bias4(const uint16_t *b, int c, int r) {
    return b ? bf2f(b[c + r]) : 0.0f;
}

// Epilogue of one 16x16 output tile: this lane's row m and columns n .. n + 3
// (c[r] is column n + r); m < M and n < N.
template <int EPI>
__device__ __forceinline__ void epi_tile(const GemmArgs &a, int m, int n, const f32x4 c) {
    if constexpr (EPI == EE_RESID) {
        float4 *px = reinterpret_cast<float4 *>(a.x + (size_t)m * a.N + n);
        float4 xv = *px;
        xv.x += c[0] + bias4(a.b0, n, 0);
        xv.y += c[1] + bias4(a.b0, n, 1);
        xv.z += c[2] + bias4(a.b0, n, 2);
        xv.w += c[3] + bias4(a.b0, n, 3);
        *px = xv;
    } else if constexpr (EPI == EE_GELU || EPI == EE_CONV1) {
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = gelu(c[r] + bias4(a.b0, n, r));
        size_t row = m;
        if constexpr (EPI == EE_CONV1) {
            const int rq = m / a.Tm;
            row = (size_t)rq * (a.Tm + 2) + 1 + (m - rq * a.Tm);
        }
        *reinterpret_cast<u32x2 *>(a.out + row * a.N + n) =
            u32x2{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
    } else if constexpr (EPI == EE_CONV2) {
        const int t = m % a.F;
        const float4 pv = *reinterpret_cast<const float4 *>(a.pos + (size_t)t * a.N + n);
        float4 xv;
        xv.x = gelu(c[0] + bias4(a.b0, n, 0)) + pv.x;
        xv.y = gelu(c[1] + bias4(a.b0, n, 1)) + pv.y;
        xv.z = gelu(c[2] + bias4(a.b0, n, 2)) + pv.z;
        xv.w = gelu(c[3] + bias4(a.b0, n, 3)) + pv.w;
        *reinterpret_cast<float4 *>(a.x + (size_t)m * a.N + n) = xv;
    } else if constexpr (EPI == EE_XKV) {
        const int rq = m / a.F, f = m - rq * a.F;
        const int slot = a.slots[rq];
        if (slot < 0 || slot >= a.max_batch) return;   // skipped request
        const int seg = n / a.seg_n, cc = n - seg * a.seg_n;
        const int h = cc / a.hd, dim = cc - h * a.hd;
        uint16_t *base = a.xkv + (size_t)slot * a.slot_stride + a.layer_off +
                         (size_t)(seg * a.H + h) * a.F_pad * a.hd;
        if (seg == 0) {   // K: the four dims are adjacent in the fragment order
            *reinterpret_cast<u32x2 *>(base + xk_index(f, dim, a.hd)) =
                u32x2{pack_h2(c[0], c[1]), pack_h2(c[2], c[3])};
        } else {          // V: [hd][32] per 32-frame step, frame at xv_pos
            uint16_t *vb = base + (size_t)(f >> 5) * a.hd * 32 + xv_pos(f & 31);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vb[(size_t)(dim + r) * 32] = f2h_bits(c[r] + bias4(a.b1, cc, r));
        }
    } else {   // EE_QKV
        const int seg = n / a.seg_n, cc = n - seg * a.seg_n;
        const int h = cc >> 6, dim = cc & 63;
        const int rq = m / a.F, t = m - rq * a.F;
        const uint16_t *bb = seg == 0 ? a.b0 : (seg == 2 ? a.b2 : nullptr);
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = c[r] + bias4(bb, cc, r);
        const size_t bh = (size_t)rq * a.H + h;
        if (seg < 2) {
            uint16_t *dst = (seg == 0 ? a.q : a.k) + (bh * a.Fq + t) * 64 + dim;
            *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
        } else {
            uint16_t *dst = a.vt + (bh * 64 + dim) * a.Fq + t;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)r * a.Fq] = (uint16_t)(pack_bf2(y[r], 0.f) & 0xffffu);
        }
    }
}

// MT x NT accumulator tiles per wave, 2 x 2 waves: a (32 MT) x (32 NT) tile per
// workgroup (4 x 8: 128 x 256, the default; 2 x 4: 64 x 128 for grids that
// would not fill the chip). A tile's shape does not change any element's
// arithmetic: every output sums its k-steps in order in one lane.
// The epilogue of a wave's MT x NT accumulator tiles: tile (i, j) gives this
// lane row mw + 16 i + r16 and columns nw + 16 j + 4 g .. + 3.
template <int EPI, int MT, int NT>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const f32x4 (&acc)[MT][NT], int mw,
                                         int nw) {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = mw + i * 16 + r16;
        if (m >= a.M) continue;
        if constexpr (EPI == EE_RESID) {
            // the residual read-modify-write: all of the row's loads first, so
            // their latencies overlap (columns past N load a valid address)
            float4 xv[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = min(nw + j * 16 + 4 * g, a.N - 4);
                xv[j] = *reinterpret_cast<const float4 *>(a.x + (size_t)m * a.N + n);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = nw + j * 16 + 4 * g;
                if (n >= a.N) continue;
                const f32x4 c = acc[i][j];
                float4 v = xv[j];
                v.x += c[0] + bias4(a.b0, n, 0);
                v.y += c[1] + bias4(a.b0, n, 1);
                v.z += c[2] + bias4(a.b0, n, 2);
                v.w += c[3] + bias4(a.b0, n, 3);
                *reinterpret_cast<float4 *>(a.x + (size_t)m * a.N + n) = v;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = nw + j * 16 + 4 * g;
                if (n < a.N) epi_tile<EPI>(a, m, n, acc[i][j]);
            }
        }
    }
}

template <int EPI, int MT, int NT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a) {
    constexpr int BM = 32 * MT, BN = 32 * NT;
    constexpr int XL = BM / 64, WL = BN / 64;       // 16-byte pieces per thread per k-step
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * GROW];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN * GROW];
    const int per = gridDim.x >> 3;
    const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lid >= a.n_wg) return;
    constexpr int GM = 8;                           // row tiles per column walk
    const int grp = lid / (GM * a.n_n);
    const int first_m = grp * GM;
    const int gsz = min(a.n_m - first_m, GM);
    const int in_grp = lid - grp * GM * a.n_n;
    const int mt = first_m + in_grp % gsz;
    const int nt = in_grp / gsz;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = mt * BM, n0 = nt * BN;

    // 16-byte pieces of a k-step: A BM rows x 4, W BN rows x 4. Rows past
    // M / N repeat the last (never stored).
    const uint16_t *xsrc[XL];
    const uint16_t *wsrc[WL];
    int xoff[XL], woff[WL];
#pragma unroll
    for (int v = 0; v < XL; ++v) {
        const int p = tid + 256 * v, row = p >> 2, pc = p & 3;
        const int m = min(m0 + row, a.M - 1);
        const int rq = m / a.rpr;
        xsrc[v] = a.A + (size_t)rq * a.sreq + (size_t)(m - rq * a.rpr) * a.srow + pc * 8;
        xoff[v] = swz(row, pc);
    }
#pragma unroll
    for (int v = 0; v < WL; ++v) {
        const int p = tid + 256 * v, row = p >> 2, pc = p & 3;
        const int n = min(n0 + row, a.N - 1);
        const int seg = n / a.seg_n;
        const uint16_t *wb = seg == 0 ? a.W0 : (seg == 1 ? a.W1 : a.W2);
        wsrc[v] = wb + (size_t)(n - seg * a.seg_n) * a.K + pc * 8;
        woff[v] = swz(row, pc);
    }
    const int KT = a.K / GBK;
    struct Stage { u32x4 x[XL], w[WL]; };
    auto gload = [&](Stage &r, int kt) {
        kt = min(kt, KT - 1);                       // past the end: a valid repeat, never stored
#pragma unroll
        for (int v = 0; v < XL; ++v) r.x[v] = ld16(xsrc[v] + kt * GBK);
#pragma unroll
        for (int v = 0; v < WL; ++v) r.w[v] = ld16(wsrc[v] + kt * GBK);
    };
    auto sstore = [&](const Stage &r, int b) {
#pragma unroll
        for (int v = 0; v < XL; ++v) *reinterpret_cast<u32x4 *>(&xs[b][xoff[v]]) = r.x[v];
#pragma unroll
        for (int v = 0; v < WL; ++v) *reinterpret_cast<u32x4 *>(&ws[b][woff[v]]) = r.w[v];
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one k-step from LDS buffer b: the W fragments in halves, so fewer
    // fragments are live at a time
    auto step = [&](int b) {
        u32x4 xf[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
            xf[i] = *reinterpret_cast<const u32x4 *>(&xs[b][swz(wm * 16 * MT + i * 16 + r16, g)]);
        __builtin_amdgcn_s_setprio(1);              // the MFMA block issues first on its SIMD
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 wf[NT / 2];
#pragma unroll
            for (int j = 0; j < NT / 2; ++j)
                wf[j] = *reinterpret_cast<const u32x4 *>(
                    &ws[b][swz(wn * 16 * NT + (NT / 2 * h + j) * 16 + r16, g)]);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT / 2; ++j)
                    acc[i][NT / 2 * h + j] = mfma_bf16_k32(wf[j], xf[i], acc[i][NT / 2 * h + j]);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // k-step kt is read from LDS buffer kt & 1; its global loads were issued
    // two k-steps earlier (register sets r0 / r1 alternate), so a load has
    // two k-steps of MFMA work to arrive
    Stage r0, r1;
    gload(r0, 0);
    gload(r1, 1);
    sstore(r0, 0);
    __syncthreads();
    // KT is even (K % 64 == 0); past the end the copies land in a buffer
    // nothing reads again
    for (int kt = 0; kt < KT; kt += 2) {
        gload(r0, kt + 2);
        step(0);
        sstore(r1, 1);
        __syncthreads();
        gload(r1, kt + 3);
        step(1);
        sstore(r0, 0);
        __syncthreads();
    }

    epilogue<EPI, MT, NT>(a, acc, m0 + wm * 16 * MT, n0 + wn * 16 * NT);
}

// Large grids: 256 x 256 tiles on eight waves, a 2 x 4 grid of 128 x 64 wave
// tiles (8 x 4 accumulator tiles), one workgroup and so two waves per SIMD
// per CU (one wave per SIMD leaves a third of the MFMA issue rate unused:
// 1.3-1.9 against 2.45 PFLOP/s in a register-only loop on MI355X). Operands
// go from global memory straight into LDS (global_load_lds, 16 bytes per
// lane) in stages of two k-steps (64 elements of K), two stage buffers of
// 64 KB. A copy instruction fills eight whole 128-byte rows, so every global
// access reads full cache lines; the eight 16-byte chunks of a row are
// XOR-swizzled (chunk c of row r sits at c ^ (r & 7)), so the copies and
// the fragment reads are free of bank conflicts without padding. Per stage:
// wait for this wave's copies of the stage, one barrier (every wave's copies
// landed, every wave done with the other buffer), the copies of the next
// stage into the other buffer, then both k-steps' fragments and their 2 x 32
// MFMAs. Every output still sums its k-steps in order in one lane with the
// same MFMA as gemm_kernel, so the two give the same bits.
constexpr int DBT = 256;                   // tile rows / columns

// gfx9 s_waitcnt immediates: vmcnt bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; the counters not waited for stay at their maxima
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0070 | (0xF << 8)); }
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_dma_kernel(GemmArgs a) {
    constexpr int MT = 8, NT = 4;
    constexpr int RPW = DBT / 8;                    // rows of each operand a wave copies
    constexpr int CPO = RPW / 8;                    // its eight-row copies per operand
    // [buffer][A rows 0..255 | W rows 0..255][64 elements]: 128 KB
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2 * DBT * 64];
    const int per = gridDim.x >> 3;
    const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lid >= a.n_wg) return;
    constexpr int GM = 4;                           // row tiles per column walk
    const int grp = lid / (GM * a.n_n);
    const int first_m = grp * GM;
    const int gsz = min(a.n_m - first_m, GM);
    const int in_grp = lid - grp * GM * a.n_n;
    const int mt = first_m + in_grp % gsz;
    const int nt = in_grp / gsz;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int wm = wave >> 2, wn = wave & 3;
    const int m0 = mt * DBT, n0 = nt * DBT;

    // copies: wave w brings rows RPW w .. RPW w + RPW - 1 of the A and W
    // tiles in eight-row copies; lane L fills row L / 8 of a copy, LDS chunk
    // L % 8, with k-chunk (L % 8) ^ (L / 8). Rows past M / N repeat the last
    // (never stored).
    const int crow = lane >> 3, cchunk = (lane & 7) ^ ((lane >> 3) & 7);
    const uint16_t *asrc[CPO], *wsrc[CPO];
#pragma unroll
    for (int i = 0; i < CPO; ++i) {
        const int r = RPW * wave + 8 * i + crow;
        const int m = min(m0 + r, a.M - 1);
        const int rq = m / a.rpr;
        asrc[i] = a.A + (size_t)rq * a.sreq + (size_t)(m - rq * a.rpr) * a.srow + cchunk * 8;
        const int n = min(n0 + r, a.N - 1);
        const int seg = n / a.seg_n;
        const uint16_t *wb = seg == 0 ? a.W0 : (seg == 1 ? a.W1 : a.W2);
        wsrc[i] = wb + (size_t)(n - seg * a.seg_n) * a.K + cchunk * 8;
    }
    const int KP = a.K / (2 * GBK);                 // stages (K % 64 == 0)
    // stage p into buffer p & 1; past the end a valid repeat of the last stage
    // into a buffer nothing reads again
    auto copy = [&](int p) {
        const int kk = min(p, KP - 1) * 2 * GBK;
        uint16_t *buf = lds[p & 1];
#pragma unroll
        for (int i = 0; i < CPO; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void *)(asrc[i] + kk),
                (__attribute__((address_space(3))) void *)&buf[(RPW * wave + 8 * i) * 64], 16, 0, 0);
#pragma unroll
        for (int i = 0; i < CPO; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void *)(wsrc[i] + kk),
                (__attribute__((address_space(3))) void *)&buf[(DBT + RPW * wave + 8 * i) * 64], 16,
                0, 0);
    };
    // k-step h of stage p: this lane's k-chunk 4 h + g of its rows
    auto frags = [&](u32x4 (&xf)[MT], u32x4 (&wf)[NT], int p, int h) {
        const uint16_t *buf = lds[p & 1];
        const int sw = ((4 * h + g) ^ (r16 & 7)) * 8;
#pragma unroll
        for (int i = 0; i < MT; ++i)
            xf[i] = *reinterpret_cast<const u32x4 *>(&buf[(wm * 128 + 16 * i + r16) * 64 + sw]);
#pragma unroll
        for (int j = 0; j < NT; ++j)
            wf[j] = *reinterpret_cast<const u32x4 *>(
                &buf[(DBT + wn * 16 * NT + 16 * j + r16) * 64 + sw]);
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfmas = [&](const u32x4 (&xc)[MT], const u32x4 (&wc)[NT]) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[i][j] = mfma_bf16_k32(wc[j], xc[i], acc[i][j]);
        __builtin_amdgcn_s_setprio(0);
    };
    copy(0);
    u32x4 xa[MT], wa[NT], xb[MT], wb[NT];
    for (int p = 0; p < KP; ++p) {
        wait_vmcnt0();                              // this wave's copies of stage p
        wait_lgkmcnt0();                            // its reads of stage p - 1
        __builtin_amdgcn_s_barrier();               // every wave's, likewise
        copy(p + 1);                                // into stage p - 1's buffer
        frags(xa, wa, p, 0);
        frags(xb, wb, p, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(xa, wa);
        mfmas(xb, wb);
    }
    wait_vmcnt0();                                  // no copy outlives the workgroup's LDS
    epilogue<EPI, MT, NT>(a, acc, m0 + wm * 128, n0 + wn * 16 * NT);
}

struct AttnArgs {
    const uint16_t *q, *k, *vt;        // [n][H][Fq][64], [n][H][Fq][64], [n][H][64][Fq]
    uint16_t *o;                       // bf16 [n][F][d]
    int H, F, Fq, d, n_qt, n_wg;
    float sl2e;                        // log2(e) / sqrt(64)
};

constexpr int AROW = 72;               // LDS row: 64 elements + 16 B pad

template <int QT>   // 16-query subtiles per wave (the workgroup takes 64 QT queries)
__global__ __launch_bounds__(256, QT == 1 ? 3 : (QT == 2 ? 2 : 1)) void attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][64 * AROW];   // [key][dim]
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][64 * AROW];   // [dim][key]
    const int per = gridDim.x >> 3;
    const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lid >= a.n_wg) return;
    const int qt = lid % a.n_qt;
    const int bh = lid / a.n_qt;                  // request * H + head
    const int rq = bh / a.H, h = bh - rq * a.H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const uint16_t *qb = a.q + (size_t)bh * a.Fq * 64;
    const uint16_t *kb = a.k + (size_t)bh * a.Fq * 64;
    const uint16_t *vb = a.vt + (size_t)bh * 64 * a.Fq;
    const int q0 = qt * 64 * QT + wave * 16 * QT;

    u32x4 qf[QT][2];
#pragma unroll
    for (int s = 0; s < QT; ++s)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            qf[s][kk] = ld16(qb + (size_t)(q0 + 16 * s + r16) * 64 + kk * 32 + g * 8);

    // staging: pieces tid, tid + 256 of K (key = p / 8), of V^T (dim = p / 8)
    u32x4 rk[2], rv[2];
    int soff[2];
    const uint16_t *ksrc[2], *vsrc[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const int p = tid + 256 * v, row = p >> 3, pc = p & 7;
        soff[v] = row * AROW + pc * 8;
        ksrc[v] = kb + (size_t)row * 64 + pc * 8;
        vsrc[v] = vb + (size_t)row * a.Fq + pc * 8;
    }
    auto gload = [&](int key0) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            rk[v] = ld16(ksrc[v] + (size_t)key0 * 64);
            rv[v] = ld16(vsrc[v] + key0);
        }
    };
    auto sstore = [&](int b) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            *reinterpret_cast<u32x4 *>(&ks[b][soff[v]]) = rk[v];
            *reinterpret_cast<u32x4 *>(&vs[b][soff[v]]) = rv[v];
        }
    };

    // row sums ride on the MFMA: a tile of ones times P^T adds, in every
    // row of lsum[s], the bf16 probabilities the PV product uses
    const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    float mrow[QT];
    f32x4 lsum[QT];
    f32x4 o[4][QT];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
        mrow[s] = -INFINITY;
        lsum[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int steps = (a.F + 63) >> 6;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
        const int b = st & 1, key0 = st * 64;
        if (st + 1 < steps) gload(key0 + 64);
        // fragments of this step, shared by the four query subtiles
        u32x4 kf[4][2], vf[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                kf[kt][kk] = *reinterpret_cast<const u32x4 *>(&ks[b][(kt * 16 + r16) * AROW + kk * 32 + g * 8]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint16_t *vrow = &vs[b][(dt * 16 + r16) * AROW + kk * 32 + 4 * g];
                const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow);
                const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 16);
                vf[dt][kk] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        const bool tail = key0 + 64 > a.F;
        // one subtile at a time (scores, softmax, PV), so one subtile's VALU
        // work can overlap the next one's MFMAs
#pragma unroll
        for (int s = 0; s < QT; ++s) {
            f32x4 sc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                sc[kt] = mfma_bf16_k32(kf[kt][0], qf[s][0], f32x4{0.f, 0.f, 0.f, 0.f});
                sc[kt] = mfma_bf16_k32(kf[kt][1], qf[s][1], sc[kt]);
            }
            if (tail) {                                  // keys past F
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (key0 + kt * 16 + 4 * g + r >= a.F) sc[kt][r] = -INFINITY;
            }
            float ml = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
#pragma unroll
            for (int kt = 1; kt < 4; ++kt)
                ml = fmaxf(ml, fmaxf(fmaxf(sc[kt][0], sc[kt][1]), fmaxf(sc[kt][2], sc[kt][3])));
            float x0, x1;
            rows16_pair(ml, x0, x1);
            ml = fmaxf(x0, x1);
            halves32_pair(ml, x0, x1);
            ml = fmaxf(x0, x1);
            // every step holds a live key, so mnew is finite; the first step's
            // mrow = -inf gives alpha = 0, a masked score exp2(-inf) = 0
            const float mnew = fmaxf(mrow[s], ml);
            const float ms = mnew * a.sl2e;
            const float alpha = __builtin_amdgcn_exp2f(__fmaf_rn(mrow[s], a.sl2e, -ms));
            mrow[s] = mnew;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sc[kt][r] = __builtin_amdgcn_exp2f(__fmaf_rn(sc[kt][r], a.sl2e, -ms));
            lsum[s] = lsum[s] * alpha;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 pf = u32x4{pack_bf2(sc[2 * kk][0], sc[2 * kk][1]),
                                       pack_bf2(sc[2 * kk][2], sc[2 * kk][3]),
                                       pack_bf2(sc[2 * kk + 1][0], sc[2 * kk + 1][1]),
                                       pack_bf2(sc[2 * kk + 1][2], sc[2 * kk + 1][3])};
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    if (kk == 0) o[dt][s] = o[dt][s] * alpha;
                    o[dt][s] = mfma_bf16_k32(vf[dt][kk], pf, o[dt][s]);
                }
                lsum[s] = mfma_bf16_k32(ones, pf, lsum[s]);
            }
        }
        if (st + 1 < steps) sstore(b ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < QT; ++s) {
        const float inv = 1.0f / lsum[s][0];      // every row of the tile holds the sum
        const int qi = q0 + 16 * s + r16;
        if (qi >= a.F) continue;
        uint16_t *dst = a.o + ((size_t)rq * a.F + qi) * a.d + h * 64 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const f32x4 v = o[dt][s];
            *reinterpret_cast<u32x2 *>(dst + dt * 16) =
                u32x2{pack_bf2(v[0] * inv, v[1] * inv), pack_bf2(v[2] * inv, v[3] * inv)};
        }
    }
}

// Layer norm of fp32 rows (one wave per row, d <= 1280, d % 4 == 0) to bf16
// rows at out + row * d.
__global__ __launch_bounds__(256) void ln_kernel(const float *x, int M, int d, const uint16_t *gam,
                                                 const uint16_t *bet, float eps, uint16_t *out) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= M) return;
    const float *xr = x + (size_t)row * d;
    float4 v[5];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int c = 4 * lane + 256 * i;
        v[i] = c < d ? *reinterpret_cast<const float4 *>(xr + c) : float4{0.f, 0.f, 0.f, 0.f};
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float mean = wave_sum(s) / (float)d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int c = 4 * lane + 256 * i;
        if (c < d) {
            const float t0 = v[i].x - mean, t1 = v[i].y - mean, t2 = v[i].z - mean, t3 = v[i].w - mean;
            q = __fmaf_rn(t0, t0, q);
            q = __fmaf_rn(t1, t1, q);
            q = __fmaf_rn(t2, t2, q);
            q = __fmaf_rn(t3, t3, q);
        }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int c = 4 * lane + 256 * i;
        if (c < d) {
            const float y0 = __fmaf_rn((v[i].x - mean) * rstd, bf2f(gam[c]), bf2f(bet[c]));
            const float y1 = __fmaf_rn((v[i].y - mean) * rstd, bf2f(gam[c + 1]), bf2f(bet[c + 1]));
            const float y2 = __fmaf_rn((v[i].z - mean) * rstd, bf2f(gam[c + 2]), bf2f(bet[c + 2]));
            const float y3 = __fmaf_rn((v[i].w - mean) * rstd, bf2f(gam[c + 3]), bf2f(bet[c + 3]));
            *reinterpret_cast<u32x2 *>(out + (size_t)row * d + c) = u32x2{pack_bf2(y0, y1), pack_bf2(y2, y3)};
        }
    }
}

// Features [n][C][T] (channel-major) to time-major rows melT[n][1 + t][C];
// rows 0 and T + 1 of each request stay zero. One workgroup per (request,
// 64 frames), staged through LDS (C <= 256).
__global__ __launch_bounds__(256) void mel_kernel(const uint16_t *mel, int C, int T, uint16_t *melT) {
    __shared__ uint16_t tile[64][257];
    const int nb = (T + 63) >> 6;
    const int rq = blockIdx.x / nb, t0 = (blockIdx.x - rq * nb) * 64;
    const uint16_t *src = mel + (size_t)rq * C * T;
    for (int e = threadIdx.x; e < C * 64; e += 256) {
        const int c = e >> 6, t = e & 63;
        if (t0 + t < T) tile[t][c] = src[(size_t)c * T + t0 + t];
    }
    __syncthreads();
    uint16_t *dst = melT + ((size_t)rq * (T + 2) + 1 + t0) * C;
    for (int e = threadIdx.x; e < C * 64; e += 256) {
        const int t = e / C, c = e - t * C;
        if (t0 + t < T) dst[(size_t)t * C + c] = tile[t][c];
    }
}

// Convolution weight [out][in][3] (PyTorch Conv1d) to [out][tap][in], the
// order of a time-major 3-row window.
__global__ void conv_relayout_kernel(const uint16_t *w, int O, int I, uint16_t *wr) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (size_t)O * I * 3) return;
    const int o = (int)(e / ((size_t)I * 3));
    const int rem = (int)(e - (size_t)o * I * 3);
    const int i = rem / 3, k = rem - i * 3;
    wr[((size_t)o * 3 + k) * I + i] = w[e];
}

// Sinusoidal positions [F][d] in fp32: channel j < d/2 holds sin(t w_j),
// channel d/2 + j holds cos(t w_j), w_j = 10000^(-j / (d/2 - 1)); the angle
// is formed in fp64.
__global__ void pos_kernel(int F, int d, float *pos) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= F * d) return;
    const int t = e / d, c = e - t * d, hh = d / 2;
    const int j = c < hh ? c : c - hh;
    const double ang = (double)t * exp(-log(10000.0) * (double)j / (double)(hh - 1));
    pos[e] = (float)(c < hh ? sin(ang) : cos(ang));
}

inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int MT, int NT>
hipError_t launch_tiles(int epi, const GemmArgs &a, hipStream_t st) {
    const dim3 grid(cdiv(a.n_wg, 8) * 8), blk(256);
    switch (epi) {
    case EE_CONV1: hipLaunchKernelGGL((gemm_kernel<EE_CONV1, MT, NT>), grid, blk, 0, st, a); break;
    case EE_CONV2: hipLaunchKernelGGL((gemm_kernel<EE_CONV2, MT, NT>), grid, blk, 0, st, a); break;
    case EE_QKV: hipLaunchKernelGGL((gemm_kernel<EE_QKV, MT, NT>), grid, blk, 0, st, a); break;
    case EE_RESID: hipLaunchKernelGGL((gemm_kernel<EE_RESID, MT, NT>), grid, blk, 0, st, a); break;
    case EE_XKV: hipLaunchKernelGGL((gemm_kernel<EE_XKV, MT, NT>), grid, blk, 0, st, a); break;
    default: hipLaunchKernelGGL((gemm_kernel<EE_GELU, MT, NT>), grid, blk, 0, st, a); break;
    }
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_dma_epi(const GemmArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((gemm_dma_kernel<EPI>), dim3(cdiv(a.n_wg, 8) * 8), dim3(512), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_dma(int epi, const GemmArgs &a, hipStream_t st) {
    switch (epi) {
    case EE_CONV1: return launch_dma_epi<EE_CONV1>(a, st);
    case EE_CONV2: return launch_dma_epi<EE_CONV2>(a, st);
    case EE_QKV: return launch_dma_epi<EE_QKV>(a, st);
    case EE_RESID: return launch_dma_epi<EE_RESID>(a, st);
    case EE_XKV: return launch_dma_epi<EE_XKV>(a, st);
    default: return launch_dma_epi<EE_GELU>(a, st);
    }
}

// 256 x 256 tiles (the LDS-copy kernel) from two rounds of workgroups on;
// else 128 x 256 tiles, or 64 x 128 when those would leave most of the 256
// CUs idle (a window or two through the d-wide projections)
hipError_t launch_gemm(int epi, GemmArgs &a, hipStream_t st) {
    if (a.K % (2 * GBK) || a.M < 1 || a.N % 4) return hipErrorInvalidValue;   // loop unrolled by 2
    if (cdiv(a.M, DBT) * cdiv(a.N, DBT) >= 512) {
        a.n_m = cdiv(a.M, DBT);
        a.n_n = cdiv(a.N, DBT);
        a.n_wg = a.n_m * a.n_n;
        return launch_dma(epi, a, st);
    }
    const bool small = cdiv(a.M, 128) * cdiv(a.N, 256) < 128;
    a.n_m = cdiv(a.M, small ? 64 : 128);
    a.n_n = cdiv(a.N, small ? 128 : 256);
    a.n_wg = a.n_m * a.n_n;
    return small ? launch_tiles<2, 4>(epi, a, st) : launch_tiles<4, 8>(epi, a, st);
}

}  // namespace enc

// A decoder layer's cross K = enc W_k^T and V = enc W_v^T + b_v for n
// requests (enc bf16 [n][F][K] rows), written in fp16 into each request's
// slot of the write-once pool: the dense GEMM above with the pool epilogue.
hipError_t launch_xkv_dense(const uint16_t *enc, int M, int K, const uint16_t *wk,
                            const uint16_t *wv, const uint16_t *bv, uint16_t *xkv,
                            long long slot_stride, long long layer_off, const int32_t *slots,
                            int F, int F_pad, int H, int hd, int max_batch, hipStream_t st) {
    enc::GemmArgs a{};
    a.A = enc;
    a.rpr = M;
    a.srow = K;
    a.W0 = wk;
    a.W1 = a.W2 = wv;
    a.b1 = bv;
    a.M = M;
    a.N = 2 * H * hd;
    a.K = K;
    a.seg_n = H * hd;
    a.F = F;
    a.H = H;
    a.xkv = xkv;
    a.slot_stride = slot_stride;
    a.layer_off = layer_off;
    a.slots = slots;
    a.F_pad = F_pad;
    a.hd = hd;
    a.max_batch = max_batch;
    return enc::launch_gemm(enc::EE_XKV, a, st);
}

namespace enc {

struct LayerW {
    const uint16_t *ln1_g, *ln1_b, *wq, *bq, *wk, *wv, *bv, *wo, *bo;
    const uint16_t *ln2_g, *ln2_b, *w1, *b1, *w2, *b2;
};

struct Layout {
    size_t melT, g1, x, h, q, k, vt, o, hid, pos, w1r, w2r, total;
};

int f_q(const wf_enc_config *c) { return cdiv(c->n_frames, 256) * 256; }

Layout layout_of(const wf_enc_config *c) {
    Layout L{};
    const size_t B = c->max_batch, F = c->n_frames, Tm = 2 * (size_t)c->n_frames, d = c->d_model;
    const size_t Fq = f_q(c), H = c->n_heads;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.melT = take(B * (Tm + 2) * c->n_mels * 2);
    L.g1 = take(B * (Tm + 2) * d * 2);
    L.x = take(B * F * d * 4);
    L.h = take(B * F * d * 2);
    L.q = take(B * H * Fq * 64 * 2);
    L.k = take(B * H * Fq * 64 * 2);
    L.vt = take(B * H * 64 * Fq * 2);
    L.o = take(B * F * d * 2);
    L.hid = take(B * F * c->d_ffn * 2);
    L.pos = take(F * d * 4);
    L.w1r = take(d * 3 * c->n_mels * 2);
    L.w2r = take(d * 3 * d * 2);
    L.total = off;
    return L;
}

bool config_ok(const wf_enc_config *c, const char **why) {
    const char *w = nullptr;
    if (!c) w = "null config";
    else if (c->n_layers < 1) w = "n_layers < 1";
    else if (c->head_dim != 64) w = "head_dim must be 64";
    else if (c->n_heads < 1 || c->n_heads * 64 != c->d_model) w = "d_model must be n_heads * 64";
    else if (c->d_model > 1280) w = "d_model above 1280";
    else if (c->d_ffn < 64 || c->d_ffn % 64) w = "d_ffn must be a positive multiple of 64";
    else if (c->n_mels < 64 || c->n_mels > 256 || c->n_mels % 64) w = "n_mels must be 64, 128, 192 or 256";
    else if (c->n_frames < 1 || c->n_frames > 4096) w = "n_frames outside [1, 4096]";
    else if (c->max_batch < 1 || (long long)c->max_batch * 2 * (c->n_frames + 1) > 0x3fffffff) w = "max_batch out of range";
    else if (!(c->ln_eps > 0.f)) w = "ln_eps must be positive";
    if (why) *why = w;
    return w == nullptr;
}

}  // namespace enc
}  // namespace wf

using namespace wf::enc;

struct wf_encoder {
    wf_enc_config c;
    Layout lay;
    std::vector<LayerW> layers;
    const uint16_t *c1b, *c2b, *lnp_g, *lnp_b;
    uint16_t *melT, *g1, *h, *q, *k, *vt, *o, *hid, *w1r, *w2r;
    float *x, *pos;
    int attn_qt = 2;   // 16-query subtiles per attention wave (measured best of 1, 2, 4)
    bool timing = false;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_used = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> spans[WF_ENC_TK_N];
};

namespace {

wf_status efail(wf_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return wf::set_error(s, buf);
}

hipEvent_t next_event(wf_encoder *e) {
    if (e->ev_used == e->ev_pool.size()) {
        hipEvent_t ev;
        if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        e->ev_pool.push_back(ev);
    }
    return e->ev_pool[e->ev_used++];
}

template <typename Fn>
wf_status timed(wf_encoder *e, int kind, hipStream_t st, Fn &&launch) {
    hipEvent_t a = nullptr, b = nullptr;
    if (e->timing) {
        a = next_event(e);
        b = next_event(e);
        if (a) (void)hipEventRecord(a, st);
    }
    const hipError_t err = launch();
    if (err != hipSuccess) return efail(WF_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    if (e->timing && a && b) {
        (void)hipEventRecord(b, st);
        e->spans[kind].push_back({a, b});
    }
    return WF_OK;
}

#define WFE_TRY(expr)                     \
    do {                                  \
        const wf_status _s = (expr);      \
        if (_s != WF_OK) return _s;       \
    } while (0)

wf_status run_ln(wf_encoder *e, int M, const uint16_t *g, const uint16_t *b, uint16_t *out,
                 hipStream_t st) {
    const wf_enc_config &c = e->c;
    return timed(e, WF_ENC_TK_LN, st, [&] {
        hipLaunchKernelGGL(ln_kernel, dim3(cdiv(M, 4)), dim3(256), 0, st, e->x, M, c.d_model, g, b,
                           c.ln_eps, out);
        return hipGetLastError();
    });
}

GemmArgs plain(const uint16_t *A, int M, int K, const uint16_t *W, const uint16_t *b, int N) {
    GemmArgs a{};
    a.A = A;
    a.rpr = M;
    a.sreq = 0;
    a.srow = K;
    a.W0 = a.W1 = a.W2 = W;
    a.b0 = b;
    a.M = M;
    a.N = N;
    a.K = K;
    a.seg_n = N;
    return a;
}

}  // namespace

extern "C" {

size_t wf_enc_workspace_bytes(const wf_enc_config *c) {
    if (!config_ok(c, nullptr)) return 0;
    return layout_of(c).total;
}

wf_status wf_enc_create(const wf_enc_config *cfg, const wf_enc_weights *w, void *workspace,
                        size_t ws_bytes, wf_encoder **out) {
    if (!out) return efail(WF_EINVAL, "out is null");
    *out = nullptr;
    const char *why = nullptr;
    if (!config_ok(cfg, &why)) return efail(WF_ESHAPE, "bad encoder config: %s", why);
    if (!w || !w->conv1_w || !w->conv1_b || !w->conv2_w || !w->conv2_b || !w->lnp_g || !w->lnp_b ||
        !w->layers)
        return efail(WF_EINVAL, "null encoder weight pointer");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const wf_enc_layer_weights &L = w->layers[l];
        const void *ps[] = {L.ln1_g, L.ln1_b, L.wq, L.bq, L.wk, L.wv, L.bv, L.wo,
                            L.bo,    L.ln2_g, L.ln2_b, L.w1, L.b1, L.w2, L.b2};
        for (const void *p : ps)
            if (!p) return efail(WF_EINVAL, "null weight pointer in encoder block %d", l);
    }
    if (!workspace) return efail(WF_EINVAL, "null workspace");
    if (ws_bytes < wf_enc_workspace_bytes(cfg)) return efail(WF_ECAPACITY, "workspace too small");
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return efail(WF_EDEVICE, "no HIP device");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return efail(WF_EDEVICE, "device is %s, not gfx950", prop.gcnArchName);

    wf_encoder *e = new wf_encoder();
    e->c = *cfg;
    e->lay = layout_of(cfg);
    const Layout &L = e->lay;
    char *ws = (char *)workspace;
    e->melT = (uint16_t *)(ws + L.melT);
    e->g1 = (uint16_t *)(ws + L.g1);
    e->x = (float *)(ws + L.x);
    e->h = (uint16_t *)(ws + L.h);
    e->q = (uint16_t *)(ws + L.q);
    e->k = (uint16_t *)(ws + L.k);
    e->vt = (uint16_t *)(ws + L.vt);
    e->o = (uint16_t *)(ws + L.o);
    e->hid = (uint16_t *)(ws + L.hid);
    e->pos = (float *)(ws + L.pos);
    e->w1r = (uint16_t *)(ws + L.w1r);
    e->w2r = (uint16_t *)(ws + L.w2r);
    e->c1b = (const uint16_t *)w->conv1_b;
    e->c2b = (const uint16_t *)w->conv2_b;
    e->lnp_g = (const uint16_t *)w->lnp_g;
    e->lnp_b = (const uint16_t *)w->lnp_b;
    e->layers.resize(cfg->n_layers);
    for (int l = 0; l < cfg->n_layers; ++l) {
        const wf_enc_layer_weights &s = w->layers[l];
        e->layers[l] = LayerW{(const uint16_t *)s.ln1_g, (const uint16_t *)s.ln1_b,
                              (const uint16_t *)s.wq,    (const uint16_t *)s.bq,
                              (const uint16_t *)s.wk,    (const uint16_t *)s.wv,
                              (const uint16_t *)s.bv,    (const uint16_t *)s.wo,
                              (const uint16_t *)s.bo,    (const uint16_t *)s.ln2_g,
                              (const uint16_t *)s.ln2_b, (const uint16_t *)s.w1,
                              (const uint16_t *)s.b1,    (const uint16_t *)s.w2,
                              (const uint16_t *)s.b2};
    }
    // zero padding everywhere (the convolution borders and the padded frames
    // of q / k / v^T are never written), then the position table and the
    // convolution weights in window order
    const int d = cfg->d_model, F = cfg->n_frames;
    bool ok = hipMemset(workspace, 0, L.total) == hipSuccess;
    if (ok) {
        hipLaunchKernelGGL(pos_kernel, dim3(cdiv(F * d, 256)), dim3(256), 0, 0, F, d, e->pos);
        hipLaunchKernelGGL(conv_relayout_kernel, dim3(cdiv(d * cfg->n_mels * 3, 256)), dim3(256), 0, 0,
                           (const uint16_t *)w->conv1_w, d, cfg->n_mels, e->w1r);
        hipLaunchKernelGGL(conv_relayout_kernel, dim3(cdiv(d * d * 3, 256)), dim3(256), 0, 0,
                           (const uint16_t *)w->conv2_w, d, d, e->w2r);
        ok = hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess;
    }
    if (!ok) {
        delete e;
        return efail(WF_EHIP, "preparing the encoder workspace failed");
    }
    *out = e;
    return WF_OK;
}

void wf_enc_destroy(wf_encoder *e) {
    if (!e) return;
    for (hipEvent_t ev : e->ev_pool) (void)hipEventDestroy(ev);
    delete e;
}

wf_status wf_encode(wf_encoder *e, int32_t n, const void *d_mel, void *d_out, void *stream) {
    if (!e || !d_mel || !d_out) return efail(WF_EINVAL, "null argument");
    const wf_enc_config &c = e->c;
    if (n < 1 || n > c.max_batch) return efail(WF_ECAPACITY, "n outside [1, max_batch]");
    hipStream_t st = (hipStream_t)stream;
    const int d = c.d_model, F = c.n_frames, Tm = 2 * F, H = c.n_heads, Fq = f_q(&c);
    const int M = n * F;
    WFE_TRY(timed(e, WF_ENC_TK_OTHER, st, [&] {
        hipLaunchKernelGGL(mel_kernel, dim3(n * cdiv(Tm, 64)), dim3(256), 0, st,
                           (const uint16_t *)d_mel, c.n_mels, Tm, e->melT);
        return hipGetLastError();
    }));
    {   // stem: conv1 (stride 1) into padded rows, conv2 (stride 2) + positions
        GemmArgs a = plain(e->melT, n * Tm, 3 * c.n_mels, e->w1r, e->c1b, d);
        a.rpr = Tm;
        a.sreq = (long long)(Tm + 2) * c.n_mels;
        a.srow = c.n_mels;
        a.out = e->g1;
        a.Tm = Tm;
        WFE_TRY(timed(e, WF_ENC_TK_STEM, st, [&] { return launch_gemm(EE_CONV1, a, st); }));
        GemmArgs b = plain(e->g1, M, 3 * d, e->w2r, e->c2b, d);
        b.rpr = F;
        b.sreq = (long long)(Tm + 2) * d;
        b.srow = 2 * d;
        b.x = e->x;
        b.pos = e->pos;
        b.F = F;
        WFE_TRY(timed(e, WF_ENC_TK_STEM, st, [&] { return launch_gemm(EE_CONV2, b, st); }));
    }
    for (int l = 0; l < c.n_layers; ++l) {
        const LayerW &w = e->layers[l];
        WFE_TRY(run_ln(e, M, w.ln1_g, w.ln1_b, e->h, st));
        GemmArgs a = plain(e->h, M, d, w.wq, w.bq, 3 * d);
        a.W1 = w.wk;
        a.W2 = w.wv;
        a.b1 = nullptr;
        a.b2 = w.bv;
        a.seg_n = d;
        a.q = e->q;
        a.k = e->k;
        a.vt = e->vt;
        a.H = H;
        a.Fq = Fq;
        a.F = F;
        WFE_TRY(timed(e, WF_ENC_TK_QKV, st, [&] { return launch_gemm(EE_QKV, a, st); }));
        AttnArgs t{};
        t.q = e->q;
        t.k = e->k;
        t.vt = e->vt;
        t.o = e->o;
        t.H = H;
        t.F = F;
        t.Fq = Fq;
        t.d = d;
        t.n_qt = Fq / (64 * e->attn_qt);
        t.n_wg = n * H * t.n_qt;
        t.sl2e = 1.4426950408889634f / 8.0f;
        WFE_TRY(timed(e, WF_ENC_TK_ATTN, st, [&] {
            if (e->attn_qt == 4)
                hipLaunchKernelGGL(attn_kernel<4>, dim3(cdiv(t.n_wg, 8) * 8), dim3(256), 0, st, t);
            else if (e->attn_qt == 1)
                hipLaunchKernelGGL(attn_kernel<1>, dim3(cdiv(t.n_wg, 8) * 8), dim3(256), 0, st, t);
            else
                hipLaunchKernelGGL(attn_kernel<2>, dim3(cdiv(t.n_wg, 8) * 8), dim3(256), 0, st, t);
            return hipGetLastError();
        }));
        GemmArgs ob = plain(e->o, M, d, w.wo, w.bo, d);
        ob.x = e->x;
        WFE_TRY(timed(e, WF_ENC_TK_OPROJ, st, [&] { return launch_gemm(EE_RESID, ob, st); }));
        WFE_TRY(run_ln(e, M, w.ln2_g, w.ln2_b, e->h, st));
        GemmArgs f1 = plain(e->h, M, d, w.w1, w.b1, c.d_ffn);
        f1.out = e->hid;
        WFE_TRY(timed(e, WF_ENC_TK_FC1, st, [&] { return launch_gemm(EE_GELU, f1, st); }));
        GemmArgs f2 = plain(e->hid, M, c.d_ffn, w.w2, w.b2, d);
        f2.x = e->x;
        WFE_TRY(timed(e, WF_ENC_TK_FC2, st, [&] { return launch_gemm(EE_RESID, f2, st); }));
    }
    return run_ln(e, M, e->lnp_g, e->lnp_b, (uint16_t *)d_out, st);
}

wf_status wf_enc_set_timing(wf_encoder *e, int32_t enable) {
    if (!e) return efail(WF_EINVAL, "null encoder");
    e->timing = enable != 0;
    for (auto &v : e->spans) v.clear();
    e->ev_used = 0;
    return WF_OK;
}

wf_status wf_enc_get_timing(wf_encoder *e, int32_t kind, double *total_ms, int32_t *count) {
    if (!e || !total_ms || !count) return efail(WF_EINVAL, "null argument");
    if (kind < 0 || kind >= WF_ENC_TK_N) return efail(WF_EINVAL, "unknown timing kind");
    double tot = 0;
    for (auto &p : e->spans[kind]) {
        if (hipEventSynchronize(p.second) != hipSuccess) return efail(WF_EHIP, "event synchronize failed");
        float ms = 0;
        if (hipEventElapsedTime(&ms, p.first, p.second) != hipSuccess)
            return efail(WF_EHIP, "elapsed time failed");
        tot += ms;
    }
    *total_ms = tot;
    *count = (int32_t)e->spans[kind].size();
    return WF_OK;
}

}  // extern "C"
