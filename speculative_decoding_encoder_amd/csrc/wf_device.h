// Device helpers for the gfx950 kernels: vector types, MFMA wrappers,
// bf16/fp16 conversions and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define WF_WAVE 64

// 16 bytes from global memory as one vector load.
__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ u32x2 ld8(const void *p) {
    return *reinterpret_cast<const u32x2 *>(p);
}
// Streaming loads (data read once): non-temporal, so they do not compete
// with reused lines in the caches.
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x2 ld8_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

__device__ __forceinline__ f32x4 mfma_bf16_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                  __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// GEMM activations (the A operand: layer-norm outputs, attention outputs,
// the MLP hidden layer, the drafter's history taps) are fp16, stored
// fragment-tiled: for each 16-row tile and 32-column step one 1 KB block in
// the lane order of the MFMA A operand (lane g*16 + r holds row r, columns
// 8g..8g+7). A fragment load is one contiguous 1 KB read. Buffers hold whole
// 16-row tiles. xh_index gives the element (m, k).
__host__ __device__ __forceinline__ size_t xh_index(int m, int k, int K) {
    return (((size_t)(m >> 4) * (size_t)(K >> 5) + (size_t)(k >> 5)) * 64 +
            (size_t)(((k >> 3) & 3) * 16 + (m & 15))) * 8 + (size_t)(k & 7);
}

// Cross-attention V blocks (one per 32-frame step, [hd][32]): the position of
// frame j (0..31 within its step). Position 8g + i holds frame 4g + i for
// i < 4 and frame 16 + 4g + i - 4 otherwise, the order in which the
// transposed score tiles leave the probabilities in a lane's registers.
__host__ __device__ __forceinline__ int xv_pos(int j) {
    return j < 16 ? 8 * (j >> 2) + (j & 3) : 8 * ((j - 16) >> 2) + 4 + (j & 3);
}

// Cross-attention K (per head, F_pad frames x hd): each 32-frame step is one
// block in the lane order of the MFMA A operand of S^T = K Q^T, a 1 KB (hd
// 64) or 512 B (hd 16) piece per 16-frame tile and operand load, so every
// load of a step reads consecutive addresses. Element offset of (frame f,
// dim c) within the head.
__host__ __device__ __forceinline__ size_t xk_index(int f, int c, int hd) {
    const size_t step = (size_t)(f >> 5) * 32 * hd;
    const int t = (f >> 4) & 1, r = f & 15;
    if (hd == 16) return step + t * 256 + ((c >> 2) * 16 + r) * 4 + (c & 3);
    return step + ((size_t)(t * (hd >> 5) + (c >> 5)) * 64 + ((c >> 3) & 3) * 16 + r) * 8 +
           (c & 7);
}

// bf16 <-> fp32. Rounding to bf16 is to nearest, ties to even.
__device__ __forceinline__ float bf2f(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f2h_bits(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float h2f_bits(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
// Two floats to packed fp16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return (uint32_t)f2h_bits(lo) | ((uint32_t)f2h_bits(hi) << 16);
}
// Eight bf16 weights to fp16 for the fp16 MFMA. Exact for |w| >= 2^-14 (every
// bf16 value there has an fp16 twin); below, fp16 subnormals keep |w| to
// 2^-24 (the packed conversion rounds toward zero).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(w[j] << 16), hi = __uint_as_float(w[j] & 0xffff0000u);
        r[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    return r;
}

// Cross-lane exchange without LDS. Within a row of 16 lanes, DPP: level 0
// and 1 of a butterfly read the xor-1 / xor-2 partner (quad_perm); levels 2
// and 3 read the mirrored lane within 8 / 16 lanes (row_half_mirror /
// row_mirror), which holds the xor-4 / xor-8 partner's value because a
// butterfly has made every quad / every 8 lanes agree by then. Across rows
// (gfx950 permlane swaps of a register with itself): the two halves of the
// result hold the values of the xor-16 (xor-32) partners in the same order in
// every lane, so a symmetric operation on them gives one result for both.
template <int S>
__device__ __forceinline__ uint32_t bfly16_u(uint32_t v) {
    constexpr int C = S == 0 ? 0xB1 : (S == 1 ? 0x4E : (S == 2 ? 0x141 : 0x140));
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, C, 0xf, 0xf, false);
}
template <int S>
__device__ __forceinline__ float bfly16(float v) { return __uint_as_float(bfly16_u<S>(__float_as_uint(v))); }
template <int S>
__device__ __forceinline__ int bfly16(int v) { return (int)bfly16_u<S>((uint32_t)v); }
__device__ __forceinline__ void rows16_pair(float v, float &a, float &b) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void halves32_pair(float v, float &a, float &b) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void rows16_pair(int v, int &a, int &b) {
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    a = (int)p[0];
    b = (int)p[1];
}
__device__ __forceinline__ void halves32_pair(int v, int &a, int &b) {
    const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    a = (int)p[0];
    b = (int)p[1];
}

// Reductions within groups of 16 lanes (lanes 16g .. 16g+15), fixed
// butterfly; every lane of the group gets the same bits.
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, bfly16<0>(v));
    v = fmaxf(v, bfly16<1>(v));
    v = fmaxf(v, bfly16<2>(v));
    v = fmaxf(v, bfly16<3>(v));
    return v;
}
__device__ __forceinline__ float sum16(float v) {
    v += bfly16<0>(v);
    v += bfly16<1>(v);
    v += bfly16<2>(v);
    v += bfly16<3>(v);
    return v;
}
// Whole-wave reductions, fixed tree (the 16-lane butterfly, then the row
// pairs, then the halves).
__device__ __forceinline__ float wave_sum(float v) {
    v = sum16(v);
    float a, b;
    rows16_pair(v, a, b);
    v = a + b;
    halves32_pair(v, a, b);
    return a + b;
}
__device__ __forceinline__ float wave_max(float v) {
    v = max16(v);
    float a, b;
    rows16_pair(v, a, b);
    v = fmaxf(a, b);
    halves32_pair(v, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ int wave_or(int v) {
    v |= bfly16<0>(v);
    v |= bfly16<1>(v);
    v |= bfly16<2>(v);
    v |= bfly16<3>(v);
    int a, b;
    rows16_pair(v, a, b);
    v = a | b;
    halves32_pair(v, a, b);
    return a | b;
}
// (value, index) argmax: larger value wins, equal values go to the lower
// index (symmetric: the merge of two candidates does not depend on order).
__device__ __forceinline__ void argmax_merge(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
template <int S>
__device__ __forceinline__ void argmax_bfly16(float &v, int &i) {
    const float v2 = bfly16<S>(v);
    const int i2 = bfly16<S>(i);
    argmax_merge(v, i, v2, i2);
}
// argmax over the 16 lanes of each group; nan: OR over the group
__device__ __forceinline__ void argmax16(float &v, int &i, int &nan) {
    argmax_bfly16<0>(v, i);
    argmax_bfly16<1>(v, i);
    argmax_bfly16<2>(v, i);
    argmax_bfly16<3>(v, i);
    nan |= bfly16<0>(nan);
    nan |= bfly16<1>(nan);
    nan |= bfly16<2>(nan);
    nan |= bfly16<3>(nan);
}
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
    argmax_bfly16<0>(v, i);
    argmax_bfly16<1>(v, i);
    argmax_bfly16<2>(v, i);
    argmax_bfly16<3>(v, i);
    float va, vb;
    int ia, ib;
    rows16_pair(v, va, vb);
    rows16_pair(i, ia, ib);
    v = va;
    i = ia;
    argmax_merge(v, i, vb, ib);
    halves32_pair(v, va, vb);
    halves32_pair(i, ia, ib);
    v = va;
    i = ia;
    argmax_merge(v, i, vb, ib);
}

// Handoff of partial results between workgroups (possibly on different
// XCDs): the producer writes with device-coherent stores (agent-scope relaxed
// atomics, which write through to the device coherence point), waits until
// all its vector memory operations have completed, then bumps an arrival
// counter; the last arriver reads the partials with device-coherent loads.
// This avoids a full L2 write-back per producer.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// cache policy of device-coherent buffer accesses (write through to, and
// read from, the device coherence point)
#define CPOL_SC1 16

// s_waitcnt vmcnt(0): every vector memory operation of this wave (stores
// included) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ int arrive(int *cnt) {
    return __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void rearm(int *cnt) {
    __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Layer norm of one row by the 16 lanes of a lane group (lanes 16q..16q+15):
// lane r16 owns the 8-column groups r16, r16+16, ... (rows up to
// 16 * 8 * LN_GPL columns), holds them in registers, and the mean and
// variance come from two passes over those registers in a fixed order with
// the sum16 butterfly. The normalised value is fma((x - mean) * rstd, gain,
// bias). The standalone kernel and the GEMM prologue both use exactly this,
// so a row normalises to the same bits either way.
#define LN_GPL 10
struct LnRow {
    float4 v[2 * LN_GPL];
};
// Loads only (clamped to the row: unconditional, so they can be in flight
// together with other loads issued after them).
__device__ __forceinline__ void ln_load16(const float *xrow, int d, int r16, LnRow &row) {
    const int last = (d >> 3) - 1;
#pragma unroll
    for (int i = 0; i < LN_GPL; ++i) {
        const int kg = min(r16 + 16 * i, last);
        row.v[2 * i] = *reinterpret_cast<const float4 *>(xrow + kg * 8);
        row.v[2 * i + 1] = *reinterpret_cast<const float4 *>(xrow + kg * 8 + 4);
    }
}
__device__ __forceinline__ void ln_reduce16(const LnRow &row, int d, int r16, float eps,
                                            float &mean, float &rstd) {
    // groups past the row add nothing (selects, not branches: the compiler
    // then waits only for this row's loads, not for every load in flight)
    const int ng = d >> 3;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < LN_GPL; ++i) {
        const float4 v0 = row.v[2 * i], v1 = row.v[2 * i + 1];
        const float t = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w));
        s = r16 + 16 * i < ng ? s + t : s;
    }
    mean = sum16(s) / (float)d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < LN_GPL; ++i) {
        const float4 v0 = row.v[2 * i], v1 = row.v[2 * i + 1];
        const float t[8] = {v0.x - mean, v0.y - mean, v0.z - mean, v0.w - mean,
                            v1.x - mean, v1.y - mean, v1.z - mean, v1.w - mean};
        float qi = q;
#pragma unroll
        for (int j = 0; j < 8; ++j) qi = __fmaf_rn(t[j], t[j], qi);
        q = r16 + 16 * i < ng ? qi : q;
    }
    const float var = sum16(q) / (float)d;
    rstd = 1.0f / sqrtf(var + eps);
}
__device__ __forceinline__ float ln_apply(float x, float mean, float rstd, float g, float b) {
    return __fmaf_rn((x - mean) * rstd, g, b);
}
// Eight consecutive columns (x at c..c+7, gains and biases as bf16x8) to one
// fp16 activation fragment.
__device__ __forceinline__ u32x4 ln_h8(float4 x0, float4 x1, u32x4 gg, u32x4 bb, float mean,
                                       float rstd) {
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float y0 = ln_apply(xv[2 * j], mean, rstd, bf2f((uint16_t)(gg[j] & 0xffffu)),
                                  bf2f((uint16_t)(bb[j] & 0xffffu)));
        const float y1 = ln_apply(xv[2 * j + 1], mean, rstd, bf2f((uint16_t)(gg[j] >> 16)),
                                  bf2f((uint16_t)(bb[j] >> 16)));
        v[j] = pack_h2(y0, y1);
    }
    return v;
}
