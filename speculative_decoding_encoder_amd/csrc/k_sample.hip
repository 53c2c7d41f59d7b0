// Temperature rejection sampling for one verification round
// (Whisper-Flash section 3.1 and appendix A.4).
//
// Candidate i (drawn by the drafter from q_i) is accepted when
// u * q_i(y) < p_i(y), u uniform on [0, 1) — the same as accepting with
// probability min(1, p_i(y) / q_i(y)). p_i = softmax(z_i / T) in fp32 with
// suppressed ids at probability 0. A rejection at candidate i draws the next
// token from (p_i - q_i)+ renormalised; when no candidate is rejected the
// extra token comes from p of the row after the last candidate. Draws use the inverse
// CDF in ascending id order. An accepted EOS ends the request with no bonus;
// the output budget works as in greedy decoding.
//
// Uniforms come from Philox4x64-10 (Salmon et al., SC'11) with key
// (seed, 0) and counter (request, step, position, stream): the top 24 bits
// of the first output word times 2^-24, exact in fp32.
//
// The row statistics (max, sum of exp) of every row come first, one
// 1024-thread workgroup per row; then one 1024-thread workgroup per request
// walks the candidate rows in order. Row statistics and the residual's
// segment sums are block reductions in a fixed order.
#include "wf_device.h"
#include "wf_internal.h"
#include "../../include/wf.h"

namespace wf {

namespace {

constexpr int NT = 1024;
constexpr uint64_t PM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t PM1 = 0xCA5A826395121157ull;
constexpr uint64_t PW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t PW1 = 0xBB67AE8584CAA73Bull;
constexpr int STREAM_ACCEPT = 0;
constexpr int STREAM_RESAMPLE = 1;

__device__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                 uint64_t k0, uint64_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += PW0;
            k1 += PW1;
        }
        const uint64_t hi0 = __umul64hi(PM0, c0), lo0 = PM0 * c0;
        const uint64_t hi1 = __umul64hi(PM1, c2), lo1 = PM1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return c0;
}

__device__ float uniform24(uint64_t seed, int req, int step, int pos, int stream) {
    const uint64_t w = philox_word0((uint64_t)(uint32_t)req, (uint64_t)(uint32_t)step,
                                    (uint64_t)(uint32_t)pos, (uint64_t)stream, seed, 0);
    return (float)(w >> 40) * 5.9604644775390625e-08f;   // 2^-24
}

// Block reductions over NT threads (fixed order: waves, then wave 0 over
// the per-wave results).
__device__ float block_max(float v, float *sh) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    if (threadIdx.x < 64) {
        float x = threadIdx.x < NT / 64 ? sh[threadIdx.x] : -INFINITY;
        x = wave_max(x);
        if (threadIdx.x == 0) sh[NT / 64] = x;
    }
    __syncthreads();
    const float r = sh[NT / 64];
    __syncthreads();
    return r;
}
__device__ float block_sum(float v, float *sh) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    if (threadIdx.x < 64) {
        float x = threadIdx.x < NT / 64 ? sh[threadIdx.x] : 0.f;
        x = wave_sum(x);
        if (threadIdx.x == 0) sh[NT / 64] = x;
    }
    __syncthreads();
    const float r = sh[NT / 64];
    __syncthreads();
    return r;
}

struct RowStats {
    float m, s;   // max of z over unsuppressed ids, sum of exp(z - m)
};

__device__ __forceinline__ float zval(const float *row, int v, float T, const uint8_t *sup) {
    if (sup && sup[v]) return -INFINITY;
    return row[v] / T;
}
__device__ __forceinline__ float zof(float x, bool suppressed, float T) {
    return suppressed ? -INFINITY : x / T;
}

// Walk thread t's elements v = t, t + NT, t + 2 NT, ... of a row in
// ascending order, calling f(v, z) with z = zval of element v (and qv, the
// draft probability, when qrow is given). The loads of a run of U elements
// go out together before any is used, so the walk waits for memory once per
// run instead of once per element; the arithmetic order is unchanged.
constexpr int kRun = 16;
template <typename F>
__device__ __forceinline__ void walk_strided(const float *row, const float *qrow, int V, float T,
                                             const uint8_t *sup, F f) {
    for (int v0 = threadIdx.x; v0 < V; v0 += NT * kRun) {
        float x[kRun], q[kRun];
        bool sp[kRun];
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int v = min(v0 + NT * u, V - 1);
            x[u] = row[v];
            q[u] = qrow ? qrow[v] : 0.f;
            sp[u] = sup ? sup[v] != 0 : false;
        }
#pragma unroll
        for (int u = 0; u < kRun; ++u)
            if (v0 + NT * u < V) f(v0 + NT * u, zof(x[u], sp[u], T), q[u]);
    }
}
// The same over a contiguous range [v0, v1), ascending.
template <typename F>
__device__ __forceinline__ void walk_range(const float *row, const float *qrow, int v0, int v1,
                                           float T, const uint8_t *sup, F f) {
    for (int b = v0; b < v1; b += kRun) {
        float x[kRun], q[kRun];
        bool sp[kRun];
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int v = min(b + u, v1 - 1);
            x[u] = row[v];
            q[u] = qrow ? qrow[v] : 0.f;
            sp[u] = sup ? sup[v] != 0 : false;
        }
#pragma unroll
        for (int u = 0; u < kRun; ++u)
            if (b + u < v1) f(b + u, zof(x[u], sp[u], T), q[u]);
    }
}

__device__ RowStats row_stats(const float *row, int V, float T, const uint8_t *sup, float *sh) {
    float m = -INFINITY;
    walk_strided(row, nullptr, V, T, sup, [&](int, float z, float) { m = fmaxf(m, z); });
    m = block_max(m, sh);
    float s = 0.f;
    walk_strided(row, nullptr, V, T, sup,
                 [&](int, float z, float) { s += (z == -INFINITY) ? 0.f : expf(z - m); });
    s = block_sum(s, sh);
    return RowStats{m, s};
}

__device__ __forceinline__ float prob_z(float z, const RowStats &st) {
    return (z == -INFINITY) ? 0.f : expf(z - st.m) / st.s;
}
__device__ __forceinline__ float prob(const float *row, int v, float T, const uint8_t *sup,
                                      const RowStats &st) {
    return prob_z(zval(row, v, T, sup), st);
}

// Inverse CDF in ascending id order over weights w_v (p_v, or (p_v - q_v)+):
// the smallest v with cumsum_v > u * total. Each thread owns a contiguous
// segment; segment sums are scanned in order through LDS.
template <bool RESID>
__device__ int icdf(const float *row, const float *qrow, int V, float T, const uint8_t *sup,
                    const RowStats &st, float u, float *sh, float *seg, int *found) {
    const int seglen = (V + NT - 1) / NT;
    const int v0 = threadIdx.x * seglen;
    const int v1 = min(v0 + seglen, V);
    auto weight_z = [&](float z, float qv) -> float {
        const float p = prob_z(z, st);
        if constexpr (RESID) return fmaxf(p - qv, 0.f);
        return p;
    };
    auto weight = [&](int v) -> float {
        return weight_z(zval(row, v, T, sup), RESID ? qrow[v] : 0.f);
    };
    const float *qr = RESID ? qrow : nullptr;
    float local = 0.f;
    walk_range(row, qr, v0, v1, T, sup, [&](int, float z, float qv) { local += weight_z(z, qv); });
    seg[threadIdx.x] = local;
    if (threadIdx.x == 0) *found = 0x7fffffff;
    __syncthreads();
    if (threadIdx.x == 0) {               // exclusive prefix over segments, in order
        float acc = 0.f;
        for (int t = 0; t < NT; ++t) {
            const float x = seg[t];
            seg[t] = acc;
            acc += x;
        }
        sh[NT / 64 + 1] = acc;
    }
    __syncthreads();
    const float total = sh[NT / 64 + 1];
    const float thr = u * total;
    float c = seg[threadIdx.x];
    if (c <= thr && v0 < v1) {
        bool hit = false;
        walk_range(row, qr, v0, v1, T, sup, [&](int v, float z, float qv) {
            if (hit) return;
            c += weight_z(z, qv);
            if (c > thr) {
                atomicMin(found, v);
                hit = true;
            }
        });
    }
    __syncthreads();
    int r = *found;
    __syncthreads();
    if (r == 0x7fffffff) {                // rounding put thr at or past the end
        int last = -1;
        for (int v = threadIdx.x; v < V; v += NT)
            if (weight(v) > 0.f) last = max(last, v);
        if (threadIdx.x == 0) *found = -1;
        __syncthreads();
        atomicMax(found, last);
        __syncthreads();
        r = *found;
        __syncthreads();
    }
    return r;
}

}  // namespace

// The softmax statistics (max, sum of exp) of every row a round may read
// (rows 0 .. n_tok - 1 of each request), one workgroup per row, all rows at
// once: the acceptance kernel then walks its candidates without reducing a
// row. Same reduction code, so the same bits.
__global__ __launch_bounds__(1024) void sample_row_stats_kernel(AcceptArgs a) {
    __shared__ float sh[NT / 64 + 2];
    const int b = blockIdx.x / a.T, i = blockIdx.x - b * a.T;
    if (i >= a.n_tok[b]) return;
    const float *row = a.logits + ((size_t)b * a.T + i) * a.V;
    const RowStats st = row_stats(row, a.V, a.temperature, a.suppress, sh);
    if (threadIdx.x == 0) {
        a.stats[2 * ((size_t)b * a.T + i)] = st.m;
        a.stats[2 * ((size_t)b * a.T + i) + 1] = st.s;
    }
}

__global__ __launch_bounds__(1024) void accept_sample_kernel(AcceptArgs a) {
    __shared__ float sh[NT / 64 + 2];
    __shared__ float seg[NT];
    __shared__ int found;
    const int b = blockIdx.x;
    const int nt = a.n_tok[b];
    int n_acc = 0, next = -1, n_emit = 0, done = 0;
    if (nt > 0) {
        const int k = nt - 1;
        const int R = a.budget[b];
        const int32_t *tok = a.tokens + (size_t)b * a.T;
        bool ok = !(R < 1 || k > R - 1 || nt > a.T);
        for (int i = 1; ok && i <= k; ++i)
            if (tok[i] < 0 || tok[i] >= a.V) ok = false;
        if (!ok) {
            n_acc = -1;
            done = 1;
        } else {
            const int req = a.request_id[b], step = a.step[b];
            const float T = a.temperature;
            int acc = 0;
            bool stopped = false;
            for (int i = 0; i < k && !stopped; ++i) {
                const float *row = a.logits + ((size_t)b * a.T + i) * a.V;
                const float *qrow = a.q + ((size_t)b * (a.T - 1) + i) * a.V;
                const RowStats st = a.stats ? RowStats{a.stats[2 * ((size_t)b * a.T + i)],
                                                       a.stats[2 * ((size_t)b * a.T + i) + 1]}
                                            : row_stats(row, a.V, T, a.suppress, sh);
                const int y = tok[i + 1];
                const float py = prob(row, y, T, a.suppress, st);
                const float qy = qrow[y];
                const float u = uniform24(a.seed, req, step, i, STREAM_ACCEPT);
                if (u * qy < py) {
                    acc = i + 1;
                    if (y == a.eos) {          // accepted EOS: finished, no bonus
                        n_emit = acc;
                        done = 1;
                        stopped = true;
                    }
                    continue;
                }
                // first rejection: draw from (p - q)+, or p when that is all zero
                const float ur = uniform24(a.seed, req, step, i, STREAM_RESAMPLE);
                float rs = 0.f;
                walk_strided(row, qrow, a.V, T, a.suppress,
                             [&](int, float z, float qv) { rs += fmaxf(prob_z(z, st) - qv, 0.f); });
                rs = block_sum(rs, sh);
                const int c = rs > 0.f
                    ? icdf<true>(row, qrow, a.V, T, a.suppress, st, ur, sh, seg, &found)
                    : icdf<false>(row, qrow, a.V, T, a.suppress, st, ur, sh, seg, &found);
                next = c;
                n_emit = acc + 1;
                done = (c == a.eos) || (acc + 1 >= R) || c < 0;
                stopped = true;
            }
            if (!stopped) {                    // every candidate accepted: bonus from row k
                const float *row = a.logits + ((size_t)b * a.T + k) * a.V;
                const RowStats st = a.stats ? RowStats{a.stats[2 * ((size_t)b * a.T + k)],
                                                       a.stats[2 * ((size_t)b * a.T + k) + 1]}
                                            : row_stats(row, a.V, T, a.suppress, sh);
                const float ub = uniform24(a.seed, req, step, k, STREAM_RESAMPLE);
                const int c = icdf<false>(row, nullptr, a.V, T, a.suppress, st, ub, sh, seg, &found);
                next = c;
                n_emit = acc + 1;
                done = (c == a.eos) || (acc + 1 >= R) || c < 0;
            }
            n_acc = acc;
        }
    }
    if (threadIdx.x == 0) {
        a.n_acc[b] = n_acc;
        a.next_token[b] = next;
        a.n_emit[b] = n_emit;
        a.done[b] = done;
    }
}

// With the row statistics in scratch the round is split so that the row a
// request draws from is spread over many workgroups:
//  1. decide (one thread per request): the candidate walk with the
//     statistics; writes the outputs of requests that end without a draw
//     (refused, accepted EOS) and, for the others, the accepted count, the
//     row to draw from (the first rejected candidate's, or row k for the
//     bonus) and the uniform;
//  2. segment sums (one workgroup per request and segment of the row): the
//     residual's and p's mass of each of kSeg segments, each thread summing
//     a contiguous run in id order, then a block reduction;
//  3. draw (one workgroup per drawing request): the residual when its total
//     mass is positive (a rejection), else p; the crossing segment by a
//     sequential prefix over the segment sums, then the crossing id inside
//     it by a sequential prefix over the threads' runs and the run's walk.
//     If rounding leaves the threshold past the mass: the last id with
//     positive weight.
// Scratch after the statistics: per request (acc, row, kind, uniform), then
// per request and segment (residual sum, p sum).
constexpr int kSeg = 64;
constexpr int kSegThreads = 256;

struct DrawScratch {
    int32_t *acc, *row;
    float *u;
    float *seg;                 // [n][kSeg][2]
};
__device__ __forceinline__ DrawScratch draw_scratch(const AcceptArgs &a) {
    float *base = a.stats + 2 * (size_t)a.n * a.T;
    DrawScratch d;
    d.acc = reinterpret_cast<int32_t *>(base);
    d.row = d.acc + a.n;
    d.u = reinterpret_cast<float *>(d.row + a.n);
    d.seg = d.u + a.n;
    return d;
}

__global__ void sample_decide_kernel(AcceptArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.n) return;
    const DrawScratch d = draw_scratch(a);
    d.row[b] = -1;
    const int nt = a.n_tok[b];
    int n_acc = 0, n_emit = 0, done = 0;
    if (nt > 0) {
        const int k = nt - 1;
        const int R = a.budget[b];
        const int32_t *tok = a.tokens + (size_t)b * a.T;
        bool ok = !(R < 1 || k > R - 1 || nt > a.T);
        for (int i = 1; ok && i <= k; ++i)
            if (tok[i] < 0 || tok[i] >= a.V) ok = false;
        if (!ok) {
            n_acc = -1;
            done = 1;
        } else {
            const int req = a.request_id[b], step = a.step[b];
            const float T = a.temperature;
            int acc = 0;
            bool stopped = false;
            for (int i = 0; i < k && !stopped; ++i) {
                const float *row = a.logits + ((size_t)b * a.T + i) * a.V;
                const float *qrow = a.q + ((size_t)b * (a.T - 1) + i) * a.V;
                const RowStats st{a.stats[2 * ((size_t)b * a.T + i)],
                                  a.stats[2 * ((size_t)b * a.T + i) + 1]};
                const int y = tok[i + 1];
                const float py = prob(row, y, T, a.suppress, st);
                const float qy = qrow[y];
                const float u = uniform24(a.seed, req, step, i, STREAM_ACCEPT);
                if (u * qy < py) {
                    acc = i + 1;
                    if (y == a.eos) {          // accepted EOS: finished, no bonus
                        n_emit = acc;
                        done = 1;
                        stopped = true;
                    }
                    continue;
                }
                d.row[b] = i;                  // first rejection: draw from row i
                d.u[b] = uniform24(a.seed, req, step, i, STREAM_RESAMPLE);
                stopped = true;
            }
            if (!stopped) {                    // every candidate accepted: bonus from row k
                d.row[b] = k;
                d.u[b] = uniform24(a.seed, req, step, k, STREAM_RESAMPLE);
            }
            d.acc[b] = acc;
            n_acc = acc;
        }
    }
    if (d.row[b] < 0) {
        a.n_acc[b] = n_acc;
        a.next_token[b] = -1;
        a.n_emit[b] = n_emit;
        a.done[b] = done;
    }
}

__device__ __forceinline__ float block_sum_t(float v, float *sh) {   // kSegThreads threads
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kSegThreads / 64; ++i) t += sh[i];
    __syncthreads();
    return t;
}

// The ids of thread t of segment g: [v0, v1).
__device__ __forceinline__ void seg_run(int V, int g, int t, int &v0, int &v1) {
    const int sl = (V + kSeg - 1) / kSeg;
    const int lo = g * sl, hi = min(lo + sl, V);
    const int rl = (sl + kSegThreads - 1) / kSegThreads;
    v0 = min(lo + t * rl, hi);
    v1 = min(v0 + rl, hi);
}

__global__ __launch_bounds__(kSegThreads) void sample_segsum_kernel(AcceptArgs a) {
    __shared__ float sh[kSegThreads / 64];
    const int b = blockIdx.x / kSeg, g = blockIdx.x - b * kSeg;
    const DrawScratch d = draw_scratch(a);
    const int r = d.row[b];
    if (r < 0) return;
    const int k = a.n_tok[b] - 1;
    const bool resid = r < k;                  // a rejection: the residual; the bonus: p
    const float *row = a.logits + ((size_t)b * a.T + r) * a.V;
    const float *qrow = resid ? a.q + ((size_t)b * (a.T - 1) + r) * a.V : nullptr;
    const RowStats st{a.stats[2 * ((size_t)b * a.T + r)], a.stats[2 * ((size_t)b * a.T + r) + 1]};
    int v0, v1;
    seg_run(a.V, g, threadIdx.x, v0, v1);
    float sr = 0.f, sp = 0.f;
    walk_range(row, qrow, v0, v1, a.temperature, a.suppress, [&](int, float z, float qv) {
        const float p = prob_z(z, st);
        sp += p;
        sr += fmaxf(p - qv, 0.f);
    });
    sr = block_sum_t(sr, sh);
    sp = block_sum_t(sp, sh);
    if (threadIdx.x == 0) {
        d.seg[((size_t)b * kSeg + g) * 2] = resid ? sr : 0.f;
        d.seg[((size_t)b * kSeg + g) * 2 + 1] = sp;
    }
}

__global__ __launch_bounds__(kSegThreads) void sample_draw_kernel(AcceptArgs a) {
    __shared__ float run[kSegThreads];
    __shared__ int sel_g, sel_t, found;
    __shared__ float sel_base, sel_thr;
    __shared__ int use_resid;
    const int b = blockIdx.x;
    const DrawScratch d = draw_scratch(a);
    const int r = d.row[b];
    if (r < 0) return;
    const int k = a.n_tok[b] - 1;
    const float *row = a.logits + ((size_t)b * a.T + r) * a.V;
    const float *qrow = r < k ? a.q + ((size_t)b * (a.T - 1) + r) * a.V : nullptr;
    const RowStats st{a.stats[2 * ((size_t)b * a.T + r)], a.stats[2 * ((size_t)b * a.T + r) + 1]};
    const float *sg = d.seg + (size_t)b * kSeg * 2;
    if (threadIdx.x == 0) {
        float rs = 0.f, ps = 0.f;
        for (int g = 0; g < kSeg; ++g) {
            rs += sg[2 * g];
            ps += sg[2 * g + 1];
        }
        const int ur = r < k && rs > 0.f;
        const float total = ur ? rs : ps;
        const float thr = d.u[b] * total;
        float acc = 0.f;
        int gsel = -1;
        for (int g = 0; g < kSeg; ++g) {
            const float x = sg[2 * g + (ur ? 0 : 1)];
            if (acc + x > thr && x > 0.f) {
                gsel = g;
                break;
            }
            acc += x;
        }
        use_resid = ur;
        sel_g = gsel;
        sel_base = acc;
        sel_thr = thr;
        found = 0x7fffffff;
    }
    __syncthreads();
    const bool ur = use_resid != 0;
    auto weight = [&](float z, float qv) {
        const float p = prob_z(z, st);
        return ur ? fmaxf(p - qv, 0.f) : p;
    };
    const int g = sel_g;
    if (g >= 0) {
        int v0, v1;
        seg_run(a.V, g, threadIdx.x, v0, v1);
        float s = 0.f;
        walk_range(row, ur ? qrow : nullptr, v0, v1, a.temperature, a.suppress,
                   [&](int, float z, float qv) { s += weight(z, qv); });
        run[threadIdx.x] = s;
        __syncthreads();
        if (threadIdx.x == 0) {                 // the crossing run, in id order
            float acc = sel_base;
            int t = 0;
            for (; t < kSegThreads; ++t) {
                if (acc + run[t] > sel_thr && run[t] > 0.f) break;
                acc += run[t];
            }
            sel_t = t;
            sel_base = acc;
        }
        __syncthreads();
        if (threadIdx.x == sel_t) {
            // the crossing id; if rounding keeps the walk under the threshold,
            // the run's last id with positive weight
            float c = sel_base;
            int hit = -1, last = -1;
            walk_range(row, ur ? qrow : nullptr, v0, v1, a.temperature, a.suppress,
                       [&](int v, float z, float qv) {
                           if (hit >= 0) return;
                           const float w = weight(z, qv);
                           c += w;
                           if (w > 0.f) last = v;
                           if (c > sel_thr) hit = v;
                       });
            found = hit >= 0 ? hit : last;
        }
        __syncthreads();
        if (sel_t == kSegThreads) {
            // no run crossed (rounding): the segment's last id with positive weight
            int last = -1;
            walk_range(row, ur ? qrow : nullptr, v0, v1, a.temperature, a.suppress,
                       [&](int v, float z, float qv) {
                           if (weight(z, qv) > 0.f) last = v;
                       });
            if (threadIdx.x == 0) found = -1;
            __syncthreads();
            atomicMax(&found, last);
            __syncthreads();
            if (found < 0 && threadIdx.x == 0) found = 0x7fffffff;
            __syncthreads();
        }
    }
    if (found == 0x7fffffff) {
        // rounding put the threshold at or past the mass: the last id with
        // positive weight (-1 when there is none)
        int last = -1;
        for (int v = threadIdx.x; v < a.V; v += kSegThreads) {
            const float w = weight(zval(row, v, a.temperature, a.suppress), ur ? qrow[v] : 0.f);
            if (w > 0.f) last = max(last, v);
        }
        __syncthreads();
        if (threadIdx.x == 0) found = -1;
        __syncthreads();
        atomicMax(&found, last);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const int c = found;
        const int acc = d.acc[b];
        const int R = a.budget[b];
        a.n_acc[b] = acc;
        a.next_token[b] = c;
        a.n_emit[b] = acc + 1;
        a.done[b] = (c == a.eos) || (acc + 1 >= R) || c < 0;
    }
}

size_t sample_scratch_floats(int n, int T) {
    return 2 * (size_t)n * T + 3 * (size_t)n + (size_t)n * kSeg * 2;
}

hipError_t launch_accept_sample(const AcceptArgs &a, hipStream_t st) {
    if (!a.stats) {
        hipLaunchKernelGGL(accept_sample_kernel, dim3(a.n), dim3(NT), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(sample_row_stats_kernel, dim3(a.n * a.T), dim3(NT), 0, st, a);
    hipLaunchKernelGGL(sample_decide_kernel, dim3((a.n + 63) / 64), dim3(64), 0, st, a);
    hipLaunchKernelGGL(sample_segsum_kernel, dim3(a.n * kSeg), dim3(kSegThreads), 0, st, a);
    hipLaunchKernelGGL(sample_draw_kernel, dim3(a.n), dim3(kSegThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace wf
