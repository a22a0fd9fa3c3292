// Stochastic verification of a verify pass by modified rejection sampling (gfx950).
//
// [Serving Efficiency] section 31.5 (Example 31.3), [Spending the Idle] section
// 12.4, [Serving] "Lossless": draft d_j, drawn from the draft distribution q_j,
// is kept with probability min(1, p(d_j) / q_j(d_j)) under the target
// distribution p at its position; at the first rejection a replacement is drawn
// from norm(max(0, p - q_j)) and verification stops; when every draft is kept,
// one more token is drawn from the target distribution after the last draft
// ([KV Cache] section 08: a pass always adds at least one token).
//
// Two kernels, both HBM-bound row streams in fp32:
//   softmax_stats_kernel: one 1024-thread workgroup per target row (the B
//     previous-pass rows, then the M rows of this pass) reduces the row's
//     maximum and sum of exp(z/T - max) with an online rescale, coalesced.
//   sample_pick_kernel: one 1024-thread workgroup per sequence. All accept tests
//     run at once, one thread per draft, and the first rejection is an LDS
//     minimum. The one inverse-CDF draw gives each thread a contiguous chunk of
//     the vocabulary; chunk sums are grouped 16 to a lane and prefixed across
//     wave 0 in lane order, and the crossing chunk is walked by a lane scan.
//     Every order is fixed, so the draw does not depend on timing. Where fp32
//     rounding leaves the cumulative sum short of the target at the end of a
//     span that must hold the draw, the span's last token of positive weight
//     is taken.
#pragma once

#include "common.h"

namespace vs {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kSampleGroup = kSampleThreads / kWave;  // chunks summed by one lane of wave 0

// p(x) = exp(z(x)/T - max) / sum. Both kernels that need a probability call this
// one function with contraction off, so a weight computed twice is the same float.
__device__ __forceinline__ float target_prob(float zx, float inv_t, float m, float s) {
#pragma clang fp contract(off)
    return expf(zx * inv_t - m) / s;
}

// Online softmax accumulation: (m, s) <- max and rescaled sum after one more y.
__device__ __forceinline__ void os_add(float& m, float& s, float y) {
    if (y > m) {
        s = s * expf(m - y) + 1.f;
        m = y;
    } else if (y > -INFINITY) {
        s += expf(y - m);
    }
}

__device__ __forceinline__ void os_merge(float& m, float& s, float m2, float s2) {
    const float mm = fmaxf(m, m2);
    if (mm == -INFINITY) return;
    s = s * expf(m - mm) + s2 * expf(m2 - mm);
    m = mm;
}

struct StatsArgs {
    const float* p0;      // [B][V]
    const float* logits;  // [M][V]
    int B, V;
    float inv_t;
    float2* stats;  // [B + M]
};

// stats[g] = (max_x z_g(x)/T, sum_x exp(z_g(x)/T - max)), g < B: p0 row g; else logits row g - B.
__global__ void __launch_bounds__(kSampleThreads) softmax_stats_kernel(StatsArgs a) {
    const int g = blockIdx.x, tid = threadIdx.x, V = a.V;
    const float inv_t = a.inv_t;
    const float* z = g < a.B ? a.p0 + (long)g * V : a.logits + (long)(g - a.B) * V;
    constexpr int U = 8;
    float m = -INFINITY, s = 0.f;
    for (int x0 = 0; x0 < V; x0 += U * kSampleThreads) {
        float y[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int x = x0 + k * kSampleThreads + tid;
            y[k] = x < V ? __builtin_nontemporal_load(z + x) * inv_t : -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) os_add(m, s, y[k]);
    }
    for (int mask = kWave / 2; mask >= 1; mask >>= 1) os_merge(m, s, shfl_xor(m, mask), shfl_xor(s, mask));
    __shared__ float2 part[kSampleWaves];
    if ((tid & (kWave - 1)) == 0) part[tid / kWave] = make_float2(m, s);
    __syncthreads();
    if (tid == 0) {
        float mm = part[0].x, ss = part[0].y;
        for (int w = 1; w < kSampleWaves; ++w) os_merge(mm, ss, part[w].x, part[w].y);
        a.stats[g] = make_float2(mm, ss);
    }
}

struct SampleArgs {
    int B, M, V;
    const int* q_start;
    const int* drafts;
    const float* p0;      // [B][V]
    const float* logits;  // [M][V]
    const float* q;       // [M][V]
    const float* u;       // [M]
    const float* v;       // [B]
    const float2* stats;  // [B + M]
    float inv_t;
    int* accept_len;
    int* token;
};

// wave-inclusive prefix sum in lane order (Hillis-Steele; fixed order)
__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
    for (int off = 1; off < kWave; off <<= 1) {
        const float t = __shfl_up(x, off, kWave);
        if (lane >= off) x += t;
    }
    return x;
}

__global__ void __launch_bounds__(kSampleThreads) sample_pick_kernel(SampleArgs a) {
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
    const int V = a.V;
    const int r0 = min(max(a.q_start[b], 0), a.M);
    const int r1 = min(max(a.q_start[b + 1], r0), a.M);
    const int K = r1 - r0;
    __shared__ int s_reject;  // index j of the first rejected draft (draft j+1), K if none
    __shared__ float s_cs[kSampleThreads];
    __shared__ int s_chunk, s_x;
    __shared__ float s_c, s_target;
    __shared__ int s_residual;

    auto row_z = [&](int j) { return j == 0 ? a.p0 + (long)b * V : a.logits + (long)(r0 + j - 1) * V; };
    auto row_st = [&](int j) { return j == 0 ? a.stats[b] : a.stats[a.B + r0 + j - 1]; };

    if (tid == 0) {
        s_reject = K;
        s_residual = 1;
    }
    __syncthreads();
    // ---- every accept test at once: draft j+1 against p_j ----
    for (int j = tid; j < K; j += kSampleThreads) {
        const int d = a.drafts[r0 + j];
        bool keep = false;
        if (d >= 0 && d < V) {
            const float2 st = row_st(j);
            const float p = target_prob(row_z(j)[d], a.inv_t, st.x, st.y);
            const float q = a.q[(long)(r0 + j) * V + d];
            keep = q > 0.f && a.u[r0 + j] < fminf(1.f, p / q);
        }
        if (!keep) atomicMin(&s_reject, j);
    }
    __syncthreads();
    const int n = s_reject;
    // ---- the one draw: from norm(max(0, p_n - q_{n+1})) after a rejection, else from p_K ----
    const float* z = row_z(n);
    const float2 st = row_st(n);
    const float* q = n < K ? a.q + (long)(r0 + n) * V : nullptr;
    const int C = (V + kSampleThreads - 1) / kSampleThreads;
    const int x0 = min(tid * C, V), x1 = min(x0 + C, V);
    auto weight = [&](int x, bool residual) {
        const float p = target_prob(z[x], a.inv_t, st.x, st.y);
        return residual ? fmaxf(0.f, p - q[x]) : p;
    };
    for (int pass = 0; pass < 2; ++pass) {
        const bool residual = q != nullptr && s_residual;
        float cs = 0.f;
        for (int x = x0; x < x1; ++x) cs += weight(x, residual);
        s_cs[tid] = cs;
        __syncthreads();
        if (tid < kWave) {
            float gs = 0.f;
            for (int i = 0; i < kSampleGroup; ++i) gs += s_cs[lane * kSampleGroup + i];
            const float incl = wave_incl_scan(gs, lane);
            const float total = __shfl(incl, kWave - 1, kWave);
            if (residual && !(total > 0.f)) {  // p == q: nothing to correct; draw from p itself
                if (lane == 0) s_residual = 0;
            } else {
                const float target = a.v[b] * total;
                const unsigned long long hit = __ballot(incl > target);
                const unsigned long long pos = __ballot(gs > 0.f);
                // the lane holding the draw; short by rounding: the last lane with weight
                const int l = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
                const float excl = __shfl_up(incl, 1, kWave);
                if (lane == l) {
                    float c = lane == 0 ? 0.f : excl;
                    int t = -1, last = -1;
                    for (int i = 0; i < kSampleGroup; ++i) {
                        const int ci = l * kSampleGroup + i;
                        if (s_cs[ci] > 0.f) last = ci;
                        if (hit && c + s_cs[ci] > target) {
                            t = ci;
                            break;
                        }
                        c += s_cs[ci];
                    }
                    if (t < 0) {  // no crossing inside the group: its last chunk with weight
                        t = last < 0 ? l * kSampleGroup : last;
                        c = -INFINITY;  // and that chunk's last token with weight
                    }
                    s_chunk = t;
                    s_c = c;
                    s_target = target;
                }
            }
        }
        __syncthreads();
        if (s_residual == (int)residual || q == nullptr) break;
    }
    // ---- walk the chunk holding the draw in 64-token pieces (wave 0) ----
    if (tid < kWave) {
        const bool residual = q != nullptr && s_residual;
        const int t = s_chunk;
        const float target = s_target;
        const bool find_last = s_c == -INFINITY;
        float c = find_last ? 0.f : s_c;
        const int lo = min(t * C, V), hi = min(lo + C, V);
        int x = -1, last = -1;
        for (int base = lo; base < hi && x < 0; base += kWave) {
            const int y = base + lane;
            const float w = y < hi ? weight(y, residual) : 0.f;
            const float incl = c + wave_incl_scan(w, lane);
            const unsigned long long pos = __ballot(w > 0.f);
            if (pos) last = base + 63 - __clzll((long long)pos);
            const unsigned long long hit = find_last ? 0ull : __ballot(incl > target && y < hi);
            if (hit) x = base + __ffsll((long long)hit) - 1;
            c = __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) s_x = x >= 0 ? x : (last >= 0 ? last : lo);
    }
    __syncthreads();
    if (tid == 0) {
        a.accept_len[b] = n;
        a.token[b] = s_x;
    }
}

}  // namespace vs
