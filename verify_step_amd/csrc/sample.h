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
//   softmax_stats_kernel: grid (rows, segments). Each 256-thread workgroup
//     reduces the maximum and the sum of exp(z/T - max) of one 2048-token
//     segment of one target row (the B previous-pass rows, then the M rows of
//     this pass) with an online rescale, from coalesced 16-byte loads. The
//     segment partials are merged in segment order where they are used.
//   sample_pick_kernel: one 1024-thread workgroup per sequence. The accept tests
//     run at once, one wave per draft (its lanes merge the row's segment
//     partials); the first rejection is an LDS minimum.
//     The one inverse-CDF draw splits the vocabulary into chunks of CS tokens,
//     tiles of 64 chunks per wave-load; chunk sums go to LDS, are summed G at a
//     time per thread and 16 at a time per lane of wave 0, and prefixed across
//     that wave in lane order; the draw then descends lane -> group -> chunk ->
//     token. Every order is fixed, so the draw does not depend on timing. Where
//     fp32 rounding leaves the running sum short of the target at the end of a
//     span that must hold the draw, the span's last entry of positive weight is
//     taken.
#pragma once

#include "common.h"

namespace vs {

constexpr int kStatsThreads = 256;
constexpr int kStatsSeg = 2048;  // tokens per statistics workgroup (8 per thread)
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kSampleMaxChunks = 8192;  // LDS chunk sums of one draw
constexpr int kLaneGroups = kSampleThreads / kWave;  // thread groups summed by one lane of wave 0
constexpr int kStatSlots = 64;  // target rows of one sequence whose merged statistics stay in LDS

__host__ __device__ constexpr int stats_segments(int V) { return (V + kStatsSeg - 1) / kStatsSeg; }
// tokens per chunk: 16, or more for vocabularies beyond 16 * kSampleMaxChunks
__host__ __device__ constexpr int sample_chunk(int V) {
    const int k = (V + 16 * kSampleMaxChunks - 1) / (16 * kSampleMaxChunks);
    return 16 * (k > 1 ? k : 1);
}

// p(x) = exp(z(x)/T - max) / sum. Every probability is computed by this one function
// with contraction off, so a weight computed twice is the same float.
__device__ __forceinline__ float target_prob(float zx, float inv_t, float m, float s) {
#pragma clang fp contract(off)
    return expf(zx * inv_t - m) / s;
}

// Online softmax accumulation: (m, s) <- max and rescaled sum after one more y.
__device__ __forceinline__ void os_add(float& m, float& s, float y) {
#pragma clang fp contract(off)
    if (y > m) {
        s = s * expf(m - y) + 1.f;
        m = y;
    } else if (y > -INFINITY) {
        s += expf(y - m);
    }
}

__device__ __forceinline__ void os_merge(float& m, float& s, float m2, float s2) {
#pragma clang fp contract(off)
    const float mm = fmaxf(m, m2);
    if (mm == -INFINITY) return;
    s = s * expf(m - mm) + s2 * expf(m2 - mm);
    m = mm;
}

struct StatsArgs {
    const float* p0;      // [B][V]
    const float* logits;  // [M][V]
    int B, V, n_seg;
    float inv_t;
    float2* part;  // [B + M][n_seg]
};

// part[g][seg] = (max z_g/T, sum exp(z_g/T - max)) over segment seg; g < B: p0 row g; else logits row g - B.
template <bool VEC4>
__global__ void __launch_bounds__(kStatsThreads) softmax_stats_kernel(StatsArgs a) {
    const int g = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, V = a.V;
    const float inv_t = a.inv_t;
    const float* z = g < a.B ? a.p0 + (long)g * V : a.logits + (long)(g - a.B) * V;
    const int x0 = seg * kStatsSeg;
    float y[8];
    if constexpr (VEC4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int x = x0 + h * (kStatsSeg / 2) + 4 * tid;
            float4_t f = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (x < V) f = *reinterpret_cast<const float4_t*>(z + x);
            y[4 * h + 0] = f.x * inv_t;
            y[4 * h + 1] = f.y * inv_t;
            y[4 * h + 2] = f.z * inv_t;
            y[4 * h + 3] = f.w * inv_t;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int x = x0 + k * kStatsThreads + tid;
            y[k] = x < V ? z[x] * inv_t : -INFINITY;
        }
    }
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) os_add(m, s, y[k]);
    for (int mask = kWave / 2; mask >= 1; mask >>= 1) os_merge(m, s, shfl_xor(m, mask), shfl_xor(s, mask));
    __shared__ float2 wp[kStatsThreads / kWave];
    if ((tid & (kWave - 1)) == 0) wp[tid / kWave] = make_float2(m, s);
    __syncthreads();
    if (tid == 0) {
        float mm = wp[0].x, ss = wp[0].y;
        for (int w = 1; w < kStatsThreads / kWave; ++w) os_merge(mm, ss, wp[w].x, wp[w].y);
        a.part[(long)g * a.n_seg + seg] = make_float2(mm, ss);
    }
}

struct SampleArgs {
    int B, M, V, n_seg;
    const int* q_start;
    const int* drafts;
    const float* p0;      // [B][V]
    const float* logits;  // [M][V]
    const float* q;       // [M][V]
    const float* u;       // [M]
    const float* v;       // [B]
    const float2* part;   // [B + M][n_seg]
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

// One level of the descent: the first entry of a[lo, hi) at which the running sum c passes the
// target, or (find_last, also when rounding leaves the sum short) the last entry of positive weight.
__device__ __forceinline__ int descend(const float* a, int lo, int hi, float& c, float target, bool& find_last) {
    int last = -1;
    for (int i = lo; i < hi; ++i) {
        if (a[i] > 0.f) last = i;
        if (!find_last && c + a[i] > target) return i;
        c += a[i];
    }
    find_last = true;
    return last >= 0 ? last : lo;
}

template <bool VEC4>
__global__ void __launch_bounds__(kSampleThreads) sample_pick_kernel(SampleArgs a) {
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int V = a.V;
    const int r0 = min(max(a.q_start[b], 0), a.M);
    const int r1 = min(max(a.q_start[b + 1], r0), a.M);
    const int K = r1 - r0;
    __shared__ float s_cs[kSampleMaxChunks];  // chunk sums
    __shared__ float s_gs[kSampleThreads];    // sums of G chunks
    __shared__ int s_reject;                  // index j of the first rejected draft (draft j+1), K if none
    __shared__ int s_residual, s_lane, s_x;
    __shared__ float s_m[kStatSlots], s_s[kStatSlots], s_c, s_target;
    __shared__ int s_find_last;

    auto row_z = [&](int j) { return j == 0 ? a.p0 + (long)b * V : a.logits + (long)(r0 + j - 1) * V; };
    // merge of the row's segment partials by one wave: lane i takes partials i, i + 64, ... in order,
    // then a fixed butterfly; every lane returns lane 0's result
    auto row_stats = [&](int j, float& m, float& s) {
        const float2* pp = a.part + (long)(j == 0 ? b : a.B + r0 + j - 1) * a.n_seg;
        m = -INFINITY;
        s = 0.f;
        for (int i = lane; i < a.n_seg; i += kWave) {
            const float2 t = pp[i];
            os_merge(m, s, t.x, t.y);
        }
        for (int mask = kWave / 2; mask >= 1; mask >>= 1) os_merge(m, s, shfl_xor(m, mask), shfl_xor(s, mask));
        m = __shfl(m, 0, kWave);
        s = __shfl(s, 0, kWave);
    };

    if (tid == 0) {
        s_reject = K;
        s_residual = 1;
    }
    __syncthreads();
    // ---- the accept tests, one wave per draft: draft j+1 against p_j. Wave j also keeps p_j's
    // statistics (and p_K's, j = K) for the draw; rows past the LDS slots are merged again later ----
    for (int j = wave; j <= K; j += kSampleWaves) {
        const bool test = j < K;
        const int d = test ? a.drafts[r0 + j] : -1;
        const bool in_vocab = d >= 0 && d < V;
        const float zd = in_vocab ? row_z(j)[d] : 0.f;
        const float qd = in_vocab ? a.q[(long)(r0 + j) * V + d] : 0.f;
        const float uj = test ? a.u[r0 + j] : 0.f;
        float m, s;
        row_stats(j, m, s);
        if (lane == 0 && j < kStatSlots) {
            s_m[j] = m;
            s_s[j] = s;
        }
        const float p = target_prob(zd, a.inv_t, m, s);
        const bool keep = in_vocab && qd > 0.f && uj < fminf(1.f, p / qd);
        if (test && !keep && lane == 0) atomicMin(&s_reject, j);
    }
    __syncthreads();
    const int n = s_reject;
    if (n >= kStatSlots && tid < kWave) {
        float m, s;
        row_stats(n, m, s);
        if (lane == 0) {
            s_m[0] = m;
            s_s[0] = s;
        }
    }
    __syncthreads();
    const int slot = n < kStatSlots ? n : 0;
    // ---- the one draw: from norm(max(0, p_n - q_{n+1})) after a rejection, else from p_K ----
    const float* z = row_z(n);
    const float* q = n < K ? a.q + (long)(r0 + n) * V : nullptr;
    const float m = s_m[slot], s = s_s[slot], inv_t = a.inv_t;
    constexpr int CS_MAX = 16;  // chunk tokens held in registers per lane (vocabularies up to 131072)
    const int CS = sample_chunk(V);
    const int n_chunks = (V + CS - 1) / CS;
    const int G = (n_chunks + kSampleThreads - 1) / kSampleThreads;
    auto weight = [&](float zx, float qx, bool residual) {
        const float p = target_prob(zx, inv_t, m, s);
        return residual ? fmaxf(0.f, p - qx) : p;
    };
    for (int pass = 0; pass < 2; ++pass) {
        const bool residual = q != nullptr && s_residual;
        // chunk sums: lane l of wave w takes chunks w*64 + l + 1024 i, two at a time (16-byte loads of
        // 16 consecutive tokens per chunk: a wave reads 4 KB contiguous per row and per chunk index)
        for (int c = wave * kWave + lane; c < n_chunks; c += 2 * kSampleThreads) {
            if (VEC4 && CS == CS_MAX) {
                float4_t zz[2][CS_MAX / 4], qq[2][CS_MAX / 4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int x0 = (c + h * kSampleThreads) * CS;
#pragma unroll
                    for (int k = 0; k < CS_MAX / 4; ++k) {
                        const int x = x0 + 4 * k;
                        zz[h][k] = float4_t{0.f, 0.f, 0.f, 0.f};
                        qq[h][k] = zz[h][k];
                        if (x < V) {
                            zz[h][k] = *reinterpret_cast<const float4_t*>(z + x);
                            if (residual) qq[h][k] = *reinterpret_cast<const float4_t*>(q + x);
                        }
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ch = c + h * kSampleThreads, x0 = ch * CS;
                    float cs = 0.f;
#pragma unroll
                    for (int k = 0; k < CS_MAX / 4; ++k) {
                        if (x0 + 4 * k < V) {
                            cs += weight(zz[h][k].x, qq[h][k].x, residual);
                            cs += weight(zz[h][k].y, qq[h][k].y, residual);
                            cs += weight(zz[h][k].z, qq[h][k].z, residual);
                            cs += weight(zz[h][k].w, qq[h][k].w, residual);
                        }
                    }
                    if (ch < n_chunks) s_cs[ch] = cs;
                }
            } else {
                for (int h = 0; h < 2; ++h) {
                    const int ch = c + h * kSampleThreads;
                    if (ch >= n_chunks) break;
                    const int x0 = ch * CS, x1 = min(x0 + CS, V);
                    float cs = 0.f;
                    for (int x = x0; x < x1; ++x) cs += weight(z[x], residual ? q[x] : 0.f, residual);
                    s_cs[ch] = cs;
                }
            }
        }
        __syncthreads();
        {  // groups of G chunks
            float gs = 0.f;
            const int c0 = tid * G, c1 = min(c0 + G, n_chunks);
            for (int c = c0; c < c1; ++c) gs += s_cs[c];
            s_gs[tid] = gs;
        }
        __syncthreads();
        if (tid < kWave) {
            float ls = 0.f;
            for (int i = 0; i < kLaneGroups; ++i) ls += s_gs[lane * kLaneGroups + i];
            const float incl = wave_incl_scan(ls, lane);
            const float total = __shfl(incl, kWave - 1, kWave);
            if (residual && !(total > 0.f)) {  // p <= q everywhere: nothing to correct; draw from p itself
                if (lane == 0) s_residual = 0;
            } else {
                const float target = a.v[b] * total;
                const unsigned long long hit = __ballot(incl > target);
                const unsigned long long pos = __ballot(ls > 0.f);
                const int l = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
                const float excl = __shfl_up(incl, 1, kWave);
                if (lane == l) {
                    s_lane = l;
                    s_c = l == 0 ? 0.f : excl;
                    s_target = target;
                    s_find_last = hit ? 0 : 1;
                }
            }
        }
        __syncthreads();
        if (s_residual == (int)residual || q == nullptr) break;
    }
    // ---- descend: lane -> group -> chunk (one thread), then token (wave 0) ----
    if (tid == 0) {
        const int l = s_lane;
        float c = s_c;
        const float target = s_target;
        bool find_last = s_find_last;
        const int g = descend(s_gs, l * kLaneGroups, (l + 1) * kLaneGroups, c, target, find_last);
        const int ch = descend(s_cs, min(g * G, n_chunks), min(g * G + G, n_chunks), c, target, find_last);
        s_x = min(ch, n_chunks - 1);
        s_c = c;
        s_find_last = find_last;
    }
    __syncthreads();
    if (tid < kWave) {
        const bool residual = q != nullptr && s_residual;
        const int ch = s_x;
        const float target = s_target;
        const bool find_last = s_find_last;
        float c = s_c;
        const int lo = min(ch * CS, V), hi = min(lo + CS, V);
        int x = -1, last = -1;
        for (int base = lo; base < hi && x < 0; base += kWave) {
            const int y = base + lane;
            const float w = y < hi ? weight(z[y], residual ? q[y] : 0.f, residual) : 0.f;
            const float incl = c + wave_incl_scan(w, lane);
            const unsigned long long pos = __ballot(w > 0.f);
            if (pos) last = base + 63 - __clzll((long long)pos);
            const unsigned long long hit = find_last ? 0ull : __ballot(incl > target && y < hi);
            if (hit) x = base + __ffsll((long long)hit) - 1;
            c = __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) {
            a.accept_len[b] = n;
            a.token[b] = x >= 0 ? x : (last >= 0 ? last : min(lo, V - 1));
        }
    }
}

}  // namespace vs
