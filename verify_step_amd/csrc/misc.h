// Small kernels of the step: row bookkeeping + rotary angles + embedding
// gather, argmax reduction with fused greedy acceptance.
#pragma once

#include "common.h"
#include "gemm.h"

namespace vs {

struct PrepArgs {
    const int* q_start;
    const int* ctx_len;
    int B, M, head_dim;
    double theta;
    const int* tokens;
    const void* embed;
    int vocab, D;
    int* row_seq;
    int* row_pos;
    float* rope_cs;  // [M][head_dim/2][2]
    float* x;        // [M][D] fp32 residual stream
    // the row's K/V slot: page * page_elems + slot * head_dim (or -1 without a valid page)
    long* row_kvoff;
    const int* block_tables;
    int max_blocks, num_pages, page_tokens;
    long page_elems;
    int* error_flags;  // optional: validation bits (VS_STEP_BAD_*)
    int* seq_group;    // optional [B]: set to -1 (no shared-prefix group), and seq_gp to 0
    int* seq_gp;
    int* merge_count;  // optional: set to 0 (the rows the group check lists for the merge kernel)
};

// One workgroup (256 threads) per row r: its sequence and position, the rotary
// (cos, sin) of every pair from the float64 angle pos * theta^(-2i/head_dim),
// and the embedding row widened into the fp32 residual stream.
template <int DT>
__global__ void __launch_bounds__(256) prep_embed_kernel(PrepArgs p) {
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    __shared__ int s_pos, s_seq;
    if (tid == 0) {
        int lo = 0, hi = p.B;  // largest b with q_start[b] <= r
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.q_start[mid] <= r) lo = mid;
            else hi = mid;
        }
        const int pos = p.ctx_len[lo] + (r - p.q_start[lo]);
        p.row_seq[r] = lo;
        p.row_pos[r] = pos;
        s_pos = pos;
        s_seq = lo;
        long off = -1;
        if (pos >= 0 && pos / p.page_tokens < p.max_blocks) {
            const int page = p.block_tables[(long)lo * p.max_blocks + pos / p.page_tokens];
            if (page >= 0 && page < p.num_pages)
                off = (long)page * p.page_elems + (long)(pos % p.page_tokens) * p.head_dim;
        }
        p.row_kvoff[r] = off;
    }
    if (p.seq_group) {
        for (long b = (long)r * blockDim.x + tid; b < p.B; b += (long)gridDim.x * blockDim.x) {
            p.seq_group[b] = -1;
            p.seq_gp[b] = 0;
        }
        if (r == 0 && tid == 0) *p.merge_count = 0;
    }
    __syncthreads();
    const int pos = s_pos;
    if (p.error_flags) {
        // validation (the kernels clamp these values anyway): the row's token, its sequence's
        // batch entries, and every block-table entry of pages 0 .. pos / page_tokens, which the row's
        // attention reads and its K/V write uses
        int bad = 0;
        if (tid == 0) {
            int lo = 0, hi = p.B;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (p.q_start[mid] <= r) lo = mid;
                else hi = mid;
            }
            const int t = p.tokens[r];
            if (t < 0 || t >= p.vocab) bad |= 1;
            if (p.q_start[lo] > r || p.q_start[lo + 1] <= r || p.ctx_len[lo] < 0) bad |= 4;
        }
        if (pos >= 0) {
            const int npg = min(pos / p.page_tokens + 1, p.max_blocks);
            if (pos / p.page_tokens >= p.max_blocks) bad |= 2;
            const int* bt = p.block_tables + (long)s_seq * p.max_blocks;
            for (int i = tid; i < npg; i += blockDim.x)
                if (bt[i] < 0 || bt[i] >= p.num_pages) bad |= 2;
        }
        if (bad) atomicOr(p.error_flags, bad);
    }
    const int half = p.head_dim / 2;
    for (int i = tid; i < half; i += blockDim.x) {
        const double inv_freq = pow(p.theta, -2.0 * (double)i / (double)p.head_dim);
        const double ang = (double)pos * inv_freq;
        p.rope_cs[((long)r * half + i) * 2 + 0] = (float)cos(ang);
        p.rope_cs[((long)r * half + i) * 2 + 1] = (float)sin(ang);
    }
    int t = p.tokens[r];
    t = t < 0 ? 0 : (t >= p.vocab ? p.vocab - 1 : t);
    const long base = (long)t * p.D;
    for (int k0 = tid * 8; k0 < p.D; k0 += blockDim.x * 8) {
        float v[8];
        load_widen<DT, 8>(reinterpret_cast<const char*>(p.embed) + (base + k0) * St<DT>::bytes, v);
        float* xr = p.x + (long)r * p.D + k0;
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[e] = v[e];
    }
}

// Shared-prefix groups ([KV Cache] section 05, prefix caching): one workgroup per group admits each
// member sequence whose block table holds the group's first sequence's prefix page ids (valid pages),
// which brings exactly one row and whose context covers the prefix: seq_group[seq] = g (the first group
// to claim a sequence keeps it), seq_gp[seq] = the prefix pages, and its row goes on the list of rows
// the merge kernel combines (merge_rows, *merge_count, in no fixed order; each row's merge is the same
// wherever it sits). A member that fails a check keeps seq_group -1 and is attended over all its own
// pages; with error_flags, the failure sets VS_STEP_BAD_BATCH (4).
struct GroupArgs {
    const int* group_seq0;
    const int* group_n;
    const int* group_pages;
    int max_group_size, max_group_pages;
    const int* q_start;
    const int* ctx_len;
    const int* block_tables;
    int B, max_blocks, num_pages, page_tokens;
    int* seq_group;
    int* seq_gp;
    int* merge_rows;   // [B]
    int* merge_count;
    int M;
    int* error_flags;
};

__global__ void __launch_bounds__(256) prefix_group_kernel(GroupArgs a) {
    const int g = blockIdx.x, tid = threadIdx.x;
    const int seq0 = a.group_seq0[g], n = a.group_n[g], gp = a.group_pages[g];
    __shared__ int bad[256];
    const bool ok_group = seq0 >= 0 && n >= 1 && n <= a.max_group_size && (long)seq0 + n <= a.B && gp >= 1 &&
                          gp <= a.max_group_pages && gp <= a.max_blocks;
    if (!ok_group) {
        if (tid == 0 && a.error_flags) atomicOr(a.error_flags, 4);
        return;
    }
    const int* bt0 = a.block_tables + (long)seq0 * a.max_blocks;
    int flag = 0;
    for (int c = 0; c < n; c += 256) {
        const int cnt = min(256, n - c);
        bad[tid] = 0;
        __syncthreads();
        for (long idx = tid; idx < (long)cnt * gp; idx += 256) {
            const int i = (int)(idx / gp), j = (int)(idx % gp);
            const int pg = bt0[j];
            if (pg < 0 || pg >= a.num_pages || a.block_tables[(long)(seq0 + c + i) * a.max_blocks + j] != pg) bad[i] = 1;
        }
        __syncthreads();
        if (tid < cnt) {
            const int seq = seq0 + c + tid;
            bool ok = !bad[tid] && a.q_start[seq + 1] - a.q_start[seq] == 1 &&
                      (long)a.ctx_len[seq] >= (long)a.page_tokens * gp;
            if (ok) ok = atomicCAS(&a.seq_group[seq], -1, g) == -1;
            if (ok) {
                a.seq_gp[seq] = gp;
                a.merge_rows[atomicAdd(a.merge_count, 1)] = min(max(a.q_start[seq], 0), a.M - 1);
            } else {
                flag = 4;
            }
        }
        __syncthreads();
    }
    if (flag && a.error_flags) atomicOr(a.error_flags, flag);
}

// y[r] = round(x[src] / sqrt(mean(x[src]^2) + eps) * gain), src = map ? map[r] : r
// (a mapped row is clamped into [0, n_src)); one 1024-thread workgroup per row,
// fixed-order reduction (per thread, per wave, then over the 16 waves in
// order). Rows up to 4096 wide take one group of four features per thread, with
// x and the gain requested together and kept in registers across the reduction.
// Used ahead of the MFMA path; the GEMV path normalises inside its own prologue.
template <int DT>
__global__ void __launch_bounds__(1024) rmsnorm_kernel(const float* x, const int* map, int n_src, const void* gain,
                                                       int D, float eps, void* y) {
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int src = map ? min(max(map[r], 0), n_src - 1) : r;
    const float* xr = x + (long)src * D;
    __shared__ float wsum[16];
    auto row_inv = [&](float ss) {
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) ss += shfl_xor(ss, mask);
        if ((tid & 63) == 0) wsum[tid >> 6] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < 16; ++w) tot += wsum[w];
        return 1.0f / sqrtf(tot / (float)D + eps);
    };
    if (D <= 4 * 1024) {
        const int k = tid * 4;
        float4_t v = (float4_t){0.f, 0.f, 0.f, 0.f};
        float gv[4] = {0.f, 0.f, 0.f, 0.f};
        float ss = 0.f;
        if (k < D) {
            load_widen<DT, 4>(reinterpret_cast<const char*>(gain) + (long)k * St<DT>::bytes, gv);
            v = *reinterpret_cast<const float4_t*>(xr + k);
            ss = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
        const float inv = row_inv(ss);
        if (k < D) {
#pragma unroll
            for (int e = 0; e < 4; ++e) store_round<DT>(y, (long)r * D + k + e, v[e] * inv * gv[e]);
        }
        return;
    }
    float ss = 0.f;
    for (int k = tid * 4; k < D; k += 1024 * 4) {
        const float4_t v = *reinterpret_cast<const float4_t*>(xr + k);
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    const float inv = row_inv(ss);
    for (int k = tid * 4; k < D; k += 1024 * 4) {
        const float4_t v = *reinterpret_cast<const float4_t*>(xr + k);
        float gv[4];
        load_widen<DT, 4>(reinterpret_cast<const char*>(gain) + (long)k * St<DT>::bytes, gv);
#pragma unroll
        for (int e = 0; e < 4; ++e) store_round<DT>(y, (long)r * D + k + e, v[e] * inv * gv[e]);
    }
}

// Per sequence: reduce each logit row's tile partials to (argmax, top-2 gap),
// then optionally run greedy acceptance over the sequence's rows and advance
// the sequence's context length by its row count.
// Grid: B workgroups of 256 threads.
__global__ void __launch_bounds__(256) argmax_accept_kernel(const ArgPart* parts, int n_tiles, const int* q_start,
                                                            int M, const int* logit_rows, int M_log,
                                                            const int* tokens, const int* g0, int* argmax, float* gap,
                                                            int* accept_len, int* bonus, int* ctx_advance) {
    const int b = blockIdx.x;
    const int r0 = min(max(q_start[b], 0), M);
    const int r1 = min(max(q_start[b + 1], r0), M);
    __shared__ float sv1[4], sv2[4];
    __shared__ int si1[4];
    if (argmax) {
        // rows without logits first (all threads), then the sequence's logit rows: one lower-bound
        // search in the ascending logit_rows finds the first, the rest follow it in order (a search
        // per row would be a chain of dependent loads for every row of a long prompt chunk)
        for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
            argmax[r] = -1;
            if (gap) gap[r] = NAN;
        }
        int lo = 0, hi = M_log;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (logit_rows[mid] < r0) lo = mid + 1;
            else hi = mid;
        }
        int hi2 = lo, top = M_log;  // the sequence's logit rows are logit_rows[lo .. hi2)
        while (hi2 < top) {
            const int mid = (hi2 + top) >> 1;
            if (logit_rows[mid] < r1) hi2 = mid + 1;
            else top = mid;
        }
        __syncthreads();  // the defaults above land before the values below
        if (hi2 - lo >= 2) {
            // several logit rows (a verify pass): up to eight rows at a time, every thread combining its
            // tiles of all of them, so the rows' partials are requested together; the combine is exact in
            // any order (largest value, lowest index on ties, second value)
            constexpr int RB = 8;
            __shared__ float bv1[RB][4], bv2[RB][4];
            __shared__ int bi1[RB][4];
            const int wave = threadIdx.x >> 6;
            for (int j0 = lo; j0 < hi2; j0 += RB) {
                const int nr = min(RB, hi2 - j0);
                float v1[RB], v2[RB];
                int i1[RB];
#pragma unroll
                for (int q = 0; q < RB; ++q) {
                    v1[q] = v2[q] = -INFINITY;
                    i1[q] = 0x7FFFFFFF;
                }
                // every load unconditional (rows past the pass's last re-read it, and are never written):
                // with a branch around a load the compiler waits for each before issuing the next
                for (int t = threadIdx.x; t < n_tiles; t += blockDim.x) {
                    ArgPart p[RB];
#pragma unroll
                    for (int q = 0; q < RB; ++q) p[q] = parts[(long)(j0 + min(q, nr - 1)) * n_tiles + t];
#pragma unroll
                    for (int q = 0; q < RB; ++q) argpart_combine(v1[q], i1[q], v2[q], p[q].v1, p[q].i1, p[q].v2);
                }
#pragma unroll
                for (int q = 0; q < RB; ++q) {
#pragma unroll
                    for (int mask = 32; mask >= 1; mask >>= 1) {
                        const float o1 = shfl_xor(v1[q], mask);
                        const int oi = shfl_xor(i1[q], mask);
                        const float o2 = shfl_xor(v2[q], mask);
                        argpart_combine(v1[q], i1[q], v2[q], o1, oi, o2);
                    }
                    if ((threadIdx.x & 63) == 0) {
                        bv1[q][wave] = v1[q];
                        bi1[q][wave] = i1[q];
                        bv2[q][wave] = v2[q];
                    }
                }
                __syncthreads();
                if (threadIdx.x < nr) {
                    const int q = threadIdx.x;
                    float a1 = bv1[q][0], a2 = bv2[q][0];
                    int ai = bi1[q][0];
                    for (int w = 1; w < 4; ++w) argpart_combine(a1, ai, a2, bv1[q][w], bi1[q][w], bv2[q][w]);
                    const int r = logit_rows[j0 + q];
                    argmax[r] = ai;
                    if (gap) gap[r] = a1 - a2;
                }
                __syncthreads();  // the rows' argmax land before the acceptance reads them; LDS is free again
            }
        }
        for (int j = lo; j < (hi2 - lo >= 2 ? lo : hi2); ++j) {
            const int r = logit_rows[j];
            float v1 = -INFINITY, v2 = -INFINITY;
            int i1 = 0x7FFFFFFF;
            for (int t = threadIdx.x; t < n_tiles; t += blockDim.x) {
                const ArgPart p = parts[(long)j * n_tiles + t];
                argpart_combine(v1, i1, v2, p.v1, p.i1, p.v2);
            }
#pragma unroll
            for (int mask = 32; mask >= 1; mask >>= 1) {
                const float o1 = shfl_xor(v1, mask);
                const int oi = shfl_xor(i1, mask);
                const float o2 = shfl_xor(v2, mask);
                argpart_combine(v1, i1, v2, o1, oi, o2);
            }
            if ((threadIdx.x & 63) == 0) {
                sv1[threadIdx.x >> 6] = v1;
                si1[threadIdx.x >> 6] = i1;
                sv2[threadIdx.x >> 6] = v2;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                float a1 = sv1[0], a2 = sv2[0];
                int ai = si1[0];
                for (int w = 1; w < 4; ++w) argpart_combine(a1, ai, a2, sv1[w], si1[w], sv2[w]);
                argmax[r] = ai;
                if (gap) gap[r] = a1 - a2;
            }
            __syncthreads();
        }
    }
    if (accept_len && threadIdx.x == 0) {
        // drafts d_1..d_K are the row tokens; g_0 is given, g_j = argmax of row j-1
        const int K = r1 - r0;
        int n = 0;
        int g = g0[b];
        while (n < K && tokens[r0 + n] == g) {
            g = argmax[r0 + n];
            ++n;
        }
        accept_len[b] = n;
        bonus[b] = g;
    }
    if (ctx_advance && threadIdx.x == 0) ctx_advance[b] += r1 - r0;
}

// Standalone greedy acceptance: one thread per sequence.
__global__ void verify_accept_kernel(int B, const int* q_start, const int* drafts, const int* g0, const int* argmax,
                                     int* accept_len, int* bonus) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int r0 = q_start[b], K = max(q_start[b + 1] - r0, 0);
    int n = 0;
    int g = g0[b];
    while (n < K && drafts[r0 + n] == g) {
        g = argmax[r0 + n];
        ++n;
    }
    accept_len[b] = n;
    bonus[b] = g;
}

// Streaming-read ceiling (a measurement aid): the rows of a buffer (8 KB each) spread round-robin over
// every wave of the grid, each row read as eight 1 KB wave-wide nontemporal loads, two rows in flight per
// wave; the words are folded into one value so the loads are kept. The same load shape as the GEMV.
__global__ void __launch_bounds__(512) stream_read_kernel(const char* __restrict__ buf, long n_rows,
                                                          unsigned* sink) {
    constexpr int CH = 8;
    const int lane = threadIdx.x & 63;
    const long G = (long)gridDim.x * 8;
    long r = (long)blockIdx.x * 8 + (threadIdx.x >> 6);
    unsigned acc = 0;
    uint4 b0[CH], b1[CH];
    auto issue = [&](uint4(&b)[CH], long row) {
#pragma unroll
        for (int c = 0; c < CH; ++c) b[c] = load_stream16(buf + row * 8192 + c * 1024 + lane * 16);
    };
    auto fold = [&](const uint4(&b)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc += b[c].x ^ b[c].y ^ b[c].z ^ b[c].w;
    };
    if (r < n_rows) {
        issue(b0, r);
        for (;;) {
            const long r1 = r + G;
            if (r1 < n_rows) issue(b1, r1);
            fold(b0);
            if (r1 >= n_rows) break;
            const long r2 = r1 + G;
            if (r2 < n_rows) issue(b0, r2);
            fold(b1);
            if (r2 >= n_rows) break;
            r = r2;
        }
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // practically never: keeps the folds live
}

}  // namespace vs
