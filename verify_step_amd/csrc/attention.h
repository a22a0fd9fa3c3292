// Paged split-KV attention for decode and verify rows (gfx950).
//
// [KV Cache] section 05: K and V are read through the sequence's block table
// from pages anywhere in the pool. Section 07, Flash-Decoding: the keys of
// one (sequence, head) are cut into splits processed in parallel; each split
// keeps the online-softmax state (running max m, running sum l, rescaled
// output o) over its keys, and the splits are merged by rescaling to a common
// maximum and dividing the summed outputs by the summed sums ([Serving
// Efficiency] section 31.4, Example 31.2: combine statistics, not normalised
// tile outputs).
//
// With a single split the workgroup's state is final: it writes the attention
// output itself (o / l in the storage type) and no merge is needed (with
// shared-prefix groups: a row outside any group whose own pages form one split).
// One workgroup of NW waves per (split, head, sequence, row-group block). Wave w takes pages
// w, w+NW, ... of the split. A prompt chunk's rows are spread over row-group blocks, so its
// row groups run in parallel. Lane l owns dims [(l%16)*DH/16, +DH/16) of key slot
// (l/16) within each group of four keys, so one page of 16 keys is four loads
// per lane for K and four for V, and the 16 lanes that share a key finish its
// dot product with DPP row sums. Each group of 16 lanes (one key slot) keeps its
// own online-softmax state over the keys it sees; the four are merged once at the
// end of the split. Every K/V byte is used by exactly one wave, so
// it goes from HBM straight to registers; each wave keeps a ring of three
// pages, two in flight while one is reduced (two pages, one in flight, for
// workgroups with four or more states, to leave registers for them). The four waves' states are merged through
// LDS and the workgroup's state is stored; a merge kernel then combines the
// splits and writes the attention output in the storage type. All rows of one sequence (up to RMAX
// at a time) share each K/V load; row i at position ctx + i keeps keys
// 0..ctx + i (causal across the rows of a pass). With grouped K/V heads
// ([KV Cache] section 04: GQA), a workgroup takes HG query heads of one K/V
// head, so each K/V load also serves HG heads: the workgroup carries RMAX x HG
// online-softmax states, state (row i, head j) at index i * HG + j. Scores are
// kept in the log2 domain (q pre-scaled by log2(e)/sqrt(DH)).
#pragma once

#include "common.h"

namespace vs {

struct AttnArgs {
    const void* q;  // [M][n_heads*DH] storage type, rotated
    const void* kv_base;
    long page_elems, layer_elems;
    int layer, n_heads, n_kv_heads, page_tokens;
    const int* block_tables;
    int max_blocks;
    int num_pages;  // page ids are clamped into [0, num_pages) before any read
    int M;          // rows in the step; q_start values are clamped into [0, M]
    const int* q_start;
    const int* ctx_len;
    int n_splits, split_pages;
    int B;             // sequences; grid z = B x row-group blocks
    int rg_blocks;     // workgroups over one sequence's row groups (each takes every rg_blocks-th group)
    float scale_log2;  // log2(e) / sqrt(DH)
    float* part;       // [M][n_heads][n_splits][part_stride(DH)]: m (log2 domain), l, -, -, o[DH]
    void* out;         // [M][n_heads*DH] storage type
    int rows_lo, rows_hi;  // a workgroup serves only sequences of rows_lo..rows_hi rows (a step that mixes
                           // one-row and longer sequences runs each kind through its own kernel)
    // Shared-prefix groups ([KV Cache] section 05, prefix caching: one copy of a common prefix's pages
    // serves several sequences). A grouped sequence (one row, seq_gp[b] = gp > 0) has the key splits
    // [0, n_pre_splits) over its group's gp prefix pages, computed once for the whole group by the
    // matrix-core kernel's group blocks, and the splits [n_pre_splits, n_splits) over its own pages
    // gp .. n_pages - 1. Any other sequence has only the splits [n_pre_splits, n_splits), over all its
    // pages (split_pages each): the workgroups of a plain launch take split n_pre_splits + blockIdx.x,
    // and the merge skips the first n_pre_splits splits of such rows. seq_gp = nullptr: no groups
    // (n_pre_splits = 0).
    const int* seq_gp;       // [B] prefix pages read by the sequence's group (0: not grouped)
    const int* seq_group;    // [B] the sequence's group (-1: none)
    const int* group_seq0;   // [n_groups] first sequence of each group (consecutive sequences)
    const int* group_n;      // [n_groups] sequences in each group
    const int* group_pages;  // [n_groups] prefix pages of each group
    int n_pre_splits, pre_split_pages;
    int gz_blocks;     // the matrix-core kernel's grid z blocks [0, gz_blocks) are group blocks: (block of
                       // 16 / HG sequences of a group) x n_pre_splits + prefix split
    int gz_per_group;  // blocks of 16 / HG sequences per group
    const int* row_seq;  // [M] each row's sequence (read by the merge kernel with groups)
    // The merge kernel's rows: merge_rows[0 .. *merge_count) (the grouped rows, when every other row
    // has a single split and was stored by the attention kernel), or nullptr: block x is row x.
    const int* merge_rows;
    const int* merge_count;
    // The matrix-core kernel's work list (nullptr: none): its plain block z - gz_blocks takes the unit
    // items[z - gz_blocks] = (sequence, first row of the row group) if below *n_items, else nothing;
    // without a list it takes sequence z % B and every rg_blocks-th row group from z / B on.
    const int2* items;
    const int* n_items;
};

// One split's statistics: m, l, two unused floats (so o starts 16-byte aligned), o[dh].
__host__ __device__ constexpr int part_stride(int dh) { return dh + 4; }
constexpr int kPartO = 4;  // offset of o in a split's statistics

// c + a.lo * b.lo + a.hi * b.hi over two packed 16-bit values, fp32 accumulation
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The pages [p_begin, p_end) of key split s >= n_pre_splits of a sequence with n_pages pages: the plain
// splits of split_pages pages, or, for a grouped sequence (gp prefix pages), its own pages gp .. n_pages - 1
// cut evenly over the splits after the prefix splits.
__device__ __forceinline__ void split_range(const AttnArgs& a, int s, int gp, int n_pages, int& p_begin, int& p_end) {
    if (gp > 0) {
        const int ss = a.n_splits - a.n_pre_splits;
        const int sp = (max(n_pages - gp, 0) + ss - 1) / ss;
        p_begin = gp + (s - a.n_pre_splits) * sp;
        p_end = min(p_begin + sp, n_pages);
    } else {
        p_begin = (s - a.n_pre_splits) * a.split_pages;
        p_end = min(p_begin + a.split_pages, n_pages);
    }
}

// o / l; a row with no visible key (l = 0, only if the block table is cut short) gives 0
__device__ __forceinline__ float safe_div(float o, float l) { return l > 0.f ? o / l : 0.f; }

template <int DT, int DH, int RMAX, int NW, int HG, int KVT = DT>  // KVT: the cache's storage type
__global__ void __launch_bounds__(NW * 64) attn_split_kernel(AttnArgs a) {
    constexpr int DPL = DH / 16;  // dims per lane
    constexpr int NS = RMAX * HG;  // online-softmax states: (row, head) pairs
    constexpr bool kDot2 = (DT == F16 || DT == BF16) && KVT == DT;  // scores by packed 16-bit dot products
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int g = lane >> 4;  // key slot within a group of four
    const int c = lane & 15;  // dim chunk
    const int s = a.n_pre_splits + blockIdx.x, h0 = blockIdx.y * HG;  // query heads h0 .. h0 + HG - 1 share K/V head hk
    const int b = blockIdx.z % a.B, rgb = blockIdx.z / a.B;
    const int group = a.n_heads / a.n_kv_heads;
    const int hk = h0 / group;

    const int r0 = min(max(a.q_start[b], 0), a.M);
    const int R = min(max(a.q_start[b + 1] - r0, 0), a.M - r0);
    if (R < a.rows_lo || R > a.rows_hi) return;  // another kernel's sequence
    const int gp = a.seq_gp ? a.seq_gp[b] : 0;  // a grouped sequence: its prefix splits come from the group
    const int ctx = max(a.ctx_len[b], 0);
    const int T = a.page_tokens;

    const int* bt = a.block_tables + (long)b * a.max_blocks;
    const long kofs = (long)a.layer * a.layer_elems + (long)hk * T * DH + (long)c * DPL;
    const long vofs = kofs + (long)a.n_kv_heads * T * DH;
    const int QLD = a.n_heads * DH;
    const char* kvb = reinterpret_cast<const char*>(a.kv_base);

    __shared__ float wst[NW][NS][DH + 2];  // per-wave (m, l, o) of each state

    // row groups of RMAX rows: this workgroup takes groups rgb, rgb + rg_blocks, ...; a group's last
    // row sits at position ctx + rg + nr - 1, so the group reads only the pages up to there
    for (int rg = rgb * RMAX; rg < R; rg += a.rg_blocks * RMAX) {
        const int nr = min(RMAX, R - rg);
        const int n_pages = min((ctx + rg + nr + T - 1) / T, a.max_blocks);
        int p_begin, p_end;
        split_range(a, s, gp, n_pages, p_begin, p_end);
        // q: with a 16-bit cache of the model's type, raw pairs for the packed dot products (the
        // products of two 16-bit values are exact in fp32; the scale is applied to the summed score);
        // otherwise widened and prescaled
        float qr[NS][DPL];
        uint32_t qw[NS][DPL / 2];
        float o[NS][DPL];
        float m[NS], l[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int i = st / HG, j = st % HG;
            m[st] = -INFINITY;
            l[st] = 0.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[st][e] = 0.f;
            const char* qp = reinterpret_cast<const char*>(a.q) +
                             ((long)(r0 + rg + (i < nr ? i : 0)) * QLD + (long)(h0 + j) * DH + c * DPL) * St<DT>::bytes;
            if constexpr (kDot2) {
                RawVec<DT, DPL> qv;
                load_raw<DT, DPL>(qv, qp);
#pragma unroll
                for (int w = 0; w < DPL / 2; ++w) qw[st][w] = i < nr ? qv.w[w] : 0u;
            } else if (i < nr) {
                load_widen<DT, DPL>(qp, qr[st]);
#pragma unroll
                for (int e = 0; e < DPL; ++e) qr[st][e] *= a.scale_log2;
            } else {
#pragma unroll
                for (int e = 0; e < DPL; ++e) qr[st][e] = 0.f;
            }
        }

        // a ring of pages per wave: while one is reduced, the next ones are in flight
        RawVec<KVT, DPL> ka[4], va[4], kb[4], vb[4], kc[4], vc[4];
        auto load_page = [&](RawVec<KVT, DPL>(&kk)[4], RawVec<KVT, DPL>(&vv)[4], int p) {
            const long pb = (long)min(max(bt[p], 0), a.num_pages - 1) * a.page_elems;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                load_raw<KVT, DPL>(kk[u], kvb + (pb + kofs + (long)(4 * u + g) * DH) * St<KVT>::bytes);
                load_raw<KVT, DPL>(vv[u], kvb + (pb + vofs + (long)(4 * u + g) * DH) * St<KVT>::bytes);
            }
        };
        auto reduce_page = [&](const RawVec<KVT, DPL>(&kk)[4], const RawVec<KVT, DPL>(&vv)[4], int p) {
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int i = st / HG;
                if (i >= nr) break;
                const int qpos = ctx + rg + i;
                float sc[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float d = 0.f;
                    if constexpr (kDot2) {
#pragma unroll
                        for (int w = 0; w < DPL / 2; ++w) d = dot2<DT>(qw[st][w], kk[u].w[w], d);
                        d = row16_sum(d) * a.scale_log2;  // the 16 lanes of a key slot hold its 16 dim chunks
                    } else {
#pragma unroll
                        for (int e = 0; e < DPL; ++e) d += qr[st][e] * raw_at<KVT, DPL>(kk[u], e);
                        d = row16_sum(d);
                    }
                    const int kp = p * T + 4 * u + g;
                    sc[u] = (kp <= qpos) ? d : -INFINITY;
                }
                // each key slot g keeps its own (m, l, o) over its keys; the four are merged once
                // per split, so a page needs no cross-lane exchange beyond the dot products
                const float pm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
                const float mn = fmaxf(m[st], pm);
                if (mn == -INFINITY) continue;  // no visible key for this slot yet
                const float alpha = exp2f(m[st] - mn);
                float ps = 0.f;
                float pu[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    pu[u] = exp2f(sc[u] - mn);
                    ps += pu[u];
                }
                l[st] = l[st] * alpha + ps;
#pragma unroll
                for (int e = 0; e < DPL; ++e) {
                    float acc = o[st][e] * alpha;
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc += pu[u] * raw_at<KVT, DPL>(vv[u], e);
                    o[st][e] = acc;
                }
                m[st] = mn;
            }
        };
        // Every load in the ring is unconditional (a page past the split re-reads the split's last
        // page, and is never reduced): with a branch around a load the compiler can only wait for
        // all outstanding loads, the pages in flight included.
        const int p0 = p_begin + wave;
        const int plast = p_end - 1;
        if (p0 < p_end) {
            if constexpr (NS >= 4) {  // many states: a ring of two pages leaves registers for them
                load_page(ka, va, p0);
                for (int p = p0;; p += 2 * NW) {
                    load_page(kb, vb, min(p + NW, plast));
                    __builtin_amdgcn_sched_barrier(0);  // the next page's loads stay ahead of this reduction
                    reduce_page(ka, va, p);
                    if (p + NW >= p_end) break;
                    load_page(ka, va, min(p + 2 * NW, plast));
                    __builtin_amdgcn_sched_barrier(0);
                    reduce_page(kb, vb, p + NW);
                    if (p + 2 * NW >= p_end) break;
                }
            } else {
                load_page(ka, va, p0);
                load_page(kb, vb, min(p0 + NW, plast));
                for (int p = p0;; p += 3 * NW) {
                    load_page(kc, vc, min(p + 2 * NW, plast));
                    __builtin_amdgcn_sched_barrier(0);
                    reduce_page(ka, va, p);
                    if (p + NW >= p_end) break;
                    load_page(ka, va, min(p + 3 * NW, plast));
                    __builtin_amdgcn_sched_barrier(0);
                    reduce_page(kb, vb, p + NW);
                    if (p + 2 * NW >= p_end) break;
                    load_page(kb, vb, min(p + 4 * NW, plast));
                    __builtin_amdgcn_sched_barrier(0);
                    reduce_page(kc, vc, p + 2 * NW);
                    if (p + 3 * NW >= p_end) break;
                }
            }
        }
        // this wave's state: merge the four key slots' states (rescaled to their common maximum),
        // park it in LDS
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            if (st / HG >= nr) break;
            float mx = fmaxf(m[st], shfl_xor(m[st], 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float f = m[st] == -INFINITY ? 0.f : exp2f(m[st] - mx);
            float ls = l[st] * f;
            ls += shfl_xor(ls, 16);
            ls += shfl_xor(ls, 32);
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                o[st][e] *= f;
                o[st][e] += shfl_xor(o[st][e], 16);
                o[st][e] += shfl_xor(o[st][e], 32);
            }
            if (lane == 0) {
                wst[wave][st][0] = mx;
                wst[wave][st][1] = ls;
            }
            if (g == 0) {
#pragma unroll
                for (int e = 0; e < DPL; ++e) wst[wave][st][2 + c * DPL + e] = o[st][e];
            }
        }
        __syncthreads();
        // merge the waves in wave order; thread t takes (state, dim) pairs
        for (int idx = tid; idx < nr * HG * DH; idx += NW * 64) {
            const int i = idx / DH, d = idx % DH;  // i: state index
            const int row = r0 + rg + i / HG, h = h0 + i % HG;
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) mx = fmaxf(mx, wst[w][i][0]);
            float ls = 0.f, os = 0.f;
            if (mx != -INFINITY) {
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float wm = wst[w][i][0];
                    if (wm == -INFINITY) continue;
                    const float f = exp2f(wm - mx);
                    ls += f * wst[w][i][1];
                    os += f * wst[w][i][2 + d];
                }
            }
            if (gp == 0 && a.n_splits - a.n_pre_splits == 1) {  // the row's only split: the state is final
                store_round<DT>(a.out, (long)row * a.n_heads * DH + (long)h * DH + d, safe_div(os, ls));
            } else {
                float* dst = a.part + (((long)row * a.n_heads + h) * a.n_splits + s) * part_stride(DH);
                if (d == 0) {
                    dst[0] = mx;
                    dst[1] = ls;
                }
                dst[kPartO + d] = os;
            }
        }
        __syncthreads();
    }

}

// One workgroup of DH threads per (row, head): rescale every split's state to
// the largest running maximum and divide the summed outputs by the summed sums.
// Split weights are computed once into LDS; thread d then sums dim d over the
// splits with independent loads.
template <int DT, int DH>
__global__ void __launch_bounds__(DH) attn_merge_kernel(AttnArgs a) {
    constexpr int kMaxSplits = 1024;
    __shared__ float sm[kMaxSplits], sw[kMaxSplits];
    __shared__ float s_red[DH / 64];
    int row = blockIdx.x;
    if (a.merge_rows) {
        if (row >= *a.merge_count) return;
        row = a.merge_rows[row];
    }
    const int h = blockIdx.y, d = threadIdx.x;
    // with prefix groups, a row outside any group has no prefix splits; with one split left, the
    // attention kernel stored its output itself
    const int s0 = a.seq_gp && a.seq_gp[a.row_seq[row]] == 0 ? a.n_pre_splits : 0;
    const int ns = min(a.n_splits - s0, kMaxSplits);
    if (ns == 1) return;
    constexpr int SD = part_stride(DH);
    const float* src = a.part + (((long)row * a.n_heads + h) * a.n_splits + s0) * SD;
    float mx = -INFINITY;
    for (int sp = d; sp < ns; sp += DH) {
        sm[sp] = src[(long)sp * SD];
        mx = fmaxf(mx, sm[sp]);
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) mx = fmaxf(mx, shfl_xor(mx, mask));
    if ((d & 63) == 0) s_red[d >> 6] = mx;
    __syncthreads();
    mx = s_red[0];
#pragma unroll
    for (int w = 1; w < DH / 64; ++w) mx = fmaxf(mx, s_red[w]);
    for (int sp = d; sp < ns; sp += DH) sw[sp] = sm[sp] == -INFINITY ? 0.f : exp2f(sm[sp] - mx);
    __syncthreads();
    float l = 0.f, o = 0.f;
#pragma unroll 4
    for (int sp = 0; sp < ns; ++sp) {
        const float w = sw[sp];
        l += w * src[(long)sp * SD + 1];
        o += w * src[(long)sp * SD + kPartO + d];
    }
    store_round<DT>(a.out, (long)row * a.n_heads * DH + (long)h * DH + d, safe_div(o, l));
}

}  // namespace vs
