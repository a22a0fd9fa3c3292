// Row-streaming weight GEMV for steps of up to MR rows (gfx950).
//
// y[m][n] = sum_k X[m][k] * W[n][k] for every row m of a small batch: the
// whole step's rows share one read of each weight row ([KV Cache] section 02;
// [Spending the Idle] section 12.2). Weight rows are streamed so that every
// wave-wide load is 1 KB of one row (64 lanes x 16 contiguous bytes): on this
// part that pattern reaches the streaming-read ceiling, where MFMA-shaped
// loads (16 rows x 64 bytes per instruction) fall well short. The products run
// on packed dot2 instructions (fp16 / bf16 pairs, fp32 accumulate); at a few
// rows per step the matrix cores would idle, and the loads are the cost.
//
// A workgroup (8 waves) owns a contiguous range of output units. A unit is
// the set of weight rows one epilogue combines: one row (residual add,
// logits), the gate and up rows of one feature (SwiGLU), or a rotary pair
// (rows i and i + head_dim/2 of one q / k / v head). Each wave takes every
// eighth unit of the range and issues the unit's loads in bursts of up to
// eight 1 KB loads per row, all in flight together; with 16 or more waves per
// CU the bursts of other waves cover each wave's wait.
// Each unit's dot products go to LDS; the epilogues (which read rotary
// tables, page ids or the residual) run after the stream, so no dependent
// global load waits behind in-flight weight batches.
//
// The workgroup's batch rows X live in LDS in the storage type, loaded once in
// a prologue that runs while the first weight batch is already in flight:
// either copied (X_PLAIN), or built from the fp32 residual stream as RMSNorm
// output, round(x * rsqrt(mean(x^2) + eps) * gain) (X_NORM), with the sum of
// squares reduced in a fixed order so every workgroup computes the same scale,
// or merged from the attention kernel's per-split statistics (X_MERGE, the
// output product's input): every split is rescaled to the largest running
// maximum and the summed outputs are divided by the summed sums ([Serving
// Efficiency] section 31.4; [KV Cache] section 07, Flash-Decoding), in the same
// order as the standalone merge kernel, so both give the same bits.
#pragma once

#include "common.h"
#include "attention.h"
#include "gemm.h"

namespace vs {

constexpr int kGemvWaves = 8;
constexpr int kGemvChunks = 8;  // 1 KB chunks per weight row in one burst of loads

struct GemvArgs {
    const void* w0;
    const void* w1;
    const void* w2;
    int n0, n1, n2;  // rows of each weight segment
    int K;           // row length, a multiple of 8
    const void* act;  // X_PLAIN: [rows][act_ld]
    int act_ld;
    const float* xin;  // X_NORM: fp32 residual [rows][xin_ld]
    int xin_ld;
    const void* gain;  // X_NORM: gain [K]
    float eps;
    const int* act_rows;  // optional GEMV row -> activation row map
    // X_MERGE: attention split statistics [rows][n_heads][n_splits][part_stride(head_dim)]
    const float* part;
    int n_splits;
    int M;                // batch rows (<= MR)
    int n_units, units_per_wg;
    // X_PLAIN rows too long for LDS: stage X k_phase elements at a time (0 = all of K at once);
    // requires one unit per wave (units_per_wg <= waves) and a multiple of one burst
    int k_phase;
    // rotary + K/V write (EPI_QKV)
    void* q_out;
    void* kv_base;
    long page_elems, layer_elems;
    int kv_dt;  // cache storage: DT, or E4M3 / E5M2
    int layer, head_dim, n_heads, n_kv_heads, page_tokens;
    const int* block_tables;
    int max_blocks, num_pages;
    const int* row_seq;
    const int* row_pos;
    const float* rope_cs;
    const long* row_kvoff;  // per row: page * page_elems + slot * head_dim of its K/V slot, or -1
    // residual (EPI_RESID)
    float* x;
    int x_ld;
    // SwiGLU (EPI_SWIGLU)
    void* h_out;
    int h_ld;
    // logits (EPI_LOGITS): partial argmax per workgroup, parts[m][wg]
    float* logits;
    int vocab;
    ArgPart* parts;
    int n_parts;
};

// fp32 sum of the 8 (or 4 for fp32) products of one 16-byte weight fragment and one activation fragment
template <int DT>
__device__ __forceinline__ float dot16(const uint4 w, const uint4 x, float acc) {
    if constexpr (DT == F16) {
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.x), __builtin_bit_cast(half2_t, x.x), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.y), __builtin_bit_cast(half2_t, x.y), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.z), __builtin_bit_cast(half2_t, x.z), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.w), __builtin_bit_cast(half2_t, x.w), acc, false);
    } else if constexpr (DT == BF16) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc,
                                              false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc,
                                              false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc,
                                              false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc,
                                              false);
    } else {
        acc += __uint_as_float(w.x) * __uint_as_float(x.x);
        acc += __uint_as_float(w.y) * __uint_as_float(x.y);
        acc += __uint_as_float(w.z) * __uint_as_float(x.z);
        acc += __uint_as_float(w.w) * __uint_as_float(x.w);
    }
    return acc;
}

// The weight rows of unit u: RU (base, row) pairs, and what the unit means.
struct UnitMap {
    const void* w[2];
    int row[2];
    int seg, head, i;  // EPI_QKV: segment (q, k, v), head inside it, rotary pair index
};

template <int EPI>
__device__ __forceinline__ UnitMap unit_map(const GemvArgs& g, int u) {
    UnitMap m;
    m.seg = 0;
    m.head = 0;
    m.i = 0;
    if constexpr (EPI == EPI_RESID || EPI == EPI_LOGITS) {
        m.w[0] = m.w[1] = g.w0;
        m.row[0] = m.row[1] = u;
    } else if constexpr (EPI == EPI_SWIGLU) {
        m.w[0] = g.w0;
        m.w[1] = g.w1;
        m.row[0] = m.row[1] = u;
    } else {
        const int half = g.head_dim / 2;
        const int qu = g.n_heads * half, ku = g.n_kv_heads * half;
        int uu = u;
        if (uu < qu) {
            m.seg = 0;
            m.w[0] = g.w0;
        } else if (uu < qu + ku) {
            m.seg = 1;
            uu -= qu;
            m.w[0] = g.w1;
        } else {
            m.seg = 2;
            uu -= qu + ku;
            m.w[0] = g.w2;
        }
        m.w[1] = m.w[0];
        m.head = uu / half;
        m.i = uu % half;
        m.row[0] = m.head * g.head_dim + m.i;
        m.row[1] = m.row[0] + half;
    }
    return m;
}

// Epilogue of one (unit, batch row m) from the unit's dot products v[0], v[1].
template <int DT, int EPI>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& g, int u, int m, float v0, float v1) {
    if constexpr (EPI == EPI_RESID) {
        g.x[(long)m * g.x_ld + u] += v0;
    } else if constexpr (EPI == EPI_LOGITS) {
        if (g.logits) g.logits[(long)m * g.vocab + u] = v0;
    } else if constexpr (EPI == EPI_SWIGLU) {
        const float s = v0 / (1.0f + expf(-v0));
        store_round<DT>(g.h_out, (long)m * g.h_ld + u, s * v1);
    } else {
        const UnitMap um = unit_map<EPI>(g, u);
        const int half = g.head_dim / 2;
        float ra = v0, rb = v1;
        if (um.seg < 2) {
            const float c = g.rope_cs[((long)m * half + um.i) * 2 + 0];
            const float s = g.rope_cs[((long)m * half + um.i) * 2 + 1];
            ra = v0 * c - v1 * s;
            rb = v1 * c + v0 * s;
        }
        if (um.seg == 0) {
            const long o = (long)m * (g.n_heads * g.head_dim) + um.head * g.head_dim + um.i;
            store_round<DT>(g.q_out, o, ra);
            store_round<DT>(g.q_out, o + half, rb);
        } else {
            const int pos = g.row_pos[m];
            if (pos < 0 || pos / g.page_tokens >= g.max_blocks) return;
            const int page = g.block_tables[(long)g.row_seq[m] * g.max_blocks + pos / g.page_tokens];
            if (page < 0 || page >= g.num_pages) return;
            const long o = (long)page * g.page_elems + (long)g.layer * g.layer_elems +
                           ((long)(um.seg - 1) * g.n_kv_heads + um.head) * g.page_tokens * g.head_dim +
                           (long)(pos % g.page_tokens) * g.head_dim + um.i;
            store_kv<DT>(g.kv_base, o, ra, g.kv_dt);
            store_kv<DT>(g.kv_base, o + half, rb, g.kv_dt);
        }
    }
}

constexpr int kGemvMaxUnits = 128;  // units per workgroup (results parked in LDS)
constexpr int kMergeMaxSplits = 8;  // X_MERGE: most key splits the prologue merges

template <int DT, int MR, int XM, int EPI, int NW = kGemvWaves, int CG = kGemvChunks>
__global__ void __launch_bounds__(NW * 64) gemv_kernel(GemvArgs g) {
    constexpr int RU = (EPI == EPI_RESID || EPI == EPI_LOGITS) ? 1 : 2;  // rows per unit
    constexpr int EPL = 16 / St<DT>::bytes;                              // elements per lane-load
    constexpr int CE = EPL * 64;                                         // elements per 1 KB chunk
    extern __shared__ __align__(16) unsigned char smem[];  // X: [M][K] in the storage type
    __shared__ float res[kGemvMaxUnits][RU][MR];           // per-unit dot products, epilogue input

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int u_begin = blockIdx.x * g.units_per_wg;
    const int n_local = min(g.units_per_wg, g.n_units - u_begin);
    const int K = g.K;
    const int NC = (K + CE - 1) / CE;      // 1 KB chunks per row
    const int NG = (NC + CG - 1) / CG;     // bursts per unit
    const int my_units = n_local > wave ? (n_local - wave + NW - 1) / NW : 0;
    const uint32_t lane_byte = (uint32_t)lane * 16;
    const uint32_t row_bytes = (uint32_t)K * St<DT>::bytes;

    // One burst: chunks [CG * gi, +CG) of each of the unit's RU rows, all loads unconditional
    // (past a row's end a lane re-reads the row's first 16 bytes; the value is masked out).
    auto issue = [&](uint4(&buf)[RU][CG], const UnitMap& um, int gi) {
#pragma unroll
        for (int r = 0; r < RU; ++r) {
            // wave-uniform row address + a 32-bit per-lane offset (scalar-base addressing)
            const char* rowp = reinterpret_cast<const char*>(r == 0 ? um.w[0] : um.w[1]) +
                               (long)(r == 0 ? um.row[0] : um.row[1]) * row_bytes;
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                const uint32_t off = (uint32_t)(gi * CG + c) * 1024u + lane_byte;
                buf[r][c] = load_stream16(rowp + (off < row_bytes ? off : 0u));
            }
        }
    };

    // ---- prologue inputs, requested before the first weight burst: loads retire in order, so anything
    // requested after the burst would wait for it. X_NORM keeps each thread's share of the fp32 rows and
    // of the gain in registers for both passes of the norm (rows up to PN * NW * 256 wide). (Fetching
    // X_MERGE's split statistics or X_PLAIN's chunks early measured no faster.)
    constexpr int PN = 2;  // float4 groups per row and thread
    float4_t pre_x[XM == X_NORM ? MR : 1][PN];
    uint32_t pre_g[XM == X_NORM ? PN : 1][St<DT>::bytes == 2 ? 2 : 4];
    const bool pre_fast = XM == X_NORM && K <= PN * NW * 256;
    if constexpr (XM == X_NORM) {
        if (pre_fast) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m >= g.M) break;
                const int src = g.act_rows ? g.act_rows[m] : m;
                const float* xr = g.xin + (long)src * g.xin_ld;
#pragma unroll
                for (int j = 0; j < PN; ++j) {
                    const int k = tid * 4 + j * NW * 256;
                    pre_x[m][j] = k < K ? *reinterpret_cast<const float4_t*>(xr + k) : (float4_t){0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int j = 0; j < PN; ++j) {
                const int k = tid * 4 + j * NW * 256;
                const uint32_t* gp = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(g.gain) +
                                                                       (long)(k < K ? k : 0) * St<DT>::bytes);
#pragma unroll
                for (int w = 0; w < (St<DT>::bytes == 2 ? 2 : 4); ++w) pre_g[j][w] = gp[w];
            }
        }
    }
    // the epilogue's own inputs (the residual, the rotary pair's cos / sin, the row's K/V slot), also
    // requested now: thread t serves (unit t / M, row t % M) when there are few enough items
    float ep_x = 0.f;
    float2 ep_cs = make_float2(1.f, 0.f);
    long ep_off = -1;
    const bool ep_fast = n_local * g.M <= NW * 64;
    if (ep_fast && tid < n_local * g.M) {
        const int ul = tid / g.M, m = tid % g.M, u = u_begin + ul;
        if constexpr (EPI == EPI_RESID) ep_x = g.x[(long)m * g.x_ld + u];
        if constexpr (EPI == EPI_QKV) {
            const UnitMap um = unit_map<EPI>(g, u);
            ep_cs = *reinterpret_cast<const float2*>(g.rope_cs + ((long)m * (g.head_dim / 2) + um.i) * 2);
            ep_off = g.row_kvoff[m];
        }
    }

    // the wave's first burst is in flight while X is staged
    uint4 buf[RU][CG];
    if (my_units > 0) issue(buf, unit_map<EPI>(g, u_begin + wave), 0);

    // ---- prologue: the batch rows into LDS ----
    if (XM == X_NORM && pre_fast) {
        __shared__ float red_f[NW][MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= g.M) break;
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < PN; ++j)
                ss += pre_x[m][j][0] * pre_x[m][j][0] + pre_x[m][j][1] * pre_x[m][j][1] +
                      pre_x[m][j][2] * pre_x[m][j][2] + pre_x[m][j][3] * pre_x[m][j][3];
#pragma unroll
            for (int mask = 32; mask >= 1; mask >>= 1) ss += shfl_xor(ss, mask);
            if (lane == 0) red_f[wave][m] = ss;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= g.M) break;
            float part[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) part[w] = red_f[w][m];
#pragma unroll
            for (int span = 1; span < NW; span <<= 1)  // fixed pairwise tree
#pragma unroll
                for (int w = 0; w + span < NW; w += 2 * span) part[w] += part[w + span];
            const float rinv = 1.0f / sqrtf(part[0] / (float)K + g.eps);
            typename St<DT>::raw* xs = reinterpret_cast<typename St<DT>::raw*>(smem) + (long)m * K;
#pragma unroll
            for (int j = 0; j < PN; ++j) {
                const int k = tid * 4 + j * NW * 256;
                if (k >= K) continue;
                float gv[4];
                if constexpr (St<DT>::bytes == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        gv[e] = St<DT>::to_f((typename St<DT>::raw)((pre_g[j][e / 2] >> (16 * (e % 2))) & 0xFFFFu));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) gv[e] = __uint_as_float(pre_g[j][e]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) xs[k + e] = St<DT>::from_f(pre_x[m][j][e] * rinv * gv[e]);
            }
        }
    } else if constexpr (XM == X_NORM) {
        __shared__ float red[NW][MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= g.M) break;
            const int src = g.act_rows ? g.act_rows[m] : m;
            const float* xr = g.xin + (long)src * g.xin_ld;
            float ss = 0.f;
#pragma unroll 4
            for (int k = tid * 4; k < K; k += NW * 64 * 4) {
                const float4_t v = *reinterpret_cast<const float4_t*>(xr + k);
                ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
            }
#pragma unroll
            for (int mask = 32; mask >= 1; mask >>= 1) ss += shfl_xor(ss, mask);
            if (lane == 0) red[wave][m] = ss;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= g.M) break;
            float part[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) part[w] = red[w][m];
#pragma unroll
            for (int span = 1; span < NW; span <<= 1)  // fixed pairwise tree
#pragma unroll
                for (int w = 0; w + span < NW; w += 2 * span) part[w] += part[w + span];
            const float tot = part[0];
            const float rinv = 1.0f / sqrtf(tot / (float)K + g.eps);
            const int src = g.act_rows ? g.act_rows[m] : m;
            const float* xr = g.xin + (long)src * g.xin_ld;
            typename St<DT>::raw* xs = reinterpret_cast<typename St<DT>::raw*>(smem) + (long)m * K;
#pragma unroll 4
            for (int k = tid * 4; k < K; k += NW * 64 * 4) {
                const float4_t v = *reinterpret_cast<const float4_t*>(xr + k);
                float gv[4];
                load_widen<DT, 4>(reinterpret_cast<const char*>(g.gain) + (long)k * St<DT>::bytes, gv);
#pragma unroll
                for (int e = 0; e < 4; ++e) xs[k + e] = St<DT>::from_f(v[e] * rinv * gv[e]);
            }
        }
    } else if constexpr (XM == X_MERGE) {
        // Thread t builds 8 consecutive elements of one head: it loads that head's (m, l) of every
        // split and its 8 output values of every split in one batch (a single L2 round trip), then
        // rescales to the largest maximum and divides the summed outputs by the summed sums, in
        // split order, as the standalone merge kernel does.
        constexpr int NS = kMergeMaxSplits;
        const int H = g.n_heads, ns = g.n_splits, Dh = g.head_dim, SD = part_stride(g.head_dim);
        const int MK = g.M * K;
        typename St<DT>::raw* xs = reinterpret_cast<typename St<DT>::raw*>(smem);
        for (int e0 = tid * 8; e0 < MK; e0 += NW * 64 * 8) {
            const int m = e0 / K, k = e0 - m * K, h = k / Dh, d0 = k - h * Dh;
            const float* src = g.part + ((long)m * H + h) * ns * SD;
            float2 ml[NS];
            float4_t oa[NS], ob[NS];
#pragma unroll
            for (int sp = 0; sp < NS; ++sp) {
                const float* ss = src + (long)(sp < ns ? sp : ns - 1) * SD;
                ml[sp] = *reinterpret_cast<const float2*>(ss);
                oa[sp] = *reinterpret_cast<const float4_t*>(ss + kPartO + d0);
                ob[sp] = *reinterpret_cast<const float4_t*>(ss + kPartO + d0 + 4);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int sp = 0; sp < NS; ++sp)
                if (sp < ns) mx = fmaxf(mx, ml[sp].x);
            float l = 0.f, o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
            for (int sp = 0; sp < NS; ++sp) {
                if (sp < ns) {
                    const float w = ml[sp].x == -INFINITY ? 0.f : exp2f(ml[sp].x - mx);
                    l += w * ml[sp].y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        o[e] += w * oa[sp][e];
                        o[4 + e] += w * ob[sp][e];
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[e0 + e] = St<DT>::from_f(l > 0.f ? o[e] / l : 0.f);
        }
    } else if (g.k_phase == 0) {  // a phased X is staged inside the main loop
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= g.M) break;
            const int src = g.act_rows ? g.act_rows[m] : m;
            const char* ar = reinterpret_cast<const char*>(g.act) + (long)src * g.act_ld * St<DT>::bytes;
            char* xs = reinterpret_cast<char*>(smem) + (long)m * K * St<DT>::bytes;
#pragma unroll 4
            for (long off = tid * 16; off < (long)K * St<DT>::bytes; off += NW * 64 * 16)
                *reinterpret_cast<uint4*>(xs + off) = *reinterpret_cast<const uint4*>(ar + off);
        }
    }
    __syncthreads();

    // The wave's work is a sequence of bursts t = 0 .. my_units * NG - 1 (unit t / NG, burst t % NG).
    // Single-row units keep the next burst in flight while the current one is consumed (two
    // buffers); two-row units, whose buffers are twice as large, load one burst at a time.
    const int total = my_units * NG;
    float acc[RU][MR];
#pragma unroll
    for (int r = 0; r < RU; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
    int xk0 = 0, xkx = K;  // X in LDS: columns [xk0, xk0 + xkx) of every row, row stride xkx
    auto consume = [&](const uint4(&cur)[RU][CG], int t) {
        const int uj = t / NG, gi = t - uj * NG;
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            const long k = (long)(gi * CG + c) * CE + lane * EPL;
            const uint32_t keep = k < K ? 0xFFFFFFFFu : 0u;
            uint4 xf[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < g.M) {
                    const uint4 v = *reinterpret_cast<const uint4*>(
                        smem + ((long)m * xkx + (keep ? k - xk0 : 0)) * St<DT>::bytes);
                    xf[m] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
                }
            }
#pragma unroll
            for (int r = 0; r < RU; ++r) {
                const uint4 w = make_uint4(cur[r][c].x & keep, cur[r][c].y & keep, cur[r][c].z & keep,
                                           cur[r][c].w & keep);
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    if (m < g.M) acc[r][m] = dot16<DT>(w, xf[m], acc[r][m]);
            }
        }
        if (gi == NG - 1) {  // unit complete: reduce over the wave, park in LDS
            const int ul = wave + NW * uj;
#pragma unroll
            for (int r = 0; r < RU; ++r)
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (m < g.M) {
                        const float s2 = wave_sum(acc[r][m]);
                        if (lane == 0) res[ul][r][m] = s2;
                    }
                    acc[r][m] = 0.f;
                }
        }
    };
    auto issue_t = [&](uint4(&dst)[RU][CG], int t) {
        const int uj = t / NG;
        issue(dst, unit_map<EPI>(g, u_begin + wave + NW * uj), t - uj * NG);
    };
    bool phased = false;
    if constexpr (XM == X_PLAIN && RU == 1) {
        if (g.k_phase > 0) {
            // X staged one phase of k_phase columns at a time; the wave's single unit streams on,
            // its next burst already in flight across each phase change
            phased = true;
            const int KP = g.k_phase;
            const int BPP = KP / (CG * CE);  // bursts per phase
            const bool has = my_units > 0;
            uint4 buf2[RU][CG];
            auto stage = [&](int ph) {
                __syncthreads();  // every wave is done with the previous phase
                const int k0 = ph * KP;
                const long nbytes = (long)min(KP, K - k0) * St<DT>::bytes;
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (m >= g.M) break;
                    const int src = g.act_rows ? g.act_rows[m] : m;
                    const char* ar =
                        reinterpret_cast<const char*>(g.act) + ((long)src * g.act_ld + k0) * St<DT>::bytes;
                    char* xs = reinterpret_cast<char*>(smem) + (long)m * KP * St<DT>::bytes;
                    for (long off = tid * 16; off < nbytes; off += NW * 64 * 16)
                        *reinterpret_cast<uint4*>(xs + off) = *reinterpret_cast<const uint4*>(ar + off);
                }
                __syncthreads();
                xk0 = k0;
                xkx = KP;
            };
            for (int t = 0; t < NG; t += 2) {
                if (has && t + 1 < NG) issue_t(buf2, t + 1);
                if (t % BPP == 0) stage(t / BPP);
                if (has) consume(buf, t);
                if (t + 1 >= NG) break;
                if (has && t + 2 < NG) issue_t(buf, t + 2);
                if ((t + 1) % BPP == 0) stage((t + 1) / BPP);
                if (has) consume(buf2, t + 1);
            }
        }
    }
    if (phased) {
    } else if constexpr (RU == 1) {
        uint4 buf2[RU][CG];
        for (int t = 0; t < total; t += 2) {
            if (t + 1 < total) issue_t(buf2, t + 1);
            consume(buf, t);
            if (t + 1 >= total) break;
            if (t + 2 < total) issue_t(buf, t + 2);
            consume(buf2, t + 1);
        }
    } else {
        for (int t = 0; t < total; ++t) {
            if (t > 0) issue_t(buf, t);
            consume(buf, t);
        }
    }
    __syncthreads();

    // ---- epilogues of the workgroup's units, all threads ----
    if (ep_fast) {
        if (tid < n_local * g.M) {
            const int ul = tid / g.M, m = tid % g.M, u = u_begin + ul;
            const float v0 = res[ul][0][m], v1 = res[ul][RU - 1][m];
            if constexpr (EPI == EPI_RESID) {
                g.x[(long)m * g.x_ld + u] = ep_x + v0;
            } else if constexpr (EPI == EPI_QKV) {
                const UnitMap um = unit_map<EPI>(g, u);
                const int half = g.head_dim / 2;
                float ra = v0, rb = v1;
                if (um.seg < 2) {
                    ra = v0 * ep_cs.x - v1 * ep_cs.y;
                    rb = v1 * ep_cs.x + v0 * ep_cs.y;
                }
                if (um.seg == 0) {
                    const long o = (long)m * (g.n_heads * g.head_dim) + um.head * g.head_dim + um.i;
                    store_round<DT>(g.q_out, o, ra);
                    store_round<DT>(g.q_out, o + half, rb);
                } else if (ep_off >= 0) {
                    const long o = ep_off + (long)g.layer * g.layer_elems +
                                   ((long)(um.seg - 1) * g.n_kv_heads + um.head) * g.page_tokens * g.head_dim + um.i;
                    store_kv<DT>(g.kv_base, o, ra, g.kv_dt);
                    store_kv<DT>(g.kv_base, o + half, rb, g.kv_dt);
                }
            } else {
                gemv_epilogue<DT, EPI>(g, u, m, v0, v1);
            }
        }
    } else {
        for (int idx = tid; idx < n_local * g.M; idx += NW * 64) {
            const int ul = idx / g.M, m = idx % g.M;
            gemv_epilogue<DT, EPI>(g, u_begin + ul, m, res[ul][0][m], res[ul][RU - 1][m]);
        }
    }
    if constexpr (EPI == EPI_LOGITS) {
        // argmax partial of this workgroup's vocabulary range, per batch row (wave w takes rows w, w+4)
        for (int m = wave; m < g.M; m += NW) {
            float v1 = -INFINITY, v2 = -INFINITY;
            int i1 = 0x7FFFFFFF;
            for (int ul = lane; ul < n_local; ul += 64) argpart_combine(v1, i1, v2, res[ul][0][m], u_begin + ul, -INFINITY);
#pragma unroll
            for (int mask = 32; mask >= 1; mask >>= 1) {
                const float o1 = shfl_xor(v1, mask);
                const int oi = shfl_xor(i1, mask);
                const float o2 = shfl_xor(v2, mask);
                argpart_combine(v1, i1, v2, o1, oi, o2);
            }
            if (lane == 0) {
                ArgPart p;
                p.v1 = v1;
                p.i1 = i1;
                p.v2 = v2;
                p.pad = 0;
                g.parts[(long)m * g.n_parts + blockIdx.x] = p;
            }
        }
    }
}

}  // namespace vs
