// Weight-streaming skinny GEMM for the decode / verify step (gfx950).
//
// C[m][n] = sum_k X[m][k] * W[n][k] for the M <= 64 rows of one 64-row group
// of a step ([KV Cache] section 02: every row passing through a weight matrix
// shares one read of it; [Spending the Idle] section 12.2: the weights have
// no idea how many tokens pass through them).
//
// This is the path for steps of more than a few rows (the row-streaming GEMV
// covers the rest). A workgroup owns one tile of 32 output features (two
// blocks of 16 weight rows, chosen by the epilogue so that values it combines,
// such as a rotary pair or a gate/up pair, land in the same lane) and all rows
// of one 64-row group. Its NW waves split the reduction axis; each wave loads
// its slice of the two 16-row blocks with 16-byte loads straight into MFMA
// operand registers and multiplies on the matrix cores (16x16x32 fp16/bf16,
// 16x16x4 fp32; rows padded to 16). The waves' partial tiles are summed in a
// fixed binary tree through LDS, so results are deterministic.
//
// Operand roles: A = weights (MFMA rows = output features), B = activations
// (MFMA columns = batch rows). Lane l supplies weight row (l % 16) and batch
// row (l % 16), both at reduction offsets (l / 16) * 8 .. +7 of each 32-wide
// chunk, and receives C[feature (l/16)*4 + r][batch row l % 16], r = 0..3.
#pragma once

#include "common.h"

namespace vs {

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// A tile workgroup multiplies one group of MT x 16 batch rows (MT <= 4); larger steps run several
// row groups per tile, launched next to each other so that they share the tile's weight reads in the
// caches (their weight loads then keep the normal cache policy instead of streaming).
enum XMode { X_PLAIN = 0, X_NORM = 1, X_MERGE = 2 };

struct ArgPart {
    float v1;  // largest value in the tile
    int i1;    // its index (lowest on exact ties)
    float v2;  // second-largest value (equal to v1 on a tie)
    int pad;
};

struct GemmArgs {
    const void* w0;
    const void* w1;
    const void* w2;
    int n0, n1, n2;  // rows of each weight segment
    int K;           // reduction length, a multiple of 32
    const void* act;  // activations [rows][act_ld] in the storage type
    int act_ld;
    int M;  // rows
    int n_tiles;
    // rotary + K/V write (EPI_QKV)
    void* q_out;  // [M][n_heads*head_dim]
    void* kv_base;
    long page_elems;   // elements per page
    long layer_elems;  // elements per layer inside a page
    int kv_dt;         // cache storage: DT, or E4M3 / E5M2
    int layer, head_dim, n_heads, n_kv_heads, page_tokens;
    const int* block_tables;
    int max_blocks;
    int num_pages;  // pool size; page ids outside [0, num_pages) are never written
    const int* row_seq;
    const int* row_pos;
    const float* rope_cs;  // [M][head_dim/2][2] (cos, sin)
    // per row: element offset of its K/V slot inside its page, page * page_elems + slot * head_dim, or -1
    // when the row has no valid page (computed once per step)
    const long* row_kvoff;
    // residual add (EPI_RESID): x += C
    float* x;
    int x_ld;
    // SwiGLU (EPI_SWIGLU)
    void* h_out;
    int h_ld;
    // logits + argmax partials (EPI_LOGITS)
    float* logits;
    int vocab;
    ArgPart* parts;
};

__device__ __forceinline__ void argpart_combine(float& v1, int& i1, float& v2, float bv1, int bi1, float bv2) {
    if (bv1 > v1 || (bv1 == v1 && bi1 < i1)) {
        v2 = fmaxf(bv2, v1);
        v1 = bv1;
        i1 = bi1;
    } else {
        v2 = fmaxf(v2, bv1);
    }
}

// Raw operand fragment of one lane: 8 consecutive storage elements.
template <int DT> struct Frag;
template <> struct Frag<F32> {
    float4_t a, b;
};
template <> struct Frag<F16> {
    uint4 a;
};
template <> struct Frag<BF16> {
    uint4 a;
};

template <int DT>
__device__ __forceinline__ void frag_zero(Frag<DT>& f) {
    if constexpr (DT == F32) {
        f.a = (float4_t){0.f, 0.f, 0.f, 0.f};
        f.b = f.a;
    } else {
        f.a = make_uint4(0u, 0u, 0u, 0u);
    }
}

template <int DT, bool STREAM = false>
__device__ __forceinline__ void frag_load(Frag<DT>& f, const void* base, long elem, bool valid) {
    if (!valid) {
        frag_zero<DT>(f);
        return;
    }
    if constexpr (DT == F32) {
        const float4_t* p = reinterpret_cast<const float4_t*>(reinterpret_cast<const float*>(base) + elem);
        if constexpr (STREAM) {
            f.a = __builtin_bit_cast(float4_t, load_stream16(p));
            f.b = __builtin_bit_cast(float4_t, load_stream16(p + 1));
        } else {
            f.a = p[0];
            f.b = p[1];
        }
    } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + elem;
        f.a = STREAM ? load_stream16(p) : *reinterpret_cast<const uint4*>(p);
    }
}

template <int DT>
__device__ __forceinline__ float4_t frag_mma(const Frag<DT>& w, const Frag<DT>& x, float4_t acc) {
    if constexpr (DT == F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, w.a), __builtin_bit_cast(half8_t, x.a),
                                                      acc, 0, 0, 0);
    } else if constexpr (DT == BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w.a),
                                                       __builtin_bit_cast(bf16x8_t, x.a), acc, 0, 0, 0);
    } else {
        // eight rank-4 updates; element e of every lane carries reduction offset (l/16)*8 + e
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w.a[e], x.a[e], acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w.b[e], x.b[e], acc, 0, 0, 0);
        return acc;
    }
}

// Which two 16-row weight blocks a tile covers, and what they mean.
struct TileMap {
    const void* w;   // segment base for block A
    const void* wb;  // segment base for block B
    int rowA, rowB;  // first weight row of each block inside its segment
    int nrows;       // rows in the segment (rows >= nrows are padding)
    int seg;         // EPI_QKV: 0 = q, 1 = k, 2 = v
    int head, j;     // EPI_QKV: head inside the segment, 16-wide slot of the head's first half
};

template <int EPI>
__device__ __forceinline__ TileMap tile_map(const GemmArgs& g, int t) {
    TileMap m;
    m.seg = 0;
    m.head = 0;
    m.j = 0;
    if constexpr (EPI == EPI_RESID || EPI == EPI_LOGITS) {  // one block of 16 rows per tile
        m.w = g.w0;
        m.wb = g.w0;
        m.rowA = 16 * t;
        m.rowB = 16 * t;
        m.nrows = g.n0;
    } else if constexpr (EPI == EPI_SWIGLU) {
        m.w = g.w0;   // gate
        m.wb = g.w1;  // up
        m.rowA = 16 * t;
        m.rowB = 16 * t;
        m.nrows = g.n0;
    } else {
        const int tph = g.head_dim / 32;  // tiles per head
        const int qt = g.n_heads * tph, kt = g.n_kv_heads * tph;
        int tt = t;
        if (tt < qt) {
            m.seg = 0;
            m.w = g.w0;
            m.nrows = g.n0;
        } else if (tt < qt + kt) {
            m.seg = 1;
            tt -= qt;
            m.w = g.w1;
            m.nrows = g.n1;
        } else {
            m.seg = 2;
            tt -= qt + kt;
            m.w = g.w2;
            m.nrows = g.n2;
        }
        m.wb = m.w;
        m.head = tt / tph;
        m.j = tt % tph;
        m.rowA = m.head * g.head_dim + 16 * m.j;
        m.rowB = m.rowA + g.head_dim / 2;
    }
    return m;
}

// Epilogue on wave 0, whose lane holds C[feature nl0 + r][row l % 16] of both blocks.
template <int DT, int MT, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, const TileMap& tm, int tile, int mg, int lane,
                                              float4_t (&acc)[MT][2]) {
    const int l16 = lane & 15;
    const int nl0 = (lane >> 4) * 4;
    if constexpr (EPI == EPI_LOGITS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mg * (16 * MT) + mt * 16 + l16;
            float v1 = -INFINITY, v2 = -INFINITY;
            int i1 = 0x7FFFFFFF;
            {
                constexpr int b = 0;  // one 16-row block per tile
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = tm.rowA + nl0 + r;
                    const float v = acc[mt][b][r];
                    if (col < g.vocab) {
                        if (m < g.M && g.logits) g.logits[(long)m * g.vocab + col] = v;
                        argpart_combine(v1, i1, v2, v, col, -INFINITY);
                    }
                }
            }
#pragma unroll
            for (int mask = 16; mask <= 32; mask <<= 1) {
                const float o1 = shfl_xor(v1, mask);
                const int oi = shfl_xor(i1, mask);
                const float o2 = shfl_xor(v2, mask);
                argpart_combine(v1, i1, v2, o1, oi, o2);
            }
            if (lane < 16 && m < g.M) {
                ArgPart p;
                p.v1 = v1;
                p.i1 = i1;
                p.v2 = v2;
                p.pad = 0;
                g.parts[(long)m * g.n_tiles + tile] = p;
            }
        }
    } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mg * (16 * MT) + mt * 16 + l16;
            if (m >= g.M) continue;
            float* xr = g.x + (long)m * g.x_ld;
#pragma unroll
            for (int r = 0; r < 4; ++r) {  // one 16-row block per tile
                const int col = tm.rowA + nl0 + r;
                if (col < tm.nrows) xr[col] += acc[mt][0][r];
            }
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mg * (16 * MT) + mt * 16 + l16;
            if (m >= g.M) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int nl = nl0 + r;
                const float a = acc[mt][0][r];
                const float b = acc[mt][1][r];
                if constexpr (EPI == EPI_SWIGLU) {
                    if (tm.rowA + nl < tm.nrows) {
                        const float s = a / (1.0f + expf(-a));
                        store_round<DT>(g.h_out, (long)m * g.h_ld + tm.rowA + nl, s * b);
                    }
                } else {  // EPI_QKV
                    const int half = g.head_dim / 2;
                    const int i = 16 * tm.j + nl;  // rotary pair index inside the head
                    float ra = a, rb = b;
                    if (tm.seg < 2) {
                        const float c = g.rope_cs[((long)m * half + i) * 2 + 0];
                        const float s = g.rope_cs[((long)m * half + i) * 2 + 1];
                        ra = a * c - b * s;
                        rb = b * c + a * s;
                    }
                    if (tm.seg == 0) {
                        const long o = (long)m * (g.n_heads * g.head_dim) + tm.head * g.head_dim + i;
                        store_round<DT>(g.q_out, o, ra);
                        store_round<DT>(g.q_out, o + half, rb);
                    } else {
                        const int pos = g.row_pos[m];
                        const int sq = g.row_seq[m];
                        if (pos < 0 || pos / g.page_tokens >= g.max_blocks) continue;
                        const int page = g.block_tables[(long)sq * g.max_blocks + pos / g.page_tokens];
                        if (page < 0 || page >= g.num_pages) continue;
                        const int slot = pos % g.page_tokens;
                        const long o = (long)page * g.page_elems + (long)g.layer * g.layer_elems +
                                       ((long)(tm.seg - 1) * g.n_kv_heads + tm.head) * g.page_tokens * g.head_dim +
                                       (long)slot * g.head_dim + i;
                        store_kv<DT>(g.kv_base, o, ra, g.kv_dt);
                        store_kv<DT>(g.kv_base, o + half, rb, g.kv_dt);
                    }
                }
            }
        }
    }
}

// STREAM: one row group (every weight byte is used once), so the weight loads carry the
// nontemporal hint.
template <int DT, int MT, int NW, int EPI, int U, bool STREAM>
__global__ void __launch_bounds__(NW * 64) gemm_skinny_kernel(GemmArgs g) {
    constexpr bool SB = EPI == EPI_RESID || EPI == EPI_LOGITS;  // tiles of one 16-row block
    constexpr int NB = SB ? 1 : 2;
    constexpr int ROWB = 256 + 16;  // LDS slab row stride in bytes (padding spreads the banks)
    constexpr int SLAB = NB * 16 * ROWB;
    constexpr int RED = (NW / 2) * MT * 8 * 64 * 4;
    // per-wave weight slabs during the main loop, the partial-tile tree afterwards
    __shared__ __align__(16) unsigned char lds[(NW * SLAB > RED ? NW * SLAB : RED)];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
    const int mg = blockIdx.x;    // 64-row group (fastest: a tile's row groups run together and share its weights)
    const int tile = blockIdx.y;
    const TileMap tm = tile_map<EPI>(g, tile);

    const int KC = g.K / 32;
    const int kc0 = (wave * KC) / NW, kc1 = ((wave + 1) * KC) / NW;

    const int l16 = lane & 15;
    const int kofs = (lane >> 4) * 8;
    const int wrowA = tm.rowA + l16, wrowB = tm.rowB + l16;
    const bool vA = wrowA < tm.nrows, vB = wrowB < tm.nrows;
    const long baseA = (long)(vA ? wrowA : 0) * g.K + kofs;
    const long baseB = (long)(vB ? wrowB : 0) * g.K + kofs;
    long xbase[MT];
    bool xv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mg * (16 * MT) + mt * 16 + l16;
        xv[mt] = m < g.M;
        xbase[mt] = (long)(xv[mt] ? m : 0) * g.act_ld + kofs;
    }

    float4_t acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        acc[mt][0] = (float4_t){0.f, 0.f, 0.f, 0.f};
        acc[mt][1] = acc[mt][0];
    }

    if constexpr (DT == F32) {
        for (int kc = kc0; kc < kc1; kc += U) {
            Frag<DT> fa[U], fb[U], fx[U][MT];
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool in = kc + u < kc1;
                const long ko = (long)(kc + u) * 32;
                frag_load<DT, true>(fa[u], tm.w, baseA + ko, in && vA);
                if constexpr (!SB) frag_load<DT, true>(fb[u], tm.wb, baseB + ko, in && vB);
    #pragma unroll
                for (int mt = 0; mt < MT; ++mt) frag_load<DT>(fx[u][mt], g.act, xbase[mt] + ko, in && xv[mt]);
            }
    #pragma unroll
            for (int u = 0; u < U; ++u) {
    #pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[mt][0] = frag_mma<DT>(fa[u], fx[u][mt], acc[mt][0]);
                    if constexpr (!SB) acc[mt][1] = frag_mma<DT>(fb[u], fx[u][mt], acc[mt][1]);
                }
            }
        }
    } else {
        // fp16 / bf16: the weights are read four rows x 256 bytes per wave instruction (lane l: row
        // l / 16 of the four, elements 8 (l % 16) .. +7 of a 128-element block), a pattern that streams
        // as fast as whole-row reads where the MFMA operand layout (16 rows x 64 bytes) does not. Each
        // block passes through a wave-private LDS slab and is read back as MFMA A fragments.
        // Blocks of 128 reduction elements = 4 k-steps; the next block's loads are in flight while
        // the current one is multiplied.
        // Every load below is unconditional (out-of-range lanes read an in-bounds address and mask the
        // result), so the loads of the next block stay in flight: with a branch around a load the
        // compiler can only wait for all outstanding loads before the current block is used.
        unsigned char* my = lds + wave * SLAB;
        const int rr = lane >> 4, cc = lane & 15;  // R4 layout: row in the group of four, 16-byte column
        long rowoff[NB][4];
        bool rowv[NB][4];
#pragma unroll
        for (int bl = 0; bl < NB; ++bl)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = (bl ? tm.rowB : tm.rowA) + 4 * j + rr;
                rowv[bl][j] = row < tm.nrows;
                rowoff[bl][j] = (long)(rowv[bl][j] ? row : 0) * g.K + 8 * cc;
            }
        const uint16_t* wA = reinterpret_cast<const uint16_t*>(tm.w);
        const uint16_t* wB = reinterpret_cast<const uint16_t*>(tm.wb);
        // Weights of k-steps outside the wave's slice (and of rows past the segment) are read from an
        // in-bounds address and zeroed when written to the slab; the zero weights cancel whatever the
        // activations hold there, so the activation loads need no mask: their out-of-slice k-steps
        // read in-bounds activations of the same row, and batch rows past M (clamped to row 0) only
        // reach output columns the epilogue does not store. No load result is touched before the
        // multiply that needs it.
        struct WBlock {
            uint4 v[NB][4];
            uint32_t keep[NB][4];
        };
        auto load_block = [&](WBlock& wb, int kc) {
            const bool kin = kc + (cc >> 2) < kc1;
            const long ko = kin ? (long)kc * 32 : -(long)(8 * cc);  // masked lanes read their row's start
#pragma unroll
            for (int bl = 0; bl < NB; ++bl)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint16_t* src = (bl ? wB : wA) + rowoff[bl][j] + ko;
                    wb.v[bl][j] = STREAM ? load_stream16(src) : *reinterpret_cast<const uint4*>(src);
                    wb.keep[bl][j] = (kin && rowv[bl][j]) ? 0xFFFFFFFFu : 0u;
                }
        };
        const long xlast = (long)(KC - 1) * 32;  // last k-step of a row: keeps clamped reads in bounds
        auto load_x = [&](Frag<DT>(&fx)[4][MT], int kc) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const long ko = min((long)(kc + ks) * 32, xlast);
                    fx[ks][mt].a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(g.act) +
                                                                    xbase[mt] + ko);
                }
        };
        auto multiply = [&](const WBlock& wb, const Frag<DT>(&fx)[4][MT]) {
#pragma unroll
            for (int bl = 0; bl < NB; ++bl)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 v = wb.v[bl][j];
                    const uint32_t kp = wb.keep[bl][j];
                    *reinterpret_cast<uint4*>(my + bl * 16 * ROWB + (4 * j + rr) * ROWB + 16 * cc) =
                        make_uint4(v.x & kp, v.y & kp, v.z & kp, v.w & kp);
                }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Frag<DT> fa, fb;
                fa.a = *reinterpret_cast<const uint4*>(my + l16 * ROWB + 64 * ks + 16 * (lane >> 4));
                if constexpr (!SB)
                    fb.a = *reinterpret_cast<const uint4*>(my + 16 * ROWB + l16 * ROWB + 64 * ks + 16 * (lane >> 4));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[mt][0] = frag_mma<DT>(fa, fx[ks][mt], acc[mt][0]);
                    if constexpr (!SB) acc[mt][1] = frag_mma<DT>(fb, fx[ks][mt], acc[mt][1]);
                }
            }
        };
        WBlock w0, w1;
        if constexpr (MT <= 2 || (SB && MT <= 4)) {  // weights and activations of the next block in flight
            Frag<DT> x0[4][MT], x1[4][MT];
            load_block(w0, kc0);
            load_x(x0, kc0);
            for (int kc = kc0; kc < kc1; kc += 8) {
                load_block(w1, kc + 4);  // past the slice: masked, in-bounds reads
                load_x(x1, kc + 4);
                __builtin_amdgcn_sched_barrier(0);  // keep the next block's loads ahead of this multiply
                multiply(w0, x0);
                if (kc + 4 >= kc1) break;
                load_block(w0, kc + 8);
                load_x(x0, kc + 8);
                __builtin_amdgcn_sched_barrier(0);
                multiply(w1, x1);
            }
        } else {  // two weight blocks of three or four row blocks: only the weights run ahead (registers)
            Frag<DT> xf[4][MT];
            load_block(w0, kc0);
            for (int kc = kc0; kc < kc1; kc += 8) {
                load_x(xf, kc);  // before the next weights, so that using it leaves those in flight
                load_block(w1, kc + 4);
                __builtin_amdgcn_sched_barrier(0);
                multiply(w0, xf);
                if (kc + 4 >= kc1) break;
                load_x(xf, kc + 4);
                load_block(w0, kc + 8);
                __builtin_amdgcn_sched_barrier(0);
                multiply(w1, xf);
            }
        }
    }

    // fixed-order tree reduction of the NW partial tiles into wave 0
    if constexpr (NW > 1) {
        float* red = reinterpret_cast<float*>(lds);
        __syncthreads();  // every wave is done with its slab
#pragma unroll
        for (int s = 1; s < NW; s <<= 1) {
            if ((wave & (2 * s - 1)) == s) {
                float* dst = red + (wave / (2 * s)) * (MT * 8 * 64);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r) dst[((mt * 2 + b) * 4 + r) * 64 + lane] = acc[mt][b][r];
            }
            __syncthreads();
            if ((wave & (2 * s - 1)) == 0) {
                const float* src = red + (wave / (2 * s)) * (MT * 8 * 64);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][b][r] += src[((mt * 2 + b) * 4 + r) * 64 + lane];
            }
            __syncthreads();
        }
    }
    if (wave != 0) return;
    gemm_epilogue<DT, MT, EPI>(g, tm, tile, mg, lane, acc);
}

}  // namespace vs
