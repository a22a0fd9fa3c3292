// Full-reduction strip GEMM for the q/k/v and gate/up products of steps with
// 8..64 rows, and for the residual products of 8..16 rows (gfx950), with their
// epilogues in the same kernel.
//
// C[n][m] = sum_k W[n][k] X[m][k] ([KV Cache] section 02: every row passing
// through a weight matrix shares one read of it). The output features are cut
// into units of 16 weight rows chosen so that the values an epilogue combines
// share a tile: for q/k/v, 8 rotary pairs (i, i + head_dim/2) of one head
// ([KV Cache] section 03: q and k are rotated before k is cached); for
// gate/up, 8 gate rows and the 8 up rows of the same features. Tile row r < 8
// holds the first member of pair r, row r + 8 the second.
//
// One workgroup of 4 waves per CU (one wave per SIMD, so each wave may hold
// up to 512 registers) owns U consecutive units and the whole reduction axis,
// so no partial sums leave the CU and no second kernel is needed. The waves
// split the reduction axis into 4 ranges of 128-element blocks; each wave
// streams, block by block, the U chunks (16 rows x 256 bytes) of its range,
// four rows x 256 bytes per load, through a wave-private LDS slab that is read
// back as MFMA A fragments (16x16x32), up to five chunks ahead of the multiply
// (20 KB in flight per wave). The batch rows X come straight from L2 as B
// fragments, one block ahead, and every weight chunk of the block reuses
// them: the wave reads its range of X once. At the end the waves' partial
// tiles are summed through LDS in wave order (fixed, so results do not depend
// on timing) and the epilogue runs on the sums.
#pragma once

#include "common.h"
#include "gemm.h"

namespace vs {

constexpr int kStripWaves = 4;
constexpr int kStripRowB = 256 + 16;          // slab row stride (bytes): fragment rows on different banks
constexpr int kStripSlab = 16 * kStripRowB;   // one wave's slab

// Units per workgroup (the accumulators take 4 MT registers per unit), and the unit counts the two
// products use (7B widths: 768 q/k/v units -> 256 workgroups; 1376 gate/up units -> 230 workgroups of
// 6; the 8B-GQA widths' 1792 gate/up units -> 256 workgroups of 7).
__host__ __device__ constexpr int strip_max_units(int MT) { return 7; }
constexpr int kStripUnitsQkv = 3;
constexpr int kStripUnitsQkvNarrow = 2;
constexpr int kStripUnitsGu = 6;
constexpr int kStripUnitsGuWide = 7;

// Wave-uniform bases of a unit's two half-tiles (rows r < 8 and r >= 8), in elements.
struct StripUnit {
    const uint16_t* h0;
    const uint16_t* h1;
};

template <int EPI>
__device__ __forceinline__ StripUnit strip_unit(const GemmArgs& g, int u) {
    StripUnit s;
    if constexpr (EPI == EPI_SWIGLU) {
        s.h0 = reinterpret_cast<const uint16_t*>(g.w0) + (long)8 * u * g.K;
        s.h1 = reinterpret_cast<const uint16_t*>(g.w1) + (long)8 * u * g.K;
    } else {
        const int uph = g.head_dim / 16;  // units per head
        const int hh = u / uph, jj = u - hh * uph;
        const uint16_t* seg;
        int head;
        if (hh < g.n_heads) {
            seg = reinterpret_cast<const uint16_t*>(g.w0);
            head = hh;
        } else if (hh < g.n_heads + g.n_kv_heads) {
            seg = reinterpret_cast<const uint16_t*>(g.w1);
            head = hh - g.n_heads;
        } else {
            seg = reinterpret_cast<const uint16_t*>(g.w2);
            head = hh - g.n_heads - g.n_kv_heads;
        }
        const long r0 = (long)head * g.head_dim + 8 * jj;
        s.h0 = seg + r0 * g.K;
        s.h1 = seg + (r0 + g.head_dim / 2) * g.K;
    }
    return s;
}

// One chunk of a wave's stream: 16 weight rows x 128 elements, as four 16-byte loads per lane
// (load i: tile rows 4 i .. 4 i + 3, lane l: row 4 i + l / 16, bytes 16 (l % 16) ..), with the mask
// that zeroes chunks past the wave's range.
struct StripChunk {
    uint4 v[4];
    uint32_t keep;
};

template <int DT, int MT, int EPI, int U>
__global__ void __launch_bounds__(kStripWaves * 64, 1) gemm_strip_kernel(GemmArgs g) {
    static_assert(U == 2 || U == 3 || U == 6 || U == 7, "the chunk ring is laid out for 2, 3, 6 or 7 units");
    typedef const __attribute__((address_space(1))) u32x4_t* gptr;
    const int K = g.K, M = g.M;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KB = K / 128;
    const int kb0 = (wave * KB) / kStripWaves, kb1 = ((wave + 1) * KB) / kStripWaves;
    const int nb = kb1 - kb0;  // blocks of this wave (0 when K is short)
    const int u_first = blockIdx.x * U;

    // this lane's byte offsets inside a half-tile: rows 4 (i & 1) + lane / 16, bytes 16 (lane % 16)
    const uint32_t loff0 = (uint32_t)((lane >> 4) * K * 2 + 16 * (lane & 15));
    const uint32_t loff1 = loff0 + (uint32_t)(4 * K * 2);
    StripUnit units[U];
#pragma unroll
    for (int j = 0; j < U; ++j) units[j] = strip_unit<EPI>(g, min(u_first + j, g.n_tiles - 1));

    // chunk of block b (of the wave's range) and unit j; past the range: masked, and read from the
    // start of the activations instead (a valid, L2-resident address: M >= 8 rows of at least K
    // elements cover the eight rows' offsets), so it costs no HBM traffic
    const char* dummy = reinterpret_cast<const char*>(g.act);
    auto load_chunk = [&](StripChunk& ck, int b, int j) {
        const bool live = b < nb;
        const char* h0 = live ? reinterpret_cast<const char*>(units[j].h0) + (long)(kb0 + b) * 256 : dummy;
        const char* h1 = live ? reinterpret_cast<const char*>(units[j].h1) + (long)(kb0 + b) * 256 : dummy;
        ck.v[0] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(h0 + loff0)));
        ck.v[1] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(h0 + loff1)));
        ck.v[2] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(h1 + loff0)));
        ck.v[3] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(h1 + loff1)));
        ck.keep = live ? 0xFFFFFFFFu : 0u;
    };
    // X fragments of one block: step s (32 elements), row tile mt; rows past M read row M - 1
    const uint16_t* A = reinterpret_cast<const uint16_t*>(g.act);
    auto load_x = [&](uint4 (&xf)[4][MT], int b) {
        const int kb = b < nb ? kb0 + b : (nb > 0 ? kb1 - 1 : 0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = min(16 * mt + (lane & 15), M - 1);
            const uint16_t* p = A + (long)m * g.act_ld + (long)kb * 128 + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < 4; ++s) xf[s][mt] = *reinterpret_cast<const uint4*>(p + 32 * s);
        }
    };

    constexpr int kSlabs = kStripWaves * kStripSlab, kRed = kStripWaves * U * MT * 1024;
    __shared__ __align__(16) unsigned char lds[kSlabs > kRed ? kSlabs : kRed];
    unsigned char* slab = lds + wave * kStripSlab;
    float4_t acc[U][MT];
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (float4_t){0.f, 0.f, 0.f, 0.f};

    auto consume = [&](const StripChunk& ck, const uint4 (&xf)[4][MT], int j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = ck.v[i];
            const uint32_t kp = ck.keep;
            *reinterpret_cast<uint4*>(slab + (4 * i + (lane >> 4)) * kStripRowB + 16 * (lane & 15)) =
                make_uint4(v.x & kp, v.y & kp, v.z & kp, v.w & kp);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            Frag<DT> fa, fx;
            fa.a = *reinterpret_cast<const uint4*>(slab + (lane & 15) * kStripRowB + 64 * s + 16 * (lane >> 4));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                fx.a = xf[s][mt];
                acc[j][mt] = frag_mma<DT>(fa, fx, acc[j][mt]);
            }
        }
    };

    // Epilogue inputs (q/k/v: each item's rotary cos / sin and its row's K/V slot), requested before the
    // stream: requested after it, they would wait behind every weight load in flight.
    constexpr int NT = kStripWaves * 64;
    constexpr int n_items = U * MT * 32 * 4;
    constexpr int NIT = (n_items + NT - 1) / NT;
    float2 rcs[NIT];
    long koff[NIT];
    if constexpr (EPI == EPI_QKV) {
        const int uph = g.head_dim / 16, half = g.head_dim / 2;
#pragma unroll
        for (int k = 0; k < NIT; ++k) {
            const int it = min((int)threadIdx.x + k * NT, n_items - 1);
            const int e = it & 3, l = (it >> 2) & 31, mt = (it >> 7) % MT, j = (it >> 7) / MT;
            const int m = min(16 * mt + (l & 15), M - 1);
            const int u = min(u_first + j, g.n_tiles - 1);
            const int i = 8 * (u % uph) + 4 * (l >> 4) + e;
            rcs[k] = *reinterpret_cast<const float2*>(g.rope_cs + ((long)m * half + i) * 2);
            koff[k] = g.row_kvoff[m];
        }
    }

    // The stream: chunk (b, j) is number c = b U + j and sits in ring slot c % R; the loads run AHEAD
    // chunks ahead (12 or 20 KB in flight per wave). Blocks go in pairs, the first of a pair multiplied
    // with X buffer xbuf[0], the second with xbuf[1]. The X of block b + 1 is requested just before chunk
    // (b + 1, 0) is, at chunk (b, U - AHEAD): the wait for it then covers only chunks needed before it
    // (loads retire in order), and its buffer is free by then because AHEAD <= U. A pair of blocks
    // fills the ring a whole number of times, so every slot index below is a constant. (Measured on
    // 7B widths: three X buffers with a deeper ring, or A fragments loaded straight from memory without
    // the slab, both ran slower.)
    constexpr int R = U == 7 ? 7 : U == 2 ? 4 : 6;  // a pair of blocks (2 U chunks) fills the ring a whole number of times
    constexpr int AHEAD = R - 1 < U ? R - 1 : U;
    constexpr int XJ = U - AHEAD;
    StripChunk ring[R];
    uint4 xbuf[2][4][MT];
    load_x(xbuf[0], 0);
#pragma unroll
    for (int c = 0; c < AHEAD; ++c) load_chunk(ring[c], c / U, c % U);
    const int np = nb > 0 ? (nb + 1) / 2 : 1;  // pairs of blocks walked
    int b = 0;
    for (int pi = 0; pi + 1 < np; ++pi, b += 2) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int c = t * U + j + AHEAD;  // chunk to request, counted from the pair's first
                if (j == XJ) load_x(xbuf[1 - t], b + t + 1);
                load_chunk(ring[c % R], b + c / U, c % U);
                __builtin_amdgcn_sched_barrier(0);
                consume(ring[(t * U + j) % R], xbuf[t], j);
            }
        }
    }
    // the last pair: no requests past the stream
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int c = t * U + j + AHEAD;
            if (t == 0 && j == XJ) load_x(xbuf[1], b + 1);
            if (c < 2 * U) load_chunk(ring[c % R], b + c / U, c % U);
            __builtin_amdgcn_sched_barrier(0);
            consume(ring[(t * U + j) % R], xbuf[t], j);
        }
    }

    // ---- the waves' partial tiles, summed in wave order ----
    __syncthreads();  // every wave is done with its slab
    float4_t* red = reinterpret_cast<float4_t*>(lds);  // [wave][unit][mt][lane]
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[((wave * U + j) * MT + mt) * 64 + lane] = acc[j][mt];
    __syncthreads();
    // item (unit j, tile mt, lane l < 32, element e): pair p = 4 (l / 16) + e of the unit, batch row
    // 16 mt + l % 16; its two members sit in lanes l and l + 32
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int it = threadIdx.x + k * NT;
        const int e = it & 3, l = (it >> 2) & 31, mt = (it >> 7) % MT, j = (it >> 7) / MT;
        const int m = 16 * mt + (l & 15);
        const int u = u_first + j;
        if (it >= n_items || m >= M || u >= g.n_tiles) continue;
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int w = 0; w < kStripWaves; ++w) {
            v0 += red[((w * U + j) * MT + mt) * 64 + l][e];
            v1 += red[((w * U + j) * MT + mt) * 64 + l + 32][e];
        }
        const int p = 4 * (l >> 4) + e;  // 0..7
        if constexpr (EPI == EPI_SWIGLU) {
            const int f = 8 * u + p;
            const float s = v0 / (1.0f + expf(-v0));
            store_round<DT>(g.h_out, (long)m * g.h_ld + f, s * v1);
        } else {
            const int uph = g.head_dim / 16, half = g.head_dim / 2;
            const int hh = u / uph, i = 8 * (u - hh * uph) + p;
            const int seg = hh < g.n_heads ? 0 : hh < g.n_heads + g.n_kv_heads ? 1 : 2;
            const int head = seg == 0 ? hh : seg == 1 ? hh - g.n_heads : hh - g.n_heads - g.n_kv_heads;
            float ra = v0, rb = v1;
            if (seg < 2) {
                ra = v0 * rcs[k].x - v1 * rcs[k].y;
                rb = v1 * rcs[k].x + v0 * rcs[k].y;
            }
            if (seg == 0) {
                const long o = (long)m * (g.n_heads * g.head_dim) + (long)head * g.head_dim + i;
                store_round<DT>(g.q_out, o, ra);
                store_round<DT>(g.q_out, o + half, rb);
            } else if (koff[k] >= 0) {
                const long o = koff[k] + (long)g.layer * g.layer_elems +
                               ((long)(seg - 1) * g.n_kv_heads + head) * g.page_tokens * g.head_dim + i;
                store_kv<DT>(g.kv_base, o, ra, g.kv_dt);
                store_kv<DT>(g.kv_base, o + half, rb, g.kv_dt);
            }
        }
    }
}

// The residual products (attention output, MLP down) of 8..16-row steps: one unit of 16 output
// features per workgroup (at 7B widths 4096 features make one unit per CU), the same wave split of the
// reduction axis and slab. With a single unit the X block of a chunk serves only that chunk, so each
// chunk carries its own X fragments and the ring of R chunks (weights and X) runs R - 1 chunks ahead.
// The epilogue adds the 16 x M sums to the residual: x[m][16 u + r] += C[r][m].
// Every CU reads all of X here (M K 2 bytes against its 32 K bytes of weights), so past 16 rows X
// outweighs the weights: measured at 7B widths (fp16, with the RMSNorm launch that follows), 8 rows:
// 11.6 / 22.0 us (O / down) against 13.4 / 26.8 us for split-K + fused norm; 32 rows: 17.7 / 33.9
// against 15.4 / 32.6; 40 rows: 21.4 / 40.3 against 16.6 / 29.9.
template <int DT, int MT>
__global__ void __launch_bounds__(kStripWaves * 64, 1) gemm_strip_resid_kernel(GemmArgs g) {
    typedef const __attribute__((address_space(1))) u32x4_t* gptr;
    constexpr int R = 5;
    const int K = g.K, M = g.M;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KB = K / 128;
    const int kb0 = (wave * KB) / kStripWaves, kb1 = ((wave + 1) * KB) / kStripWaves;
    const int nb = kb1 - kb0;
    const int u = blockIdx.x;
    const uint32_t loff0 = (uint32_t)((lane >> 4) * K * 2 + 16 * (lane & 15));
    const uint32_t loff1 = loff0 + (uint32_t)(4 * K * 2);
    const char* h0 = reinterpret_cast<const char*>(g.w0) + (long)16 * u * K * 2;
    const char* h1 = h0 + (long)8 * K * 2;
    const char* dummy = reinterpret_cast<const char*>(g.act);
    const uint16_t* A = reinterpret_cast<const uint16_t*>(g.act);
    struct Chunk {
        uint4 v[4];
        uint4 x[4][MT];
        uint32_t keep;
    };
    // chunk b of the wave's range: 16 rows x 128 elements of weights and the X fragments of the same
    // 128 elements; past the range the weights come from the activations and are masked
    auto load = [&](Chunk& ck, int b) {
        const bool live = b < nb;
        const char* a0 = live ? h0 + (long)(kb0 + b) * 256 : dummy;
        const char* a1 = live ? h1 + (long)(kb0 + b) * 256 : dummy;
        ck.v[0] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(a0 + loff0)));
        ck.v[1] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(a0 + loff1)));
        ck.v[2] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(a1 + loff0)));
        ck.v[3] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((gptr)(a1 + loff1)));
        ck.keep = live ? 0xFFFFFFFFu : 0u;
        const int kb = live ? kb0 + b : (nb > 0 ? kb1 - 1 : 0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = min(16 * mt + (lane & 15), M - 1);
            const uint16_t* p = A + (long)m * g.act_ld + (long)kb * 128 + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < 4; ++s) ck.x[s][mt] = *reinterpret_cast<const uint4*>(p + 32 * s);
        }
    };
    constexpr int kSlabs = kStripWaves * kStripSlab, kRed = kStripWaves * MT * 1024;
    __shared__ __align__(16) unsigned char lds[kSlabs > kRed ? kSlabs : kRed];
    unsigned char* slab = lds + wave * kStripSlab;
    float4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const Chunk& ck) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = ck.v[i];
            const uint32_t kp = ck.keep;
            *reinterpret_cast<uint4*>(slab + (4 * i + (lane >> 4)) * kStripRowB + 16 * (lane & 15)) =
                make_uint4(v.x & kp, v.y & kp, v.z & kp, v.w & kp);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            Frag<DT> fa, fx;
            fa.a = *reinterpret_cast<const uint4*>(slab + (lane & 15) * kStripRowB + 64 * s + 16 * (lane >> 4));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                fx.a = ck.x[s][mt];
                acc[mt] = frag_mma<DT>(fa, fx, acc[mt]);
            }
        }
    };
    // the residual values the epilogue adds to, requested before the stream (thread t: rows pair
    // p = 4 (l / 16) + e of tile mt, l < 32, as in the epilogue below)
    constexpr int NT = kStripWaves * 64;
    constexpr int n_items = MT * 32 * 4;
    constexpr int NIT = (n_items + NT - 1) / NT;
    float2 xr[NIT];
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int it = min((int)threadIdx.x + k * NT, n_items - 1);
        const int e = it & 3, l = (it >> 2) & 31, mt = it >> 7;
        const int m = min(16 * mt + (l & 15), M - 1), f = 16 * u + 4 * (l >> 4) + e;
        xr[k] = make_float2(g.x[(long)m * g.x_ld + f], g.x[(long)m * g.x_ld + f + 8]);
    }
    // the stream: slot of chunk c is c % R (the loop body is R chunks); the loads run R - 1 ahead
    Chunk ring[R];
#pragma unroll
    for (int c = 0; c < R - 1; ++c) load(ring[c], c);
    for (int c0 = 0; c0 < nb; c0 += R) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
            if (c0 + t >= nb) break;
            load(ring[(t + R - 1) % R], c0 + t + R - 1);
            __builtin_amdgcn_sched_barrier(0);
            consume(ring[t]);
        }
    }
    __syncthreads();
    float4_t* red = reinterpret_cast<float4_t*>(lds);  // [wave][mt][lane]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int it = threadIdx.x + k * NT;
        const int e = it & 3, l = (it >> 2) & 31, mt = it >> 7;
        const int m = 16 * mt + (l & 15);
        if (it >= n_items || m >= M) continue;
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int w = 0; w < kStripWaves; ++w) {
            v0 += red[(w * MT + mt) * 64 + l][e];
            v1 += red[(w * MT + mt) * 64 + l + 32][e];
        }
        const int f = 16 * u + 4 * (l >> 4) + e;
        g.x[(long)m * g.x_ld + f] = xr[k].x + v0;
        g.x[(long)m * g.x_ld + f + 8] = xr[k].y + v1;
    }
}

}  // namespace vs
