// Pipelined MFMA GEMM for steps of more than 64 rows, such as a prompt chunk
// (gfx950).
//
// C[n][m] = sum_k W[n][k] X[m][k] with the epilogues of the skinny tile GEMM
// ([KV Cache] section 06, chunked prefill: the rows of a prompt chunk go
// through the same weight products as the decode rows of their step; at
// hundreds of rows the product is a dense contraction and the matrix cores
// set its pace). A workgroup of sixteen waves owns 256 weight rows x 128 batch
// rows; each wave multiplies 32 weight rows (two 16-row blocks) by 64 batch
// rows (four 16-row tiles) with MFMA 16x16x32, 8 accumulators of four floats.
// Four waves share each SIMD, so one wave's LDS and barrier waits are covered
// by the others' matrix work. Measured on the 576-row 7B step (the four
// products per step by dispatch events, the residual products' slice sums
// included): four waves of 128 x 64, 11.97 ms (the matrix cores busy about
// 38 % of the time; a probe on LDS data alone reached 43 % at one wave per
// SIMD); eight waves of 64 x 64, 10.86 ms; sixteen waves of 64 x 32 or
// 32 x 64, 10.58 and 10.56 ms. The q/k/v and gate/up products pair their
// blocks the way their epilogues need (rotary halves; the gate and up rows of
// the same features), so a wave holds one whole output tile of those
// products, two of the others.
//
// Both operands go straight from global memory into LDS (gfx950's LDS-direct
// loads, 16 bytes a lane) in 64-element steps of the reduction, through a ring
// of three LDS stages: the loads of step k + 2 are issued while step k is
// multiplied, and no register holds staged data, so the register file keeps
// the accumulators and fragments. One such load writes 1 KB of LDS in lane
// order (eight rows of 128 bytes), so rows cannot be padded against bank
// conflicts; instead the 16-byte chunks of a row are stored XOR-swizzled
// (chunk q of row r in slot q ^ ((r / 2) % 8)), which puts the sixteen rows of
// a fragment read on sixteen different bank groups. The loads are issued in
// inline assembly, and the waits for them are explicit: the compiler, seeing
// the builtin form, waits for every outstanding load before any LDS read,
// which would leave nothing in flight. (Measured on this part: staging one
// step ahead through registers left the matrix cores idle most of the time,
// and three register stages did not fit beside the accumulators and
// fragments; LDS read bandwidth is not the limit at these wave tiles.)
//
// Workgroups are placed for the chip's eight L2 slices: workgroup L runs on
// XCD L % 8, and the workgroups that share a block of weight rows (all row
// blocks of one block of features, and one slice of the reduction) get
// numbers with the same remainder, so their weights come through one L2.
//
// The residual products (4096 output features at 7B widths: too few blocks to
// fill the chip) may split the reduction into slices; each slice then writes
// fp32 partial sums part[slice][m][n], which the residual + RMSNorm reduction
// adds in slice order (so results do not depend on timing).
#pragma once

#include "common.h"
#include "gemm.h"

namespace vs {

constexpr int kTileK = 64;                 // reduction elements per stage
constexpr int kTileRowB = kTileK * 2;      // bytes of one staged row
constexpr int kTileStages = 3;             // LDS stages (two in flight while one is multiplied)
constexpr int kTileWN = 8, kTileWM = 2;    // waves along the features and along the batch rows
constexpr int kTileWaves = kTileWN * kTileWM;
constexpr int kTileTN = 2;                 // 16-row weight blocks per wave
constexpr int kTileTM = 4;                 // 16-row batch tiles per wave
constexpr int kTileRowsN = kTileWN * kTileTN * 16;  // weight rows per workgroup
constexpr int kTileRowsM = kTileWM * kTileTM * 16;  // batch rows per workgroup

// epilogue tiles (the skinny GEMM's tiling) per workgroup
__host__ __device__ constexpr int tile_tiles_per_wg(int EPI) {
    return (EPI == EPI_QKV || EPI == EPI_SWIGLU) ? kTileWN * kTileTN / 2 : kTileWN * kTileTN;
}
// workgroups of a launch: 8 x ceil(column blocks / 8) x row blocks (the padding ones return at once)
__host__ __device__ inline int tile_grid(int n_tiles, int EPI, int n_slices, int M) {
    const int tpg = tile_tiles_per_wg(EPI);
    const int cols = ((n_tiles + tpg - 1) / tpg) * n_slices;
    return 8 * ((cols + 7) / 8) * ((M + kTileRowsM - 1) / kTileRowsM);
}

// n_slices > 1 (EPI_RESID only): slice s of the reduction writes its sums to part[s][m][n] (n < g.n0)
// instead of adding them to x.
template <int DT, int EPI>
__global__ void __launch_bounds__(kTileWaves * 64, 1) gemm_tile_kernel(GemmArgs g, int n_slices, float* part) {
    constexpr bool PAIRED = EPI == EPI_QKV || EPI == EPI_SWIGLU;
    constexpr int TPG = tile_tiles_per_wg(EPI);
    constexpr int BN = kTileRowsN, BM = kTileRowsM;
    constexpr int A_PER = BN / 8 / kTileWaves, B_PER = BM / 8 / kTileWaves;  // LDS-direct loads (8 rows each) per wave and stage
    static_assert(A_PER % 2 == 0 && B_PER >= 1, "whole 16-row weight blocks and 8-row batch groups per wave");
    constexpr int STAGE_B = (BN + BM) * kTileRowB;          // bytes of one stage: weight rows, then batch rows
    __shared__ __align__(1024) unsigned char lds[kTileStages * STAGE_B];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % kTileWN, wm = wave / kTileWN;  // this wave's weight block and row block

    // workgroup -> (column block, row block): column block c = 8 (r / row blocks) + L % 8
    const int L = blockIdx.x, r = L >> 3;
    const int mblk = (g.M + BM - 1) / BM;
    const int c = 8 * (r / mblk) + (L & 7), im = r % mblk;
    const int nblk = (g.n_tiles + TPG - 1) / TPG;
    if (c >= nblk * n_slices) return;
    const int nb = c / n_slices, sl = c - nb * n_slices;
    const int m0 = im * BM, t0 = nb * TPG;
    const int last_tile = g.n_tiles - 1;
    const int nk_all = g.K / kTileK;
    const int kb0 = (int)(((long)sl * nk_all) / n_slices), nkb = (int)(((long)(sl + 1) * nk_all) / n_slices) - kb0;

    // Loads. Row group j (rows 8 j .. 8 j + 7 of an operand tile) is one load: lane l fills LDS row
    // 8 j + l / 8, slot l % 8, with chunk (l % 8) ^ ((4 j + l / 16) % 8) of that row. Wave w loads weight
    // groups A_PER w .. A_PER w + A_PER - 1 (whole 16-row blocks: block bases are wave-uniform) and batch
    // groups B_PER w .. B_PER w + B_PER - 1. Batch rows past M read row M - 1 (never stored); weight rows are whole 16-row
    // blocks of valid rows (the host checks the segment sizes).
    const int lr = lane >> 3, ls = lane & 7;
    const char* abase[A_PER / 2];  // per 16-row block of the wave
#pragma unroll
    for (int i = 0; i < A_PER / 2; ++i) {
        const int blk = (A_PER / 2) * wave + i;
        const int t = min(t0 + (PAIRED ? blk / 2 : blk), last_tile);
        const TileMap tm = tile_map<EPI>(g, t);
        const bool second = PAIRED && (blk & 1);
        const int row0 = second ? tm.rowB : tm.rowA;
        const char* bp =
            reinterpret_cast<const char*>(second ? tm.wb : tm.w) + ((long)row0 * g.K + (long)kb0 * kTileK) * 2;
        // wave-uniform in scalar registers, both halves of the address (the builtin moves 32 bits)
        const unsigned long long u = reinterpret_cast<unsigned long long>(bp);
        const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u), hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
        abase[i] = reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
    }
    // lane offsets inside a block: the block's first group (rows 0..7) and its second (rows 8..15)
    const uint32_t aoff0 = (uint32_t)((lr * g.K + 8 * (ls ^ ((lane >> 4) & 7))) * 2);
    const uint32_t aoff1 = (uint32_t)(((8 + lr) * g.K + 8 * (ls ^ ((4 + (lane >> 4)) & 7))) * 2);
    const char* act = reinterpret_cast<const char*>(g.act) + (long)kb0 * kTileK * 2;
    uint32_t boff[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int j = B_PER * wave + i;
        const int m = min(m0 + 8 * j + lr, g.M - 1);
        boff[i] = (uint32_t)((m * g.act_ld + 8 * (ls ^ ((4 * j + (lane >> 4)) & 7))) * 2);
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)lds);
    // One LDS-direct load: M0 holds the wave's LDS destination, lane l's 16 bytes land at M0 + 16 l.
    // The compiler keeps M0 for itself and warns about the clobber; in these kernels it uses M0 for
    // nothing else (every M0 write in their code is the one below, right before its load).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    auto dma = [](const char* sbase, uint32_t voff, uint32_t ldsaddr) {
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(ldsaddr), "v"(voff), "s"(sbase)
                     : "memory", "m0");
    };
#pragma clang diagnostic pop
    // step j of the slice into stage buffer sb (past the end: the last step again, never multiplied);
    // A_PER + B_PER loads per wave
    auto issue = [&](int j, int sb) {
        const long ko = (long)min(j, nkb - 1) * kTileRowB;
        const uint32_t base = lds0 + (uint32_t)(sb * STAGE_B);
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            dma(abase[i / 2] + ko, (i & 1) ? aoff1 : aoff0, base + (uint32_t)((A_PER * wave + i) * 1024));
#pragma unroll
        for (int i = 0; i < B_PER; ++i)
            dma(act + ko, boff[i], base + (uint32_t)(BN * kTileRowB + (B_PER * wave + i) * 1024));
    };

    float4_t acc[kTileTN][kTileTM];
#pragma unroll
    for (int b = 0; b < kTileTN; ++b)
#pragma unroll
        for (int i = 0; i < kTileTM; ++i) acc[b][i] = (float4_t){0.f, 0.f, 0.f, 0.f};
    const int l16 = lane & 15, kq = lane >> 4;
    // fragment reads: row 16 x + l16, chunk 4 s + kq, stored in slot (4 s + kq) ^ ((l16 / 2) % 8)
    const int sw = (l16 >> 1) & 7;
    const int frow = l16 * kTileRowB;
    const int fslot0 = 16 * (kq ^ sw), fslot1 = 16 * ((4 + kq) ^ sw);
    auto compute = [&](int sb) {
        const unsigned char* stA = lds + sb * STAGE_B + (wn * kTileTN * 16) * kTileRowB + frow;
        const unsigned char* stB = lds + sb * STAGE_B + BN * kTileRowB + (wm * kTileTM * 16) * kTileRowB + frow;
#pragma unroll
        for (int s = 0; s < kTileK / 32; ++s) {
            const int fs = s ? fslot1 : fslot0;
            Frag<DT> fa[kTileTN], fb[kTileTM];
#pragma unroll
            for (int b = 0; b < kTileTN; ++b) fa[b].a = *reinterpret_cast<const uint4*>(stA + b * 16 * kTileRowB + fs);
#pragma unroll
            for (int i = 0; i < kTileTM; ++i) fb[i].a = *reinterpret_cast<const uint4*>(stB + i * 16 * kTileRowB + fs);
#pragma unroll
            for (int b = 0; b < kTileTN; ++b)
#pragma unroll
                for (int i = 0; i < kTileTM; ++i) acc[b][i] = frag_mma<DT>(fa[b], fb[i], acc[b][i]);
        }
    };

    // The ring: step k sits in stage buffer k % 3. Before step k is multiplied the wave waits until at
    // most one step's loads (A_PER + B_PER) are outstanding, i.e. its own loads of step k have landed, and the
    // barrier then covers every wave's; the same barrier frees the buffer of step k - 1, which takes
    // step k + 2.
    issue(0, 0);
    issue(1, 1);
    for (int k0 = 0; k0 < nkb; k0 += kTileStages) {
#pragma unroll
        for (int u = 0; u < kTileStages; ++u) {
            const int k = k0 + u;
            if (k >= nkb) break;
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(A_PER + B_PER) : "memory");
            __syncthreads();
            issue(k + 2, (u + 2) % kTileStages);
            compute(u);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the ring's last loads (past the end) have landed

    // ---- epilogues: the wave's output tiles ----
    const int mg = im * kTileWM + wm;  // row group of 16 kTileTM rows
    if (n_slices > 1) {
        if constexpr (EPI == EPI_RESID) {
            const int nl0 = kq * 4;
#pragma unroll
            for (int j = 0; j < kTileTN; ++j) {
                const int t = t0 + wn * kTileTN + j;
                if (t > last_tile) break;
                const int n = 16 * t + nl0;
#pragma unroll
                for (int i = 0; i < kTileTM; ++i) {
                    const int m = mg * 16 * kTileTM + i * 16 + l16;
                    if (m >= g.M) continue;
                    float* dst = part + ((long)sl * g.M + m) * g.n0 + n;
                    if (n + 3 < g.n0) {
                        *reinterpret_cast<float4_t*>(dst) = acc[j][i];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < g.n0) dst[e] = acc[j][i][e];
                    }
                }
            }
        }
        return;
    }
    constexpr int TPW = PAIRED ? kTileTN / 2 : kTileTN;  // output tiles per wave
    if constexpr (EPI == EPI_QKV) {
        // rotary + q / K/V stores ([KV Cache] section 03), as the skinny GEMM's epilogue computes them,
        // with every input requested before the first use: each row's K/V slot (row_kvoff, -1 for a row
        // without a valid page) and the (cos, sin) of the four rotary pairs a lane holds per tile and row
        const int half = g.head_dim / 2, nl0 = kq * 4;
        int mrow[kTileTM];
        long koff[kTileTM];
#pragma unroll
        for (int i = 0; i < kTileTM; ++i) {
            mrow[i] = mg * 16 * kTileTM + i * 16 + l16;
            koff[i] = g.row_kvoff[min(mrow[i], g.M - 1)];
        }
        TileMap tms[TPW];
        float4_t cs[TPW][kTileTM][2];  // (cos, sin) of pairs nl0 .. nl0 + 3: (c0 s0 c1 s1), (c2 s2 c3 s3)
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            tms[j] = tile_map<EPI>(g, min(t0 + wn * TPW + j, last_tile));
#pragma unroll
            for (int i = 0; i < kTileTM; ++i) {
                const float* p = g.rope_cs + ((long)min(mrow[i], g.M - 1) * half + 16 * tms[j].j + nl0) * 2;
                cs[j][i][0] = *reinterpret_cast<const float4_t*>(p);
                cs[j][i][1] = *reinterpret_cast<const float4_t*>(p + 4);
            }
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            if (t0 + wn * TPW + j > last_tile) break;
            const TileMap& tm = tms[j];
#pragma unroll
            for (int i = 0; i < kTileTM; ++i) {
                const int m = mrow[i];
                if (m >= g.M) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a = acc[2 * j][i][r], b = acc[2 * j + 1][i][r];
                    const int ip = 16 * tm.j + nl0 + r;  // rotary pair inside the head
                    float ra = a, rb = b;
                    if (tm.seg < 2) {
                        const float c = cs[j][i][r >> 1][2 * (r & 1)], sn = cs[j][i][r >> 1][2 * (r & 1) + 1];
                        ra = a * c - b * sn;
                        rb = b * c + a * sn;
                    }
                    if (tm.seg == 0) {
                        const long o = (long)m * (g.n_heads * g.head_dim) + (long)tm.head * g.head_dim + ip;
                        store_round<DT>(g.q_out, o, ra);
                        store_round<DT>(g.q_out, o + half, rb);
                    } else if (koff[i] >= 0) {
                        const long o = koff[i] + (long)g.layer * g.layer_elems +
                                       ((long)(tm.seg - 1) * g.n_kv_heads + tm.head) * g.page_tokens * g.head_dim + ip;
                        store_kv<DT>(g.kv_base, o, ra, g.kv_dt);
                        store_kv<DT>(g.kv_base, o + half, rb, g.kv_dt);
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const int t = t0 + wn * TPW + j;
        if (t > last_tile) break;
        float4_t e[kTileTM][2];
#pragma unroll
        for (int i = 0; i < kTileTM; ++i) {
            e[i][0] = acc[PAIRED ? 2 * j : j][i];
            e[i][1] = PAIRED ? acc[2 * j + 1][i] : (float4_t){0.f, 0.f, 0.f, 0.f};
        }
        gemm_epilogue<DT, kTileTM, EPI>(g, tile_map<EPI>(g, t), t, mg, lane, e);
    }
}

}  // namespace vs
