// LDS-tiled MFMA GEMM for steps of more than 64 rows, such as a prompt chunk
// (gfx950).
//
// C[m][n] = sum_k X[m][k] * W[n][k] with the epilogues of the skinny tile GEMM
// ([KV Cache] section 06, chunked prefill: a chunk of prompt rows runs through
// the same weight products as the decode rows of its step). At these sizes the
// product is a real dense contraction, so the work is tiled for the matrix
// cores: a workgroup of 4 waves owns two tiles of the skinny GEMM's feature
// tiling (16 or 32 features each, paired the way its epilogue needs: rotary
// halves, gate and up) and 128 rows; every 64-element step of the reduction,
// both operands go global -> registers -> LDS with 16-byte loads (double
// buffered, one barrier a step), and each wave multiplies its tile against 64
// rows with MFMA 16x16x32 from LDS fragments. Rows and features past the ends
// read in-bounds data whose results are never stored.
#pragma once

#include "common.h"
#include "gemm.h"

namespace vs {

constexpr int kBigRows = 128;  // rows per workgroup (two waves of 64)
constexpr int kBigK = 64;      // reduction elements per LDS stage
constexpr int kBigLd = kBigK + 8;  // LDS row stride in elements (16 bytes of padding against bank conflicts)

template <int DT, int EPI>
__global__ void __launch_bounds__(256) gemm_big_kernel(GemmArgs g) {
    constexpr bool SB = EPI == EPI_RESID || EPI == EPI_LOGITS;
    constexpr int NB = SB ? 1 : 2;    // 16-feature blocks per tile
    constexpr int AR = 2 * NB * 16;   // weight rows staged per step (two tiles)
    constexpr int CH = kBigK / 8;     // 16-byte chunks per staged row
    constexpr int A_PER = AR * CH / 256, B_PER = kBigRows * CH / 256;  // chunks per thread
    __shared__ __align__(16) uint16_t lA[2][AR * kBigLd];
    __shared__ __align__(16) uint16_t lB[2][kBigRows * kBigLd];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave & 1, wc = wave >> 1;  // row half, tile column
    const int m0 = blockIdx.x * kBigRows;     // row block (fastest: the row blocks of a tile share its weights)
    const int t0 = blockIdx.y * 2;
    const int last_tile = g.n_tiles - 1;
    const TileMap tm0 = tile_map<EPI>(g, min(t0, last_tile));
    const TileMap tm1 = tile_map<EPI>(g, min(t0 + 1, last_tile));

    // this thread's staging chunks: weight rows (tile column, block, row) and batch rows
    const uint16_t* asrc[A_PER];
    int adst[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int c = tid + 256 * i;
        const int r = c / CH, q = c % CH;
        const int col = r / (16 * NB), blk = (r / 16) % NB, ri = r % 16;
        // select fields, not a reference to one of the two maps (that would put them in scratch memory)
        const int rowA = col ? tm1.rowA : tm0.rowA, rowB = col ? tm1.rowB : tm0.rowB;
        const int nrows = col ? tm1.nrows : tm0.nrows;
        const void* wa = col ? tm1.w : tm0.w;
        const void* wbp = col ? tm1.wb : tm0.wb;
        int row = (blk ? rowB : rowA) + ri;
        if (row >= nrows) row = 0;
        asrc[i] = reinterpret_cast<const uint16_t*>(blk ? wbp : wa) + (long)row * g.K + 8 * q;
        adst[i] = r * kBigLd + 8 * q;
    }
    const uint16_t* bsrc[B_PER];
    int bdst[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int c = tid + 256 * i;
        const int r = c / CH, q = c % CH;
        const int m = m0 + r < g.M ? m0 + r : 0;
        bsrc[i] = reinterpret_cast<const uint16_t*>(g.act) + (long)m * g.act_ld + 8 * q;
        bdst[i] = r * kBigLd + 8 * q;
    }
    // staged chunks as native vectors (an array of the HIP vector struct ends up in scratch memory)
    u32x4_t ra[A_PER], rb[B_PER];
    auto fetch = [&](int kb) {
        const long ko = (long)kb * kBigK;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(asrc[i] + ko);
#pragma unroll
        for (int i = 0; i < B_PER; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(bsrc[i] + ko);
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) *reinterpret_cast<u32x4_t*>(&lA[buf][adst[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PER; ++i) *reinterpret_cast<u32x4_t*>(&lB[buf][bdst[i]]) = rb[i];
    };

    float4_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i][0] = (float4_t){0.f, 0.f, 0.f, 0.f};
        acc[i][1] = acc[i][0];
    }
    const int l16 = lane & 15, kq = lane >> 4;
    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < kBigK / 32; ++s) {
            const int ko = s * 32 + kq * 8;
            Frag<DT> fa[NB], fb[4];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                fa[b].a = *reinterpret_cast<const uint4*>(&lA[buf][((wc * NB + b) * 16 + l16) * kBigLd + ko]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fb[i].a = *reinterpret_cast<const uint4*>(&lB[buf][(wr * 64 + i * 16 + l16) * kBigLd + ko]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[i][b] = frag_mma<DT>(fa[b], fb[i], acc[i][b]);
        }
    };

    const int nkb = g.K / kBigK;
    fetch(0);
    stage(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        // the next stage's loads are in flight while this one is multiplied (the last step refetches
        // its own data into the buffer nobody reads any more: no branch keeps the operands in registers)
        fetch(min(kb + 1, nkb - 1));
        compute(kb & 1);
        stage((kb + 1) & 1);
        __syncthreads();
    }

    const int t = t0 + wc;
    if (t > last_tile) return;
    if (wc == 0) gemm_epilogue<DT, 4, EPI>(g, tm0, t, (m0 + 64 * wr) / 64, lane, acc);
    else gemm_epilogue<DT, 4, EPI>(g, tm1, t, (m0 + 64 * wr) / 64, lane, acc);
}

}  // namespace vs
