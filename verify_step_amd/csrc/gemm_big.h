// LDS-tiled MFMA GEMM for steps of more than 64 rows, such as a prompt chunk
// (gfx950).
//
// C[m][n] = sum_k X[m][k] * W[n][k] with the epilogues of the skinny tile GEMM
// ([KV Cache] section 06, chunked prefill: a chunk of prompt rows runs through
// the same weight products as the decode rows of its step). At these sizes the
// product is a real dense contraction, so the work is tiled for the matrix
// cores: a workgroup owns T tiles of the skinny GEMM's feature tiling and 128
// rows, one wave per (tile, group of 128 / RG rows): eight tiles of 32 weight
// rows (paired the way the epilogue needs: rotary halves, gate and up), one
// row group; or, for the residual and logit products, two tiles of 16 rows,
// two row groups (more, smaller workgroups: at 4096 features larger ones left
// the CUs unevenly loaded); every 64-element step of the reduction,
// both operands go global -> registers -> LDS with 16-byte loads (double
// buffered, one barrier a step), and each wave multiplies its tile against its
// rows with MFMA 16x16x32 from LDS fragments. Each weight byte then serves 128
// rows and each activation byte 32 or 256 weight rows from LDS (the
// activations are what the many paired tiles re-read from L2). Rows and
// features past the ends read in-bounds data whose results are never stored.
#pragma once

#include "common.h"
#include "gemm.h"

namespace vs {

constexpr int kBigRows = 128;  // rows per workgroup
// feature tiles per workgroup and row groups per tile (waves = tiles x row groups)
__host__ __device__ constexpr int big_tiles(int EPI) { return EPI == EPI_RESID || EPI == EPI_LOGITS ? 2 : 8; }
__host__ __device__ constexpr int big_rgroups(int EPI) { return EPI == EPI_RESID || EPI == EPI_LOGITS ? 2 : 1; }
constexpr int kBigK = 64;      // reduction elements per LDS stage
constexpr int kBigLd = kBigK + 8;  // LDS row stride in elements (16 bytes of padding against bank conflicts)

template <int DT, int EPI>
__global__ void __launch_bounds__(big_tiles(EPI) * big_rgroups(EPI) * 64) gemm_big_kernel(GemmArgs g) {
    constexpr int kBigTiles = big_tiles(EPI), RG = big_rgroups(EPI);
    constexpr bool SB = EPI == EPI_RESID || EPI == EPI_LOGITS;
    constexpr int NB = SB ? 1 : 2;              // 16-feature blocks per tile
    constexpr int NT = kBigTiles * RG * 64;     // threads
    constexpr int AR = kBigTiles * NB * 16;     // weight rows staged per step
    constexpr int CH = kBigK / 8;               // 16-byte chunks per staged row
    constexpr int A_PER = AR * CH / NT, B_PER = kBigRows * CH / NT;  // chunks per thread
    static_assert(AR * CH % NT == 0 && kBigRows * CH % NT == 0, "staging split");
    __shared__ __align__(16) uint16_t lA[2][AR * kBigLd];
    __shared__ __align__(16) uint16_t lB[2][kBigRows * kBigLd];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % RG, wc = wave / RG;  // this wave's row group and tile
    const int m0 = blockIdx.x * kBigRows;  // row block (fastest: the row blocks of a tile share its weights)
    const int t0 = blockIdx.y * kBigTiles;
    const int last_tile = g.n_tiles - 1;

    // this thread's staging chunks: weight rows (tile, block, row) and batch rows
    const uint16_t* asrc[A_PER];
    int adst[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int c = tid + NT * i;
        const int r = c / CH, q = c % CH;
        const int col = r / (16 * NB), blk = (r / 16) % NB, ri = r % 16;
        const TileMap tm = tile_map<EPI>(g, min(t0 + col, last_tile));
        int row = (blk ? tm.rowB : tm.rowA) + ri;
        if (row >= tm.nrows) row = 0;
        asrc[i] = reinterpret_cast<const uint16_t*>(blk ? tm.wb : tm.w) + (long)row * g.K + 8 * q;
        adst[i] = r * kBigLd + 8 * q;
    }
    const uint16_t* bsrc[B_PER];
    int bdst[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int c = tid + NT * i;
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

    constexpr int MTB = kBigRows / RG / 16;  // row tiles of 16 per wave
    float4_t acc[MTB][2];
#pragma unroll
    for (int i = 0; i < MTB; ++i) {
        acc[i][0] = (float4_t){0.f, 0.f, 0.f, 0.f};
        acc[i][1] = acc[i][0];
    }
    const int l16 = lane & 15, kq = lane >> 4;
    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < kBigK / 32; ++s) {
            const int ko = s * 32 + kq * 8;
            Frag<DT> fa[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                fa[b].a = *reinterpret_cast<const uint4*>(&lA[buf][((wc * NB + b) * 16 + l16) * kBigLd + ko]);
#pragma unroll
            for (int i = 0; i < MTB; ++i) {
                Frag<DT> fb;
                fb.a = *reinterpret_cast<const uint4*>(&lB[buf][((wr * MTB + i) * 16 + l16) * kBigLd + ko]);
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[i][b] = frag_mma<DT>(fa[b], fb, acc[i][b]);
            }
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
    gemm_epilogue<DT, MTB, EPI>(g, tile_map<EPI>(g, t), t, blockIdx.x * RG + wr, lane, acc);
}

}  // namespace vs
