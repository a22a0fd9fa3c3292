// Split-K tile GEMM for the weight products of steps with 17..64 rows (gfx950),
// with the reductions that finish them: the residual products (attention output,
// MLP down) add their sums to x, the q/k/v and gate/up products run their
// epilogues on the summed values.
//
// x[m][n] += sum_k X[m][k] * W[n][k] ([KV Cache] section 02: every row passing
// through a weight matrix shares one read of it). A workgroup of 8 waves owns
// one slice of at most 512 reduction elements and a run of consecutive blocks
// of 128 output features (16 per wave per block). It stages its slice of all
// the step's rows (X) in LDS once, with coalesced loads, and every wave reads
// its MFMA B fragments from there for every block of the run: the activation
// bytes fetched from L2 are 1/8 (or less) of what a 16-feature tile per
// workgroup would fetch, where they cost as much as the weight stream itself.
// Each wave streams its 16 weight rows four rows x 256 bytes per load through a
// wave-private LDS slab (read back as MFMA A fragments), two 128-element blocks
// ahead of the multiply; the stream runs on from one feature block to the next,
// so a run of blocks pays the workgroup's start (X staging, first loads) once. Workgroups along the reduction write fp32 partial sums
// [slice][row][feature]; resid_reduce_kernel adds them to x in slice order, so
// the result does not depend on timing (resid_norm_kernel does the same and also
// writes the RMSNorm of the new x that the next product reads).
#pragma once

#include "common.h"
#include "gemm.h"

namespace vs {

constexpr int kKsRows = 128;  // output features per workgroup (8 waves x 16)
constexpr int kKsXPad = 8;    // LDS row padding (elements): a fragment's 16 rows fall on different banks
// most reduction elements per workgroup: 1024 for 33..48 rows and 768 for 49..64 (the X slice then
// fills most of the LDS of the one workgroup a CU holds at those sizes anyway), 512 otherwise (with
// up to 32 rows two or more workgroups fit a CU)
__host__ __device__ constexpr int ks_slice(int MT) { return MT == 3 ? 1024 : MT == 4 ? 768 : 512; }

// LDS of one workgroup (X slice + eight weight slabs), for the workgroups a CU can hold
__host__ __device__ constexpr int ks_lds_bytes(int MT) {
    return MT * 16 * (ks_slice(MT) + kKsXPad) * 2 + 8 * 16 * (256 + 16);
}

struct KsplitArgs {
    // W [N][K] in the storage type, up to three segments stacked along N: rows [0, n0) of w0,
    // then [n0, n0 + n1) of w1, then the rest of w2 (one matrix: n0 = N, w1 = w2 = w0). n0 and
    // n1 are multiples of 128, so that no block of 128 features spans two segments.
    const void* w0;
    const void* w1;
    const void* w2;
    int n0, n1;
    int N, K;       // K a multiple of 32
    const void* act;  // [M][act_ld] storage type
    int act_ld, M;    // M <= 16 * MT
    int n_slices;     // workgroups along K (gridDim.y); slices are whole 128-element blocks, at most
                      // ks_slice(MT) elements each: n_slices >= ceil(ceil(K / 128) / (ks_slice(MT) / 128))
    float* part;      // [n_slices][M][N] fp32
    int fb_per_wg;    // 128-feature blocks per workgroup (gridDim.x = ceil(ceil(N / 128) / fb_per_wg))
};

// One 128-element block of a wave's 16 weight rows, R4 layout (lane: row 4 j + lane / 16 of the 16,
// bytes 16 (lane % 16) .. +15), with the masks applied on the way into the slab.
struct KsBlock {
    uint4 v[4];
    uint32_t keep[4];
};

// Loads element q = (feature block i, K block b) = (q / nb, q % nb) of a wave's stream. Steps past
// the slice or the stream read their row's first chunk (rows past N: row 0) and are masked.
// f0: first feature of the workgroup's run; r0: this lane's first row inside a block (wave * 16 +
// lane / 16).
template <bool STREAM>
__device__ __forceinline__ void ks_load_block(KsBlock& wb, int q, int nb, int nfb, int total, int nsteps, int f0,
                                              int r0, int cc, long kbase, const uint16_t* W0, const uint16_t* W1,
                                              const uint16_t* W2, int n0s, int n01, int N, int K) {
    const int i = min(q / nb, nfb - 1), b = q - (q / nb) * nb;
    const bool kin = q < total && 4 * b + (cc >> 2) < nsteps;
    const long ko = kin ? kbase + 8 * cc + (long)b * 128 : 0;
    // the block's segment (wave-uniform): its base and its first row inside it
    const int b0 = f0 + i * kKsRows;
    const bool in0 = b0 < n0s, in1 = b0 < n01;
    const uint16_t* seg = in0 ? W0 : in1 ? W1 : W2;
    const int sb = in0 ? b0 : in1 ? b0 - n0s : b0 - n01;
    // a global-memory pointer, said explicitly: after the choice among three pointers the compiler
    // no longer infers it, and would issue generic loads
    typedef const __attribute__((address_space(1))) u32x4_t* gptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = r0 + 4 * j;  // row inside the block
        const bool rv = b0 + r < N;
        const gptr src = (gptr)(seg + (long)(rv ? sb + r : 0) * K + ko);
        wb.v[j] = __builtin_bit_cast(uint4, STREAM ? __builtin_nontemporal_load(src) : *src);
        wb.keep[j] = (kin && rv) ? 0xFFFFFFFFu : 0u;
    }
}

template <int DT, int MT, bool STREAM>
__global__ void __launch_bounds__(512) gemm_ksplit_kernel(KsplitArgs g) {
    // the fields the lambdas below use, as plain values (a lambda holding a reference to the whole
    // argument block keeps the block in scratch memory)
    const int N = g.N, K = g.K, M = g.M, n0s = g.n0, n01 = g.n0 + g.n1;
    float* const part = g.part;
    constexpr int ROWB = 256 + 16;  // slab row stride in bytes
    constexpr int SLAB = 16 * ROWB;
    constexpr int XLD = ks_slice(MT) + kKsXPad;  // X row stride in LDS, elements
    static_assert(MT * 16 * XLD * 2 + 8 * SLAB == ks_lds_bytes(MT), "LDS size");
    __shared__ __align__(16) uint16_t xs[MT * 16 * XLD];
    __shared__ __align__(16) unsigned char slabs[8 * SLAB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int fb0 = blockIdx.x * g.fb_per_wg;  // this workgroup's feature blocks fb0 .. fb0 + nfb - 1
    const int nfb = min(g.fb_per_wg, (N + kKsRows - 1) / kKsRows - fb0);
    const int sl = blockIdx.y;
    // slices on whole 128-element blocks (a block cut by a slice boundary would be loaded whole and
    // partly masked); only the last block of K may be short
    const int KC = K / 32, KB = (KC + 3) / 4;
    const int c0 = min(4 * (int)(((long)sl * KB) / g.n_slices), KC);
    const int c1 = min(4 * (int)(((long)(sl + 1) * KB) / g.n_slices), KC);
    const int nsteps = c1 - c0;  // 32-element steps of this slice (<= ks_slice(MT) / 32)
    const long kbase = (long)c0 * 32;

    // ---- weights: 16 rows of this wave per feature block, blocks of 128 elements (4 steps), R4 layout.
    // The wave's stream is the sequence q = (feature block i, K block b) = (q / nb, q % nb).
    const int nb = (nsteps + 3) / 4;  // K blocks per feature block
    const int total = nfb * nb;
    const int rr = lane >> 4, cc = lane & 15;
    const uint16_t* W0 = reinterpret_cast<const uint16_t*>(g.w0);
    const uint16_t* W1 = reinterpret_cast<const uint16_t*>(g.w1);
    const uint16_t* W2 = reinterpret_cast<const uint16_t*>(g.w2);
    // (a free function: inside a lambda, the choice among the captured pointers becomes a load
    // from the closure at a run-time offset, which keeps the closure in scratch memory)
    auto load_block = [&](KsBlock& wb, int q) {
        ks_load_block<STREAM>(wb, q, nb, nfb, total, nsteps, fb0 * kKsRows, wave * 16 + rr, cc, kbase, W0, W1, W2,
                              n0s, n01, N, K);
    };
    KsBlock w0, w1, w2;
    load_block(w0, 0);
    load_block(w1, 1);

    // ---- stage X[row][kbase .. kbase + 32 * nsteps) (rows past M read row 0: their outputs are never stored)
    {
        const int cpr = nsteps * 4;  // 16-byte chunks per row
        const uint16_t* A = reinterpret_cast<const uint16_t*>(g.act);
        for (int c = threadIdx.x; c < MT * 16 * cpr; c += 512) {
            const int r = c / cpr, q = c - r * cpr;
            const int m = r < M ? r : 0;
            const uint4 v = *reinterpret_cast<const uint4*>(A + (long)m * g.act_ld + kbase + 8 * q);
            *reinterpret_cast<uint4*>(xs + r * XLD + 8 * q) = v;
        }
    }
    __syncthreads();

    float4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    // partial sums of feature block i, then a fresh accumulator: lane holds
    // C[feature n0 + 4 kq + r][row 16 mt + l16], r = 0..3
    auto flush = [=, &acc](int i) {
        const int n = (fb0 + i) * kKsRows + wave * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + (lane & 15);
            if (m < M) {
                float* dst = part + ((long)sl * M + m) * N + n;
                if (n + 3 < N) {
                    *reinterpret_cast<float4_t*>(dst) = acc[mt];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) dst[r] = acc[mt][r];
                }
            }
            acc[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
        }
    };
    unsigned char* my = slabs + wave * SLAB;
    const int l16 = lane & 15, kq = lane >> 4;
    auto multiply = [=, &acc](const KsBlock& wb, int b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 v = wb.v[j];
            const uint32_t kp = wb.keep[j];
            *reinterpret_cast<uint4*>(my + (4 * j + rr) * ROWB + 16 * cc) =
                make_uint4(v.x & kp, v.y & kp, v.z & kp, v.w & kp);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int kk = 4 * b + s;
            if (kk >= nsteps) break;  // X past the slice is not staged
            Frag<DT> fa, fx;
            fa.a = *reinterpret_cast<const uint4*>(my + l16 * ROWB + 64 * s + 16 * kq);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                fx.a = *reinterpret_cast<const uint4*>(xs + (mt * 16 + l16) * XLD + kk * 32 + kq * 8);
                acc[mt] = frag_mma<DT>(fa, fx, acc[mt]);
            }
        }
    };
    // multiply stream element q; after a feature block's last K block, write its partial sums
    auto step = [=, &acc](const KsBlock& wb, int q) {
        const int i = q / nb, b = q - i * nb;
        multiply(wb, b);
        if (b == nb - 1) flush(i);
    };
    // three blocks in the ring: while one is multiplied, the next two are in flight
    for (int q = 0; q < total; q += 3) {
        load_block(w2, q + 2);
        __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of this multiply
        step(w0, q);
        if (q + 1 >= total) break;
        load_block(w0, q + 3);
        __builtin_amdgcn_sched_barrier(0);
        step(w1, q + 1);
        if (q + 2 >= total) break;
        load_block(w1, q + 4);
        __builtin_amdgcn_sched_barrier(0);
        step(w2, q + 2);
    }
}

// sum over slices of part[slice][j] (plane apart), in slice order; the loads of eight slices at a
// time are issued before the first add (the index is clamped, not branched around)
__device__ __forceinline__ float slice_sum(const float* p, long plane, int n_slices) {
    float s = 0.f;
    for (int s0 = 0; s0 < n_slices; s0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p[min(s0 + j, n_slices - 1) * plane];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + j < n_slices) s = s0 + j == 0 ? v[j] : s + v[j];
    }
    return s;
}

// q, k, v of the step's rows from the split-K partial sums of the stacked [Wq; Wk; Wv] product
// (N = (n_heads + 2 n_kv_heads) head_dim): the epilogue of the skinny tile GEMM on summed values
// ([KV Cache] section 03: rotary on q and k, q to q_out, k and v into the row's page slot). One
// thread per (row, head of the stack, rotary pair i, i + head_dim / 2).
template <int DT>
__global__ void __launch_bounds__(256) qkv_reduce_kernel(GemmArgs g, const float* __restrict__ part, int n_slices,
                                                         int N) {
    const int half = g.head_dim / 2;
    const int units = (g.n_heads + 2 * g.n_kv_heads) * half;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)g.M * units) return;
    const int m = (int)(idx / units), u = (int)(idx - (long)m * units);
    const int hh = u / half, i = u - hh * half;  // head of the stack, pair index
    const int seg = hh < g.n_heads ? 0 : hh < g.n_heads + g.n_kv_heads ? 1 : 2;
    const int head = seg == 0 ? hh : seg == 1 ? hh - g.n_heads : hh - g.n_heads - g.n_kv_heads;
    const long plane = (long)g.M * N;
    const float* src = part + (long)m * N + (long)hh * g.head_dim + i;
    const float a = slice_sum(src, plane, n_slices);
    const float b = slice_sum(src + half, plane, n_slices);
    float ra = a, rb = b;
    if (seg < 2) {
        const float c = g.rope_cs[((long)m * half + i) * 2 + 0];
        const float sn = g.rope_cs[((long)m * half + i) * 2 + 1];
        ra = a * c - b * sn;
        rb = b * c + a * sn;
    }
    if (seg == 0) {
        const long o = (long)m * (g.n_heads * g.head_dim) + (long)head * g.head_dim + i;
        store_round<DT>(g.q_out, o, ra);
        store_round<DT>(g.q_out, o + half, rb);
    } else {
        const int pos = g.row_pos[m];
        const int sq = g.row_seq[m];
        if (pos < 0 || pos / g.page_tokens >= g.max_blocks) return;
        const int page = g.block_tables[(long)sq * g.max_blocks + pos / g.page_tokens];
        if (page < 0 || page >= g.num_pages) return;
        const int slot = pos % g.page_tokens;
        const long o = (long)page * g.page_elems + (long)g.layer * g.layer_elems +
                       ((long)(seg - 1) * g.n_kv_heads + head) * g.page_tokens * g.head_dim +
                       (long)slot * g.head_dim + i;
        store_kv<DT>(g.kv_base, o, ra, g.kv_dt);
        store_kv<DT>(g.kv_base, o + half, rb, g.kv_dt);
    }
}

// h = silu(gate) * up from the split-K partial sums of the stacked [W_gate; W_up] product
// (N = 2F): the SwiGLU epilogue of the skinny tile GEMM on summed values. One thread per
// (row, feature).
template <int DT>
__global__ void __launch_bounds__(256) swiglu_reduce_kernel(const float* __restrict__ part, int n_slices, int M,
                                                            int F, void* h_out, int h_ld) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)M * F) return;
    const int m = (int)(idx / F), f = (int)(idx - (long)m * F);
    const long plane = (long)M * 2 * F;
    const float* src = part + (long)m * 2 * F + f;
    const float a = slice_sum(src, plane, n_slices);
    const float b = slice_sum(src + F, plane, n_slices);
    const float s = a / (1.0f + expf(-a));
    store_round<DT>(h_out, (long)m * h_ld + f, s * b);
}

// Logits of the step's logit rows from the split-K partial sums of the LM head (N = vocab), and the
// argmax partials of every 16-feature tile, as the skinny tile GEMM's logits epilogue writes them
// (largest value, its lowest index on ties, second largest). One thread per (row, tile): the tile's
// 16 logits summed over the slices in order, written (when logits is not null) and folded in
// column order.
__global__ void __launch_bounds__(256) logits_reduce_kernel(const float* __restrict__ part, int n_slices, int M,
                                                           int V, float* logits, ArgPart* parts, int n_tiles) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)M * n_tiles) return;
    const int m = (int)(idx / n_tiles), t = (int)(idx - (long)m * n_tiles);
    const long plane = (long)M * V;
    const float* src = part + (long)m * V + 16 * t;
    float acc[16];
    if (16 * t + 16 <= V && (V & 3) == 0) {
        // a whole tile in 16-byte loads, four slices' worth in flight at a time, added in slice order
        for (int s0 = 0; s0 < n_slices; s0 += 4) {
            float4_t a[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[j][q] = *reinterpret_cast<const float4_t*>(src + min(s0 + j, n_slices - 1) * plane + 4 * q);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (s0 + j < n_slices) acc[4 * q + e] = s0 + j == 0 ? a[j][q][e] : acc[4 * q + e] + a[j][q][e];
        }
    } else {  // the vocabulary's last, partial tile (or rows not 16-byte aligned): column by column
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 16 * t + j < V ? slice_sum(src + j, plane, n_slices) : 0.f;
    }
    float v1 = -INFINITY, v2 = -INFINITY;
    int i1 = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int col = 16 * t + j;
        if (col < V) {
            if (logits) logits[(long)m * V + col] = acc[j];
            argpart_combine(v1, i1, v2, acc[j], col, -INFINITY);
        }
    }
    ArgPart p;
    p.v1 = v1;
    p.i1 = i1;
    p.v2 = v2;
    p.pad = 0;
    parts[(long)m * n_tiles + t] = p;
}

// x[m][n] += sum over slices of part[slice][m][n], slices in order; four features per thread.
__global__ void __launch_bounds__(256) resid_reduce_kernel(float* __restrict__ x, int x_ld,
                                                           const float* __restrict__ part, int n_slices, int M,
                                                           int N) {
    const long i4 = (long)blockIdx.x * 256 + threadIdx.x;  // index of a group of four features
    const int groups = (N + 3) / 4;
    if (i4 >= (long)M * groups) return;
    const int m = (int)(i4 / groups), n = (int)(i4 - (long)m * groups) * 4;
    const long plane = (long)M * N;
    const float* src = part + (long)m * N + n;
    if (n + 3 < N) {
        float4_t s = *reinterpret_cast<const float4_t*>(src);
        for (int sl = 1; sl < n_slices; ++sl) s += *reinterpret_cast<const float4_t*>(src + sl * plane);
        float* xr = x + (long)m * x_ld + n;
        xr[0] += s[0];
        xr[1] += s[1];
        xr[2] += s[2];
        xr[3] += s[3];
    } else {
        for (int r = 0; r < 4 && n + r < N; ++r) {
            float s = src[r];
            for (int sl = 1; sl < n_slices; ++sl) s += src[sl * plane + r];
            x[(long)m * x_ld + n + r] += s;
        }
    }
}

// The residual add above fused with the RMSNorm that reads its result (in the pre-norm block of
// [KV Cache] section 03 every residual add is followed by the next sublayer's RMSNorm): for one
// row m per workgroup, x[m] += sum over slices of part[slice][m] (slices in order, as resid_reduce_kernel),
// then y[m] = round(x[m] / sqrt(mean(x[m]^2) + eps) * gain). A step's few rows leave few
// workgroups, so every thread keeps its four features' partial sums of all slices in flight at
// once; the mean of squares is summed in a fixed order (per thread, then per wave, then over the
// waves in order). D must be a multiple of 4.
// The sum over slices of four features' partials (src: slice 0's, the slices plane floats apart), in
// slice order: JB slices' loads at a time, all issued before the first add (the slice index is clamped
// instead of branched around, so none of them waits for another).
template <int JB>
__device__ __forceinline__ float4_t ks_slice_sum4(const float* src, long plane, int n_slices) {
    float4_t s = (float4_t){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_slices; s0 += JB) {
        float4_t v[JB];
#pragma unroll
        for (int j = 0; j < JB; ++j) v[j] = *reinterpret_cast<const float4_t*>(src + min(s0 + j, n_slices - 1) * plane);
#pragma unroll
        for (int j = 0; j < JB; ++j)
            if (s0 + j < n_slices) s = s0 + j == 0 ? v[j] : s + v[j];
    }
    return s;
}

template <int DT, int JB>  // JB: slices' loads issued at a time (4, 12 or 16, whichever fits the slice count)
__global__ void __launch_bounds__(1024) resid_norm_kernel(float* __restrict__ x, const float* __restrict__ part,
                                                          int n_slices, int M, int D, const void* gain, float eps,
                                                          void* y) {
    const int m = blockIdx.x, tid = threadIdx.x;
    const long plane = (long)M * D;
    float* xr = x + (long)m * D;
    auto slice_sum4 = [&](int k) { return ks_slice_sum4<JB>(part + (long)m * D + k, plane, n_slices); };
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
        // one group of four features per thread: the residual, the gain and the partials are all
        // requested at once, and the new residual stays in registers across the row's reduction
        const int k = tid * 4;
        float4_t v = (float4_t){0.f, 0.f, 0.f, 0.f};
        float gv[4] = {0.f, 0.f, 0.f, 0.f};
        float ss = 0.f;
        if (k < D) {
            load_widen<DT, 4>(reinterpret_cast<const char*>(gain) + (long)k * St<DT>::bytes, gv);
            v = *reinterpret_cast<const float4_t*>(xr + k);
            const float4_t s = slice_sum4(k);
            v[0] += s[0];
            v[1] += s[1];
            v[2] += s[2];
            v[3] += s[3];
            *reinterpret_cast<float4_t*>(xr + k) = v;
            ss = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
        const float inv = row_inv(ss);
        if (k < D) {
#pragma unroll
            for (int e = 0; e < 4; ++e) store_round<DT>(y, (long)m * D + k + e, v[e] * inv * gv[e]);
        }
        return;
    }
    float ss = 0.f;
    for (int k = tid * 4; k < D; k += 1024 * 4) {
        const float4_t s = slice_sum4(k);
        float4_t v = *reinterpret_cast<const float4_t*>(xr + k);
        v[0] += s[0];
        v[1] += s[1];
        v[2] += s[2];
        v[3] += s[3];
        *reinterpret_cast<float4_t*>(xr + k) = v;
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    const float inv = row_inv(ss);
    for (int k = tid * 4; k < D; k += 1024 * 4) {
        const float4_t v = *reinterpret_cast<const float4_t*>(xr + k);  // this thread's own writes above
        float gv[4];
        load_widen<DT, 4>(reinterpret_cast<const char*>(gain) + (long)k * St<DT>::bytes, gv);
#pragma unroll
        for (int e = 0; e < 4; ++e) store_round<DT>(y, (long)m * D + k + e, v[e] * inv * gv[e]);
    }
}

}  // namespace vs
