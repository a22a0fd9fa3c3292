// Paged split-KV attention on the matrix cores, for workgroups whose query
// states share each K/V page: the rows of a verify pass or prompt chunk of one
// sequence, times the query heads of one grouped K/V head (gfx950).
//
// Same method and outputs as attn_split_kernel ([KV Cache] sections 05 and 07;
// [Serving Efficiency] section 31.4): pages read through the block table, an
// online softmax per query state over each split of the keys, the splits'
// (max, sum, output) statistics merged afterwards. Up to 16 states
// (R rows x HG heads, state s = row s / HG, head s % HG) form the rows of MFMA
// tiles; one 16-key page per wave step:
//   scores   S[16 states][16 keys] = Q K^T: four MFMA 16x16x32 over the head
//            dimension, q fragments held in registers for the whole split, K
//            loaded from the page straight into B-operand layout;
//   softmax  per state in fp32 (log2 domain), row reductions by DPP over the 16
//            lanes that hold one state's 16 keys;
//   output   O[16 states][128] += P V: eight MFMA 16x16x16 per term. P is
//            carried as two storage-type terms (hi + lo, about 16 significant
//            bits) transposed through a wave-private LDS tile; V is staged in a
//            wave-private LDS tile and read back key-wise for the B operand.
// A lane's output rows are the same four states as its score rows, so the
// softmax rescale needs no exchange. The waves' states are merged through LDS
// at the end of the split, in wave order.
#pragma once

#include "attention.h"
#include "common.h"

namespace vs {

// maximum over the 16 lanes of each DPP row, the same result in every lane of the row
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    return v;
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// O(16 x 16) += A(16 x 16) B(16 x 16), operands as four storage-type elements per lane (raw bits)
template <int DT>
__device__ __forceinline__ float4_t mma16(uint2 a, uint2 b, float4_t acc) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b),
                                                     acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                         __builtin_bit_cast(short4_t, b), acc, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ float4_t mma32(uint4 a, uint4 b, float4_t acc) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                      acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       acc, 0, 0, 0);
}

constexpr int kAmWaves = 4;
constexpr int kAmDh = 128;
constexpr int kAmPLd = 16;  // P tile row stride (elements): a half-wave's transposed read covers the banks once
// V tile row stride (elements): 288 bytes, so consecutive rows start 8 banks apart and the eight
// rows of a half-wave's transposed read (32 bytes each) cover the 64 banks once
constexpr int kAmVLd = kAmDh + 16;

// two 8-bit floats (bytes 0, 1 of a word, or 2, 3 with HI) widened to two storage-type elements packed
// in one word. Every e4m3 and e5m2 value is exact in fp16 and in bf16, so no rounding is involved:
// an e5m2 byte is the high byte of the binary16 of its value; otherwise the packed conversion to
// fp32 is exact and bf16 keeps the upper half of each fp32, fp16 converts it (exactly).
template <int DT, int KVT, bool HI>
__device__ __forceinline__ uint32_t widen2(uint32_t word) {
    typedef float float2_t __attribute__((ext_vector_type(2)));
    if constexpr (KVT == E5M2 && DT == F16) {
        return __builtin_amdgcn_perm(0u, word, HI ? 0x030C020Cu : 0x010C000Cu);
    } else {
        float2_t f;
        if constexpr (KVT == E4M3) f = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
        else f = __builtin_amdgcn_cvt_pk_f32_bf8((int)word, HI);
        if constexpr (DT == BF16) {
            return __builtin_amdgcn_perm(__float_as_uint(f.y), __float_as_uint(f.x), 0x07060302u);
        } else {
            return (uint32_t)St<F16>::from_f(f.x) | ((uint32_t)St<F16>::from_f(f.y) << 16);
        }
    }
}

// eight 8-bit floats (two words) widened to eight storage-type elements
template <int DT, int KVT>
__device__ __forceinline__ uint4 widen8(uint2 w) {
    return make_uint4(widen2<DT, KVT, false>(w.x), widen2<DT, KVT, true>(w.x), widen2<DT, KVT, false>(w.y),
                      widen2<DT, KVT, true>(w.y));
}

// The matrix-core kernel's work list: every row group (R rows from the first row of the sequence on) of
// every sequence of rows_lo..rows_hi rows, as (sequence, first row within it), in sequence order and within
// a sequence last group first (a causal pass's last group reads the most pages: the longest units start
// first); *n_items the count, at most cap (one workgroup, blocks of 1024 sequences, an exclusive scan per
// block).
__global__ void __launch_bounds__(1024) attn_items_kernel(const int* q_start, int B, int M, int R, int rows_lo,
                                                          int rows_hi, int2* items, int cap, int* n_items) {
    __shared__ int sc[1024];
    const int tid = threadIdx.x;
    int base = 0;
    for (int b0 = 0; b0 < B; b0 += 1024) {
        const int b = b0 + tid;
        int n = 0;
        if (b < B) {
            const int r0 = min(max(q_start[b], 0), M);
            const int rn = min(max(q_start[b + 1] - r0, 0), M - r0);
            if (rn >= rows_lo && rn <= rows_hi) n = (rn + R - 1) / R;
        }
        sc[tid] = n;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan (Hillis-Steele)
            const int v = tid >= off ? sc[tid - off] : 0;
            __syncthreads();
            sc[tid] += v;
            __syncthreads();
        }
        const int at = base + sc[tid] - n;
        for (int k = 0; k < n && at + k < cap; ++k) items[at + k] = make_int2(b, (n - 1 - k) * R);
        base += sc[1023];
        __syncthreads();
    }
    if (tid == 0) *n_items = min(base, cap);
}

// Two waves per SIMD (at most 256 registers, no scratch): with one page in flight per wave, a
// decode step's few states leave the kernel bound by load latency, and the second resident
// workgroup is what hides it.
// EXT: group blocks, grouped sequences (seq_gp) and the work list may be present; without it the kernel
// takes plain blocks only (every sequence x row-group block) and none of that code is compiled in.
template <int DT, int HG, int KVT, bool EXT>
__global__ void __launch_bounds__(kAmWaves * 64, 2) attn_mfma_kernel(AttnArgs a) {
    constexpr int DH = kAmDh;
    constexpr int R = 16 / HG;  // rows per group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kq = lane >> 4;
    const int h0 = blockIdx.y * HG;
    const int hk = h0 / (a.n_heads / a.n_kv_heads);
    const int T = a.page_tokens;
    // A group block (blockIdx.z < gz_blocks) takes R sequences of one shared-prefix group as its row
    // slots (each one row, at its own position) and one of the prefix splits [0, n_pre_splits) of its
    // prefix pages, read through the block table of the group's first sequence (every member's table holds
    // the same prefix page ids, checked before: a member that fails the check has seq_group -1 and
    // takes the plain path). Any other block takes row groups of one sequence, as below, and the key
    // split n_pre_splits + blockIdx.x.
    const bool grp = EXT && (int)blockIdx.z < a.gz_blocks;
    int s = blockIdx.x, b, rgb, rg_step, r0, Rn, ctx, gp, gi = 0, j0 = 0, gn = 0;
    if (grp) {  // z = (group block) x n_pre_splits + prefix split; blocks past x = 0 are not needed
        if (s > 0) return;
        s = blockIdx.z % a.n_pre_splits;
        const int gz = blockIdx.z / a.n_pre_splits;
        rg_step = R;
        gi = gz / a.gz_per_group;
        j0 = (gz % a.gz_per_group) * R;
        gn = a.group_n[gi];
        b = min(max(a.group_seq0[gi], 0), a.B - 1);
        rgb = 0;
        r0 = 0;
        Rn = 1;  // one pass over the row slots
        ctx = 0;
        gp = min(max(a.group_pages[gi], 0), a.max_blocks);
    } else {
        if constexpr (EXT) {
            s += a.n_pre_splits;
            if (s >= a.n_splits) return;
        }
        const int z = blockIdx.z - (EXT ? a.gz_blocks : 0);
        if (EXT && a.items) {  // one unit of the work list
            if (z >= *a.n_items) return;
            const int2 it = a.items[z];
            b = min(max(it.x, 0), a.B - 1);
            rgb = max(it.y, 0) / R;
            rg_step = 1 << 30;
        } else {
            b = z % a.B;
            rgb = z / a.B;
            rg_step = a.rg_blocks * R;
        }
        r0 = min(max(a.q_start[b], 0), a.M);
        Rn = min(max(a.q_start[b + 1] - r0, 0), a.M - r0);
        if (Rn < a.rows_lo || Rn > a.rows_hi) return;  // another kernel's sequence
        gp = EXT && a.seq_gp ? a.seq_gp[b] : 0;  // a grouped sequence: its prefix splits come from the group blocks
        ctx = max(a.ctx_len[b], 0);
    }
    const int* bt = a.block_tables + (long)b * a.max_blocks;
    const long kofs = (long)a.layer * a.layer_elems + (long)hk * T * DH;
    const long vofs = kofs + (long)a.n_kv_heads * T * DH;
    const int QLD = a.n_heads * DH;
    const unsigned char* kv = reinterpret_cast<const unsigned char*>(a.kv_base);
    constexpr int KB = St<KVT>::bytes;
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q);

    __shared__ __align__(16) uint16_t pt[kAmWaves][2][16 * kAmPLd];  // P hi / lo, [key][state]
    __shared__ __align__(16) uint16_t vt[kAmWaves][16 * kAmVLd];     // V page, [key][dim]
    __shared__ float wst[kAmWaves][16][DH + 2];                      // per-wave (m, l, o) of each state
    __shared__ int srow[R], spos[R];  // a group block's row slots: q / output row (-1: none) and position

    for (int rg = rgb * R; rg < Rn; rg += rg_step) {
        if (grp) {  // the member sequences' rows and positions (group blocks only: a plain block's follow from rg)
            if (tid < R) {
                int row = -1, pos = 0;
                const int seq = a.group_seq0[gi] + j0 + tid;
                if (j0 + tid < gn && seq >= 0 && seq < a.B && a.seq_group[seq] == gi) {
                    row = min(max(a.q_start[seq], 0), a.M - 1);
                    pos = max(a.ctx_len[seq], 0);
                }
                srow[tid] = row;
                spos[tid] = pos;
            }
            __syncthreads();
        }
        // row slot i's q / output row (-1: none) and its position
        auto slot_row = [&](int i) { return grp ? srow[i] : rg + i < Rn ? r0 + rg + i : -1; };
        auto slot_pos = [&](int i) { return grp ? spos[i] : ctx + rg + i; };
        int p_begin, p_end;
        if (grp) {
            bool any = false;
#pragma unroll
            for (int i = 0; i < R; ++i) any |= srow[i] >= 0;
            p_begin = s * a.pre_split_pages;
            p_end = any ? min(p_begin + a.pre_split_pages, gp) : p_begin;
        } else {
            const int nr = min(R, Rn - rg);
            split_range(a, s, gp, min((ctx + rg + nr + T - 1) / T, a.max_blocks), p_begin, p_end);
        }
        // q fragments (A operand of the scores): state l16, dims 8 kq + 32 step
        uint4 qf[4];
        {
            const int i = l16 / HG, j = l16 % HG;
            const int row = slot_row(i);
            const bool ok = row >= 0;
            const long qrow = (long)(ok ? row : max(slot_row(0), 0)) * QLD + (long)(h0 + j) * DH + 8 * kq;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint4 v = *reinterpret_cast<const uint4*>(qb + qrow + 32 * st);
                qf[st] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
            }
        }
        // this lane's four states (score and output rows): 4 kq + r
        int qpos[4];
        bool sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = (4 * kq + r) / HG;
            sv[r] = slot_row(i) >= 0;
            qpos[r] = slot_pos(i);
        }
        float m[4], l[4];
        float4_t o[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            m[r] = -INFINITY;
            l[r] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] = (float4_t){0.f, 0.f, 0.f, 0.f};

        // K (B operand of the scores) and V of one page: key slot l16, dims 8 kq + 32 step
        auto load_page = [&](uint4(&kk)[4], uint4(&vv)[4], int p) {
            const long pb = (long)min(max(bt[p], 0), a.num_pages - 1) * a.page_elems + (long)l16 * DH + 8 * kq;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if constexpr (KB == 2) {
                    kk[st] = load_stream16(kv + (pb + kofs + 32 * st) * 2);
                    vv[st] = load_stream16(kv + (pb + vofs + 32 * st) * 2);
                } else {  // an 8-bit cache: eight values per lane, widened (exactly) to the storage type
                    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
                    const u32x2_t k8 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(kv + pb + kofs + 32 * st));
                    const u32x2_t v8 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(kv + pb + vofs + 32 * st));
                    kk[st] = widen8<DT, KVT>(make_uint2(k8.x, k8.y));
                    vv[st] = widen8<DT, KVT>(make_uint2(v8.x, v8.y));
                }
            }
        };
        uint16_t* my_p = &pt[wave][0][0];
        uint16_t* my_v = &vt[wave][0];
        auto reduce_page = [&](const uint4(&kk)[4], const uint4(&vv)[4], int p) {
            // V to LDS, natural layout [key][dim]
#pragma unroll
            for (int st = 0; st < 4; ++st) *reinterpret_cast<uint4*>(my_v + l16 * kAmVLd + 8 * kq + 32 * st) = vv[st];
            __builtin_amdgcn_wave_barrier();
            float4_t sc = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) sc = mma32<DT>(qf[st], kk[st], sc);
            const int kp = p * T + l16;
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = (sv[r] && kp <= qpos[r]) ? sc[r] * a.scale_log2 : -INFINITY;
                const float mn = fmaxf(m[r], row16_max(x));
                const float alpha = mn == -INFINITY ? 1.f : exp2f(m[r] - mn);
                const float e = mn == -INFINITY ? 0.f : exp2f(x - mn);
                l[r] = l[r] * alpha + row16_sum(e);
                m[r] = mn;
                pr[r] = e;
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t][r] *= alpha;
            }
            // P as hi + lo storage-type terms, as the lane holds it: [key l16][states 4 kq .. +3], one 8-byte
            // store per term
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const uint16_t h0 = St<DT>::from_f(pr[r]), h1 = St<DT>::from_f(pr[r + 1]);
                const uint16_t l0 = St<DT>::from_f(pr[r] - St<DT>::to_f(h0));
                const uint16_t l1 = St<DT>::from_f(pr[r + 1] - St<DT>::to_f(h1));
                hw[r / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lw[r / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
            *reinterpret_cast<uint2*>(my_p + l16 * kAmPLd + 4 * kq) = make_uint2(hw[0], hw[1]);
            *reinterpret_cast<uint2*>(my_p + 16 * kAmPLd + l16 * kAmPLd + 4 * kq) = make_uint2(lw[0], lw[1]);
            __builtin_amdgcn_wave_barrier();  // the wave's LDS writes above come before its reads below
            // The transposing LDS read (gfx950) hands lane i of each 16-lane group, as element e, element
            // i % 4 of the 8 bytes that lane 4 e + i / 4 of the group addressed. A operand P[state l16][keys
            // 4 kq .. +3]: lane (kq, s) addresses [key 4 kq + s / 4][state 4 (s % 4)], so lane (kq, i)
            // receives [key 4 kq + e][state i] as element e.
            typedef __attribute__((address_space(3))) short4_t lds_short4;
            lds_short4* prow = (lds_short4*)(my_p + (4 * kq + (l16 >> 2)) * kAmPLd + 4 * (l16 & 3));
            const uint2 ph = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(prow));
            const uint2 pl = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(prow + 16 * kAmPLd / 4));
            // B operand V[keys 4 kq .. +3][dim 16 t + l16], by the same read: lane (kq, s) addresses
            // V[4 kq + s / 4][16 t + 4 (s % 4)], and lane (kq, i) receives V[4 kq + e][16 t + i] as element e.
            lds_short4* vrow = (lds_short4*)(my_v + (4 * kq + (l16 >> 2)) * kAmVLd + 4 * (l16 & 3));
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint2 vb = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(vrow + 4 * t));
                o[t] = mma16<DT>(ph, vb, o[t]);
                o[t] = mma16<DT>(pl, vb, o[t]);
            }
        };
        // a ring of two pages per wave. Every load in the loop is unconditional (a page past the
        // split re-reads the split's last page, and is never reduced): with a branch around a load
        // the compiler can only wait for all outstanding loads, the one in flight included.
        const int p0 = p_begin + wave;
        if (p0 < p_end) {
            const int plast = p_end - 1;
            uint4 ka[4], va[4], kb2[4], vb2[4];
            load_page(ka, va, p0);
            for (int p = p0;; p += 2 * kAmWaves) {
                load_page(kb2, vb2, min(p + kAmWaves, plast));
                __builtin_amdgcn_sched_barrier(0);  // the next page's loads stay ahead of this reduction
                reduce_page(ka, va, p);
                if (p + kAmWaves >= p_end) break;
                load_page(ka, va, min(p + 2 * kAmWaves, plast));
                __builtin_amdgcn_sched_barrier(0);
                reduce_page(kb2, vb2, p + kAmWaves);
                if (p + 2 * kAmWaves >= p_end) break;
            }
        }
        // this wave's states to LDS: lane holds o[state 4 kq + r][dim 16 t + l16]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int st = 4 * kq + r;
            if (l16 == 0) {
                wst[wave][st][0] = m[r];
                wst[wave][st][1] = l[r];
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) wst[wave][st][2 + 16 * t + l16] = o[t][r];
        }
        __syncthreads();
        // a row with one key split (no group, one plain split) is final here; the merge kernel skips it
        const bool single = !grp && gp == 0 && a.n_splits - a.n_pre_splits == 1;
        // merge the waves in wave order; thread t takes (state, dim) pairs of the valid states
        const int n_st = grp ? 16 : min(R, Rn - rg) * HG;  // a plain block's valid states come first
        for (int idx = tid; idx < n_st * DH; idx += kAmWaves * 64) {
            const int st = idx / DH, d = idx % DH;
            const int row = slot_row(st / HG), h = h0 + st % HG;
            if (row < 0) continue;
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kAmWaves; ++w) mx = fmaxf(mx, wst[w][st][0]);
            float ls = 0.f, os = 0.f;
            if (mx != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kAmWaves; ++w) {
                    const float wm = wst[w][st][0];
                    if (wm == -INFINITY) continue;
                    const float f = exp2f(wm - mx);
                    ls += f * wst[w][st][1];
                    os += f * wst[w][st][2 + d];
                }
            }
            if (single) {
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

}  // namespace vs
