// decode_step / verify_accept: host-side validation, workspace plan and the
// launch sequence of one batched decode / verify step on gfx950.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>

#include "../../include/verify_step.h"
#include "attention.h"
#include "attention_mfma.h"
#include "common.h"
#include "error.h"
#include "gemm.h"
#include "gemm_big.h"
#include "gemm_tile.h"
#include "gemm_ksplit.h"
#include "gemm_strip.h"
#include "gemv.h"
#include "misc.h"
#include "sample.h"

const vs_pool_desc* vs_pool_geometry(const vs_pool* pool);

namespace {
thread_local std::string g_err;
}

vs_status vs_fail(vs_status code, const std::string& msg) {
    g_err = msg;
    return code;
}
vs_status vs_ok() { return VS_OK; }

extern "C" const char* vs_last_error(void) { return g_err.c_str(); }

namespace {

using namespace vs;

constexpr int kPageTokens = 16;

// ---- optional per-kernel event timing (measurement aid) -------------------
struct KernelTimer {
    int kind = VS_KERNEL_NONE;
    void* const* start = nullptr;
    void* const* stop = nullptr;
    int capacity = 0;
    int count = 0;
} g_timer;

// Launch of a kernel that takes one argument struct. When the timer is armed for
// `kind`, the start / stop events come from the dispatch itself (hipExtLaunchKernel),
// so they bracket the kernel's execution and nothing queued around it.
template <typename T>
void launch1(int kind, void (*kern)(T), dim3 grid, dim3 block, size_t lds, hipStream_t s, T arg) {
    void* argv[] = {&arg};
    if (kind != VS_KERNEL_NONE && g_timer.kind == kind && g_timer.count < g_timer.capacity) {
        const int i = g_timer.count++;
        (void)hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, lds, s,
                                 static_cast<hipEvent_t>(g_timer.start[i]), static_cast<hipEvent_t>(g_timer.stop[i]),
                                 0);
    } else {
        (void)hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, lds, s);
    }
}

// The same for a kernel of several arguments (the split-K reductions, timed with their product's kind).
template <typename... P, typename... A>
void launchn(int kind, void (*kern)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A... args) {
    std::tuple<P...> packed(static_cast<P>(args)...);
    std::apply(
        [&](auto&... e) {
            void* argv[] = {static_cast<void*>(&e)...};
            if (kind != VS_KERNEL_NONE && g_timer.kind == kind && g_timer.count < g_timer.capacity) {
                const int i = g_timer.count++;
                (void)hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, lds, s,
                                         static_cast<hipEvent_t>(g_timer.start[i]),
                                         static_cast<hipEvent_t>(g_timer.stop[i]), 0);
            } else {
                (void)hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, lds, s);
            }
        },
        packed);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// A second stream per device (default priority) for attention work beside the caller's stream: the
// one-row sequences' VALU kernel beside the matrix-core kernel, forked from and joined back into the
// caller's stream by events. It is made on the first step on the device whose stream is not under
// graph capture (until then the two kernels run one after the other). The fork / join sequence of one
// step holds the device's lock, so steps on several host threads never wait on each other's events.
constexpr int kMaxAuxDevices = 64;
struct AuxStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
};
AuxStream g_aux[kMaxAuxDevices];
std::mutex g_aux_make;

AuxStream* aux_stream(hipStream_t s) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxAuxDevices) return nullptr;
    AuxStream& a = g_aux[dev];
    std::lock_guard<std::mutex> lk(g_aux_make);
    if (a.s) return &a;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
        if (f) (void)hipEventDestroy(f);
        (void)hipStreamDestroy(st);
        return nullptr;
    }
    a.fork = f;
    a.join = j;
    a.s = st;
    return &a;
}

// The chip: 256 CUs of 160 KB LDS (MI355X).
constexpr int kNumCUs = 256;
constexpr int kLdsPerCu = 160 * 1024;

// Slices along K and 128-feature blocks per workgroup of a split-K product (N features, K, M rows).
// Slices are whole 128-element blocks of K, at most ks_slice(MT) elements each; a workgroup takes a
// run of fb feature blocks of one slice, so that the grid is about one round of the workgroups the
// CUs hold (the start of a workgroup, X staging and the first loads, is paid once per run). From 33
// rows on, slices may be longer than 512 elements, and the slice count minimises an estimate of the
// time: rounds x the longest workgroup's blocks (fb x blocks per slice), times 1 + the fp32 partial
// sums' bytes (written and read again) over the weight bytes, 4 s M / K; ties go to fewer slices.
// (The estimate reproduces the measured best choice for the 7B and 8B-GQA products at 40 and 64
// rows.)
struct KsShape {
    int slices, fb;
};
KsShape ks_shape(int N, int K, int M) {
    const int MT = (M + 15) / 16, nblk = (N + kKsRows - 1) / kKsRows, KB = (K / 32 + 3) / 4,
              mb = ks_slice(MT) / 128;
    const long resident = (long)kNumCUs * std::max(1, (int)(kLdsPerCu / ks_lds_bytes(MT)));
    auto fb_of = [&](int s) { return (int)std::max<long>(1, ((long)nblk * s + resident - 1) / resident); };
    int s = (KB + mb - 1) / mb;
    if (MT >= 3) {
        int best = s;
        double best_cost = 0.0;
        for (int t = s; t <= KB; ++t) {
            const int fb = fb_of(t);
            const long wgs = (long)((nblk + fb - 1) / fb) * t;
            const long rounds = (wgs + resident - 1) / resident;
            const double cost =
                (double)rounds * fb * ((KB + t - 1) / t) * (1.0 + 4.0 * t * std::max(M, 1) / (double)K);
            if (t == s || cost < best_cost - 1e-9) {
                best_cost = cost;
                best = t;
            }
        }
        s = best;
    }
    return {s, fb_of(s)};
}

int kv_elem_bytes(int dtype) { return dtype == VS_F32 ? 4 : (dtype == VS_FP8_E4M3 || dtype == VS_FP8_E5M2) ? 1 : 2; }

// Rows of a step at which the row-streaming GEMV gives way to the MFMA tiles (beyond four rows the
// GEMV's LDS reads of the batch rows outrun the weight stream),
// and the LDS the GEMV may use for its batch rows.
constexpr int kGemvMaxRows = 4;
constexpr size_t kGemvMaxLds = 96 * 1024;
// A plain-input product whose rows exceed this much LDS stages X in phases, so that two
// workgroups still fit on a CU.
constexpr size_t kGemvPhaseLds = 64 * 1024;
// Waves per attention workgroup (fewer where more rows per sequence need more registers),
// and the workgroups the key splits aim for (one per CU).
int attn_waves(int states, int dt) { return states == 1 || (states == 2 && dt != VS_F32) ? 8 : 4; }
constexpr long kAttnTargetWaves = 2048;  // eight-wave workgroups: 256 (one per CU)
// four-wave workgroups (several rows per sequence): two per CU
constexpr long kAttnTargetWgsFew = 512;
// matrix-core attention: one per CU (measured: each further split adds its start-up and, past one
// split, the merge kernel; at 8 x 5 verify rows one split per sequence and head ran 5.44 -> 5.21 ms
// per 7B step)
constexpr long kAttnTargetWgsMfma = 256;
// Output units per workgroup of the output GEMV when it merges the key splits itself.
constexpr int kGemvMergeUnits = 16;

struct Plan {
    int B, M, M_log, D, H, Hkv, Dh, F, V, L, dt, esz;
    int n_splits, split_pages, rmax, attn_hg, attn_waves, rg_blocks;
    bool attn_mfma;  // matrix-core attention: up to 16 (row, head) states per workgroup
    bool attn_mixed;  // matrix-core attention for sequences of 2+ rows, the VALU kernel for one-row ones
    int attn_hg1;     // head group of the VALU kernel's one-row sequences
    int attn_nw1;     // waves per VALU workgroup of one (row, head) state: 4 or 8
    // shared-prefix groups: the matrix-core kernel's group blocks (head groups of grp_hg heads) take each
    // group's prefix pages once, over the first n_pre_splits key splits
    bool groups;
    int grp_hg, n_pre_splits, pre_split_pages, gz_per_group, gz_blocks;
    // the matrix-core kernel's blocks go by a work list of (sequence, row group) units when the plain
    // grid (every sequence x rg_blocks) would be mostly empty: a prompt chunk beside many decode rows
    bool attn_items;
    int items_cap;
    bool ksplit;  // residual products through the split-K tile GEMM
    bool ksplit_qkv, ksplit_gu;  // the q/k/v and gate/up products too (their epilogues after the sums)
    bool ksplit_lm;              // the LM head too (logits and argmax partials after the sums)
    int strip_qkv;               // q/k/v through the full-reduction strip GEMM (epilogue in-kernel): units per
                                 // workgroup (3 or 2), 0 when not
    int strip_gu;                // gate/up through it: its units per workgroup (6 or 7), 0 when not
    bool strip_o, strip_down;    // the residual products through its one-unit variant (8..16 rows)
    int tile_slices;             // > 1: more than 64 rows, residual products split K over this many slices
    int ks_slices;  // most slices of one of them (sizes the partial sums)
    bool gemv;      // the row-streaming path serves every product of the step
    bool merge_in_o; // the output product's prologue merges the key splits (no merge kernel)
    int n_lm_parts; // argmax partials per logit row
    size_t off_grp;  // seq_group[B], seq_gp[B], merge_rows[B], merge_count
    size_t off_items, off_n_items;
    size_t off_row_seq, off_row_pos, off_kvoff, off_rope, off_x, off_xn, off_q, off_attn, off_h, off_part, off_xf, off_lmpart,
        off_ksp;
    size_t total;
};

vs_status check_dims(const vs_model_desc* m) {
    if (m->dtype != VS_F32 && m->dtype != VS_F16 && m->dtype != VS_BF16)
        return vs_fail(VS_ERR_INVALID, "model dtype must be VS_F32, VS_F16 or VS_BF16");
    if (m->head_dim != 64 && m->head_dim != 128) return vs_fail(VS_ERR_SHAPE, "head_dim must be 64 or 128");
    if (m->n_heads <= 0 || m->n_kv_heads <= 0 || m->n_heads % m->n_kv_heads != 0)
        return vs_fail(VS_ERR_SHAPE, "n_heads must be a positive multiple of n_kv_heads");
    if (m->d_model != m->n_heads * m->head_dim) return vs_fail(VS_ERR_SHAPE, "d_model must equal n_heads * head_dim");
    if (m->ffn <= 0 || m->ffn % 32 != 0) return vs_fail(VS_ERR_SHAPE, "ffn must be a positive multiple of 32");
    if (m->vocab < 2 || m->n_layers <= 0) return vs_fail(VS_ERR_SHAPE, "vocab >= 2 and n_layers >= 1 required");
    if (!(m->eps > 0.f) || !(m->rope_theta > 0.f)) return vs_fail(VS_ERR_INVALID, "eps and rope_theta must be > 0");
    return vs_ok();
}

// Units per GEMV workgroup: the units spread evenly over about 512 workgroups (two per
// CU, so every CU streams the same number of bytes), at most kGemvMaxUnits.
int gemv_units_per_wg(int n_units) {
    const int u = (n_units + 511) / 512;
    return std::min(std::max(u, 1), kGemvMaxUnits);
}

vs_status make_plan(const vs_batch_desc* d, const vs_model_desc* m, Plan* p) {
    if (!d || !m || !p) return vs_fail(VS_ERR_INVALID, "null argument");
    vs_status st = check_dims(m);
    if (st != VS_OK) return st;
    if (d->B < 1 || d->B > 65535 || d->M < 0 || d->M_log < 0 || d->M_log > d->M || d->max_rows < 1 ||
        d->max_ctx < 1 || d->max_blocks < 1)
        return vs_fail(VS_ERR_INVALID, "batch sizes out of range (1 <= B <= 65535, 0 <= M_log <= M, max_* >= 1)");
    if ((long)d->max_blocks * kPageTokens < d->max_ctx)
        return vs_fail(VS_ERR_SHAPE, "max_blocks * 16 must cover max_ctx");
    p->B = d->B;
    p->M = d->M;
    p->M_log = d->M_log;
    p->D = m->d_model;
    p->H = m->n_heads;
    p->Hkv = m->n_kv_heads;
    p->Dh = m->head_dim;
    p->F = m->ffn;
    p->V = m->vocab;
    p->L = m->n_layers;
    p->dt = m->dtype;
    p->esz = m->dtype == VS_F32 ? 4 : 2;
    // key splits: about one workgroup per CU over B x heads, at least two pages per wave of a split
    // rows per attention row group (5: a verify pass of five drafts fits one group exactly)
    p->rmax = d->max_rows <= 1 ? 1 : d->max_rows <= 2 ? 2 : d->max_rows <= 4 ? 4 : d->max_rows <= 5 ? 5 : 8;
    p->attn_hg = 1;
    {
        // grouped K/V heads: a workgroup may take HG query heads of one K/V head, up to 4 (row, head)
        // states (more leave one wave per SIMD, which measured slower than plain row groups); pick
        // the (rows, HG) that reads each K/V page the fewest times, the plain row groups on a tie
        const int group = m->n_heads / m->n_kv_heads;
        auto reads = [&](int r, int hg) { return (long)((d->max_rows + r - 1) / r) * (group / hg); };
        long best = reads(p->rmax, 1);
        for (int hg : {2, 4}) {
            if (group % hg) continue;
            for (int r : {1, 2}) {
                if (r * hg > 4 || reads(r, hg) >= best) continue;
                best = reads(r, hg);
                p->rmax = r;
                p->attn_hg = hg;
            }
        }
    }
    p->attn_waves = attn_waves(p->rmax * p->attn_hg, m->dtype);
    {
        // several rows per sequence or grouped heads (fp16 / bf16, head_dim 128): the states that share
        // each page run as MFMA tiles of 16: HG heads of one K/V group (the largest power of two up to
        // 16 dividing the group) x 16 / HG rows
        const int group = m->n_heads / m->n_kv_heads;
        // One-row sequences with grouped heads take the matrix cores only while (sequence, K/V head)
        // pairs are fewer than the CUs: with more, the VALU kernel's four-head workgroups stream K/V
        // faster (measured at 8B widths, bf16, 64 decode rows, contexts 128..4096: 4.48 against 4.92 ms
        // of attention per step; at one row the matrix cores win, 0.48 against 0.53 ms).
        p->attn_mfma = m->dtype != VS_F32 && m->head_dim == kAmDh &&
                       (d->max_rows >= 2 || (group >= 2 && (long)d->B * m->n_kv_heads < kNumCUs));
        // rows differ between sequences (a prompt chunk among decode rows): the one-row sequences,
        // which would fill one of the 16 states, go to the VALU kernel, whose one-state workgroups
        // stream K/V faster
        p->attn_mixed = p->attn_mfma && d->max_rows >= 2 && (long)d->M < (long)d->B * d->max_rows;
        p->attn_hg1 = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
        if (p->attn_mfma) {
            int hg = 1;
            while (hg < 16 && group % (2 * hg) == 0) hg *= 2;
            p->attn_hg = hg;
            p->rmax = 16 / hg;
            p->attn_waves = kAmWaves;
        }
    }
    // shared-prefix groups: used for fp16 / bf16 models with head_dim 128 (the matrix-core kernel's group
    // blocks), ignored otherwise
    if (d->n_prefix_groups < 0) return vs_fail(VS_ERR_INVALID, "n_prefix_groups must be >= 0");
    p->groups = d->n_prefix_groups > 0 && m->dtype != VS_F32 && m->head_dim == kAmDh && d->M > 0;
    p->grp_hg = 1;
    p->n_pre_splits = p->pre_split_pages = p->gz_per_group = p->gz_blocks = 0;
    if (p->groups) {
        if (!d->group_seq0 || !d->group_n || !d->group_pages || d->max_group_size < 1 || d->max_group_pages < 1 ||
            d->n_prefix_groups > d->B || d->max_group_size > d->B || d->max_group_pages > d->max_blocks)
            return vs_fail(VS_ERR_INVALID,
                           "prefix groups need device arrays, 1 <= n_prefix_groups <= B, 1 <= max_group_size <= B, "
                           "1 <= max_group_pages <= max_blocks");
        const int group = m->n_heads / m->n_kv_heads;
        while (p->grp_hg < 16 && group % (2 * p->grp_hg) == 0) p->grp_hg *= 2;
        const int per_block = 16 / p->grp_hg;  // sequences per group block
        p->gz_per_group = (d->max_group_size + per_block - 1) / per_block;
        const long gz = (long)d->n_prefix_groups * p->gz_per_group;
        if (gz + d->B > 65535) return vs_fail(VS_ERR_INVALID, "too many prefix-group blocks (groups x ceil(max_group_size / 16 x HG) + B > 65535)");
        p->gz_blocks = (int)gz;
    }
    const int max_pages = (d->max_ctx + kPageTokens - 1) / kPageTokens;
    // row groups of a sequence go to separate workgroups (a prompt chunk's groups run in parallel)
    const int rg_needed = (d->max_rows + p->rmax - 1) / p->rmax;
    p->rg_blocks = (int)std::max<long>(1, std::min<long>(rg_needed, (65535L - p->gz_blocks) / d->B));
    const long pairs = (long)d->B * (m->n_heads / p->attn_hg) * p->rg_blocks;  // workgroups per split
    const long wgs_target = p->attn_mfma          ? kAttnTargetWgsMfma
                            : p->attn_waves == 8 ? kAttnTargetWaves / 8
                                                 : kAttnTargetWgsFew;
    const int ns = (int)std::min<long>(std::max(1, max_pages / (2 * p->attn_waves)),
                                       std::max<long>(1, (wgs_target + pairs - 1) / pairs));
    p->split_pages = (max_pages + ns - 1) / ns;
    p->n_splits = (max_pages + p->split_pages - 1) / p->split_pages;
    if (p->groups) {
        // the prefix splits, ahead of the others: the group blocks take about half of the CUs (the other
        // attention work runs beside them), at least two pages per wave. Measured on 7B, 64 decode rows
        // in 4 groups of 1024-token prefixes + a 512-row chunk (128 group blocks per split): 1 prefix
        // split 15.91 ms per step, 2: 16.04, 4: 16.18.
        const long gwgs = (long)p->gz_blocks * (m->n_heads / p->grp_hg);  // group blocks per prefix split
        p->n_pre_splits = (int)std::max<long>(
            1, std::min<long>(d->max_group_pages / (2 * kAmWaves), (long)kNumCUs / 2 / gwgs));
        if ((long)p->gz_blocks * p->n_pre_splits + (long)d->B * p->rg_blocks > 65535)
            p->n_pre_splits = std::max(1, (int)((65535L - (long)d->B * p->rg_blocks) / p->gz_blocks));
        p->pre_split_pages = (d->max_group_pages + p->n_pre_splits - 1) / p->n_pre_splits;
        p->n_splits += p->n_pre_splits;
        p->gz_blocks *= p->n_pre_splits;  // the group blocks' z range: every (block, prefix split) pair
    }
    // one-state VALU workgroups (decode rows, one head each): four waves, each with twice the pages,
    // when the launch has no more workgroups than CUs or its sequences are grouped (few own pages
    // after the prefix); eight otherwise. Measured (7B): batch 1 at context 2048, 2.869 -> 2.846 ms per
    // step; batch 8, contexts 128..4096, 4.364 -> 4.309; 64 decode rows on shared prefixes + a 512-row
    // chunk, 17.06 -> 16.64; batch 64 (2048 workgroups of about 130 pages) 14.13 with eight waves
    // against 14.61 with four.
    p->attn_nw1 = (long)d->B * m->n_heads * (p->n_splits - p->n_pre_splits) <= kNumCUs || p->groups ? 4 : 8;
    p->attn_items = false;
    p->items_cap = 0;
    if (p->attn_mfma) {
        // units: at most ceil(rows / R) per sequence of rows_lo+ rows
        const int R = 16 / p->attn_hg, lo = p->attn_mixed ? 2 : 1;
        const long nq = std::min<long>(d->B, std::max(d->M, 1) / lo);
        const long cap = ((long)d->M + (R - 1) * nq + R - 1) / R;
        if ((long)d->B * p->rg_blocks > 2 * cap && cap <= 65535L - p->gz_blocks) {
            p->attn_items = true;
            p->items_cap = (int)std::max<long>(cap, 1);
        }
    }
    // the row-streaming GEMV serves steps of up to kGemvMaxRows rows (beyond, the products' VALU work
    // outgrows the weight stream); RMSNorm-input products stage all of X, plain-input ones may phase it
    p->gemv = d->M <= kGemvMaxRows && (size_t)std::max(d->M, 1) * p->D * p->esz <= kGemvMaxLds;
    p->merge_in_o = p->gemv && p->n_splits > 1 && p->n_splits <= kMergeMaxSplits && !p->groups;
    p->n_lm_parts = p->gemv ? (p->V + gemv_units_per_wg(p->V) - 1) / gemv_units_per_wg(p->V) : (p->V + 15) / 16;
    // 17..64 rows in fp16 / bf16: the weight products split K over workgroups, the X slice staged
    // once per workgroup in LDS (up to 16 rows the 16-feature tiles read no more activation bytes
    // than weight bytes)
    p->ksplit = !p->gemv && p->dt != VS_F32 && d->M > 16 && d->M <= 64;
    p->ks_slices = std::max(ks_shape(p->D, p->H * p->Dh, d->M).slices, ks_shape(p->D, p->F, d->M).slices);
    // (the stacked products' segments must start on 128-feature blocks). The q/k/v product takes
    // it from 5 rows on (measured at 8 rows: 25 against 29 us per layer at the 7B shape; the other
    // products are faster as 16-feature tiles there)
    p->ksplit_qkv = !p->gemv && p->dt != VS_F32 && d->M <= 64 && (p->H * p->Dh) % kKsRows == 0 &&
                    (p->Hkv * p->Dh) % kKsRows == 0;
    p->ksplit_gu = p->ksplit && p->F % kKsRows == 0;
    // 8..64 rows: the q/k/v and gate/up products through the strip GEMM when its units (16 weight
    // rows each) spread over the CUs in whole workgroups of U units with at most 15 % of them idle
    // (at 7B widths: 3 q/k/v units on every CU, 6 gate/up units on 230 CUs). At least 8 rows: masked
    // chunks read eight rows' offsets from the activations.
    {
        const int MT = (d->M + 15) / 16;
        auto strip_ok = [&](long units, int U) {
            const long wgs = (units + U - 1) / U;
            return U <= strip_max_units(MT) && wgs <= kNumCUs && wgs * 100 >= 85L * kNumCUs;
        };
        const bool base = p->dt != VS_F32 && !p->gemv && d->M >= 8 && d->M <= 64 && p->D % 128 == 0;
        // q/k/v units that do not fill whole three-unit workgroups (the 8B-GQA widths: 384 units) may go two
        // to a workgroup on 75 % of the CUs up to 48 rows (8 x 5 verify rows: 19.6 against 21.3 us per layer
        // for split-K + its rotary reduction; at 64 rows 25.2 against 24.5, so split-K stays there)
        const long qkv_units = (long)(p->H + 2 * p->Hkv) * p->Dh / 16;
        const bool narrow_ok = MT <= 3 && (qkv_units + 1) / 2 <= kNumCUs && (qkv_units + 1) / 2 * 100 >= 70L * kNumCUs;
        p->strip_qkv = !(base && p->Dh % 16 == 0)           ? 0
                       : strip_ok(qkv_units, kStripUnitsQkv) ? kStripUnitsQkv
                       : narrow_ok                           ? kStripUnitsQkvNarrow
                                                             : 0;
        p->strip_gu = !(base && p->F % 8 == 0) ? 0
                      : strip_ok(p->F / 8, kStripUnitsGu)     ? kStripUnitsGu
                      : strip_ok(p->F / 8, kStripUnitsGuWide) ? kStripUnitsGuWide
                                                                : 0;
        // the residual products: one unit per workgroup, up to 16 rows (one row tile; every CU reads
        // all of X, which past 16 rows outweighs its share of the weights)
        const bool base_r = base && d->M <= 16 && p->D % 16 == 0 && strip_ok(p->D / 16, 1);
        p->strip_o = base_r && (p->H * p->Dh) % 128 == 0;
        p->strip_down = base_r && p->F % 128 == 0;
    }
    // more than 64 rows (the pipelined tile GEMM): the residual products have D / 256 feature blocks
    // x ceil(M / 128) row blocks of workgroups, too few for the CUs at prompt-chunk sizes; their
    // reduction is then split into slices to make about one workgroup per CU (at most 8 slices, each
    // at least one 64-element step). Measured at 7B widths and 576 rows (O / down): 1 slice 92 / 218 us,
    // 2 slices 48 / 115, 3 slices 41 / 87, 4 slices 56 / 124.
    p->tile_slices = 1;
    if (p->dt != VS_F32 && d->M > 64 && p->D % 16 == 0 && (p->H * p->Dh) % kTileK == 0 && p->F % kTileK == 0) {
        const long wgs = (long)((p->D / 16 + 15) / 16) * ((d->M + kTileRowsM - 1) / kTileRowsM);
        const int nk = std::min(p->H * p->Dh, p->F) / kTileK;
        p->tile_slices = (int)std::max<long>(1, std::min<long>({8L, (long)kNumCUs / wgs, (long)nk}));
    }
    // the LM head goes by its own rows: 17..64 logit rows through split-K also in a longer step (a prompt
    // chunk beside 64 decode rows), where the 16-feature tiles took 155 us per step
    p->ksplit_lm = p->dt != VS_F32 && !p->gemv && d->M_log > 0 && d->M_log <= 64 && (p->ksplit || d->M_log > 16);
    const long n_qkv = (long)(p->H + 2 * p->Hkv) * p->Dh, n_gu = 2L * p->F;
    long ks_floats = std::max<long>((long)p->ks_slices * p->D,
                                    std::max((long)ks_shape(n_qkv, p->D, d->M).slices * n_qkv,
                                             (long)ks_shape(n_gu, p->D, d->M).slices * n_gu));
    // (the LM head's partial sums cover only the logit rows: per-row size scaled to M below)
    if (p->ksplit_lm)
        ks_floats = std::max<long>(ks_floats, ((long)ks_shape(p->V, p->D, d->M_log).slices * p->V * d->M_log +
                                               std::max(d->M, 1) - 1) / std::max(d->M, 1));
    const size_t M = (size_t)std::max(d->M, 1), ML = (size_t)std::max(d->M_log, 1);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + std::max<size_t>(bytes, 4));
        return at;
    };
    p->off_row_seq = take(M * 4);
    p->off_row_pos = take(M * 4);
    p->off_kvoff = take(M * 8);
    p->off_rope = take(M * (p->Dh / 2) * 2 * 4);
    p->off_x = take(M * p->D * 4);
    p->off_xn = take(M * p->D * p->esz);
    p->off_q = take(M * p->H * p->Dh * p->esz);
    p->off_attn = take(M * p->H * p->Dh * p->esz);
    p->off_h = take(M * p->F * p->esz);
    p->off_part = take(M * p->H * p->n_splits * part_stride(p->Dh) * 4);
    p->off_xf = take(ML * p->D * p->esz);
    p->off_lmpart = take(ML * p->n_lm_parts * sizeof(ArgPart));
    if (p->tile_slices > 1) ks_floats = std::max<long>(ks_floats, (long)p->tile_slices * p->D);
    p->off_ksp = take(p->ksplit || p->ksplit_qkv || p->ksplit_lm || p->tile_slices > 1 ? (size_t)ks_floats * M * 4 : 4);
    p->off_grp = take(p->groups ? (3 * (size_t)d->B + 1) * 4 : 4);  // seq_group, seq_gp, merge_rows, count
    p->off_items = take((size_t)std::max(p->items_cap, 1) * 8);
    p->off_n_items = take(4);
    p->total = o;
    return vs_ok();
}

// ---- launches ------------------------------------------------------------

template <int DT, int MT, int EPI>
void launch_gemm_mt(int kind, const GemmArgs& g, int NW, int n_mgroups, hipStream_t s) {
    constexpr int U = (DT == F32 ? 4 : 8) / MT > 0 ? (DT == F32 ? 4 : 8) / MT : 1;
    dim3 grid(n_mgroups, g.n_tiles);
    // one row group streams the weights (nontemporal); several share them through the caches
    if constexpr (DT != F32) {
        if (n_mgroups == 1) {
            if (NW >= 8) launch1(kind, gemm_skinny_kernel<DT, MT, 8, EPI, U, true>, grid, dim3(8 * 64), 0, s, g);
            else launch1(kind, gemm_skinny_kernel<DT, MT, 4, EPI, U, true>, grid, dim3(4 * 64), 0, s, g);
            return;
        }
    }
    if (NW >= 8) launch1(kind, gemm_skinny_kernel<DT, MT, 8, EPI, U, false>, grid, dim3(8 * 64), 0, s, g);
    else launch1(kind, gemm_skinny_kernel<DT, MT, 4, EPI, U, false>, grid, dim3(4 * 64), 0, s, g);
}

// x += W a for 5..64 rows: the split-K tile GEMM writes per-slice partial sums, then they are added
// to x in slice order. With a gain, the same kernel that adds them also writes RMSNorm(x) * gain to
// y (x rows of exactly N features).
// Partial sums part[slice][M][N] of W a for 5..64 rows through the split-K tile GEMM, W up to
// three stacked segments (w0: rows [0, n0), w1: [n0, n0 + n1), w2: the rest); returns the slices.
template <int DT>
int launch_ksplit(int kind, const void* w0, const void* w1, const void* w2, int n0, int n1, int N, int K,
                  const void* act, int act_ld, int M, float* part, hipStream_t s) {
    if constexpr (DT == F32) {
        return 0;  // fp32 models keep the tile GEMM (the plan never selects this for them)
    } else {
    const int MT = (M + 15) / 16, nblk = (N + kKsRows - 1) / kKsRows;
    const KsShape sh = ks_shape(N, K, M);
    const int slices = sh.slices, fb = sh.fb;
    const KsplitArgs a{w0, w1, w2, n0, n1, N, K, act, act_ld, M, slices, part, fb};
    const dim3 grid((nblk + fb - 1) / fb, a.n_slices), block(512);
    switch (MT) {
        case 1: launch1(kind, gemm_ksplit_kernel<DT, 1, true>, grid, block, 0, s, a); break;
        case 2: launch1(kind, gemm_ksplit_kernel<DT, 2, true>, grid, block, 0, s, a); break;
        case 3: launch1(kind, gemm_ksplit_kernel<DT, 3, true>, grid, block, 0, s, a); break;
        default: launch1(kind, gemm_ksplit_kernel<DT, 4, true>, grid, block, 0, s, a); break;
    }
    return slices;
    }
}

// The strip GEMM (q/k/v or gate/up with its epilogue): one workgroup of eight waves per U units.
template <int DT, int EPI, int U>
void launch_strip(int kind, const GemmArgs& g, hipStream_t s) {
    if constexpr (DT == F32) {
        return;  // fp16 / bf16 only (the plan never selects this for fp32 models)
    } else {
        const dim3 grid((g.n_tiles + U - 1) / U), block(kStripWaves * 64);
        switch ((g.M + 15) / 16) {
            case 1: launch1(kind, gemm_strip_kernel<DT, 1, EPI, U>, grid, block, 0, s, g); break;
            case 2: launch1(kind, gemm_strip_kernel<DT, 2, EPI, U>, grid, block, 0, s, g); break;
            case 3: launch1(kind, gemm_strip_kernel<DT, 3, EPI, U>, grid, block, 0, s, g); break;
            default:
                if constexpr (U <= strip_max_units(4)) launch1(kind, gemm_strip_kernel<DT, 4, EPI, U>, grid, block, 0, s, g);
                break;
        }
    }
}

// x += W a through the one-unit strip GEMM (8..16 rows: one row tile), one workgroup per 16 features.
template <int DT>
void launch_strip_resid(int kind, const GemmArgs& g, hipStream_t s) {
    if constexpr (DT == F32) {
        return;  // fp16 / bf16 only (the plan never selects this for fp32 models)
    } else {
        launch1(kind, gemm_strip_resid_kernel<DT, 1>, dim3(g.n_tiles), dim3(kStripWaves * 64), 0, s, g);
    }
}

template <int DT>
void launch_resid_ksplit(int kind, const void* w, int N, int K, const void* act, int act_ld, int M, float* x,
                         int x_ld, float* part, hipStream_t s, const void* gain = nullptr, float eps = 0.f,
                         void* y = nullptr) {
    if constexpr (DT == F32) {
        return;  // fp32 models keep the tile GEMM (the plan never selects this for them)
    } else {
    const int slices = launch_ksplit<DT>(kind, w, w, w, N, 0, N, K, act, act_ld, M, part, s);
    if (gain) {
        // loads in as few rounds as possible without many clamped (repeated) ones: 4 up to four slices,
        // 16 for 13..16, 12 otherwise (23 slices: 12 + 11)
        auto rn = slices <= 4                    ? resid_norm_kernel<DT, 4>
                  : slices > 12 && slices <= 16 ? resid_norm_kernel<DT, 16>
                                                 : resid_norm_kernel<DT, 12>;
        launchn(kind, rn, dim3(M), dim3(1024), 0, s, x, part, slices, M, N, gain, eps, y);
    } else {
        const long groups = (long)M * ((N + 3) / 4);
        launchn(kind, resid_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, x, x_ld,
                           part, slices, M, N);
    }
    }
}

// The pipelined tile GEMM takes a product when its reduction is whole 64-element steps and its weight
// segments whole 16-row blocks (q/k/v: whole 32-row tiles of each head); the LM head keeps the LDS-tiled
// GEMM (its epilogue folds argmax partials per 16-feature tile).
template <int EPI>
bool tile_ok(const GemmArgs& g) {
    if (EPI == EPI_LOGITS || g.K % kTileK != 0 || g.n0 % 16 != 0) return false;
    if (EPI == EPI_QKV) return g.head_dim % 32 == 0 && g.n1 % 16 == 0 && g.n2 % 16 == 0;
    return true;
}

// x += W a for more than 64 rows through the tile GEMM, the reduction split into `slices` slices whose
// partial sums are added in slice order; with a gain the same reduction writes RMSNorm(x) * gain to y.
template <int DT>
void launch_resid_tile(int kind, const GemmArgs& g, int slices, float* part, hipStream_t s, const void* gain = nullptr,
                       float eps = 0.f, void* y = nullptr) {
    if constexpr (DT == F32) {
        return;  // fp16 / bf16 only (the plan never selects this for fp32 models)
    } else {
        launchn(kind, gemm_tile_kernel<DT, EPI_RESID>, dim3(tile_grid(g.n_tiles, EPI_RESID, slices, g.M)), dim3(kTileWaves * 64), 0,
                s, g, slices, part);
        if (gain) {
            auto rn = slices <= 4 ? resid_norm_kernel<DT, 4> : resid_norm_kernel<DT, 12>;
            launchn(kind, rn, dim3(g.M), dim3(1024), 0, s, g.x, (const float*)part, slices, g.M, g.n0, gain, eps, y);
        } else {
            const long groups = (long)g.M * ((g.n0 + 3) / 4);
            launchn(kind, resid_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, g.x, g.x_ld,
                    (const float*)part, slices, g.M, g.n0);
        }
    }
}

template <int DT, int EPI>
void launch_gemm(int kind, const GemmArgs& g, hipStream_t s) {
    const int M = g.M;
    if (M <= 0) return;
    if constexpr (DT != F32) {
        // more than 64 rows (a prompt chunk): LDS-tiled MFMA GEMM, eight paired (or two single) feature
        // tiles x 128 rows per workgroup
        if (M > 64 && tile_ok<EPI>(g)) {
            launchn(kind, gemm_tile_kernel<DT, EPI>, dim3(tile_grid(g.n_tiles, EPI, 1, M)), dim3(kTileWaves * 64), 0, s, g, 1,
                    (float*)nullptr);
            return;
        }
        if (M > 64 && g.K % kBigK == 0) {
            constexpr int T = big_tiles(EPI);
            const dim3 grid((M + kBigRows - 1) / kBigRows, (g.n_tiles + T - 1) / T);
            launch1(kind, gemm_big_kernel<DT, EPI>, grid, dim3(T * big_rgroups(EPI) * 64), 0, s, g);
            return;
        }
    }
    const int MT = std::min((M + 15) / 16, 4);  // row blocks of 16 per group
    const int n_mgroups = (M + 16 * MT - 1) / (16 * MT);
    const long wgs = (long)g.n_tiles * n_mgroups;
    int NW = wgs < 1024 ? 8 : 4;
    const int KC = g.K / 32;
    while (NW > 4 && NW > KC) NW >>= 1;
    if (MT == 1) launch_gemm_mt<DT, 1, EPI>(kind, g, NW, n_mgroups, s);
    else if (MT == 2) launch_gemm_mt<DT, 2, EPI>(kind, g, NW, n_mgroups, s);
    else if (MT == 3) launch_gemm_mt<DT, 3, EPI>(kind, g, NW, n_mgroups, s);
    else launch_gemm_mt<DT, 4, EPI>(kind, g, NW, n_mgroups, s);
}

template <int DT, int MR, int XM, int EPI>
void launch_gemv_mr(int kind, const GemvArgs& g, hipStream_t s) {
    const size_t lds = (size_t)g.M * (g.k_phase > 0 ? g.k_phase : g.K) * St<DT>::bytes;
    static bool attr_set = false;  // per instantiation: allow more than 64 KB of dynamic LDS
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_kernel<DT, MR, XM, EPI>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemvMaxLds);
        attr_set = true;
    }
    const int n_wg = (g.n_units + g.units_per_wg - 1) / g.units_per_wg;
    launch1(kind, gemv_kernel<DT, MR, XM, EPI>, dim3(n_wg), dim3(kGemvWaves * 64), lds, s, g);
}

template <int DT, int XM, int EPI>
void launch_gemv(int kind, GemvArgs g, hipStream_t s, int units_per_wg = 0) {
    if (g.M <= 0) return;
    g.units_per_wg = units_per_wg > 0 ? units_per_wg : gemv_units_per_wg(g.n_units);
    g.k_phase = 0;
    if (XM == X_PLAIN && (size_t)g.M * g.K * St<DT>::bytes > kGemvPhaseLds) {
        // phases of whole bursts (kGemvChunks 1 KB chunks), one unit per wave
        const int burst = kGemvChunks * (1024 / St<DT>::bytes);
        g.k_phase = (int)(kGemvPhaseLds / ((size_t)g.M * St<DT>::bytes)) / burst * burst;
        g.units_per_wg = std::min(g.units_per_wg, kGemvWaves);
    }
    if (g.M <= 1) launch_gemv_mr<DT, 1, XM, EPI>(kind, g, s);
    else if (g.M <= 2) launch_gemv_mr<DT, 2, XM, EPI>(kind, g, s);
    else if (g.M <= 4) launch_gemv_mr<DT, 4, XM, EPI>(kind, g, s);
    else launch_gemv_mr<DT, 8, XM, EPI>(kind, g, s);
}

// The split pass, then the merge kernel unless the splits are merged elsewhere (one split
// needs none; the output GEMV can merge them in its prologue).
template <int DT, int DH, int KVT>
void launch_attention_kv(const AttnArgs& a, int B, int M, int rmax, int hg, bool merge_kernel, hipStream_t s, int nw1) {
    dim3 grid(a.n_splits - a.n_pre_splits, a.n_heads / hg, B * a.rg_blocks);
    const int nw = rmax * hg == 1 ? nw1 : attn_waves(rmax * hg, DT);
    dim3 block(nw * 64);
    auto go = [&](auto kern) { launch1(VS_KERNEL_ATTN, kern, grid, block, 0, s, a); };
    switch (hg * 16 + rmax) {
        case 16 + 1:
            if (nw == 4) go(attn_split_kernel<DT, DH, 1, 4, 1, KVT>);
            else go(attn_split_kernel<DT, DH, 1, 8, 1, KVT>);
            break;
        case 16 + 2:
            if (nw == 8) go(attn_split_kernel<DT, DH, 2, DT == F32 ? 4 : 8, 1, KVT>);
            else go(attn_split_kernel<DT, DH, 2, 4, 1, KVT>);
            break;
        case 16 + 4: go(attn_split_kernel<DT, DH, 4, 4, 1, KVT>); break;
        case 16 + 5: go(attn_split_kernel<DT, DH, 5, 4, 1, KVT>); break;
        case 32 + 1:
            if (nw == 8) go(attn_split_kernel<DT, DH, 1, DT == F32 ? 4 : 8, 2, KVT>);
            else go(attn_split_kernel<DT, DH, 1, 4, 2, KVT>);
            break;
        case 32 + 2: go(attn_split_kernel<DT, DH, 2, 4, 2, KVT>); break;
        case 64 + 1: go(attn_split_kernel<DT, DH, 1, 4, 4, KVT>); break;
        default: go(attn_split_kernel<DT, DH, 8, 4, 1, KVT>); break;
    }
    if (merge_kernel && a.n_splits > 1)
        launch1(VS_KERNEL_MERGE, attn_merge_kernel<DT, DH>, dim3(M, a.n_heads), dim3(DH), 0, s, a);
}

// The cache's storage type picks the K/V loads: the model's type, or (fp16 / bf16 models with
// head_dim 128) an 8-bit float.
// Matrix-core attention: grid (splits, head groups of HG, prefix-group blocks + plain blocks); z_seq = 0
// launches the group blocks alone.
template <int DT, int KVT>
void launch_attention_mfma(const AttnArgs& a, int z_seq, int hg, hipStream_t s) {
    const int nx = z_seq == 0 ? 1 : a.n_splits - a.n_pre_splits;  // the group blocks carry their split in z
    const dim3 grid(nx, a.n_heads / hg, a.gz_blocks + z_seq), block(kAmWaves * 64);
    // the kernel with group blocks, grouped sequences and the work list compiled in only where used
    const bool ext = a.gz_blocks > 0 || a.items || a.seq_gp;
    auto go = [&](auto plain, auto full) { launch1(VS_KERNEL_ATTN, ext ? full : plain, grid, block, 0, s, a); };
    switch (hg) {
        case 1: go(attn_mfma_kernel<DT, 1, KVT, false>, attn_mfma_kernel<DT, 1, KVT, true>); break;
        case 2: go(attn_mfma_kernel<DT, 2, KVT, false>, attn_mfma_kernel<DT, 2, KVT, true>); break;
        case 4: go(attn_mfma_kernel<DT, 4, KVT, false>, attn_mfma_kernel<DT, 4, KVT, true>); break;
        case 8: go(attn_mfma_kernel<DT, 8, KVT, false>, attn_mfma_kernel<DT, 8, KVT, true>); break;
        default: go(attn_mfma_kernel<DT, 16, KVT, false>, attn_mfma_kernel<DT, 16, KVT, true>); break;
    }
}

// The attention kernels of one layer; two of them (the matrix-core kernel and the VALU kernel of the
// one-row sequences, or the group blocks and the VALU kernel) take disjoint rows and key splits, so with
// a second stream the second runs beside the first.
template <int DT, int KVT>
void launch_attention_kvt(const AttnArgs& a, const Plan& p, hipStream_t s, AuxStream* aux) {
    constexpr int DH = kAmDh;
    const bool two = p.attn_mfma ? p.attn_mixed : p.groups;
    std::unique_lock<std::mutex> lk;
    hipStream_t s2 = s;
    if (two && aux) {
        lk = std::unique_lock<std::mutex>(aux->mu);
        (void)hipEventRecord(aux->fork, s);
        (void)hipStreamWaitEvent(aux->s, aux->fork, 0);
        s2 = aux->s;
    }
    if (p.attn_mfma) {
        if (p.attn_mixed) {  // the one-row sequences: one-row groups of the VALU kernel, same splits
            AttnArgs av = a;
            av.rows_hi = 1;
            av.rg_blocks = 1;
            av.items = nullptr;
            launch_attention_kv<DT, DH, KVT>(av, p.B, p.M, 1, p.attn_hg1, false, s2, p.attn_nw1);
        }
        // the matrix cores take the prefix-group blocks and the sequences of 2+ rows (all, unless mixed)
        AttnArgs am = a;
        if (p.attn_mixed) am.rows_lo = 2;
        launch_attention_mfma<DT, KVT>(am, p.attn_items ? p.items_cap : p.B * p.rg_blocks, p.attn_hg, s);
    } else {
        if (p.groups) launch_attention_mfma<DT, KVT>(a, 0, p.grp_hg, s2);  // the group blocks alone
        launch_attention_kv<DT, DH, KVT>(a, p.B, p.M, p.rmax, p.attn_hg, false, s, p.attn_nw1);
    }
    if (s2 != s) {
        (void)hipEventRecord(aux->join, s2);
        (void)hipStreamWaitEvent(s, aux->join, 0);
    }
}

template <int DT, int DH>
void launch_attention(const AttnArgs& a, const Plan& p, int kv_dt, hipStream_t s, AuxStream* aux) {
    const bool merge_kernel = !p.merge_in_o;
    if constexpr (DT != F32 && DH == kAmDh) {
        if (p.attn_mfma || p.groups) {
            if (kv_dt == E4M3) launch_attention_kvt<DT, E4M3>(a, p, s, aux);
            else if (kv_dt == E5M2) launch_attention_kvt<DT, E5M2>(a, p, s, aux);
            else launch_attention_kvt<DT, DT>(a, p, s, aux);
            if (merge_kernel && a.n_splits > 1)
                launch1(VS_KERNEL_MERGE, attn_merge_kernel<DT, DH>, dim3(a.merge_rows ? p.B : p.M, a.n_heads),
                        dim3(DH), 0, s, a);
            return;
        }
    }
    if constexpr (DT != F32 && DH == 128) {
        if (kv_dt == E4M3)
            return launch_attention_kv<DT, DH, E4M3>(a, p.B, p.M, p.rmax, p.attn_hg, merge_kernel, s, p.attn_nw1);
        if (kv_dt == E5M2)
            return launch_attention_kv<DT, DH, E5M2>(a, p.B, p.M, p.rmax, p.attn_hg, merge_kernel, s, p.attn_nw1);
    }
    launch_attention_kv<DT, DH, DT>(a, p.B, p.M, p.rmax, p.attn_hg, merge_kernel, s, p.attn_nw1);
}

// Common epilogue fields of both product paths.
template <typename A>
void fill_epilogue(A& g, const Plan& p, const vs_batch_desc* d, const int32_t* bt, const vs_pool_desc* pg,
                   const int* row_seq, const int* row_pos, const float* rope_cs, const long* row_kvoff = nullptr) {
    g.row_kvoff = row_kvoff;
    g.block_tables = bt;
    g.max_blocks = d->max_blocks;
    g.num_pages = pg->num_pages;
    g.row_seq = row_seq;
    g.row_pos = row_pos;
    g.rope_cs = rope_cs;
    g.kv_base = kv_pool_base(d->pool);
    g.kv_dt = pg->dtype;  // the pool's codes are the kernels' storage types
    g.page_elems = (long)(kv_page_bytes(pg) / kv_elem_bytes(pg->dtype));
    g.layer_elems = 2L * p.Hkv * kPageTokens * p.Dh;
    g.head_dim = p.Dh;
    g.n_heads = p.H;
    g.n_kv_heads = p.Hkv;
    g.page_tokens = kPageTokens;
}

template <int DT>
vs_status run_step(const Plan& p, const vs_batch_desc* d, const int32_t* bt, const vs_weights* w,
                   const vs_step_out* out, char* ws, hipStream_t s, bool allow_aux) {
    const vs_pool_desc* pg = vs_pool_geometry(d->pool);
    int* row_seq = reinterpret_cast<int*>(ws + p.off_row_seq);
    int* row_pos = reinterpret_cast<int*>(ws + p.off_row_pos);
    long* row_kvoff = reinterpret_cast<long*>(ws + p.off_kvoff);
    float* rope_cs = reinterpret_cast<float*>(ws + p.off_rope);
    float* x = reinterpret_cast<float*>(ws + p.off_x);
    void* xn = ws + p.off_xn;
    void* qb = ws + p.off_q;
    void* attn = ws + p.off_attn;
    void* hmid = ws + p.off_h;
    float* part = reinterpret_cast<float*>(ws + p.off_part);
    void* xf = ws + p.off_xf;
    ArgPart* lmpart = reinterpret_cast<ArgPart*>(ws + p.off_lmpart);
    float* ksp = reinterpret_cast<float*>(ws + p.off_ksp);
    const float eps = w->dims.eps;

    PrepArgs pa;
    pa.q_start = d->q_start;
    pa.ctx_len = d->ctx_len;
    pa.B = p.B;
    pa.M = p.M;
    pa.head_dim = p.Dh;
    pa.theta = (double)w->dims.rope_theta;
    pa.tokens = d->tokens;
    pa.embed = w->embed;
    pa.vocab = p.V;
    pa.D = p.D;
    pa.row_seq = row_seq;
    pa.row_pos = row_pos;
    pa.rope_cs = rope_cs;
    pa.x = x;
    pa.row_kvoff = row_kvoff;
    pa.block_tables = bt;
    pa.max_blocks = d->max_blocks;
    pa.num_pages = pg->num_pages;
    pa.page_tokens = kPageTokens;
    pa.page_elems = (long)(kv_page_bytes(pg) / kv_elem_bytes(pg->dtype));
    pa.error_flags = d->error_flags;
    int* seq_group = reinterpret_cast<int*>(ws + p.off_grp);
    int* seq_gp = seq_group + p.B;
    int* merge_rows = seq_gp + p.B;
    int* merge_count = merge_rows + p.B;
    pa.seq_group = p.groups ? seq_group : nullptr;
    pa.seq_gp = p.groups ? seq_gp : nullptr;
    pa.merge_count = p.groups ? merge_count : nullptr;
    hipLaunchKernelGGL((prep_embed_kernel<DT>), dim3(p.M), dim3(256), 0, s, pa);
    if (p.groups) {
        GroupArgs ga;
        ga.group_seq0 = d->group_seq0;
        ga.group_n = d->group_n;
        ga.group_pages = d->group_pages;
        ga.max_group_size = d->max_group_size;
        ga.max_group_pages = d->max_group_pages;
        ga.q_start = d->q_start;
        ga.ctx_len = d->ctx_len;
        ga.block_tables = bt;
        ga.B = p.B;
        ga.max_blocks = d->max_blocks;
        ga.num_pages = pg->num_pages;
        ga.page_tokens = kPageTokens;
        ga.seq_group = seq_group;
        ga.seq_gp = seq_gp;
        ga.merge_rows = merge_rows;
        ga.merge_count = merge_count;
        ga.M = p.M;
        ga.error_flags = d->error_flags;
        hipLaunchKernelGGL(prefix_group_kernel, dim3(d->n_prefix_groups), dim3(256), 0, s, ga);
    }

    GemvArgs gv = {};
    fill_epilogue(gv, p, d, bt, pg, row_seq, row_pos, rope_cs, row_kvoff);
    gv.M = p.M;
    gv.xin = x;
    gv.xin_ld = p.D;
    gv.eps = eps;
    GemmArgs gm = {};
    fill_epilogue(gm, p, d, bt, pg, row_seq, row_pos, rope_cs, row_kvoff);
    gm.M = p.M;

    AttnArgs a = {};
    a.rows_lo = 0;
    a.rows_hi = 0x7fffffff;  // every sequence (the mixed launch narrows it)
    a.q = qb;
    a.kv_base = kv_pool_base(d->pool);
    a.page_elems = (long)(kv_page_bytes(pg) / kv_elem_bytes(pg->dtype));
    a.layer_elems = 2L * p.Hkv * kPageTokens * p.Dh;
    a.n_heads = p.H;
    a.n_kv_heads = p.Hkv;
    a.page_tokens = kPageTokens;
    a.block_tables = bt;
    a.max_blocks = d->max_blocks;
    a.num_pages = pg->num_pages;
    a.M = p.M;
    a.q_start = d->q_start;
    a.ctx_len = d->ctx_len;
    a.n_splits = p.n_splits;
    a.split_pages = p.split_pages;
    a.B = p.B;
    a.rg_blocks = p.rg_blocks;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p.Dh));
    a.part = part;
    a.out = attn;
    a.row_seq = row_seq;
    AuxStream* aux = allow_aux && ((p.attn_mfma && p.attn_mixed) || p.groups) ? aux_stream(s) : nullptr;
    if (p.attn_items) {
        a.items = reinterpret_cast<int2*>(ws + p.off_items);
        a.n_items = reinterpret_cast<int*>(ws + p.off_n_items);
        hipLaunchKernelGGL(attn_items_kernel, dim3(1), dim3(1024), 0, s, d->q_start, p.B, p.M, 16 / p.attn_hg,
                           p.attn_mixed ? 2 : 0, 0x7fffffff, reinterpret_cast<int2*>(ws + p.off_items), p.items_cap,
                           reinterpret_cast<int*>(ws + p.off_n_items));
    }
    if (p.groups) {
        a.seq_gp = seq_gp;
        a.seq_group = seq_group;
        a.group_seq0 = d->group_seq0;
        a.group_n = d->group_n;
        a.group_pages = d->group_pages;
        a.n_pre_splits = p.n_pre_splits;
        a.pre_split_pages = p.pre_split_pages;
        a.gz_blocks = p.gz_blocks;
        a.gz_per_group = p.gz_per_group;
        if (p.n_splits - p.n_pre_splits == 1) {  // only the grouped rows have splits to merge
            a.merge_rows = merge_rows;
            a.merge_count = merge_count;
        }
    }

    // the split-K residual products hand the next RMSNorm's output over in xn (fused into their
    // partial-sum reduction): the norm ahead of the next product is then already done
    bool xn_ready = false;
    for (int l = 0; l < p.L; ++l) {
        const vs_layer_weights& lw = w->layers[l];
        // RMSNorm(x) -> q, k, v; rotary; K/V into the pages
        if (p.gemv) {
            GemvArgs q = gv;
            q.w0 = lw.wq;
            q.w1 = lw.wk;
            q.w2 = lw.wv;
            q.K = p.D;
            q.gain = lw.attn_norm;
            q.q_out = qb;
            q.layer = l;
            q.n_units = (p.H + 2 * p.Hkv) * p.Dh / 2;
            launch_gemv<DT, X_NORM, EPI_QKV>(VS_KERNEL_QKV, q, s);
        } else {
            if (!xn_ready)
                hipLaunchKernelGGL((rmsnorm_kernel<DT>), dim3(p.M), dim3(1024), 0, s, x, (const int*)nullptr, p.M,
                                   lw.attn_norm, p.D, eps, xn);
            xn_ready = false;
            GemmArgs q = gm;
            q.w0 = lw.wq;
            q.w1 = lw.wk;
            q.w2 = lw.wv;
            q.n0 = p.H * p.Dh;
            q.n1 = p.Hkv * p.Dh;
            q.n2 = p.Hkv * p.Dh;
            q.K = p.D;
            q.act = xn;
            q.act_ld = p.D;
            q.n_tiles = (p.H + 2 * p.Hkv) * p.Dh / 32;
            q.q_out = qb;
            q.layer = l;
            if (p.strip_qkv) {
                q.n_tiles = (p.H + 2 * p.Hkv) * p.Dh / 16;
                if (p.strip_qkv == kStripUnitsQkvNarrow)
                    launch_strip<DT, EPI_QKV, kStripUnitsQkvNarrow>(VS_KERNEL_QKV, q, s);
                else
                    launch_strip<DT, EPI_QKV, kStripUnitsQkv>(VS_KERNEL_QKV, q, s);
            } else if (p.ksplit_qkv) {
                const int N = q.n0 + q.n1 + q.n2;
                const int slices = launch_ksplit<DT>(VS_KERNEL_QKV, lw.wq, lw.wk, lw.wv, q.n0, q.n1, N, p.D, xn, p.D,
                                                     p.M, ksp, s);
                const long threads = (long)p.M * (p.H + 2 * p.Hkv) * (p.Dh / 2);
                launchn(VS_KERNEL_QKV, qkv_reduce_kernel<DT>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                                   q, ksp, slices, N);
            } else {
                launch_gemm<DT, EPI_QKV>(VS_KERNEL_QKV, q, s);
            }
        }

        a.layer = l;
        if (p.Dh == 128) launch_attention<DT, 128>(a, p, pg->dtype, s, aux);
        else launch_attention<DT, 64>(a, p, pg->dtype, s, aux);

        // x += W_o attn
        if (p.gemv) {
            GemvArgs o = gv;
            o.w0 = lw.wo;
            o.K = p.H * p.Dh;
            o.act = attn;
            o.act_ld = p.H * p.Dh;
            o.x = x;
            o.x_ld = p.D;
            o.n_units = p.D;
            if (p.merge_in_o) {
                o.part = part;
                o.n_splits = p.n_splits;
                // fewer, wider workgroups: each one reads every split's statistics from L2
                launch_gemv<DT, X_MERGE, EPI_RESID>(VS_KERNEL_OPROJ, o, s, kGemvMergeUnits);
            } else {
                launch_gemv<DT, X_PLAIN, EPI_RESID>(VS_KERNEL_OPROJ, o, s);
            }
        } else {
            GemmArgs o = gm;
            o.w0 = lw.wo;
            o.n0 = p.D;
            o.K = p.H * p.Dh;
            o.act = attn;
            o.act_ld = p.H * p.Dh;
            o.n_tiles = (p.D + 15) / 16;
            o.x = x;
            o.x_ld = p.D;
            if (p.strip_o) {
                launch_strip_resid<DT>(VS_KERNEL_OPROJ, o, s);
            } else if (p.tile_slices > 1 && tile_ok<EPI_RESID>(o)) {
                launch_resid_tile<DT>(VS_KERNEL_OPROJ, o, p.tile_slices, ksp, s, lw.ffn_norm, eps, xn);
                xn_ready = true;
            } else if (p.ksplit) {
                launch_resid_ksplit<DT>(VS_KERNEL_OPROJ, lw.wo, p.D, p.H * p.Dh, attn, p.H * p.Dh, p.M, x, p.D, ksp, s,
                                        lw.ffn_norm, eps, xn);
                xn_ready = true;
            } else
                launch_gemm<DT, EPI_RESID>(VS_KERNEL_OPROJ, o, s);
        }

        // RMSNorm(x) -> silu(gate) * up
        if (p.gemv) {
            GemvArgs gu = gv;
            gu.w0 = lw.wg;
            gu.w1 = lw.wu;
            gu.K = p.D;
            gu.gain = lw.ffn_norm;
            gu.h_out = hmid;
            gu.h_ld = p.F;
            gu.n_units = p.F;
            launch_gemv<DT, X_NORM, EPI_SWIGLU>(VS_KERNEL_GATEUP, gu, s);
        } else {
            if (!xn_ready)
                hipLaunchKernelGGL((rmsnorm_kernel<DT>), dim3(p.M), dim3(1024), 0, s, x, (const int*)nullptr, p.M,
                                   lw.ffn_norm, p.D, eps, xn);
            xn_ready = false;
            GemmArgs gu = gm;
            gu.w0 = lw.wg;
            gu.w1 = lw.wu;
            gu.n0 = p.F;
            gu.n1 = p.F;
            gu.K = p.D;
            gu.act = xn;
            gu.act_ld = p.D;
            gu.n_tiles = (p.F + 15) / 16;
            gu.h_out = hmid;
            gu.h_ld = p.F;
            if (p.strip_gu) {
                gu.n_tiles = p.F / 8;
                if (p.strip_gu == kStripUnitsGuWide)
                    launch_strip<DT, EPI_SWIGLU, kStripUnitsGuWide>(VS_KERNEL_GATEUP, gu, s);
                else
                    launch_strip<DT, EPI_SWIGLU, kStripUnitsGu>(VS_KERNEL_GATEUP, gu, s);
            } else if (p.ksplit_gu) {
                const int slices = launch_ksplit<DT>(VS_KERNEL_GATEUP, lw.wg, lw.wu, lw.wu, p.F, p.F, 2 * p.F, p.D, xn,
                                                     p.D, p.M, ksp, s);
                const long threads = (long)p.M * p.F;
                launchn(VS_KERNEL_GATEUP, swiglu_reduce_kernel<DT>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                                   s, ksp, slices, p.M, p.F, hmid, p.F);
            } else {
                launch_gemm<DT, EPI_SWIGLU>(VS_KERNEL_GATEUP, gu, s);
            }
        }

        // x += W_d h
        if (p.gemv) {
            GemvArgs dn = gv;
            dn.w0 = lw.wd;
            dn.K = p.F;
            dn.act = hmid;
            dn.act_ld = p.F;
            dn.x = x;
            dn.x_ld = p.D;
            dn.n_units = p.D;
            launch_gemv<DT, X_PLAIN, EPI_RESID>(VS_KERNEL_DOWN, dn, s);
        } else {
            GemmArgs dn = gm;
            dn.w0 = lw.wd;
            dn.n0 = p.D;
            dn.K = p.F;
            dn.act = hmid;
            dn.act_ld = p.F;
            dn.n_tiles = (p.D + 15) / 16;
            dn.x = x;
            dn.x_ld = p.D;
            if (p.strip_down) {
                launch_strip_resid<DT>(VS_KERNEL_DOWN, dn, s);
            } else if (p.tile_slices > 1 && tile_ok<EPI_RESID>(dn)) {
                if (l + 1 < p.L) {
                    launch_resid_tile<DT>(VS_KERNEL_DOWN, dn, p.tile_slices, ksp, s, w->layers[l + 1].attn_norm, eps, xn);
                    xn_ready = true;
                } else {
                    launch_resid_tile<DT>(VS_KERNEL_DOWN, dn, p.tile_slices, ksp, s);
                }
            } else if (p.ksplit && l + 1 < p.L) {
                launch_resid_ksplit<DT>(VS_KERNEL_DOWN, lw.wd, p.D, p.F, hmid, p.F, p.M, x, p.D, ksp, s,
                                        w->layers[l + 1].attn_norm, eps, xn);
                xn_ready = true;
            } else if (p.ksplit) {
                launch_resid_ksplit<DT>(VS_KERNEL_DOWN, lw.wd, p.D, p.F, hmid, p.F, p.M, x, p.D, ksp, s);
            } else
                launch_gemm<DT, EPI_RESID>(VS_KERNEL_DOWN, dn, s);
        }
    }

    if (p.M_log > 0) {  // final RMSNorm of the logit rows -> LM head, argmax partials
        if (p.gemv) {
            GemvArgs lm = gv;
            lm.w0 = w->lm_head;
            lm.K = p.D;
            lm.gain = w->final_norm;
            lm.act_rows = d->logit_rows;
            lm.M = p.M_log;
            lm.logits = out->logits;
            lm.vocab = p.V;
            lm.parts = lmpart;
            lm.n_parts = p.n_lm_parts;
            lm.n_units = p.V;
            launch_gemv<DT, X_NORM, EPI_LOGITS>(VS_KERNEL_LMHEAD, lm, s);
        } else {
            hipLaunchKernelGGL((rmsnorm_kernel<DT>), dim3(p.M_log), dim3(1024), 0, s, x, d->logit_rows, p.M,
                               w->final_norm, p.D, eps, xf);
            GemmArgs lm = gm;
            lm.w0 = w->lm_head;
            lm.n0 = p.V;
            lm.K = p.D;
            lm.act = xf;
            lm.act_ld = p.D;
            lm.M = p.M_log;
            lm.n_tiles = p.n_lm_parts;
            lm.logits = out->logits;
            lm.vocab = p.V;
            lm.parts = lmpart;
            if (p.ksplit_lm) {
                const int slices = launch_ksplit<DT>(VS_KERNEL_LMHEAD, w->lm_head, w->lm_head, w->lm_head, p.V, 0, p.V,
                                                     p.D, xf, p.D, p.M_log, ksp, s);
                const long threads = (long)p.M_log * p.n_lm_parts;
                launchn(VS_KERNEL_LMHEAD, logits_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, ksp,
                                   slices, p.M_log, p.V, out->logits, lmpart, p.n_lm_parts);
            } else {
                launch_gemm<DT, EPI_LOGITS>(VS_KERNEL_LMHEAD, lm, s);
            }
        }
    }
    if (out->argmax || d->ctx_advance) {
        hipLaunchKernelGGL(argmax_accept_kernel, dim3(p.B), dim3(256), 0, s, lmpart, p.n_lm_parts, d->q_start, p.M,
                           d->logit_rows, p.M_log, d->tokens, out->g0, out->argmax, out->top2_gap, out->accept_len,
                           out->bonus, d->ctx_advance);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return vs_fail(VS_ERR_HIP, std::string("decode_step launch: ") + hipGetErrorString(e));
    return vs_ok();
}

}  // namespace

extern "C" vs_status decode_step_workspace_bytes(const vs_batch_desc* desc, const vs_model_desc* dims, size_t* bytes) {
    if (!bytes) return vs_fail(VS_ERR_INVALID, "decode_step_workspace_bytes: null output");
    Plan p;
    vs_status st = make_plan(desc, dims, &p);
    if (st != VS_OK) return st;
    *bytes = p.total;
    return vs_ok();
}

namespace {

// Argument checks shared by decode_step and decode_step_noalloc; fills the plan.
vs_status check_step(const vs_batch_desc* desc, const int32_t* block_tables, const vs_weights* weights,
                     const vs_step_out* out, Plan* p) {
    if (!desc || !weights || !out) return vs_fail(VS_ERR_INVALID, "decode_step: null argument");
    vs_status st = make_plan(desc, &weights->dims, p);
    if (st != VS_OK) return st;
    if (p->M == 0) return vs_ok();
    if (!desc->pool || !desc->q_start || !desc->ctx_len || !desc->tokens || !block_tables)
        return vs_fail(VS_ERR_INVALID, "decode_step: pool, q_start, ctx_len, tokens and block_tables are required");
    if (p->M_log > 0 && (!desc->logit_rows || !out->argmax))
        return vs_fail(VS_ERR_INVALID, "decode_step: logit rows need logit_rows and out->argmax");
    const bool fused = out->accept_len || out->bonus || out->g0;
    if (fused && !(out->accept_len && out->bonus && out->g0 && out->argmax))
        return vs_fail(VS_ERR_INVALID, "decode_step: fused acceptance needs g0, accept_len, bonus and argmax");
    if (!weights->embed || !weights->final_norm || !weights->lm_head || !weights->layers)
        return vs_fail(VS_ERR_INVALID, "decode_step: missing weight pointer");
    for (int l = 0; l < p->L; ++l) {
        const vs_layer_weights& lw = weights->layers[l];
        if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.ffn_norm || !lw.wg || !lw.wu || !lw.wd)
            return vs_fail(VS_ERR_INVALID, "decode_step: missing weight pointer in layer " + std::to_string(l));
    }
    const vs_pool_desc* pg = vs_pool_geometry(desc->pool);
    if (pg->page_tokens != kPageTokens || pg->n_layers != p->L || pg->n_kv_heads != p->Hkv || pg->head_dim != p->Dh)
        return vs_fail(VS_ERR_SHAPE, "decode_step: pool geometry does not match the model");
    const bool kv8 = pg->dtype == VS_FP8_E4M3 || pg->dtype == VS_FP8_E5M2;
    if (pg->dtype != p->dt && !(kv8 && p->dt != VS_F32 && p->Dh == 128))
        return vs_fail(VS_ERR_SHAPE, "decode_step: the pool's dtype must be the model's, or an 8-bit float for an "
                                     "fp16 / bf16 model with head_dim 128");
    return vs_ok();
}

// allow_aux: the step may make and use the device's second stream (the allocation-free entry point
// keeps to the caller's stream)
vs_status run_checked(const Plan& p, const vs_batch_desc* desc, const int32_t* block_tables,
                      const vs_weights* weights, const vs_step_out* out, char* w, hipStream_t stream, bool allow_aux) {
    switch (p.dt) {
        case VS_F32: return run_step<F32>(p, desc, block_tables, weights, out, w, stream, allow_aux);
        case VS_F16: return run_step<F16>(p, desc, block_tables, weights, out, w, stream, allow_aux);
        default: return run_step<BF16>(p, desc, block_tables, weights, out, w, stream, allow_aux);
    }
}

}  // namespace

extern "C" vs_status decode_step(const vs_batch_desc* desc, const int32_t* block_tables, const vs_weights* weights,
                                 const vs_step_out* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    Plan p;
    vs_status st = check_step(desc, block_tables, weights, out, &p);
    if (st != VS_OK || p.M == 0) return st;
    if (!ws || ws_bytes < p.total)
        return vs_fail(VS_ERR_SHAPE, "decode_step: workspace needs " + std::to_string(p.total) + " bytes");
    return run_checked(p, desc, block_tables, weights, out, static_cast<char*>(ws), stream, true);
}

// ---- the allocation-free variant: the workspace is a device array of the library itself -------
//
// One copy per GPU, alive until the process ends. In host code the array's name is only a host-side
// stand-in; its device address comes from hipGetSymbolAddress, taken once per device with that
// device current, and that address is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[VS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

vs_status scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return vs_fail(VS_ERR_HIP, std::string("decode_step_noalloc: hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return vs_fail(VS_ERR_INVALID, "decode_step_noalloc: device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return vs_fail(VS_ERR_HIP, std::string("decode_step_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return vs_ok();
}
}  // namespace

extern "C" vs_status decode_step_noalloc(const vs_batch_desc* desc, const int32_t* block_tables,
                                         const vs_weights* weights, const vs_step_out* out, hipStream_t stream) {
    Plan p;
    vs_status st = check_step(desc, block_tables, weights, out, &p);
    if (st != VS_OK || p.M == 0) return st;
    if (p.total > (size_t)VS_NOALLOC_SCRATCH_BYTES)
        return vs_fail(VS_ERR_SHAPE, "decode_step_noalloc: this batch needs " + std::to_string(p.total) +
                                         " bytes of workspace, more than the library's " +
                                         std::to_string((size_t)VS_NOALLOC_SCRATCH_BYTES) +
                                         "-byte scratch array; use decode_step with a caller workspace");
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != VS_OK) return st;
    return run_checked(p, desc, block_tables, weights, out, static_cast<char*>(ws), stream, false);
}

extern "C" vs_status verify_accept(int32_t B, const int32_t* q_start, const int32_t* drafts, const int32_t* g0,
                                   const int32_t* argmax, int32_t* accept_len, int32_t* bonus, hipStream_t stream) {
    if (B < 0) return vs_fail(VS_ERR_INVALID, "verify_accept: B < 0");
    if (B == 0) return vs_ok();
    if (!q_start || !drafts || !g0 || !argmax || !accept_len || !bonus)
        return vs_fail(VS_ERR_INVALID, "verify_accept: null argument");
    hipLaunchKernelGGL(verify_accept_kernel, dim3((B + 63) / 64), dim3(64), 0, stream, B, q_start, drafts, g0, argmax,
                       accept_len, bonus);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return vs_fail(VS_ERR_HIP, std::string("verify_accept launch: ") + hipGetErrorString(e));
    return vs_ok();
}

extern "C" vs_status verify_sample_workspace_bytes(int32_t B, int32_t M, int32_t V, size_t* bytes) {
    if (!bytes) return vs_fail(VS_ERR_INVALID, "verify_sample_workspace_bytes: null output");
    if (B < 0 || M < 0 || V < 1) return vs_fail(VS_ERR_INVALID, "verify_sample_workspace_bytes: bad sizes");
    *bytes = sizeof(float2) * (size_t)((int64_t)B + M) * (size_t)stats_segments(V);
    return vs_ok();
}

extern "C" vs_status verify_sample(int32_t B, int32_t M, int32_t V, const int32_t* q_start, const int32_t* drafts,
                                   const float* p0_logits, const float* logits, const float* q_probs, const float* u,
                                   const float* v, float temperature, int32_t* accept_len, int32_t* token, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
    if (B < 0 || M < 0) return vs_fail(VS_ERR_INVALID, "verify_sample: B < 0 or M < 0");
    if (B == 0) return vs_ok();
    if (V < 1) return vs_fail(VS_ERR_INVALID, "verify_sample: V < 1");
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return vs_fail(VS_ERR_INVALID, "verify_sample: temperature must be positive and finite");
    if (!q_start || !p0_logits || !v || !accept_len || !token || !ws)
        return vs_fail(VS_ERR_INVALID, "verify_sample: null argument");
    if (M > 0 && (!drafts || !logits || !q_probs || !u))
        return vs_fail(VS_ERR_INVALID, "verify_sample: drafts, logits, q_probs and u are required when M > 0");
    if ((int64_t)B + M > INT32_MAX) return vs_fail(VS_ERR_SHAPE, "verify_sample: B + M too large");
    const int n_seg = stats_segments(V);
    if (n_seg > 65535) return vs_fail(VS_ERR_SHAPE, "verify_sample: V too large");
    const size_t need = sizeof(float2) * (size_t)(B + M) * (size_t)n_seg;
    if (ws_bytes < need) return vs_fail(VS_ERR_SHAPE, "verify_sample: workspace needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) % alignof(float2))
        return vs_fail(VS_ERR_INVALID, "verify_sample: workspace must be 8-byte aligned");
    auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    const bool vec4 = V % 4 == 0 && a16(p0_logits) && a16(logits) && a16(q_probs);
    float2* part = static_cast<float2*>(ws);
    const float inv_t = 1.f / temperature;
    const StatsArgs sa{p0_logits, logits, B, V, n_seg, inv_t, part};
    const SampleArgs pa{B, M, V, n_seg, q_start, drafts, p0_logits, logits, q_probs, u, v, part, inv_t, accept_len, token};
    const dim3 sgrid(B + M, n_seg);
    if (vec4) {
        launch1(VS_KERNEL_SMSTATS, softmax_stats_kernel<true>, sgrid, dim3(kStatsThreads), 0, stream, sa);
        launch1(VS_KERNEL_SAMPLE, sample_pick_kernel<true>, dim3(B), dim3(kSampleThreads), 0, stream, pa);
    } else {
        launch1(VS_KERNEL_SMSTATS, softmax_stats_kernel<false>, sgrid, dim3(kStatsThreads), 0, stream, sa);
        launch1(VS_KERNEL_SAMPLE, sample_pick_kernel<false>, dim3(B), dim3(kSampleThreads), 0, stream, pa);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return vs_fail(VS_ERR_HIP, std::string("verify_sample launch: ") + hipGetErrorString(e));
    return vs_ok();
}

extern "C" vs_status vs_time_kernel(int32_t kind, void* const* start_events, void* const* stop_events,
                                    int32_t capacity) {
    if (kind < VS_KERNEL_NONE || kind > VS_KERNEL_SAMPLE) return vs_fail(VS_ERR_INVALID, "vs_time_kernel: bad kind");
    if (kind != VS_KERNEL_NONE && (capacity < 0 || (capacity > 0 && (!start_events || !stop_events))))
        return vs_fail(VS_ERR_INVALID, "vs_time_kernel: events required");
    g_timer.kind = kind;
    g_timer.start = start_events;
    g_timer.stop = stop_events;
    g_timer.capacity = kind == VS_KERNEL_NONE ? 0 : capacity;
    g_timer.count = 0;
    return vs_ok();
}

extern "C" int32_t vs_timed_launches(void) { return g_timer.count; }

extern "C" vs_status vs_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
    if (!buf || !sink) return vs_fail(VS_ERR_INVALID, "vs_stream_read: null argument");
    if (bytes == 0 || bytes % 8192 != 0) return vs_fail(VS_ERR_INVALID, "vs_stream_read: bytes must be a multiple of 8192");
    hipLaunchKernelGGL(stream_read_kernel, dim3(512), dim3(512), 0, stream, static_cast<const char*>(buf),
                       (long)(bytes / 8192), reinterpret_cast<unsigned*>(sink));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return vs_fail(VS_ERR_HIP, std::string("vs_stream_read launch: ") + hipGetErrorString(e));
    return vs_ok();
}
