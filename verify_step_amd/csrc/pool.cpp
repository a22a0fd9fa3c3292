// Host-side bookkeeping of the paged KV cache: a free list, per-page reference
// counts, block-table growth and copy-on-write of a shared, partly filled last
// page ([KV Cache] section 05 "The block table" and "Block sharing and
// copy-on-write"; [Serving Efficiency] section 31.3), and the prefix-cache
// index over full blocks ([KV Cache] section 05 "Prefix caching").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/verify_step.h"
#include "error.h"

struct vs_pool {
    vs_pool_desc desc;
    char* base;
    size_t bytes;
    size_t page_bytes;
    std::vector<int32_t> ref;        // reference count per page
    std::vector<int32_t> free_list;  // stack of free page ids (top = back)
    // prefix-cache index: chain hash of a full block -> the page holding it (one reference each)
    struct Entry {
        uint64_t parent;              // chain hash of the block before it (the root for block 0)
        std::vector<int32_t> tokens;  // the block's token ids (a hash match must also match these)
        int32_t page, depth;          // depth: the block's index in its chain
        uint64_t last_use;
    };
    std::unordered_map<uint64_t, Entry> index;
    uint64_t clock = 0;
};

extern "C" size_t kv_page_bytes(const vs_pool_desc* d) {
    if (!d) return 0;
    const size_t elem = d->dtype == VS_F32 ? 4 : (d->dtype == VS_FP8_E4M3 || d->dtype == VS_FP8_E5M2) ? 1 : 2;
    return (size_t)d->n_layers * 2 * d->n_kv_heads * d->page_tokens * d->head_dim * elem;
}

extern "C" vs_status kv_pool_create(const vs_pool_desc* desc, void* dev_base, size_t dev_bytes, vs_pool** out) {
    if (!desc || !out) return vs_fail(VS_ERR_INVALID, "kv_pool_create: null argument");
    *out = nullptr;
    if (desc->num_pages <= 0 || desc->page_tokens <= 0 || desc->n_layers <= 0 || desc->n_kv_heads <= 0 ||
        desc->head_dim <= 0)
        return vs_fail(VS_ERR_INVALID, "kv_pool_create: every size must be positive");
    if (desc->dtype < VS_F32 || desc->dtype > VS_FP8_E5M2)
        return vs_fail(VS_ERR_INVALID, "kv_pool_create: unknown dtype");
    const size_t pb = kv_page_bytes(desc);
    if (!dev_base || dev_bytes < pb * (size_t)desc->num_pages)
        return vs_fail(VS_ERR_INVALID, "kv_pool_create: device region smaller than num_pages pages");
    vs_pool* p = new vs_pool;
    p->desc = *desc;
    p->base = static_cast<char*>(dev_base);
    p->bytes = dev_bytes;
    p->page_bytes = pb;
    p->ref.assign(desc->num_pages, 0);
    p->free_list.reserve(desc->num_pages);
    for (int32_t i = desc->num_pages - 1; i >= 0; --i) p->free_list.push_back(i);  // pops 0, 1, 2, ...
    *out = p;
    return vs_ok();
}

extern "C" void kv_pool_destroy(vs_pool* pool) { delete pool; }

extern "C" vs_status kv_alloc(vs_pool* pool, int32_t n, int32_t* out_ids) {
    if (!pool || (n > 0 && !out_ids)) return vs_fail(VS_ERR_INVALID, "kv_alloc: null argument");
    if (n < 0) return vs_fail(VS_ERR_INVALID, "kv_alloc: negative count");
    if ((size_t)n > pool->free_list.size())
        return vs_fail(VS_ERR_OOM, "kv_alloc: " + std::to_string(n) + " pages requested, " +
                                       std::to_string(pool->free_list.size()) + " free");
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = pool->free_list.back();
        pool->free_list.pop_back();
        pool->ref[id] = 1;
        out_ids[i] = id;
    }
    return vs_ok();
}

static bool valid_id(const vs_pool* pool, int32_t id) { return id >= 0 && id < pool->desc.num_pages; }

extern "C" vs_status kv_share(vs_pool* pool, const int32_t* ids, int32_t n) {
    if (!pool || (n > 0 && !ids) || n < 0) return vs_fail(VS_ERR_INVALID, "kv_share: bad argument");
    for (int32_t i = 0; i < n; ++i)
        if (!valid_id(pool, ids[i]) || pool->ref[ids[i]] == 0)
            return vs_fail(VS_ERR_INVALID, "kv_share: page " + std::to_string(ids[i]) + " is not in use");
    for (int32_t i = 0; i < n; ++i) pool->ref[ids[i]] += 1;
    return vs_ok();
}

extern "C" vs_status kv_free(vs_pool* pool, const int32_t* ids, int32_t n) {
    if (!pool || (n > 0 && !ids) || n < 0) return vs_fail(VS_ERR_INVALID, "kv_free: bad argument");
    // check every drop first (a page listed k times needs k references), then apply
    std::unordered_map<int32_t, int32_t> drops;
    for (int32_t i = 0; i < n; ++i) {
        if (!valid_id(pool, ids[i])) return vs_fail(VS_ERR_INVALID, "kv_free: page id out of range");
        drops[ids[i]] += 1;
    }
    for (const auto& kv : drops) {
        if (pool->ref[kv.first] < kv.second)
            return vs_fail(VS_ERR_INVALID, "kv_free: page " + std::to_string(kv.first) + " has fewer references (" +
                                               std::to_string(pool->ref[kv.first]) + ") than drops");
    }
    for (int32_t i = 0; i < n; ++i) {
        if (--pool->ref[ids[i]] == 0) pool->free_list.push_back(ids[i]);
    }
    return vs_ok();
}

extern "C" vs_status kv_append(vs_pool* pool, int32_t* bt_row, int32_t* n_blocks, int32_t max_blocks, int32_t cur_len,
                               int32_t n_new, hipStream_t stream) {
    if (!pool || !bt_row || !n_blocks) return vs_fail(VS_ERR_INVALID, "kv_append: null argument");
    if (cur_len < 0 || n_new < 0) return vs_fail(VS_ERR_INVALID, "kv_append: negative length");
    const int32_t T = pool->desc.page_tokens;
    const int32_t have = *n_blocks;
    if (have != (cur_len + T - 1) / T)
        return vs_fail(VS_ERR_INVALID, "kv_append: block count does not match the sequence length");
    const int32_t need = (cur_len + n_new + T - 1) / T;
    if (need > max_blocks) return vs_fail(VS_ERR_SHAPE, "kv_append: block table row too short");
    for (int32_t i = 0; i < have; ++i)
        if (!valid_id(pool, bt_row[i]) || pool->ref[bt_row[i]] == 0)
            return vs_fail(VS_ERR_INVALID, "kv_append: block table holds a page that is not in use");
    const bool cow = n_new > 0 && (cur_len % T) != 0 && pool->ref[bt_row[have - 1]] > 1;
    const int32_t n_alloc = (need - have) + (cow ? 1 : 0);
    if ((size_t)n_alloc > pool->free_list.size())
        return vs_fail(VS_ERR_OOM, "kv_append: " + std::to_string(n_alloc) + " pages needed, " +
                                       std::to_string(pool->free_list.size()) + " free");
    if (cow) {
        const int32_t old = bt_row[have - 1];
        const int32_t fresh = pool->free_list.back();
        hipError_t e = hipMemcpyAsync(pool->base + (size_t)fresh * pool->page_bytes,
                                      pool->base + (size_t)old * pool->page_bytes, pool->page_bytes,
                                      hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return vs_fail(VS_ERR_HIP, std::string("kv_append: page copy: ") + hipGetErrorString(e));
        pool->free_list.pop_back();
        pool->ref[fresh] = 1;
        pool->ref[old] -= 1;  // still > 0: another sequence holds it
        bt_row[have - 1] = fresh;
    }
    for (int32_t i = have; i < need; ++i) {
        const int32_t id = pool->free_list.back();
        pool->free_list.pop_back();
        pool->ref[id] = 1;
        bt_row[i] = id;
    }
    *n_blocks = need;
    return vs_ok();
}

extern "C" int32_t kv_num_free(const vs_pool* pool) { return pool ? (int32_t)pool->free_list.size() : -1; }

extern "C" int32_t kv_refcount(const vs_pool* pool, int32_t page) {
    if (!pool || !valid_id(pool, page)) return -1;
    return pool->ref[page];
}

extern "C" void* kv_pool_base(const vs_pool* pool) { return pool ? pool->base : nullptr; }

// ---- prefix-cache index ([KV Cache] section 05 "Prefix caching"; [Serving Efficiency] section 31.3)

namespace {

// 64-bit FNV-1a (Fowler, Noll, Vo): offset basis 0xcbf29ce484222325, prime 0x100000001b3.
uint64_t fnv1a64(uint64_t h, const void* data, size_t n) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 0x100000001b3ULL;
    }
    return h;
}
constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ULL;

// one block: FNV-1a over the parent's 8 little-endian bytes, then each token id's 4
uint64_t block_hash(uint64_t parent, const int32_t* tokens, int32_t T) {
    unsigned char buf[8];
    for (int i = 0; i < 8; ++i) buf[i] = (unsigned char)(parent >> (8 * i));
    uint64_t h = fnv1a64(kFnvBasis, buf, 8);
    for (int32_t t = 0; t < T; ++t) {
        const uint32_t v = (uint32_t)tokens[t];
        const unsigned char b[4] = {(unsigned char)v, (unsigned char)(v >> 8), (unsigned char)(v >> 16),
                                    (unsigned char)(v >> 24)};
        h = fnv1a64(h, b, 4);
    }
    return h;
}

}  // namespace

extern "C" vs_status kv_prefix_root(const void* key, size_t len, uint64_t* root) {
    if (!root || (len > 0 && !key)) return vs_fail(VS_ERR_INVALID, "kv_prefix_root: null argument");
    *root = fnv1a64(kFnvBasis, key, len);
    return vs_ok();
}

extern "C" vs_status kv_prefix_chain(uint64_t root, const int32_t* tokens, int32_t n_tokens, int32_t page_tokens,
                                     uint64_t* hashes) {
    if (n_tokens < 0 || page_tokens <= 0) return vs_fail(VS_ERR_INVALID, "kv_prefix_chain: bad size");
    const int32_t n = n_tokens / page_tokens;
    if (n > 0 && (!tokens || !hashes)) return vs_fail(VS_ERR_INVALID, "kv_prefix_chain: null argument");
    uint64_t h = root;
    for (int32_t i = 0; i < n; ++i) hashes[i] = h = block_hash(h, tokens + (size_t)i * page_tokens, page_tokens);
    return vs_ok();
}

extern "C" vs_status kv_prefix_insert(vs_pool* pool, uint64_t root, const uint64_t* hashes, const int32_t* tokens,
                                      const int32_t* pages, int32_t n_blocks, int32_t* n_added) {
    if (!pool || n_blocks < 0 || (n_blocks > 0 && (!hashes || !tokens || !pages)))
        return vs_fail(VS_ERR_INVALID, "kv_prefix_insert: bad argument");
    const int32_t T = pool->desc.page_tokens;
    for (int32_t i = 0; i < n_blocks; ++i) {
        if (!valid_id(pool, pages[i]) || pool->ref[pages[i]] == 0)
            return vs_fail(VS_ERR_INVALID, "kv_prefix_insert: page " + std::to_string(pages[i]) + " is not in use");
        const uint64_t parent = i == 0 ? root : hashes[i - 1];
        if (block_hash(parent, tokens + (size_t)i * T, T) != hashes[i])
            return vs_fail(VS_ERR_INVALID, "kv_prefix_insert: hash " + std::to_string(i) +
                                               " is not the chain hash of its block");
    }
    const uint64_t now = ++pool->clock;
    int32_t added = 0;
    for (int32_t i = 0; i < n_blocks; ++i) {
        auto it = pool->index.find(hashes[i]);
        if (it != pool->index.end()) {  // already held (another sequence computed it first)
            it->second.last_use = now;
            continue;
        }
        vs_pool::Entry e;
        e.parent = i == 0 ? root : hashes[i - 1];
        e.tokens.assign(tokens + (size_t)i * T, tokens + (size_t)(i + 1) * T);
        e.page = pages[i];
        e.depth = i;
        e.last_use = now;
        pool->index.emplace(hashes[i], std::move(e));
        pool->ref[pages[i]] += 1;  // the index's own reference
        ++added;
    }
    if (n_added) *n_added = added;
    return vs_ok();
}

extern "C" vs_status kv_prefix_lookup(vs_pool* pool, uint64_t root, const uint64_t* hashes, const int32_t* tokens,
                                      int32_t n_blocks, int32_t* pages_out, int32_t* n_hit) {
    if (!pool || !n_hit || n_blocks < 0 || (n_blocks > 0 && (!hashes || !tokens || !pages_out)))
        return vs_fail(VS_ERR_INVALID, "kv_prefix_lookup: bad argument");
    const int32_t T = pool->desc.page_tokens;
    const uint64_t now = ++pool->clock;
    int32_t hit = 0;
    for (; hit < n_blocks; ++hit) {
        auto it = pool->index.find(hashes[hit]);
        if (it == pool->index.end()) break;
        const vs_pool::Entry& e = it->second;
        const uint64_t parent = hit == 0 ? root : hashes[hit - 1];
        if (e.parent != parent || std::memcmp(e.tokens.data(), tokens + (size_t)hit * T, sizeof(int32_t) * T) != 0)
            break;  // a hash collision: not this prefix
    }
    for (int32_t i = 0; i < hit; ++i) {
        vs_pool::Entry& e = pool->index.find(hashes[i])->second;
        e.last_use = now;
        pool->ref[e.page] += 1;  // the caller's reference
        pages_out[i] = e.page;
    }
    *n_hit = hit;
    return vs_ok();
}

extern "C" vs_status kv_prefix_evict(vs_pool* pool, int32_t n_pages, int32_t* n_freed) {
    if (!pool || n_pages < 0) return vs_fail(VS_ERR_INVALID, "kv_prefix_evict: bad argument");
    // candidates: entries only the index still holds; least recently used first, deeper blocks first
    std::vector<std::tuple<uint64_t, int32_t, uint64_t>> cand;  // (last_use, -depth, hash)
    for (const auto& kv : pool->index)
        if (pool->ref[kv.second.page] == 1) cand.emplace_back(kv.second.last_use, -kv.second.depth, kv.first);
    std::sort(cand.begin(), cand.end());
    int32_t freed = 0;
    for (const auto& c : cand) {
        if (freed >= n_pages) break;
        auto it = pool->index.find(std::get<2>(c));
        const int32_t page = it->second.page;
        pool->index.erase(it);
        pool->ref[page] = 0;
        pool->free_list.push_back(page);
        ++freed;
    }
    if (n_freed) *n_freed = freed;
    return vs_ok();
}

extern "C" int32_t kv_prefix_entries(const vs_pool* pool) { return pool ? (int32_t)pool->index.size() : -1; }

// internal accessors for the step
const vs_pool_desc* vs_pool_geometry(const vs_pool* pool) { return &pool->desc; }
