// C ABI entry points: argument validation on the host, then kernel launches
// on the caller's stream.  Nothing is enqueued when validation fails.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "mi_internal.h"

namespace mi {
size_t build_index_lds_bytes(int32_t N, int32_t n_slash);
}

// The built-in schedule buffer of mi_sparse_prefill_noalloc: one copy per
// GPU, in the library's device globals, held until the process ends.  Host
// code never passes the array's name to a kernel (in host code it is a
// host-side stand-in); it uses the device address hipGetSymbolAddress
// returns, looked up once per device with that device current
// (scratch_pointer below).
static __device__ __align__(256) int32_t scratch[MI_NOALLOC_SCHEDULE_ENTRIES];

namespace {

thread_local std::string g_last_error;

mi_status fail(mi_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mi_status fail(mi_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

constexpr size_t kMaxLds = 150 * 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mi_status check_desc(const mi_attn_desc* d) {
    if (!d) return fail(MI_ERR_NULL, "desc is NULL");
    if (d->batch < 1 || d->heads_q < 1 || d->heads_kv < 1)
        return fail(MI_ERR_SHAPE, "batch, heads_q and heads_kv must be >= 1");
    if (d->heads_q > MI_MAX_HEADS)
        return fail(MI_ERR_SHAPE, "heads_q %d exceeds %d", d->heads_q, MI_MAX_HEADS);
    if (d->heads_q % d->heads_kv != 0)
        return fail(MI_ERR_SHAPE, "heads_q %d is not a multiple of heads_kv %d", d->heads_q, d->heads_kv);
    if (d->seq_len < MI_BLOCK || d->seq_len % MI_BLOCK != 0)
        return fail(MI_ERR_SHAPE, "seq_len %d must be a positive multiple of 64", d->seq_len);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(MI_ERR_SHAPE, "head_dim %d not in {64, 128}", d->head_dim);
    if (d->dtype != MI_F32 && d->dtype != MI_BF16) return fail(MI_ERR_DTYPE, "unknown dtype %d", d->dtype);
    if (!(d->scale > 0.f) || !std::isfinite(d->scale))
        return fail(MI_ERR_SHAPE, "scale must be finite and > 0");
    const int64_t* strides[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
    const char* names[4] = {"q", "k", "v", "o"};
    for (int t = 0; t < 4; ++t)
        for (int i = 0; i < 3; ++i)
            if (strides[t][i] < 0 || strides[t][i] % 8 != 0)
                return fail(MI_ERR_SHAPE, "%s_stride[%d] = %lld must be a non-negative multiple of 8",
                            names[t], i, (long long)strides[t][i]);
    return MI_OK;
}

mi_status check_heads(const mi_attn_desc* d, const int32_t* heads, int32_t n_heads) {
    if (!heads) return fail(MI_ERR_NULL, "heads is NULL");
    if (n_heads < 1 || n_heads > d->heads_q)
        return fail(MI_ERR_PATTERN, "n_heads %d out of [1, %d]", n_heads, d->heads_q);
    for (int i = 0; i < n_heads; ++i) {
        if (heads[i] < 0 || heads[i] >= d->heads_q)
            return fail(MI_ERR_PATTERN, "heads[%d] = %d out of range", i, heads[i]);
        if (i > 0 && heads[i] <= heads[i - 1])
            return fail(MI_ERR_PATTERN, "heads must be strictly increasing");
    }
    return MI_OK;
}

mi_status check_patterns(const mi_attn_desc* d, const int32_t* pat) {
    for (int h = 0; h < d->heads_q; ++h)
        if (pat[h] < MI_ASHAPE || pat[h] > MI_VSLASH_EXACT)
            return fail(MI_ERR_PATTERN, "head_pattern[%d] = %d is not a pattern code", h, pat[h]);
    return MI_OK;
}

int ashape_max_blocks(int nb, int sink, int local) {
    const int v = (sink + 63) / 64 + (local + 126) / 64;
    return v < nb ? v : nb;
}

void copy_strides(int64_t* dst, const int64_t* src) {
    for (int i = 0; i < 3; ++i) dst[i] = src[i];
}

mi_status launched(hipError_t e) {
    if (e != hipSuccess) return fail(MI_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    return MI_OK;
}

// Validation and argument packing shared by the two attention entry points.
mi_status prepare_attn(const mi_attn_desc* d, const void* q, const void* k, const void* v,
                       const int32_t* head_pattern, const mi_index* idx, int32_t sink_tokens,
                       int32_t local_tokens, void* o, float* lse, mi::AttnArgs& a) {
    mi_status st = check_desc(d);
    if (st != MI_OK) return st;
    if (!q || !k || !v || !o) return fail(MI_ERR_NULL, "q, k, v or o is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(MI_ERR_SHAPE, "q, k, v and o must be 16-byte aligned");
    bool any_sparse = false, any_vs = false, any_a = false, any_exact = false;
    if (head_pattern) {
        if ((st = check_patterns(d, head_pattern)) != MI_OK) return st;
        for (int h = 0; h < d->heads_q; ++h) {
            any_sparse |= head_pattern[h] != MI_DENSE;
            any_vs |= head_pattern[h] == MI_VSLASH || head_pattern[h] == MI_VSLASH_EXACT;
            any_exact |= head_pattern[h] == MI_VSLASH_EXACT;
            any_a |= head_pattern[h] == MI_ASHAPE;
        }
    }
    if (any_sparse) {
        if (!idx || !idx->block_count || !idx->block_idx)
            return fail(MI_ERR_NULL, "sparse heads need idx with block_count and block_idx");
        if (idx->block_cap < 1) return fail(MI_ERR_BUDGET, "idx->block_cap must be >= 1");
        if (any_vs && (!idx->col_count || !idx->col_idx || idx->col_cap < 1))
            return fail(MI_ERR_NULL, "Vertical-Slash heads need idx->col_count, col_idx and col_cap >= 1");
        if (any_exact && !idx->vs_bits) return fail(MI_ERR_NULL, "exact Vertical-Slash heads need idx->vs_bits");
    }
    if (any_a && (sink_tokens < 0 || local_tokens < 1))
        return fail(MI_ERR_BUDGET, "A-shape needs sink_tokens >= 0 and local_tokens >= 1");
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    copy_strides(a.qs, d->q_stride);
    copy_strides(a.ks, d->k_stride);
    copy_strides(a.vs, d->v_stride);
    copy_strides(a.os, d->o_stride);
    a.B = d->batch; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.N = d->seq_len; a.D = d->head_dim;
    a.dtype = d->dtype; a.scale = d->scale;
    if (any_sparse) {
        a.block_count = idx->block_count; a.block_idx = idx->block_idx;
        a.col_count = idx->col_count; a.col_idx = idx->col_idx;
        a.block_cap = idx->block_cap; a.col_cap = idx->col_cap;
        a.vs_bits = any_exact ? idx->vs_bits : nullptr;
    }
    a.sink = sink_tokens; a.local = local_tokens;
    a.all_dense = head_pattern ? 0 : 1;
    for (int h = 0; h < d->heads_q; ++h) a.pattern[h] = head_pattern ? (uint8_t)head_pattern[h] : (uint8_t)MI_DENSE;
    const size_t es = d->dtype == MI_BF16 ? 2 : 4;
    if ((uint64_t)d->k_stride[2] * es * MI_BLOCK >= (1ull << 31) || (uint64_t)d->v_stride[2] * es * MI_BLOCK >= (1ull << 31))
        return fail(MI_ERR_SHAPE, "K/V token strides too large (64 rows must span < 2 GiB)");
    // the attention addresses a head's K and V rows by 32-bit byte offsets
    if ((uint64_t)d->k_stride[2] * es * d->seq_len >= (1ull << 32) ||
        (uint64_t)d->v_stride[2] * es * d->seq_len >= (1ull << 32))
        return fail(MI_ERR_SHAPE, "K/V token strides too large (seq_len rows must span < 4 GiB)");
    const size_t lds = mi::sparse_attn_lds_bytes(a);
    if (lds > mi::kAttnMaxLds)
        return fail(MI_ERR_SHAPE, "attention needs %zu bytes of LDS (> %zu): seq_len or col_cap too large", lds,
                    mi::kAttnMaxLds);
    return MI_OK;
}

// Builds the item schedule into `sched` (device memory) and launches the
// attention that reads it, both on stream s.
mi_status launch_scheduled(mi::AttnArgs& a, int32_t* sched, hipStream_t s) {
    mi_status st = launched(mi::launch_attn_schedule(a, sched, s));
    if (st != MI_OK) return st;
    a.sched = sched;
    a.sched_len = mi::attn_schedule_len(a);
    return launched(mi::launch_sparse_attn(a, s));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

mi_status scratch_pointer(int32_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(MI_ERR_LAUNCH, "no current HIP device (or device id >= %d)", kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MI_ERR_LAUNCH, "hipGetSymbolAddress of the schedule buffer failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<int32_t*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return MI_OK;
}

}  // namespace

extern "C" {

const char* mi_status_str(mi_status s) {
    switch (s) {
        case MI_OK: return "ok";
        case MI_ERR_NULL: return "null pointer";
        case MI_ERR_SHAPE: return "unsupported shape";
        case MI_ERR_BUDGET: return "budget out of range";
        case MI_ERR_DTYPE: return "unknown dtype";
        case MI_ERR_WORKSPACE: return "workspace too small";
        case MI_ERR_LAUNCH: return "kernel launch failed";
        case MI_ERR_PATTERN: return "bad head list or pattern";
    }
    return "unknown status";
}

const char* mi_last_error(void) { return g_last_error.c_str(); }

size_t mi_workspace_bytes(const mi_attn_desc* d, int32_t op, int32_t p0, int32_t p1) {
    (void)p1;
    if (check_desc(d) != MI_OK || p0 < 0) return 0;
    switch (op) {
        case MI_OP_VS_ESTIMATE: return mi::vs_workspace_bytes(d->batch, p0, d->seq_len, false);
        case MI_OP_BLOCK_ESTIMATE:
            return mi::bs_workspace_bytes(d->batch, p0, d->heads_kv, d->seq_len, d->head_dim, false);
        case MI_OP_SPARSE_PREFILL:
            return (mi::attn_schedule_bytes(d->batch, d->heads_q, d->heads_kv, d->seq_len) + 255) & ~size_t(255);
        case MI_OP_ANTIDIAG_ESTIMATE: return mi::ad_workspace_bytes(d->batch, p0, d->seq_len, false);
    }
    return 0;
}

mi_status mi_vs_estimate(const mi_attn_desc* d, const void* q, const void* k, const int32_t* heads,
                         int32_t n_heads, int32_t last_q, int32_t n_vertical, int32_t n_slash,
                         int32_t force_vertical, int32_t force_slash, int32_t* vertical_idx,
                         int32_t* slash_idx, float* vertical_score, float* slash_score, void* ws,
                         size_t ws_bytes, void* stream) {
    mi_status st = check_desc(d);
    if (st != MI_OK) return st;
    if (!q || !k || !vertical_idx || !slash_idx) return fail(MI_ERR_NULL, "q, k, vertical_idx or slash_idx is NULL");
    if (!aligned16(q) || !aligned16(k)) return fail(MI_ERR_SHAPE, "q and k must be 16-byte aligned");
    if ((vertical_score == nullptr) != (slash_score == nullptr))
        return fail(MI_ERR_NULL, "vertical_score and slash_score must both be given or both be NULL");
    if ((st = check_heads(d, heads, n_heads)) != MI_OK) return st;
    if (last_q < 1 || last_q > 64 || last_q > d->seq_len)
        return fail(MI_ERR_BUDGET, "last_q %d out of [1, min(64, seq_len)]", last_q);
    if (n_vertical < 1 || n_slash < 1) return fail(MI_ERR_BUDGET, "budgets must be >= 1");
    if (force_vertical < 1 || force_vertical > n_vertical || force_vertical > d->seq_len)
        return fail(MI_ERR_BUDGET, "force_vertical %d out of [1, min(n_vertical, seq_len)]", force_vertical);
    if (force_slash < 1 || force_slash > n_slash || force_slash > d->seq_len)
        return fail(MI_ERR_BUDGET, "force_slash %d out of [1, min(n_slash, seq_len)]", force_slash);
    const size_t need = mi::vs_workspace_bytes(d->batch, n_heads, d->seq_len, vertical_score != nullptr);
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(MI_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    mi::VsArgs a{};
    a.q = q; a.k = k;
    copy_strides(a.qs, d->q_stride);
    copy_strides(a.ks, d->k_stride);
    a.B = d->batch; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.N = d->seq_len; a.D = d->head_dim;
    a.dtype = d->dtype; a.scale = d->scale;
    a.n_heads = n_heads;
    for (int i = 0; i < n_heads; ++i) a.heads[i] = heads[i];
    a.last_q = last_q;
    a.n_vertical = n_vertical; a.n_slash = n_slash;
    a.force_vertical = force_vertical; a.force_slash = force_slash;
    a.vertical_idx = vertical_idx; a.slash_idx = slash_idx;
    a.vscore = vertical_score; a.sscore = slash_score;
    a.ws = ws;
    return launched(mi::launch_vs_estimate(a, static_cast<hipStream_t>(stream)));
}

mi_status mi_block_estimate(const mi_attn_desc* d, const void* q, const void* k, const int32_t* heads,
                            int32_t n_heads, int32_t top_blocks, int32_t* block_idx,
                            int32_t* block_count, float* block_score, void* ws, size_t ws_bytes,
                            void* stream) {
    mi_status st = check_desc(d);
    if (st != MI_OK) return st;
    if (!q || !k || !block_idx || !block_count) return fail(MI_ERR_NULL, "q, k, block_idx or block_count is NULL");
    if (!aligned16(q) || !aligned16(k)) return fail(MI_ERR_SHAPE, "q and k must be 16-byte aligned");
    if ((st = check_heads(d, heads, n_heads)) != MI_OK) return st;
    if (top_blocks < 2) return fail(MI_ERR_BUDGET, "top_blocks %d must be >= 2 (blocks 0 and a are kept)", top_blocks);
    const int nb = d->seq_len / MI_BLOCK;
    if ((size_t)nb * 4 + 12 * 1024 > kMaxLds)
        return fail(MI_ERR_SHAPE, "seq_len %d too long for the block estimate (nb <= %zu)", d->seq_len,
                    (kMaxLds - 12 * 1024) / 4);
    const size_t need = mi::bs_workspace_bytes(d->batch, n_heads, d->heads_kv, d->seq_len, d->head_dim,
                                               block_score != nullptr);
    if (ws_bytes < need || !ws) return fail(MI_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    mi::BsArgs a{};
    a.q = q; a.k = k;
    copy_strides(a.qs, d->q_stride);
    copy_strides(a.ks, d->k_stride);
    a.B = d->batch; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.N = d->seq_len; a.D = d->head_dim;
    a.dtype = d->dtype; a.scale = d->scale;
    a.n_heads = n_heads;
    for (int i = 0; i < n_heads; ++i) a.heads[i] = heads[i];
    a.top = top_blocks;
    a.block_idx = block_idx; a.block_count = block_count;
    a.w = block_score;
    a.ws = ws;
    return launched(mi::launch_block_estimate(a, static_cast<hipStream_t>(stream)));
}

mi_status mi_antidiag_estimate(const mi_attn_desc* d, const void* q, const void* k, const int32_t* heads,
                               int32_t n_heads, int32_t top_blocks, int32_t* block_idx, int32_t* block_count,
                               float* block_score, void* ws, size_t ws_bytes, void* stream) {
    mi_status st = check_desc(d);
    if (st != MI_OK) return st;
    if (!q || !k || !block_idx || !block_count) return fail(MI_ERR_NULL, "q, k, block_idx or block_count is NULL");
    if (!aligned16(q) || !aligned16(k)) return fail(MI_ERR_SHAPE, "q and k must be 16-byte aligned");
    if ((st = check_heads(d, heads, n_heads)) != MI_OK) return st;
    if (top_blocks < 2) return fail(MI_ERR_BUDGET, "top_blocks %d must be >= 2 (blocks 0 and a are kept)", top_blocks);
    const int nb = d->seq_len / MI_BLOCK;
    if ((size_t)nb * 4 + 12 * 1024 > kMaxLds)
        return fail(MI_ERR_SHAPE, "seq_len %d too long for the block estimate (nb <= %zu)", d->seq_len,
                    (kMaxLds - 12 * 1024) / 4);
    const size_t need = mi::ad_workspace_bytes(d->batch, n_heads, d->seq_len, block_score != nullptr);
    if (ws_bytes < need || !ws) return fail(MI_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    mi::BsArgs a{};
    a.q = q; a.k = k;
    copy_strides(a.qs, d->q_stride);
    copy_strides(a.ks, d->k_stride);
    a.B = d->batch; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.N = d->seq_len; a.D = d->head_dim;
    a.dtype = d->dtype; a.scale = d->scale;
    a.n_heads = n_heads;
    for (int i = 0; i < n_heads; ++i) a.heads[i] = heads[i];
    a.top = top_blocks;
    a.block_idx = block_idx; a.block_count = block_count;
    a.w = block_score;
    a.ws = ws;
    return launched(mi::launch_antidiag_estimate(a, static_cast<hipStream_t>(stream)));
}

mi_status mi_build_index(const mi_attn_desc* d, const int32_t* head_pattern, const int32_t* vertical_idx,
                         int32_t n_vertical, const int32_t* slash_idx, int32_t n_slash,
                         const int32_t* bs_block_idx, const int32_t* bs_block_count, int32_t top_blocks,
                         int32_t sink_tokens, int32_t local_tokens, const mi_index* out, void* stream) {
    mi_status st = check_desc(d);
    if (st != MI_OK) return st;
    if (!head_pattern) return fail(MI_ERR_NULL, "head_pattern is NULL");
    if ((st = check_patterns(d, head_pattern)) != MI_OK) return st;
    if (!out || !out->block_count || !out->block_idx || !out->col_count)
        return fail(MI_ERR_NULL, "out, out->block_count, out->block_idx or out->col_count is NULL");
    const int nb = d->seq_len / MI_BLOCK;
    bool any_vs = false, any_bs = false, any_a = false, any_exact = false;
    for (int h = 0; h < d->heads_q; ++h) {
        any_vs |= head_pattern[h] == MI_VSLASH || head_pattern[h] == MI_VSLASH_EXACT;
        any_exact |= head_pattern[h] == MI_VSLASH_EXACT;
        any_bs |= head_pattern[h] == MI_BSPARSE;
        any_a |= head_pattern[h] == MI_ASHAPE;
    }
    if (out->block_cap < 1) return fail(MI_ERR_BUDGET, "block_cap must be >= 1");
    if (any_vs) {
        if (!vertical_idx || !slash_idx || !out->col_idx)
            return fail(MI_ERR_NULL, "Vertical-Slash heads need vertical_idx, slash_idx and out->col_idx");
        if (n_vertical < 1 || n_slash < 1) return fail(MI_ERR_BUDGET, "budgets must be >= 1");
        const int need_b = std::min<int64_t>(nb, 2 * (int64_t)n_slash);
        if (out->block_cap < need_b)
            return fail(MI_ERR_BUDGET, "block_cap %d < min(nb, 2 n_slash) = %d", out->block_cap, need_b);
        const int need_c = std::min(n_vertical, d->seq_len);
        if (out->col_cap < need_c)
            return fail(MI_ERR_BUDGET, "col_cap %d < min(n_vertical, seq_len) = %d", out->col_cap, need_c);
        const size_t lds = mi::build_index_lds_bytes(d->seq_len, n_slash);
        if (lds > kMaxLds) return fail(MI_ERR_SHAPE, "index build needs %zu bytes of LDS", lds);
        if (any_exact && !out->vs_bits) return fail(MI_ERR_NULL, "exact Vertical-Slash heads need out->vs_bits");
    }
    if (any_bs) {
        if (!bs_block_idx || !bs_block_count)
            return fail(MI_ERR_NULL, "Block-Sparse heads need bs_block_idx and bs_block_count");
        if (top_blocks < 1) return fail(MI_ERR_BUDGET, "top_blocks must be >= 1");
        if (out->block_cap < std::min(top_blocks, nb))
            return fail(MI_ERR_BUDGET, "block_cap %d < top_blocks %d", out->block_cap, top_blocks);
    }
    if (any_a) {
        if (sink_tokens < 0 || local_tokens < 1)
            return fail(MI_ERR_BUDGET, "A-shape needs sink_tokens >= 0 and local_tokens >= 1");
        const int need_a = ashape_max_blocks(nb, sink_tokens, local_tokens);
        if (out->block_cap < need_a)
            return fail(MI_ERR_BUDGET, "block_cap %d < A-shape maximum %d", out->block_cap, need_a);
    }
    mi::IndexArgs a{};
    a.B = d->batch; a.Hq = d->heads_q; a.N = d->seq_len;
    for (int h = 0; h < d->heads_q; ++h) a.pattern[h] = (uint8_t)head_pattern[h];
    a.vertical_idx = vertical_idx; a.n_vertical = n_vertical;
    a.slash_idx = slash_idx; a.n_slash = n_slash;
    a.bs_idx = bs_block_idx; a.bs_count = bs_block_count; a.top = top_blocks;
    a.sink = sink_tokens; a.local = local_tokens;
    a.block_count = out->block_count; a.block_idx = out->block_idx;
    a.col_count = out->col_count; a.col_idx = out->col_idx;
    a.block_cap = out->block_cap; a.col_cap = out->col_cap;
    a.vs_bits = any_exact ? out->vs_bits : nullptr;
    return launched(mi::launch_build_index(a, static_cast<hipStream_t>(stream)));
}

mi_status mi_sparse_prefill(const mi_attn_desc* d, const void* q, const void* k, const void* v,
                            const int32_t* head_pattern, const mi_index* idx, int32_t sink_tokens,
                            int32_t local_tokens, void* o, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
    mi::AttnArgs a{};
    mi_status st = prepare_attn(d, q, k, v, head_pattern, idx, sink_tokens, local_tokens, o, lse, a);
    if (st != MI_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (ws) {
        // the item schedule: built into ws by a kernel on the stream, read by
        // the attention kernel
        const size_t bytes = (size_t)mi::attn_schedule_len(a) * sizeof(int32_t);
        if (ws_bytes < bytes) return fail(MI_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, bytes);
        if (!aligned16(ws)) return fail(MI_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        return launch_scheduled(a, static_cast<int32_t*>(ws), s);
    }
    return launched(mi::launch_sparse_attn(a, s));
}

mi_status mi_sparse_prefill_noalloc(const mi_attn_desc* d, const void* q, const void* k, const void* v,
                                    const int32_t* head_pattern, const mi_index* idx, int32_t sink_tokens,
                                    int32_t local_tokens, void* o, float* lse, void* stream) {
    mi::AttnArgs a{};
    mi_status st = prepare_attn(d, q, k, v, head_pattern, idx, sink_tokens, local_tokens, o, lse, a);
    if (st != MI_OK) return st;
    const int32_t len = mi::attn_schedule_len(a);
    if (len > MI_NOALLOC_SCHEDULE_ENTRIES)
        return fail(MI_ERR_WORKSPACE,
                    "the item schedule needs %d entries, more than the %d of the built-in buffer "
                    "(batch * heads_q * ceil(seq_len / 256) too large): use mi_sparse_prefill with a workspace",
                    len, MI_NOALLOC_SCHEDULE_ENTRIES);
    int32_t* buf = nullptr;
    if ((st = scratch_pointer(&buf)) != MI_OK) return st;
    return launch_scheduled(a, buf, static_cast<hipStream_t>(stream));
}

int32_t mi_attn_schedule(const mi_attn_desc* d, const int32_t* head_pattern, int32_t sink_tokens,
                         int32_t local_tokens, int32_t block_cap, int32_t* out, int32_t cap) {
    if (check_desc(d) != MI_OK) return -1;
    if (head_pattern && check_patterns(d, head_pattern) != MI_OK) return -1;
    mi::AttnArgs a{};
    a.B = d->batch; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.N = d->seq_len;
    a.sink = sink_tokens; a.local = local_tokens; a.block_cap = block_cap;
    a.all_dense = head_pattern ? 0 : 1;
    for (int h = 0; h < d->heads_q; ++h) a.pattern[h] = head_pattern ? (uint8_t)head_pattern[h] : (uint8_t)MI_DENSE;
    const std::vector<int32_t> sched = mi::attn_schedule_host(a);
    if (out)
        for (int32_t i = 0; i < cap && i < (int32_t)sched.size(); ++i) out[i] = sched[i];
    return (int32_t)sched.size();
}

}  // extern "C"
