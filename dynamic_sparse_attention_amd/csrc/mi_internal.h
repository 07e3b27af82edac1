// Host-side interface between the C ABI layer (abi.hip) and the kernel
// launchers in the other translation units.  Not part of the public ABI.
#pragma once

#include <vector>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mi_sparse.h"

namespace mi {

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t qs[3], ks[3], vs[3], os[3];
    int32_t B, Hq, Hkv, N, D, dtype;
    float scale;
    const int32_t* block_count;
    const int32_t* block_idx;
    const int32_t* col_count;
    const int32_t* col_idx;
    int32_t block_cap, col_cap;
    int32_t sink, local;
    int32_t all_dense;
    uint8_t pattern[MI_MAX_HEADS];
    const int32_t* sched;  // device item schedule (NULL: the default order)
    int32_t sched_len;     // entries (a multiple of 4)
    const uint32_t* vs_bits;  // membership maps of exact Vertical-Slash heads (mi_index.vs_bits)
};
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s);
// Item schedule of the attention kernel (schedule.hip): bytes (an upper
// bound for any pattern set), entries for these arguments, the device build
// into `out` (enqueued on the stream), and the same order built on the host.
size_t attn_schedule_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N);
int32_t attn_schedule_len(const AttnArgs& a);
hipError_t launch_attn_schedule(const AttnArgs& a, int32_t* out, hipStream_t s);
std::vector<int32_t> attn_schedule_host(const AttnArgs& a);
// LDS of one attention workgroup: four K/V staging tiles, the four column
// lists of a run of query blocks and its step list (grows with seq_len and
// col_cap).
constexpr size_t kAttnMaxLds = 160 * 1024;
int attn_col_stride(const AttnArgs& a);
size_t sparse_attn_lds_bytes(const AttnArgs& a);

struct VsArgs {
    const void* q;
    const void* k;
    int64_t qs[3], ks[3];
    int32_t B, Hq, Hkv, N, D, dtype;
    float scale;
    int32_t n_heads;
    int32_t heads[MI_MAX_HEADS];
    int32_t last_q;
    int32_t n_vertical, n_slash, force_vertical, force_slash;
    int32_t* vertical_idx;
    int32_t* slash_idx;
    float* vscore;  // caller [B, Hq, N] score rows, or NULL (then kept in ws)
    float* sscore;
    void* ws;       // workspace laid out by the launcher (vs_workspace_bytes)
};
size_t vs_workspace_bytes(int32_t B, int32_t n_heads, int32_t N, bool caller_scores);
hipError_t launch_vs_estimate(const VsArgs& a, hipStream_t s);

// Top-k over the two score rows (vertical, slash) of each listed head: for
// each row select k = min(budget, n) positions, [0, forced) plus the best
// others by (score desc, index asc), written ascending to the head's output
// row [B, Hq, budget], with -1 beyond k.
struct TopkList {
    const float* score;
    int32_t* out;
    int32_t budget;
    int32_t forced;
};
struct TopkRows {
    int32_t B, Hq, n_heads, n;
    int32_t heads[MI_MAX_HEADS];
    int32_t score_by_head;
    int64_t srow_b, srow_h;
    TopkList list[2];
    uint32_t* scratch;  // topk_scratch_bytes(2 * B * n_heads) of device memory
};
// The first-digit histograms of the rows (mi_topk.h) must already be in
// `scratch`, built by the score kernels after the scratch was cleared.
hipError_t launch_topk_rows(const TopkRows& t, hipStream_t s);
size_t topk_scratch_bytes(int32_t rows);

struct BsArgs {
    const void* q;
    const void* k;
    int64_t qs[3], ks[3];
    int32_t B, Hq, Hkv, N, D, dtype;
    float scale;
    int32_t n_heads;
    int32_t heads[MI_MAX_HEADS];
    int32_t top;
    int32_t* block_idx;
    int32_t* block_count;
    float* w;              // caller [B, Hq, nb, nb] weights, or NULL (then kept in ws)
    void* ws;              // workspace laid out by the launcher (bs_workspace_bytes)
};
size_t bs_workspace_bytes(int32_t B, int32_t n_heads, int32_t Hkv, int32_t N, int32_t D,
                          bool caller_scores);
hipError_t launch_block_estimate(const BsArgs& a, hipStream_t s);
// Antidiagonal block scores with the same selection (BsArgs.w: caller weights
// or NULL; ws: the score rows, ad_workspace_bytes).
size_t ad_workspace_bytes(int32_t B, int32_t n_heads, int32_t N, bool caller_scores);
hipError_t launch_antidiag_estimate(const BsArgs& a, hipStream_t s);

struct IndexArgs {
    int32_t B, Hq, N;
    uint8_t pattern[MI_MAX_HEADS];
    const int32_t* vertical_idx;
    int32_t n_vertical;
    const int32_t* slash_idx;
    int32_t n_slash;
    const int32_t* bs_idx;
    const int32_t* bs_count;
    int32_t top;
    int32_t sink, local;
    int32_t* block_count;
    int32_t* block_idx;
    int32_t* col_count;
    int32_t* col_idx;
    int32_t block_cap, col_cap;
    uint32_t* vs_bits;
};
hipError_t launch_build_index(const IndexArgs& a, hipStream_t s);

}  // namespace mi
