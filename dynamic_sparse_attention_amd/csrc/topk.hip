// Top-k of the Vertical-Slash score rows: one workgroup of 1024 threads per
// (batch, listed head, list).  Vertical list: the first force_vertical keys
// are forced; slash list: the first force_slash offsets are forced (the sink
// and the main diagonal).  Rows are read from global memory (L2) once per
// radix pass.
#include "mi_internal.h"
#include "mi_select.h"

namespace mi {
namespace {

constexpr int kNT = 1024;

struct TopkP {
    TopkRows t;
};

__global__ void __launch_bounds__(kNT) topk_rows_kernel(TopkP p) {
    __shared__ SelectSmem sm;
    const TopkRows& t = p.t;
    const int row = blockIdx.x;
    const int which = row % 2;
    const int bl = row / 2;
    const int b = bl / t.n_heads, li = bl % t.n_heads;
    const int h = t.heads[li];
    const TopkList& L = t.list[which];
    const float* score = L.score + b * t.srow_b + (int64_t)(t.score_by_head ? h : li) * t.srow_h;
    int32_t* out = L.out + ((int64_t)b * t.Hq + h) * L.budget;
    const int forced = L.forced;
    auto key = [&](int i) -> uint32_t { return i < forced ? kForcedKey : order_key(score[i]); };
    const int k = min(L.budget, t.n);
    select_topk<kNT>(key, t.n, k, L.budget, out, sm);
}

}  // namespace

hipError_t launch_topk_rows(const TopkRows& t, hipStream_t s) {
    TopkP p{t};
    hipLaunchKernelGGL(topk_rows_kernel, dim3(2 * t.B * t.n_heads), dim3(kNT), 0, s, p);
    return hipGetLastError();
}

}  // namespace mi
