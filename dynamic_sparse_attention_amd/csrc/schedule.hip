// Work schedule of the attention kernel.
//
// A work item is (batch, query head, run of four query blocks).  The kernel's
// default order is run-major with the query heads of one kv group as four
// consecutive items that go to one XCD, so that they walk the same K/V tiles
// at the same time and share them in that XCD's L2.  That only holds when the
// four heads follow the same pattern: a Vertical-Slash head walks every key
// block, an A-shape head only the sink and its local window, a Block-Sparse
// head its own blocks.  Mixed groups then fetch most tiles once per head.
//
// The schedule groups items by (batch, kv group, pattern class) instead:
// within a sequence (b, g, class), items are listed run-major (longest
// first) over the class's heads of the group and cut into chunks of four, so
// a chunk holds heads of one class of one kv group, extended over
// consecutive runs when the group has fewer than four such heads
// (consecutive runs of a head walk nearly the same key blocks).  Chunks are
// then ordered by estimated length, longest first, ties in sequence order.
// Entries are packed items ((b * Hq + h) * nruns + run); chunks shorter than
// four are padded with -1.
//
// The schedule is built on the device, by one thread per chunk, into the
// caller's workspace just before the attention launch: no host memory is
// involved, nothing is cached between calls.  A chunk's estimate is a
// non-increasing function of its position in its sequence, so the ordered
// position of chunk c of sequence s with estimate e is
//     #{chunks with estimate > e}
//   + #{chunks with estimate == e in sequences before s}
//   + #{chunks of s before c with estimate == e},
// each term a closed-form count per sequence (the estimate is a step
// function of the run).  mi_attn_schedule() returns the
// same order built on the host by a plain stable sort.
#include <algorithm>
#include <vector>

#include "mi_internal.h"

namespace mi {
namespace {

constexpr int kRunBlocks = 4;  // query blocks per work item
constexpr int kChunk = 4;      // items per chunk (one XCD)
constexpr int kSchedThreads = 256;

__host__ __device__ inline int pattern_class(int p) {
    if (p == MI_ASHAPE) return 1;
    if (p == MI_BSPARSE) return 2;
    return 0;  // Vertical-Slash and dense walk (nearly) every causal key block
}

struct SchedShape {
    int32_t B, Hq, Hkv, nb, nruns, all_dense, sink, local, block_cap;
};

// Bound on the key blocks of an item of a sparse class (the causal span
// bounds every class).
__host__ __device__ inline long class_cap(int cls, const SchedShape& k) {
    if (cls == 1) return (long)((k.sink + 63) / 64 + (k.local + 126) / 64 + kRunBlocks);
    if (cls == 2) return (long)kRunBlocks * k.block_cap;
    return (long)k.nb;
}

// Key blocks an item of this class is expected to visit:
// min(4 (run + 1), nb, class bound), non-decreasing in the run.
__host__ __device__ inline long estimate(int cls, int run, const SchedShape& k) {
    const long full = (long)(run + 1) * kRunBlocks;
    const long span = full < k.nb ? full : (long)k.nb;
    const long cap = class_cap(cls, k);
    return span < cap ? span : cap;
}

// ---------------------------------------------------------------- host

std::vector<int32_t> build_host(const SchedShape& k, const uint8_t* pat) {
    const int group = k.Hq / k.Hkv;
    struct Chunk {
        long est;
        int32_t it[kChunk];
    };
    std::vector<Chunk> chunks;
    std::vector<int> heads;
    for (int b = 0; b < k.B; ++b)
        for (int g = 0; g < k.Hkv; ++g)
            for (int cls = 0; cls < 3; ++cls) {
                heads.clear();
                for (int h = g * group; h < (g + 1) * group; ++h)
                    if (pattern_class(k.all_dense ? MI_DENSE : pat[h]) == cls) heads.push_back(h);
                if (heads.empty()) continue;
                Chunk c{};
                int fill = 0;
                for (int pos = 0; pos < k.nruns; ++pos) {
                    const int run = k.nruns - 1 - pos;
                    for (int h : heads) {
                        if (fill == 0) c.est = estimate(cls, run, k);
                        c.it[fill++] = (int32_t)(((int64_t)b * k.Hq + h) * k.nruns + run);
                        if (fill == kChunk) {
                            chunks.push_back(c);
                            fill = 0;
                        }
                    }
                }
                if (fill > 0) {
                    for (; fill < kChunk; ++fill) c.it[fill] = -1;
                    chunks.push_back(c);
                }
            }
    std::stable_sort(chunks.begin(), chunks.end(), [](const Chunk& x, const Chunk& y) { return x.est > y.est; });
    std::vector<int32_t> out;
    out.reserve(chunks.size() * kChunk);
    for (const Chunk& c : chunks) out.insert(out.end(), c.it, c.it + kChunk);
    return out;
}

// ---------------------------------------------------------------- device

struct SchedParams {
    SchedShape k;
    int32_t per_batch;  // chunks of one batch entry
    int32_t* out;
    uint8_t pattern[MI_MAX_HEADS];
};

// Sequence q = 3 g + class of one batch entry: its head count and chunks.
struct Seq {
    int nh, nchunks;
};

// Head classes and per-sequence head counts, staged in LDS by each
// workgroup once: the lookups below then never touch the argument memory.
struct SchedLds {
    uint8_t cls[MI_MAX_HEADS];
    int16_t nh[3 * MI_MAX_HEADS];
};

__device__ inline Seq seq_of(const SchedParams& p, const SchedLds& L, int q) {
    const int nh = L.nh[q];
    return Seq{nh, (p.k.nruns * nh + kChunk - 1) / kChunk};
}

// Estimate of chunk c of a sequence with nh heads (from its first item).
__device__ inline long chunk_est(const SchedParams& p, int cls, int nh, int c) {
    const int run = p.k.nruns - 1 - (kChunk * c) / nh;
    return estimate(cls, run, p.k);
}

// Number of chunks of a sequence whose estimate exceeds e.  The estimate
// exceeds e exactly for runs >= R = floor(e / 4) (when nb and the class
// bound exceed e at all), i.e. for item positions below nruns - R: the
// first ceil((nruns - R) nh / 4) chunks.
__device__ inline int count_above(const SchedParams& p, int cls, const Seq& s, long e) {
    if ((long)p.k.nb <= e || class_cap(cls, p.k) <= e) return 0;
    const long R = e / kRunBlocks < p.k.nruns ? e / kRunBlocks : (long)p.k.nruns;
    const long n = ((p.k.nruns - R) * s.nh + kChunk - 1) / kChunk;
    return (int)(n < s.nchunks ? n : s.nchunks);
}

__global__ void __launch_bounds__(kSchedThreads) attn_schedule_kernel(SchedParams p) {
    __shared__ SchedLds L;
    const int group = p.k.Hq / p.k.Hkv;
    for (int h = threadIdx.x; h < p.k.Hq; h += kSchedThreads)
        L.cls[h] = (uint8_t)pattern_class(p.k.all_dense ? MI_DENSE : p.pattern[h]);
    __syncthreads();
    for (int q = threadIdx.x; q < 3 * p.k.Hkv; q += kSchedThreads) {
        int nh = 0;
        for (int h = (q / 3) * group; h < (q / 3 + 1) * group; ++h) nh += L.cls[h] == q % 3;
        L.nh[q] = (int16_t)nh;
    }
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kSchedThreads + threadIdx.x;
    const int64_t total = (int64_t)p.k.B * p.per_batch;
    if (t >= total) return;
    const int b = (int)(t / p.per_batch);
    int r = (int)(t % p.per_batch);
    // locate the thread's sequence (g, cls) and chunk c
    int g = 0, cls = 0;
    Seq s{0, 0};
    for (int q = 0; q < 3 * p.k.Hkv; ++q) {
        s = seq_of(p, L, q);
        if (r < s.nchunks) {
            g = q / 3;
            cls = q % 3;
            break;
        }
        r -= s.nchunks;
    }
    const int c = r;
    const long e = chunk_est(p, cls, s.nh, c);
    // ordered position
    int64_t gt = 0, eq_before = 0;
    const int me = 3 * g + cls;
    for (int q = 0; q < 3 * p.k.Hkv; ++q) {
        const int cq = q % 3;
        const Seq sq = seq_of(p, L, q);
        if (sq.nchunks == 0) continue;
        const int n_gt = count_above(p, cq, sq, e);      // chunks with estimate > e
        const int n_ge = count_above(p, cq, sq, e - 1);  // chunks with estimate >= e (e >= 1)
        gt += n_gt;
        eq_before += (int64_t)(n_ge - n_gt) * b + (q < me ? n_ge - n_gt : 0);
        if (q == me) eq_before += c - n_gt;
    }
    const int64_t rank = gt * p.k.B + eq_before;
    if (rank < 0 || rank >= total) return;  // unreachable: ranks are a permutation of the chunks
    int32_t* dst = p.out + rank * kChunk;
    const int g_heads = s.nh;
    const int64_t len = (int64_t)p.k.nruns * g_heads;
    for (int j = 0; j < kChunk; ++j) {
        const int64_t i = (int64_t)kChunk * c + j;
        int32_t item = -1;
        if (i < len) {
            const int pos = (int)(i / g_heads), hk = (int)(i % g_heads);
            // the hk-th head of class cls in group g
            int h = g * group, seen = -1;
            for (; h < (g + 1) * group; ++h) {
                seen += L.cls[h] == cls;
                if (seen == hk) break;
            }
            const int run = p.k.nruns - 1 - pos;
            item = (int32_t)(((int64_t)b * p.k.Hq + h) * p.k.nruns + run);
        }
        dst[j] = item;
    }
}

SchedShape shape_of(const AttnArgs& a) {
    SchedShape k{};
    k.B = a.B; k.Hq = a.Hq; k.Hkv = a.Hkv; k.nb = a.N / 64;
    k.nruns = (k.nb + kRunBlocks - 1) / kRunBlocks;
    k.all_dense = a.all_dense; k.sink = a.sink; k.local = a.local;
    k.block_cap = std::max(a.block_cap, 1);
    return k;
}

}  // namespace

size_t attn_schedule_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N) {
    const size_t nruns = (N / 64 + kRunBlocks - 1) / kRunBlocks;
    // every (batch, kv group, class) sequence pads to a multiple of 4
    return ((size_t)B * Hq * nruns + (size_t)B * Hkv * 3 * (kChunk - 1)) * sizeof(int32_t);
}

int32_t attn_schedule_len(const AttnArgs& a) {
    const SchedShape k = shape_of(a);
    const int group = k.Hq / k.Hkv;
    int64_t per_batch = 0;
    for (int g = 0; g < k.Hkv; ++g)
        for (int cls = 0; cls < 3; ++cls) {
            int nh = 0;
            for (int h = g * group; h < (g + 1) * group; ++h)
                nh += pattern_class(k.all_dense ? MI_DENSE : a.pattern[h]) == cls;
            per_batch += (k.nruns * (int64_t)nh + kChunk - 1) / kChunk;
        }
    return (int32_t)(per_batch * k.B * kChunk);
}

std::vector<int32_t> attn_schedule_host(const AttnArgs& a) { return build_host(shape_of(a), a.pattern); }

hipError_t launch_attn_schedule(const AttnArgs& a, int32_t* out, hipStream_t s) {
    SchedParams p{};
    p.k = shape_of(a);
    p.per_batch = attn_schedule_len(a) / (kChunk * p.k.B);
    p.out = out;
    for (int h = 0; h < MI_MAX_HEADS; ++h) p.pattern[h] = a.pattern[h];
    const int64_t total = (int64_t)p.k.B * p.per_batch;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_schedule_kernel, dim3((unsigned)((total + kSchedThreads - 1) / kSchedThreads)),
                       dim3(kSchedThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mi
