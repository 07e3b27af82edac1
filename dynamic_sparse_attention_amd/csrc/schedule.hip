// Host-side work schedule of the attention kernel.
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
// within a class, items are listed run-major (longest first) and cut into
// chunks of four, so a chunk holds heads of one class of one kv group,
// extended over consecutive runs when the group has fewer than four such
// heads (consecutive runs of a head walk nearly the same key blocks).
// Chunks are then ordered by estimated length, longest first.  Entries are
// packed items ((b * Hq + h) * nruns + run); chunks shorter than four are
// padded with -1.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "mi_internal.h"

namespace mi {
namespace {

constexpr int kRunBlocks = 4;  // query blocks per work item
constexpr int kChunk = 4;      // items per chunk (one XCD)

struct Key {
    int B, Hq, Hkv, nb, all_dense, sink, local, block_cap;
    std::vector<int> pat;
    bool operator<(const Key& o) const {
        return std::tie(B, Hq, Hkv, nb, all_dense, sink, local, block_cap, pat) <
               std::tie(o.B, o.Hq, o.Hkv, o.nb, o.all_dense, o.sink, o.local, o.block_cap, o.pat);
    }
};

int pattern_class(int p) {
    if (p == MI_ASHAPE) return 1;
    if (p == MI_BSPARSE) return 2;
    return 0;  // Vertical-Slash and dense walk (nearly) every causal key block
}

// Key blocks an item of this class is expected to visit.
long estimate(int cls, int run, const Key& k) {
    const long span = std::min(k.nb, (run + 1) * kRunBlocks);
    if (cls == 1) return std::min<long>(span, (k.sink + 63) / 64 + (k.local + 126) / 64 + kRunBlocks);
    if (cls == 2) return std::min<long>(span, (long)kRunBlocks * k.block_cap);
    return span;
}

std::vector<int32_t> build(const Key& k) {
    const int nruns = (k.nb + kRunBlocks - 1) / kRunBlocks;
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
                    if (pattern_class(k.all_dense ? MI_DENSE : k.pat[h]) == cls) heads.push_back(h);
                if (heads.empty()) continue;
                Chunk c{};
                int fill = 0;
                for (int pos = 0; pos < nruns; ++pos) {
                    const int run = nruns - 1 - pos;
                    for (int h : heads) {
                        if (fill == 0) c.est = estimate(cls, run, k);
                        c.it[fill++] = (int32_t)(((int64_t)b * k.Hq + h) * nruns + run);
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

}  // namespace

size_t attn_schedule_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N) {
    const size_t nruns = (N / 64 + kRunBlocks - 1) / kRunBlocks;
    // every (batch, kv group, class) sequence pads to a multiple of 4
    return ((size_t)B * Hq * nruns + (size_t)B * Hkv * 3 * (kChunk - 1)) * sizeof(int32_t);
}

// The schedule for these arguments.  Schedules are kept for the life of the
// process (one per distinct layer shape and pattern set), so the host memory
// an asynchronous copy reads stays valid.
const std::vector<int32_t>& attn_schedule(const AttnArgs& a) {
    static std::mutex mu;
    static std::map<Key, std::vector<int32_t>> cache;
    Key k{a.B, a.Hq, a.Hkv, a.N / 64, a.all_dense, a.sink, a.local, std::max(a.block_cap, 1), {}};
    k.pat.assign(a.pattern, a.pattern + a.Hq);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(k);
    if (it == cache.end()) it = cache.emplace(k, build(k)).first;
    return it->second;
}

}  // namespace mi
