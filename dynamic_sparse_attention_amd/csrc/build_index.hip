// Conversion of the online estimates into per-query-block work lists
// (aifetchly guide, "1. The Vertical-Slash Kernel Mechanics" and "2. The
// Block-Sparse Kernel Mechanics": vertical keys read as coalesced chunks,
// only active 64x64 tiles computed).
//
// One workgroup per (batch, head, run of kAPerWG query blocks).
//  Vertical-Slash: a slash offset o is computed as whole aligned tiles; its
//    diagonal crosses key blocks a - floor(o/64) and a - ceil(o/64) of query
//    block a.  The set T of such tile distances is the same for every a
//    (translation invariance), so each workgroup builds T once as an LDS
//    bitmap, compacts it to an ascending list, and writes
//        block list of a = a - T[p-1], ..., a - T[0]   (p = #{t in T : t <= a})
//    which is ascending.  Columns: verticals j <= 64a+63 whose key block is
//    not a listed tile, in the order of the (ascending) vertical list, by an
//    ordered wave-ballot compaction.
//  Block-Sparse: copy of the estimated lists.
//  A-shape: sink blocks [0, ceil(sink/64)) and window blocks
//    [a - floor((local+62)/64), a], merged.
//  Dense: counts only.
// Entries beyond a list's count are -1 (rows of dense heads, and column rows
// of non-Vertical-Slash heads, are not written).
#include "mi_internal.h"
#include "mi_select.h"

namespace mi {
namespace {

constexpr int kNT = 256;
constexpr int kAPerWG = 16;

struct IdxP {
    IndexArgs a;
    int32_t nb;
    int32_t t_cap;  // LDS capacity of the tile-distance list
};

__global__ void __launch_bounds__(kNT) build_index_kernel(IdxP P) {
    extern __shared__ uint32_t dyn[];  // [bitmap words][tile list]
    __shared__ SelectSmem sm;
    __shared__ int32_t s_count;
    const IndexArgs& A = P.a;
    const int nb = P.nb;
    const int runs = (nb + kAPerWG - 1) / kAPerWG;
    const int bh = blockIdx.x / runs;
    const int a0 = (blockIdx.x % runs) * kAPerWG;
    const int a1 = min(a0 + kAPerWG, nb);
    const int b = bh / A.Hq, h = bh % A.Hq;
    const int pattern = A.pattern[h];
    const int64_t row0 = (int64_t)bh * nb;
    const int t = threadIdx.x;

    if (pattern == MI_DENSE) {
        for (int a = a0 + t; a < a1; a += kNT) {
            A.block_count[row0 + a] = a + 1;
            A.col_count[row0 + a] = 0;
        }
        return;
    }
    if (pattern == MI_BSPARSE) {
        for (int a = a0; a < a1; ++a) {
            const int64_t src = ((int64_t)bh * nb + a) * A.top;
            const int cnt = min(max(A.bs_count[row0 + a], 0), A.top);
            int32_t* dst = A.block_idx + (row0 + a) * A.block_cap;
            for (int m = t; m < A.block_cap; m += kNT) dst[m] = (m < cnt) ? A.bs_idx[src + m] : -1;
            if (t == 0) {
                A.block_count[row0 + a] = cnt;
                A.col_count[row0 + a] = 0;
            }
        }
        return;
    }
    if (pattern == MI_ASHAPE) {
        const int sink_blocks = (A.sink + 63) / 64;           // blocks holding a sink key
        const int wb = (A.local + 62) / 64;                   // window reach in blocks
        for (int a = a0; a < a1; ++a) {
            const int s_hi = min(a, sink_blocks - 1);         // sink range [0, s_hi]
            const int w_lo = max(0, a - wb);                  // window range [w_lo, a]
            int cnt;
            if (s_hi + 1 >= w_lo) cnt = a + 1;                // ranges touch: [0, a]
            else cnt = (s_hi + 1) + (a - w_lo + 1);
            cnt = min(cnt, A.block_cap);
            int32_t* dst = A.block_idx + (row0 + a) * A.block_cap;
            for (int m = t; m < A.block_cap; m += kNT) {
                int v = -1;
                if (m < cnt) v = (s_hi + 1 >= w_lo || m <= s_hi) ? m : w_lo + (m - s_hi - 1);
                dst[m] = v;
            }
            if (t == 0) {
                A.block_count[row0 + a] = cnt;
                A.col_count[row0 + a] = 0;
            }
        }
        return;
    }

    // ---- Vertical-Slash
    const int words = (nb + 31) / 32;
    uint32_t* bits = dyn;
    int32_t* tl = reinterpret_cast<int32_t*>(dyn + words);
    for (int w = t; w < words; w += kNT) bits[w] = 0u;
    __syncthreads();
    const int32_t* S = A.slash_idx + ((int64_t)b * A.Hq + h) * A.n_slash;
    for (int i = t; i < A.n_slash; i += kNT) {
        const int o = S[i];
        if (o < 0 || o >= A.N) continue;
        const int lo = o / 64, hi = (o + 63) / 64;
        if (lo < nb) atomicOr(&bits[lo / 32], 1u << (lo % 32));
        if (hi < nb) atomicOr(&bits[hi / 32], 1u << (hi % 32));
    }
    __syncthreads();
    // compact the bitmap into the ascending list tl[0..nt)
    int nt = 0;
    for (int w0 = 0; w0 < words; w0 += kNT) {
        const int w = w0 + t;
        const uint32_t word = (w < words) ? bits[w] : 0u;
        int tot;
        const int before = block_int_scan<kNT>(__popc(word), sm, tot);
        int pos = nt + before;
        uint32_t x = word;
        while (x) {
            const int bit = __ffs(x) - 1;
            x &= x - 1;
            if (pos < P.t_cap) tl[pos] = w * 32 + bit;
            ++pos;
        }
        nt += tot;
    }
    __syncthreads();
    nt = min(nt, P.t_cap);
    const int32_t* V = A.vertical_idx + ((int64_t)b * A.Hq + h) * A.n_vertical;
    for (int a = a0; a < a1; ++a) {
        // p = number of tile distances <= a (binary search in the ascending list)
        int lo = 0, hi = nt;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (tl[mid] <= a) lo = mid + 1; else hi = mid;
        }
        const int p = min(lo, A.block_cap);
        int32_t* dst = A.block_idx + (row0 + a) * A.block_cap;
        for (int m = t; m < A.block_cap; m += kNT) dst[m] = (m < p) ? a - tl[p - 1 - m] : -1;
        // columns: verticals j <= 64a+63 whose block a - floor(j/64) is not in T
        const int jmax = 64 * a + 63;
        int32_t* cdst = A.col_idx + (row0 + a) * A.col_cap;
        int run = 0;
        for (int base = 0; base < A.n_vertical; base += kNT) {
            const int i = base + t;
            const int j = (i < A.n_vertical) ? V[i] : -1;
            bool keep = false;
            if (j >= 0 && j <= jmax && j < A.N) {
                const int dist = a - j / 64;
                keep = ((bits[dist / 32] >> (dist % 32)) & 1u) == 0u;
            }
            int tot;
            const int before = block_flag_scan<kNT>(keep, sm, tot);
            if (keep && run + before < A.col_cap) cdst[run + before] = j;
            run += tot;
        }
        run = min(run, A.col_cap);
        for (int m = run + t; m < A.col_cap; m += kNT) cdst[m] = -1;
        if (t == 0) {
            A.block_count[row0 + a] = p;
            A.col_count[row0 + a] = run;
        }
    }
    (void)s_count;
}

}  // namespace

size_t build_index_lds_bytes(int32_t N, int32_t n_slash) {
    const int nb = N / 64;
    const int words = (nb + 31) / 32;
    const int tcap = min(nb, 2 * n_slash);
    return (size_t)(words + tcap) * 4;
}

hipError_t launch_build_index(const IndexArgs& a, hipStream_t s) {
    IdxP p{};
    p.a = a;
    p.nb = a.N / 64;
    bool any_vs = false;
    for (int h = 0; h < a.Hq; ++h) any_vs |= a.pattern[h] == MI_VSLASH;
    p.t_cap = any_vs ? min(p.nb, 2 * a.n_slash) : 0;
    const size_t dyn = any_vs ? build_index_lds_bytes(a.N, a.n_slash) : 0;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_index_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    const int runs = (p.nb + kAPerWG - 1) / kAPerWG;
    hipLaunchKernelGGL(build_index_kernel, dim3(a.B * a.Hq * runs), dim3(kNT), dyn, s, p);
    return hipGetLastError();
}

}  // namespace mi
