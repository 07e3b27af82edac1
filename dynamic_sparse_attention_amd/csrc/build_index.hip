// Conversion of the online estimates into per-query-block work lists
// (aifetchly guide, "1. The Vertical-Slash Kernel Mechanics" and "2. The
// Block-Sparse Kernel Mechanics": vertical keys read as coalesced chunks,
// only active 64x64 tiles computed).
//
// One workgroup per (batch, head, run of kAPerWG query blocks), one wave per
// query block.
//  Vertical-Slash: a slash offset o is computed as whole aligned tiles; its
//    diagonal crosses key blocks a - floor(o/64) and a - ceil(o/64) of query
//    block a.  The set T of such tile distances is the same for every a
//    (translation invariance), so a first kernel builds T once per head (LDS
//    byte flags compacted to an ascending list) and stores it as the list of
//    the last query block; every workgroup of the second kernel reads it back
//    and writes
//        block list of a = a - T[p-1], ..., a - T[0]   (p = #{t in T : t <= a})
//    which is ascending.  Columns: verticals j <= 64a+63 whose key block is
//    not a listed tile, in the order of the (ascending) vertical list, by an
//    ordered wave-ballot compaction.
//    Exact Vertical-Slash heads get the same lists, plus membership maps of
//    their vertical keys and slash offsets (vs_bits_kernel) from which the
//    attention masks each element of a listed tile.
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
constexpr int kAPerWG = 64;
constexpr int kTS = 1024;  // threads of the per-head tile-set kernel

struct IdxP {
    IndexArgs a;
    int32_t nb;
    int32_t t_cap;  // LDS capacity of the tile-distance list
};

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// LDS of both kernels: one byte flag per key-block distance (plain stores,
// no atomics on shared words), padded to whole 32-flag units of 8 words,
// followed by the ascending tile-distance list.
__host__ __device__ inline int flag_words(int nb) { return (nb + 127) / 128 * 32; }

// Block lists are written once and read by a later kernel, long after they
// would have left the caches: their whole-row 16-byte stores are
// non-temporal (streamed past the caches), which writes them measurably
// faster.  Column rows are written by partial-wave stores and stay ordinary
// stores (non-temporal partial lines are slower).
__device__ __forceinline__ void st_stream(int32_t* p, int32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_stream4(int32_t* p, i32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(p));
}

// One wave writes a list row: f(m) for m < cnt, -1 for cnt <= m < cap, as
// 16-byte stores when the rows are 16-byte aligned.
template <class F>
__device__ __forceinline__ void wave_fill(int32_t* dst, int cap, int cnt, bool vec, int lane, F f) {
    if (vec) {
        for (int m = 4 * lane; m < cap; m += 256) {
            i32x4 v;
            v.x = (m + 0 < cnt) ? f(m + 0) : -1;
            v.y = (m + 1 < cnt) ? f(m + 1) : -1;
            v.z = (m + 2 < cnt) ? f(m + 2) : -1;
            v.w = (m + 3 < cnt) ? f(m + 3) : -1;
            st_stream4(dst + m, v);
        }
    } else {
        for (int m = lane; m < cap; m += 64) st_stream(dst + m, (m < cnt) ? f(m) : -1);
    }
}

// Tile-distance set T of one Vertical-Slash head (one workgroup per head):
// LDS flags of floor(o/64) and ceil(o/64) over the slash offsets o,
// compacted in ascending order, written as the block list of the last query
// block (nb-1 - T[nt-1], ..., nb-1 - T[0]) with its count.
__global__ void __launch_bounds__(kTS) tile_set_kernel(IdxP P) {
    extern __shared__ uint32_t dyn[];  // [flag bytes][tile list]
    __shared__ SelectSmem sm;
    const IndexArgs& A = P.a;
    const int nb = P.nb;
    const int bh = blockIdx.x;
    const int b = bh / A.Hq, h = bh % A.Hq;
    if (A.pattern[h] != MI_VSLASH && A.pattern[h] != MI_VSLASH_EXACT) return;
    const int t = threadIdx.x;
    const int fw = flag_words(nb);
    uint8_t* flag = reinterpret_cast<uint8_t*>(dyn);
    int32_t* tl = reinterpret_cast<int32_t*>(dyn + fw);
    for (int w = t; w < fw; w += kTS) dyn[w] = 0u;
    __syncthreads();
    const int32_t* S = A.slash_idx + ((int64_t)b * A.Hq + h) * A.n_slash;
    for (int i0 = 0; i0 < A.n_slash; i0 += 4 * kTS) {
        int o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kTS + t;
            o[u] = (i < A.n_slash) ? S[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (o[u] < 0 || o[u] >= A.N) continue;
            const int lo = o[u] / 64, hi = (o[u] + 63) / 64;
            if (lo < nb) flag[lo] = 1;
            if (hi < nb) flag[hi] = 1;
        }
    }
    __syncthreads();
    // compact the flags into the ascending list tl[0..nt): thread u packs
    // flags [32u, 32u+32) into a mask, then a workgroup scan places them
    const int units = fw / 8;
    int nt = 0;
    for (int u0 = 0; u0 < units; u0 += kTS) {
        const int u = u0 + t;
        uint32_t mask = 0;
        if (u < units) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t x = dyn[8 * u + k];  // four 0/1 bytes
                mask |= ((x & 1u) | ((x >> 7) & 2u) | ((x >> 14) & 4u) | ((x >> 21) & 8u)) << (4 * k);
            }
        }
        int tot;
        const int before = block_int_scan<kTS>(__popc(mask), sm, tot);
        int pos = nt + before;
        while (mask) {
            const int bit = __ffs(mask) - 1;
            mask &= mask - 1;
            if (pos < P.t_cap) tl[pos] = u * 32 + bit;
            ++pos;
        }
        nt += tot;
    }
    __syncthreads();
    nt = min(min(nt, P.t_cap), A.block_cap);
    const int64_t last = (int64_t)bh * nb + nb - 1;
    int32_t* dst = A.block_idx + last * A.block_cap;
    for (int m = t; m < A.block_cap; m += kTS) st_stream(dst + m, (m < nt) ? (nb - 1) - tl[nt - 1 - m] : -1);
    if (t == 0) A.block_count[last] = nt;
}

__global__ void __launch_bounds__(kNT) build_index_kernel(IdxP P) {
    extern __shared__ uint32_t dyn[];  // [flag bytes][tile list]
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
    const int lane = t & 63;
    const bool vec_b = (A.block_cap & 3) == 0 && (reinterpret_cast<uintptr_t>(A.block_idx) & 15) == 0;

    if (pattern == MI_DENSE) {
        for (int a = a0 + t; a < a1; a += kNT) {
            A.block_count[row0 + a] = a + 1;
            A.col_count[row0 + a] = 0;
        }
        return;
    }
    if (pattern == MI_BSPARSE) {
        for (int a = a0 + (t >> 6); a < a1; a += kNT / 64) {
            const int32_t* src = A.bs_idx + ((int64_t)bh * nb + a) * A.top;
            const int cnt = min(max(A.bs_count[row0 + a], 0), A.top);
            int32_t* dst = A.block_idx + (row0 + a) * A.block_cap;
            wave_fill(dst, A.block_cap, cnt, vec_b, lane, [&](int m) { return src[m]; });
            if (lane == 0) {
                A.block_count[row0 + a] = cnt;
                A.col_count[row0 + a] = 0;
            }
        }
        return;
    }
    if (pattern == MI_ASHAPE) {
        const int sink_blocks = (A.sink + 63) / 64;           // blocks holding a sink key
        const int wb = (A.local + 62) / 64;                   // window reach in blocks
        for (int a = a0 + (t >> 6); a < a1; a += kNT / 64) {
            const int s_hi = min(a, sink_blocks - 1);         // sink range [0, s_hi]
            const int w_lo = max(0, a - wb);                  // window range [w_lo, a]
            int cnt;
            if (s_hi + 1 >= w_lo) cnt = a + 1;                // ranges touch: [0, a]
            else cnt = (s_hi + 1) + (a - w_lo + 1);
            cnt = min(cnt, A.block_cap);
            int32_t* dst = A.block_idx + (row0 + a) * A.block_cap;
            const bool merged = s_hi + 1 >= w_lo;
            wave_fill(dst, A.block_cap, cnt, vec_b, lane,
                      [&](int m) { return (merged || m <= s_hi) ? m : w_lo + (m - s_hi - 1); });
            if (lane == 0) {
                A.block_count[row0 + a] = cnt;
                A.col_count[row0 + a] = 0;
            }
        }
        return;
    }

    // ---- Vertical-Slash: recover T from the last query block's list, which
    // tile_set_kernel wrote (block list of nb-1 = nb-1 - T[nt-1], ..., nb-1 - T[0];
    // the capacity check on the host guarantees it holds all of T).
    const int fw = flag_words(nb);
    uint8_t* flag = reinterpret_cast<uint8_t*>(dyn);
    int32_t* tl = reinterpret_cast<int32_t*>(dyn + fw);
    for (int w = t; w < fw; w += kNT) dyn[w] = 0u;
    const int64_t last = row0 + nb - 1;
    const int nt = min(A.block_count[last], P.t_cap);
    __syncthreads();
    const int32_t* lrow = A.block_idx + last * A.block_cap;
    for (int m = t; m < nt; m += kNT) {
        const int d = (nb - 1) - lrow[nt - 1 - m];
        tl[m] = d;
        flag[d] = 1;
    }
    __syncthreads();
    // One wave per query block from here on: no workgroup barriers.
    const int32_t* V = A.vertical_idx + ((int64_t)b * A.Hq + h) * A.n_vertical;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const bool vec_c = (A.col_cap & 3) == 0 && (reinterpret_cast<uintptr_t>(A.col_idx) & 15) == 0;
    for (int a = a0 + (t >> 6); a < a1; a += kNT / 64) {
        // p = number of tile distances <= a (binary search in the ascending list)
        int lo = 0, hi = nt;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (tl[mid] <= a) lo = mid + 1; else hi = mid;
        }
        const int p = min(lo, A.block_cap);
        int32_t* dst = A.block_idx + (row0 + a) * A.block_cap;
        if (a != nb - 1)  // written by tile_set_kernel, read by the other workgroups
            wave_fill(dst, A.block_cap, p, vec_b, lane, [&](int m) { return a - tl[p - 1 - m]; });
        // columns: verticals j <= 64a+63 whose block a - floor(j/64) is not in T,
        // compacted in list order by wave ballots
        const int jmax = 64 * a + 63;
        int32_t* cdst = A.col_idx + (row0 + a) * A.col_cap;
        int run = 0;
        for (int base = 0; base < A.n_vertical; base += 256) {
            int jj[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = base + 64 * u + lane;
                jj[u] = (i < A.n_vertical) ? V[i] : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = jj[u];
                bool keep = false;
                if (j >= 0 && j <= jmax && j < A.N) {
                    const int dist = a - j / 64;
                    keep = flag[dist] == 0;
                }
                const uint64_t m = __ballot(keep);
                const int pos = run + __popcll(m & below);
                if (keep && pos < A.col_cap) cdst[pos] = j;
                run += __popcll(m);
            }
        }
        run = min(run, A.col_cap);
        if (vec_c) {
            const int r4 = min((run + 3) & ~3, A.col_cap);
            if (run + lane < r4) cdst[run + lane] = -1;
            for (int m = r4 + 4 * lane; m < A.col_cap; m += 256)
                *reinterpret_cast<i32x4*>(cdst + m) = i32x4{-1, -1, -1, -1};
        } else {
            for (int m = run + lane; m < A.col_cap; m += 64) cdst[m] = -1;
        }
        if (lane == 0) {
            if (a != nb - 1) A.block_count[row0 + a] = p;
            A.col_count[row0 + a] = run;
        }
    }
}

// Membership maps of an exact Vertical-Slash head (one workgroup per head):
// words [0, W) hold bit 64 + j for each vertical key j, words [W, 2W) bit
// 64 + o for each slash offset o (W = N/32 + 4; the first 64 bits and the
// tail stay zero).  Cleared, then set with atomic ORs.
__global__ void __launch_bounds__(kTS) vs_bits_kernel(IdxP P) {
    const IndexArgs& A = P.a;
    const int bh = blockIdx.x;
    const int b = bh / A.Hq, h = bh % A.Hq;
    if (A.pattern[h] != MI_VSLASH_EXACT) return;
    const int W = A.N / 32 + 4;
    uint32_t* vb = A.vs_bits + (int64_t)bh * 2 * W;
    uint32_t* sb = vb + W;
    const int t = threadIdx.x;
    for (int w = t; w < 2 * W; w += kTS) vb[w] = 0u;
    __syncthreads();
    const int32_t* V = A.vertical_idx + ((int64_t)b * A.Hq + h) * A.n_vertical;
    const int32_t* S = A.slash_idx + ((int64_t)b * A.Hq + h) * A.n_slash;
    for (int i = t; i < A.n_vertical; i += kTS) {
        const int j = V[i];
        if (j >= 0 && j < A.N) atomicOr(vb + ((j + 64) >> 5), 1u << ((j + 64) & 31));
    }
    for (int i = t; i < A.n_slash; i += kTS) {
        const int o = S[i];
        if (o >= 0 && o < A.N) atomicOr(sb + ((o + 64) >> 5), 1u << ((o + 64) & 31));
    }
}

}  // namespace

size_t build_index_lds_bytes(int32_t N, int32_t n_slash) {
    const int nb = N / 64;
    const int tcap = min(nb, 2 * n_slash);
    return (size_t)(flag_words(nb) + tcap) * 4;
}

hipError_t launch_build_index(const IndexArgs& a, hipStream_t s) {
    IdxP p{};
    p.a = a;
    p.nb = a.N / 64;
    bool any_vs = false;
    bool any_exact = false;
    for (int h = 0; h < a.Hq; ++h) {
        any_vs |= a.pattern[h] == MI_VSLASH || a.pattern[h] == MI_VSLASH_EXACT;
        any_exact |= a.pattern[h] == MI_VSLASH_EXACT;
    }
    p.t_cap = any_vs ? min(p.nb, 2 * a.n_slash) : 0;
    const size_t dyn = any_vs ? build_index_lds_bytes(a.N, a.n_slash) : 0;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_index_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    if (any_vs) {
        if (dyn > 48 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(tile_set_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(tile_set_kernel, dim3(a.B * a.Hq), dim3(kTS), dyn, s, p);
    }
    const int runs = (p.nb + kAPerWG - 1) / kAPerWG;
    hipLaunchKernelGGL(build_index_kernel, dim3(a.B * a.Hq * runs), dim3(kNT), dyn, s, p);
    if (any_exact) hipLaunchKernelGGL(vs_bits_kernel, dim3(a.B * a.Hq), dim3(kTS), 0, s, p);
    return hipGetLastError();
}

}  // namespace mi
