// Exact, deterministic top-k selection for one workgroup of NT threads.
//
// Candidates 0..n-1 carry 32-bit keys that order them: a score is mapped to
// an unsigned key whose integer order is the float order, and forced members
// get the largest key 0xFFFFFFFF (no float maps there).  Selection is by
// (key desc, index asc): the k-th largest key T is found by a 3-pass radix
// select over 11/11/10-bit digits with an LDS histogram, then one ordered
// pass keeps every key > T and the first `need` keys == T in index order, so
// the output is ascending and independent of thread timing.  Histogram
// counts are integer atomics, whose sums do not depend on order.  The
// ordered pass gives each wavefront a contiguous segment of candidates: one
// counting sweep, one exchange of the per-wavefront counts through LDS, and
// one writing sweep in which ballots order the members of each 64-candidate
// chunk.
#pragma once

#include "mi_device.h"

namespace mi {

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;  // -0 and +0 tie
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr uint32_t kForcedKey = 0xFFFFFFFFu;

struct SelectSmem {
    uint32_t hist[2048];
    int32_t wave_tot[17];
    int32_t seg_gt[16], seg_eq[16];  // per-wavefront counts of the ordered pass
    uint32_t found_digit;
    int32_t found_above;
};

// Exclusive prefix over the workgroup of a 0/1 predicate (wave ballot +
// per-wave totals in LDS).  Returns the prefix; `total` gets the sum.
template <int NT>
__device__ __forceinline__ int block_flag_scan(bool pred, SelectSmem& sm, int& total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t m = __ballot(pred);
    const int in_wave = __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    if (lane == 0) sm.wave_tot[wave] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = sm.wave_tot[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();  // wave_tot may be reused by the next scan
    total = tot;
    return before + in_wave;
}

// Exclusive prefix of an integer over the workgroup (in thread order).
template <int NT>
__device__ __forceinline__ int block_int_scan(int v, SelectSmem& sm, int& total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) sm.wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = sm.wave_tot[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// Finds the k-th largest key T (1 <= k <= n) and how many candidates with
// key == T must be taken (need).  KeyFn: uint32_t(int i).
template <int NT, class KeyFn>
__device__ void radix_threshold(KeyFn key, int n, int k, SelectSmem& sm, uint32_t& T, int& need) {
    uint32_t prefix = 0, pmask = 0;
    int rem = k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        for (int i = threadIdx.x; i < 2048; i += NT) sm.hist[i] = 0u;
        __syncthreads();
        // eight independent loads per thread before their atomics, so that
        // the loop is not bound by one memory latency per element
        for (int i0 = threadIdx.x; i0 < n; i0 += 8 * NT) {
            uint32_t kk[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * NT;
                kk[u] = i < n ? key(i) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u * NT < n && (kk[u] & pmask) == prefix)
                    atomicAdd(&sm.hist[(kk[u] >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        // thread t owns bins in descending order: positions [t*BPT, (t+1)*BPT)
        constexpr int BPT = 2048 / NT;
        const int bpt = nbins / NT > 0 ? nbins / NT : 1;
        int local = 0;
        const int p0 = threadIdx.x * bpt;
        for (int q = 0; q < bpt; ++q) {
            const int pos = p0 + q;
            if (pos < nbins) local += sm.hist[nbins - 1 - pos];
        }
        int tot;
        int above = block_int_scan<NT>(local, sm, tot);
        for (int q = 0; q < bpt; ++q) {
            const int pos = p0 + q;
            if (pos >= nbins) break;
            const int bin = nbins - 1 - pos;
            const int c = sm.hist[bin];
            if (above < rem && above + c >= rem) {
                sm.found_digit = (uint32_t)bin;
                sm.found_above = above;
            }
            above += c;
        }
        (void)BPT;
        __syncthreads();
        const uint32_t dv = sm.found_digit;
        rem -= sm.found_above;
        prefix |= dv << shift;
        pmask |= uint32_t(nbins - 1) << shift;
        __syncthreads();
    }
    T = prefix;
    need = rem;
}

// Writes the selected indices ascending to out[0..k); out[k..budget) = -1.
template <int NT, class KeyFn>
__device__ void select_topk(KeyFn key, int n, int k, int budget, int32_t* out, SelectSmem& sm) {
    if (k >= n) {
        for (int i = threadIdx.x; i < budget; i += NT) out[i] = (i < n) ? i : -1;
        return;
    }
    uint32_t T;
    int need;
    radix_threshold<NT>(key, n, k, sm, T, need);
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes < this one
    const int seg = (n + NW * 64 - 1) / (NW * 64) * 64;  // candidates per wavefront
    const int s0 = wave * seg, s1 = min(n, s0 + seg);
    // sweep 1: counts of keys > T and == T in this wavefront's segment
    // (four 64-candidate chunks loaded together)
    int gt = 0, eq = 0;
    for (int base = s0; base < s1; base += 256) {
        uint32_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + 64 * u + lane;
            kk[u] = (i < s1) ? key(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + 64 * u + lane;
            gt += __popcll(__ballot(i < s1 && kk[u] > T));
            eq += __popcll(__ballot(i < s1 && kk[u] == T));
        }
    }
    if (lane == 0) {
        sm.seg_gt[wave] = gt;
        sm.seg_eq[wave] = eq;
    }
    __syncthreads();
    int sel_base = 0, eq_before = 0;
    for (int w = 0; w < wave; ++w) {
        const int e = sm.seg_eq[w];
        const int take = min(max(need - eq_before, 0), e);
        sel_base += sm.seg_gt[w] + take;
        eq_before += e;
    }
    const int eq_take = min(max(need - eq_before, 0), eq);  // first eq_take keys == T of the segment
    // sweep 2: ordered writes
    int run_eq = 0, run_sel = 0;
    for (int base = s0; base < s1; base += 256) {
        uint32_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + 64 * u + lane;
            kk[u] = (i < s1) ? key(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + 64 * u + lane;
            const bool g = i < s1 && kk[u] > T;
            const bool e = i < s1 && kk[u] == T;
            const uint64_t me = __ballot(e);
            const bool sel = g || (e && run_eq + __popcll(me & below) < eq_take);
            const uint64_t ms = __ballot(sel);
            if (sel) out[sel_base + run_sel + __popcll(ms & below)] = i;
            run_eq += __popcll(me);
            run_sel += __popcll(ms);
        }
    }
    for (int i = k + threadIdx.x; i < budget; i += NT) out[i] = -1;
}

}  // namespace mi
