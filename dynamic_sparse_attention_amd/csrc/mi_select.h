// Exact, deterministic top-k selection for one workgroup of NT threads.
//
// Candidates 0..n-1 carry 32-bit keys that order them: a score is mapped to
// an unsigned key whose integer order is the float order, and forced members
// get the largest key 0xFFFFFFFF (no float maps there).  Selection is by
// (key desc, index asc): the k-th largest key T is found by a 3-pass radix
// select over 11/11/10-bit digits with an LDS histogram, then one ordered
// pass keeps every key > T and the first `need` keys == T in index order, so
// the output is ascending and independent of thread timing.  Histogram
// counts are integer atomics, whose sums do not depend on order.
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
        for (int i = threadIdx.x; i < n; i += NT) {
            const uint32_t kk = key(i);
            if ((kk & pmask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & (nbins - 1)], 1u);
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
    int run_eq = 0, run_sel = 0;
    for (int base = 0; base < n && run_sel < k; base += NT) {
        const int i = base + threadIdx.x;
        const uint32_t kk = (i < n) ? key(i) : 0u;
        const bool gt = (i < n) && kk > T;
        const bool eq = (i < n) && kk == T;
        int eq_tot;
        const int eq_before = block_flag_scan<NT>(eq, sm, eq_tot);
        const bool sel = gt || (eq && run_eq + eq_before < need);
        int sel_tot;
        const int sel_before = block_flag_scan<NT>(sel, sm, sel_tot);
        if (sel) out[run_sel + sel_before] = i;
        run_eq += eq_tot;
        run_sel += sel_tot;
    }
    for (int i = k + threadIdx.x; i < budget; i += NT) out[i] = -1;
}

}  // namespace mi
