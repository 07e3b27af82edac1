// Top-k of the Vertical-Slash score rows (vertical list: the first
// force_vertical keys are forced; slash list: the first force_slash offsets,
// the sink and the main diagonal).  Exact and deterministic: selection by
// (key desc, index asc) with order_key(), output ascending.
//
// A row is split into S segments, one 256-thread workgroup each, so that the
// 2 rows per listed head keep the whole GPU busy.  Six launches over
// (row, segment):
//   0. clear the per-row global histograms;
//   1-3. radix passes over 11/11/10-bit digits: every workgroup adds the
//      histogram of its segment (restricted to the prefix found so far) to
//      the row's global histogram with one atomic per non-empty bin, after
//      finding the digit of the previous pass from that pass's complete
//      histogram (every workgroup finds the same digit; segment 0 records it);
//   4. with the k-th key T known, each wavefront counts the keys > T and == T
//      of its contiguous slice of the segment;
//   5. each wavefront writes the selected indices of its slice at the offset
//      given by the counts of the slices before it: all keys > T, and keys
//      == T while the row's first `need` of them (in index order) are not
//      exhausted.
// Histogram sums are integer atomics, whose totals do not depend on order.
#include "mi_internal.h"
#include "mi_select.h"

namespace mi {
namespace {

constexpr int kNT = 256;
constexpr int kNW = kNT / 64;
constexpr int kMaxSeg = 64;  // segments per row

// Per-row scratch (uint32 words): three histograms, the state after each
// pass (prefix, remaining rank) and the (gt, eq) counts of every wavefront
// slice of every segment.
constexpr int kHistWords = 2048 + 2048 + 1024;
constexpr int kRowWords = kHistWords + 8 + 2 * kMaxSeg * kNW;
constexpr int kBatch = 16;  // keys per lane loaded together by the count and write sweeps

struct TopkP {
    TopkRows t;
    int32_t nseg, seg;  // segments per row, keys per segment (multiple of 256)
};

struct RowView {
    const float* score;
    int32_t* out;
    int k, budget, forced, n;
    uint32_t* scr;
};

__device__ __forceinline__ RowView row_view(const TopkP& p, int row) {
    const TopkRows& t = p.t;
    const int which = row % 2, bl = row / 2;
    const int b = bl / t.n_heads, li = bl % t.n_heads;
    const int h = t.heads[li];
    const TopkList& L = t.list[which];
    RowView v;
    v.score = L.score + b * t.srow_b + (int64_t)(t.score_by_head ? h : li) * t.srow_h;
    v.out = L.out + ((int64_t)b * t.Hq + h) * L.budget;
    v.k = min(L.budget, t.n);
    v.budget = L.budget;
    v.forced = L.forced;
    v.n = t.n;
    v.scr = t.scratch + (int64_t)row * kRowWords;
    return v;
}

__device__ __forceinline__ uint32_t key_of(const RowView& v, int i) {
    return i < v.forced ? kForcedKey : order_key(v.score[i]);
}

struct Smem {
    uint32_t hist[2048];
    int32_t tot[kNW];
    uint32_t digit;
    int32_t above;
};

// Finds, in a complete histogram of nbins bins, the bin that holds the
// rem-th largest key (rem >= 1) and how many keys lie in higher bins.
__device__ void find_bin(const uint32_t* hist, int nbins, int rem, Smem& sm, uint32_t& digit, int& above) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int bpt = nbins / kNT;  // 8 or 4 bins per thread, descending
    int local = 0;
    for (int q = 0; q < bpt; ++q) local += (int)hist[nbins - 1 - (t * bpt + q)];
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) sm.tot[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += sm.tot[w];
    for (int q = 0; q < bpt; ++q) {
        const int bin = nbins - 1 - (t * bpt + q);
        const int c = (int)hist[bin];
        if (run < rem && run + c >= rem) {
            sm.digit = (uint32_t)bin;
            sm.above = run;
        }
        run += c;
    }
    __syncthreads();
    digit = sm.digit;
    above = sm.above;
    __syncthreads();
}

__global__ void __launch_bounds__(kNT) topk_clear(TopkP p) {
    const int64_t words = (int64_t)2 * p.t.B * p.t.n_heads * kRowWords;
    for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < words; i += (int64_t)gridDim.x * kNT)
        p.t.scratch[i] = 0u;
}

// Radix pass `pass` (0..2) over segment s of a row.
__global__ void __launch_bounds__(kNT) topk_hist(TopkP p, int pass) {
    __shared__ Smem sm;
    const int row = blockIdx.x / p.nseg, s = blockIdx.x % p.nseg;
    const RowView v = row_view(p, row);
    if (v.k >= v.n) return;  // everything is selected
    uint32_t* st = v.scr + kHistWords;  // state: [pass] = (prefix, rem)
    const int i0 = s * p.seg, i1 = min(v.n, i0 + p.seg);
    // the first keys are in flight while the previous digit is found
    uint32_t kk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = i0 + (int)threadIdx.x + u * kNT;
        kk[u] = i < i1 ? key_of(v, i) : 0u;
    }
    uint32_t prefix = 0, pmask = 0;
    int rem = v.k;
    if (pass > 0) {
        // the digit of the previous pass, from its complete histogram
        const uint32_t* ph = v.scr + (pass == 1 ? 0 : 2048);
        if (pass == 2) {
            prefix = st[0];
            rem = (int)st[1];
        }
        uint32_t d;
        int above;
        find_bin(ph, 2048, rem, sm, d, above);
        const int shift = pass == 1 ? 21 : 10;
        prefix |= d << shift;
        rem -= above;
        pmask = pass == 1 ? 0xFFE00000u : 0xFFFFFC00u;
        if (s == 0 && threadIdx.x == 0) {
            st[2 * (pass - 1)] = prefix;
            st[2 * (pass - 1) + 1] = (uint32_t)rem;
        }
    }
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int i = threadIdx.x; i < nbins; i += kNT) sm.hist[i] = 0u;
    __syncthreads();
    for (int base = i0 + (int)threadIdx.x; base < i1; base += 8 * kNT) {
        if (base != i0 + (int)threadIdx.x) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = base + u * kNT;
                kk[u] = i < i1 ? key_of(v, i) : 0u;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (base + u * kNT < i1 && (kk[u] & pmask) == prefix)
                atomicAdd(&sm.hist[(kk[u] >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    uint32_t* gh = v.scr + (pass == 0 ? 0 : (pass == 1 ? 2048 : 4096));
    for (int i = threadIdx.x; i < nbins; i += kNT)
        if (sm.hist[i]) atomicAdd(&gh[i], sm.hist[i]);
}

// The threshold key T and the number of keys == T to take, from the last
// histogram; every workgroup of the row finds the same values.
__device__ void threshold(const RowView& v, Smem& sm, uint32_t& T, int& need) {
    const uint32_t* st = v.scr + kHistWords;
    uint32_t d;
    int above;
    find_bin(v.scr + 4096, 1024, (int)st[3], sm, d, above);
    T = st[2] | d;
    need = (int)st[3] - above;
}

// Keys of wavefront slice [w0, w1) in batches of kBatch per lane: lane l of
// batch b holds key w0 + 64 (kBatch b + u) + l in kk[u] (0 past w1).
__device__ __forceinline__ void load_batch(const RowView& v, int base, int w1, uint32_t (&kk)[kBatch]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int i = base + 64 * u + lane;
        kk[u] = i < w1 ? key_of(v, i) : 0u;
    }
}

// Each wavefront counts, over its contiguous slice of the segment (the
// slices topk_write walks), the keys > T and == T.
__global__ void __launch_bounds__(kNT) topk_count(TopkP p) {
    __shared__ Smem sm;
    const int row = blockIdx.x / p.nseg, s = blockIdx.x % p.nseg;
    const RowView v = row_view(p, row);
    if (v.k >= v.n) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i0 = s * p.seg, i1 = min(v.n, i0 + p.seg);
    const int wseg = p.seg / kNW;
    const int w0 = i0 + wave * wseg, w1 = min(i1, w0 + wseg);
    // the first batch of keys is in flight while the threshold is found
    uint32_t kk[kBatch];
    load_batch(v, w0, w1, kk);
    uint32_t T;
    int need;
    threshold(v, sm, T, need);
    int gt = 0, eq = 0;
    for (int base = w0; base < w1; base += 64 * kBatch) {
        if (base != w0) load_batch(v, base, w1, kk);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const bool in = base + 64 * u + lane < w1;
            gt += (in && kk[u] > T) ? 1 : 0;
            eq += (in && kk[u] == T) ? 1 : 0;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        gt += __shfl_xor(gt, off, 64);
        eq += __shfl_xor(eq, off, 64);
    }
    if (lane == 0) {
        uint32_t* wcnt = v.scr + kHistWords + 8 + 2 * (s * kNW + wave);
        wcnt[0] = (uint32_t)gt;
        wcnt[1] = (uint32_t)eq;
    }
}

__global__ void __launch_bounds__(kNT) topk_write(TopkP p) {
    __shared__ Smem sm;
    const int row = blockIdx.x / p.nseg, s = blockIdx.x % p.nseg;
    const RowView v = row_view(p, row);
    if (v.k >= v.n) {
        // every candidate is selected: out = 0..n-1, then -1 padding
        if (s == 0)
            for (int i = threadIdx.x; i < v.budget; i += kNT) v.out[i] = i < v.n ? i : -1;
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i0 = s * p.seg, i1 = min(v.n, i0 + p.seg);
    const int wseg = p.seg / kNW;
    const int w0 = i0 + wave * wseg, w1 = min(i1, w0 + wseg);
    // the first batch of keys is in flight while the threshold is found
    uint32_t kk[kBatch];
    load_batch(v, w0, w1, kk);
    uint32_t T;
    int need;
    threshold(v, sm, T, need);
    // selected entries and keys == T in the wavefront slices before this one
    // (slices are ordered by key index: segment-major, then wavefront)
    const uint32_t* wcnt = v.scr + kHistWords + 8;
    const int before = s * kNW + wave;
    int sel_base = 0, eq_before = 0;
    for (int q = lane; q < before; q += 64) {
        sel_base += (int)wcnt[2 * q];
        eq_before += (int)wcnt[2 * q + 1];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        sel_base += __shfl_xor(sel_base, off, 64);
        eq_before += __shfl_xor(eq_before, off, 64);
    }
    // keys == T are taken in index order until `need` are selected
    sel_base += min(eq_before, need);
    const int eq_left = max(need - eq_before, 0);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int run_eq = 0, run_sel = 0;
    for (int base = w0; base < w1; base += 64 * kBatch) {
        if (base != w0) load_batch(v, base, w1, kk);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = base + 64 * u + lane;
            const bool g = i < w1 && kk[u] > T;
            const bool e = i < w1 && kk[u] == T;
            const uint64_t me = __ballot(e);
            const bool sel = g || (e && run_eq + __popcll(me & below) < eq_left);
            const uint64_t ms = __ballot(sel);
            if (sel) v.out[sel_base + run_sel + __popcll(ms & below)] = i;
            run_eq += __popcll(me);
            run_sel += __popcll(ms);
        }
    }
    if (s == 0)
        for (int i = v.k + threadIdx.x; i < v.budget; i += kNT) v.out[i] = -1;
}

}  // namespace

size_t topk_scratch_bytes(int32_t rows) { return (size_t)rows * kRowWords * sizeof(uint32_t); }

hipError_t launch_topk_rows(const TopkRows& t, hipStream_t s) {
    TopkP p{t, 1, 0};
    const int rows = 2 * t.B * t.n_heads;
    // segments of at least 4096 keys, at most kMaxSeg per row
    int nseg = (t.n + 4095) / 4096;
    nseg = max(1, min(kMaxSeg, nseg));
    int seg = (t.n + nseg - 1) / nseg;
    seg = (seg + kNT - 1) / kNT * kNT;
    nseg = (t.n + seg - 1) / seg;
    p.nseg = nseg;
    p.seg = seg;
    const int clear_blocks = min(1024, (int)((topk_scratch_bytes(rows) / 4 + kNT - 1) / kNT));
    hipLaunchKernelGGL(topk_clear, dim3(clear_blocks), dim3(kNT), 0, s, p);
    hipError_t e = hipGetLastError();
    for (int pass = 0; pass < 3 && e == hipSuccess; ++pass) {
        hipLaunchKernelGGL(topk_hist, dim3(rows * nseg), dim3(kNT), 0, s, p, pass);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_count, dim3(rows * nseg), dim3(kNT), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_write, dim3(rows * nseg), dim3(kNT), 0, s, p);
    return hipGetLastError();
}

}  // namespace mi
