// Top-k of the Vertical-Slash score rows (vertical list: the first
// force_vertical keys are forced; slash list: the first force_slash offsets,
// the sink and the main diagonal).  Exact and deterministic: selection by
// (key desc, index asc) with order_key(), output ascending.
//
// The key is resolved as three radix digits (mi_topk.h).  The histogram of
// the first digit is built by the score kernels while they hold the scores,
// so the rows are read here three times, in three launches over (row,
// segment), a row being split into up to 64 segments of one 256-thread
// workgroup so that the 2 rows per listed head keep the GPU busy:
//   pass 2: finds digit 1 from its complete histogram (every workgroup finds
//           the same digit; segment 0 records it) and adds the histogram of
//           digit 2 over the keys with that prefix, one atomic per non-empty
//           bin;
//   pass 3: finds digit 2 the same way, so the 22-bit prefix P of the k-th
//           key is known; each wavefront sweeps its contiguous slice of the
//           segment, counts the keys above P and the keys sharing it, keeps
//           the last digit of the first four of those, and adds them to the
//           digit-3 histogram;
//   write:  finds digit 3, hence the k-th key T and how many keys equal to T
//           to take; each wavefront turns the slice records of the slices
//           before it into its output offset (a slice holding more than four
//           keys with prefix P is counted again by a sweep, which only
//           degenerate rows with many near-equal scores need) and writes the
//           selected indices of its slice: all keys > T, and keys == T while
//           the row's first `need` of them (in index order) are not
//           exhausted.
// Histogram sums are integer atomics, whose totals do not depend on order.
#include "mi_internal.h"
#include "mi_topk.h"

namespace mi {
namespace {

constexpr int kNT = 256;
constexpr int kNW = kTopkNW;
static_assert(kNT / 64 == kNW, "one slice per wavefront");
constexpr int kBatch = 16;  // keys per lane loaded together by the slice sweeps
constexpr uint32_t kMask1 = 0xFFC00000u;  // digit 1
constexpr uint32_t kMask12 = 0xFFFFF800u;  // digits 1 and 2

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
    v.scr = t.scratch + (int64_t)row * kTopkRowWords;
    return v;
}

__device__ __forceinline__ uint32_t key_of(const RowView& v, int i) { return topk_key(v.score[i], i, v.forced); }

struct Smem {
    uint32_t hist[2048];
    int32_t tot[kNW];
    uint32_t digit;
    int32_t above;
    uint16_t list[kNW][kTopkSliceList];
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

// Slice [w0, w1) of wavefront `wave` of segment s.
__device__ __forceinline__ void slice_of(const TopkP& p, const RowView& v, int s, int wave, int& w0, int& w1) {
    const int i0 = s * p.seg, i1 = min(v.n, i0 + p.seg);
    const int wseg = p.seg / kNW;
    w0 = i0 + wave * wseg;
    w1 = min(i1, w0 + wseg);
}

// Pass 2 over segment s of a row.
__global__ void __launch_bounds__(kNT) topk_pass2(TopkP p) {
    __shared__ Smem sm;
    const int row = blockIdx.x / p.nseg, s = blockIdx.x % p.nseg;
    const RowView v = row_view(p, row);
    if (v.k >= v.n) return;  // everything is selected
    uint32_t* st = v.scr + kTopkOffState;
    const int i0 = s * p.seg, i1 = min(v.n, i0 + p.seg);
    // the first keys are in flight while digit 1 is found
    uint32_t kk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = i0 + (int)threadIdx.x + u * kNT;
        kk[u] = i < i1 ? key_of(v, i) : 0u;
    }
    uint32_t d;
    int above;
    find_bin(v.scr, kTopkH1, v.k, sm, d, above);
    const uint32_t prefix = d << 22;
    if (s == 0 && threadIdx.x == 0) {
        st[0] = prefix;
        st[1] = (uint32_t)(v.k - above);
    }
    for (int i = threadIdx.x; i < kTopkH2; i += kNT) sm.hist[i] = 0u;
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
            if (base + u * kNT < i1 && (kk[u] & kMask1) == prefix) atomicAdd(&sm.hist[(kk[u] >> 11) & 2047u], 1u);
    }
    __syncthreads();
    uint32_t* gh = v.scr + kTopkOffH2;
    for (int i = threadIdx.x; i < kTopkH2; i += kNT)
        if (sm.hist[i]) atomicAdd(&gh[i], sm.hist[i]);
}

// Pass 3 over segment s of a row: digit-3 histogram and the slice records.
__global__ void __launch_bounds__(kNT) topk_pass3(TopkP p) {
    __shared__ Smem sm;
    const int row = blockIdx.x / p.nseg, s = blockIdx.x % p.nseg;
    const RowView v = row_view(p, row);
    if (v.k >= v.n) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t* st = v.scr + kTopkOffState;
    int w0, w1;
    slice_of(p, v, s, wave, w0, w1);
    uint32_t kk[kBatch];
    load_batch(v, w0, w1, kk);
    const int rem1 = (int)st[1];
    uint32_t d;
    int above;
    find_bin(v.scr + kTopkOffH2, kTopkH2, rem1, sm, d, above);
    const uint32_t P = st[0] | (d << 11);
    if (s == 0 && threadIdx.x == 0) {
        st[2] = P;
        st[3] = (uint32_t)(rem1 - above);
    }
    for (int i = threadIdx.x; i < kTopkH3; i += kNT) sm.hist[i] = 0u;
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int gt = 0, eq = 0;  // eq: wave-uniform count of keys with prefix P so far
    for (int base = w0; base < w1; base += 64 * kBatch) {
        if (base != w0) load_batch(v, base, w1, kk);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const bool in = base + 64 * u + lane < w1;
            const uint32_t hi = kk[u] & kMask12;
            gt += (in && hi > P) ? 1 : 0;
            const bool e = in && hi == P;
            const uint64_t me = __ballot(e);
            if (e) {
                atomicAdd(&sm.hist[kk[u] & 2047u], 1u);
                const int pos = eq + __popcll(me & below);
                if (pos < kTopkSliceList) sm.list[wave][pos] = (uint16_t)(kk[u] & 2047u);
            }
            eq += __popcll(me);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) gt += __shfl_xor(gt, off, 64);
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) {
        uint32_t* rec = v.scr + kTopkOffSlices + kTopkSliceWords * (s * kNW + wave);
        uint32_t lo = 0u, hi2 = 0u;
        const int nl = min(eq, kTopkSliceList);
        for (int j = 0; j < nl; ++j) {
            const uint32_t x = sm.list[wave][j];
            if (j < 2) lo |= x << (16 * j);
            else hi2 |= x << (16 * (j - 2));
        }
        rec[0] = (uint32_t)gt;
        rec[1] = (uint32_t)eq;
        rec[2] = lo;
        rec[3] = hi2;
    }
    __syncthreads();
    uint32_t* gh = v.scr + kTopkOffH3;
    for (int i = threadIdx.x; i < kTopkH3; i += kNT)
        if (sm.hist[i]) atomicAdd(&gh[i], sm.hist[i]);
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
    int w0, w1;
    slice_of(p, v, s, wave, w0, w1);
    // the first batch of keys is in flight while the threshold is found
    uint32_t kk[kBatch];
    load_batch(v, w0, w1, kk);
    const uint32_t* st = v.scr + kTopkOffState;
    const int rem2 = (int)st[3];
    uint32_t d3;
    int above;
    find_bin(v.scr + kTopkOffH3, kTopkH3, rem2, sm, d3, above);
    const uint32_t T = st[2] | d3;
    const int need = rem2 - above;
    // selected entries and keys == T in the slices before this one (slices
    // are ordered by key index: segment-major, then wavefront)
    const uint32_t* recs = v.scr + kTopkOffSlices;
    const int before = s * kNW + wave;
    int sel_base = 0, eq_before = 0;
    for (int q = lane; q < before; q += 64) {
        const uint32_t* rec = recs + kTopkSliceWords * q;
        const int eqn = (int)rec[1];
        int g = 0, e = 0;
        if (eqn <= kTopkSliceList) {
            g = (int)rec[0];
            for (int j = 0; j < eqn; ++j) {
                const uint32_t x = (rec[2 + j / 2] >> (16 * (j % 2))) & 0xFFFFu;
                g += x > d3 ? 1 : 0;
                e += x == d3 ? 1 : 0;
            }
        } else {
            // many keys share the prefix: count the slice against T
            int q0, q1;
            slice_of(p, v, q / kNW, q % kNW, q0, q1);
            for (int i = q0; i < q1; ++i) {
                const uint32_t key = key_of(v, i);
                g += key > T ? 1 : 0;
                e += key == T ? 1 : 0;
            }
        }
        sel_base += g;
        eq_before += e;
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

size_t topk_scratch_bytes(int32_t rows) { return (size_t)rows * kTopkRowWords * sizeof(uint32_t); }

hipError_t launch_topk_rows(const TopkRows& t, hipStream_t s) {
    TopkP p{t, 1, 0};
    const int rows = 2 * t.B * t.n_heads;
    // segments of at least 4096 keys, at most kTopkMaxSeg per row
    int nseg = (t.n + 4095) / 4096;
    nseg = max(1, min(kTopkMaxSeg, nseg));
    int seg = (t.n + nseg - 1) / nseg;
    seg = (seg + kNT - 1) / kNT * kNT;
    nseg = (t.n + seg - 1) / seg;
    p.nseg = nseg;
    p.seg = seg;
    hipLaunchKernelGGL(topk_pass2, dim3(rows * nseg), dim3(kNT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_pass3, dim3(rows * nseg), dim3(kNT), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_write, dim3(rows * nseg), dim3(kNT), 0, s, p);
    return hipGetLastError();
}

}  // namespace mi
