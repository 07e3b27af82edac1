// Block-Sparse estimate for gfx950 (hotpaper.ai summary of arXiv 2407.02490,
// key idea: 64-token mean pooling gives block-level attention weights;
// aifetchly guide, "2. The Block-Sparse Kernel Mechanics": mean key per
// 64-token block, dot products with the query block, top-k key blocks).
//
//   1. pool:   fp32 means of the 64 rows of every query block of the listed
//              heads and every key block of their kv heads (HBM-bound read of
//              Q and K once);
//   2. scores: z[a][c] = scale * Qbar_a . Kbar_c for c <= a, 64x64 tiles of
//              the lower triangle, fp32 FMA from LDS;
//   3. select: per query block a, softmax over c <= a (the block-level
//              attention weights, written out), then the exact top-k with
//              blocks 0 and a forced (mi_select.h).
#include "mi_internal.h"
#include "mi_select.h"

namespace mi {
namespace {

struct BsP {
    const char* q;
    const char* k;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2;
    int32_t B, Hq, N, nb, D, group, n_heads, n_kv, top;
    float scale;
    int32_t heads[MI_MAX_HEADS];
    int32_t kvlist[MI_MAX_HEADS];
    int32_t kvslot[MI_MAX_HEADS];  // kv head -> row of kbar (or -1)
    float* qbar;  // [B, n_heads, nb, D]
    float* kbar;  // [B, n_kv, nb, D]
    float* w;     // score rows
    int64_t w_b, w_h;  // strides of (batch, head row)
    int32_t w_by_head;
    int32_t* block_idx;    // [B, Hq, nb, top]
    int32_t* block_count;  // [B, Hq, nb]
};

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// One workgroup per (pooled row set, block); thread d sums column d.
template <typename T>
__global__ void __launch_bounds__(128) bs_pool(BsP p) {
    const int a = blockIdx.x % p.nb;
    const int r = blockIdx.x / p.nb;  // [0, B*n_heads) queries, then [.., + B*n_kv) keys
    const int d = threadIdx.x;
    if (d >= p.D) return;
    const T* src;
    float* dst;
    if (r < p.B * p.n_heads) {
        const int b = r / p.n_heads, li = r % p.n_heads;
        src = reinterpret_cast<const T*>(p.q) + b * p.qs0 + p.heads[li] * p.qs1 + (int64_t)a * 64 * p.qs2;
        dst = p.qbar + ((int64_t)r * p.nb + a) * p.D;
        float acc = 0.f;
        for (int i = 0; i < 64; ++i) acc += ld(src + (int64_t)i * p.qs2 + d);
        dst[d] = acc * (1.0f / 64.0f);
    } else {
        const int rk = r - p.B * p.n_heads;
        const int b = rk / p.n_kv, ki = rk % p.n_kv;
        src = reinterpret_cast<const T*>(p.k) + b * p.ks0 + p.kvlist[ki] * p.ks1 + (int64_t)a * 64 * p.ks2;
        dst = p.kbar + ((int64_t)rk * p.nb + a) * p.D;
        float acc = 0.f;
        for (int i = 0; i < 64; ++i) acc += ld(src + (int64_t)i * p.ks2 + d);
        dst[d] = acc * (1.0f / 64.0f);
    }
}

// Lower-triangle 64x64 tiles of z; thread (ty, tx) computes rows 4ty.., cols 4tx..
__global__ void __launch_bounds__(256) bs_scores(BsP p) {
    constexpr int KC = 32;
    __shared__ float qs[64][KC + 1];
    __shared__ float ks[64][KC + 1];
    const int T = (p.nb + 63) / 64;
    const int per = T * (T + 1) / 2;
    const int bl = blockIdx.x / per;
    int x = blockIdx.x % per;
    int ta = 0;
    while (x >= ta + 1) { x -= ta + 1; ++ta; }
    const int tc = x;
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int kslot = p.kvslot[p.heads[li] / p.group];
    const float* Q = p.qbar + (int64_t)bl * p.nb * p.D;
    const float* K = p.kbar + ((int64_t)b * p.n_kv + kslot) * p.nb * p.D;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.D; k0 += KC) {
        for (int e = threadIdx.x; e < 64 * KC; e += 256) {
            const int rr = e / KC, cc = e % KC;
            const int ar = ta * 64 + rr, cr = tc * 64 + rr;
            qs[rr][cc] = ar < p.nb ? Q[(int64_t)ar * p.D + k0 + cc] : 0.f;
            ks[rr][cc] = cr < p.nb ? K[(int64_t)cr * p.D + k0 + cc] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < KC; ++kk) {
            float qa[4], kc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) qa[i] = qs[ty * 4 + i][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) kc[j] = ks[tx * 4 + j][kk];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(qa[i], kc[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* W = p.w + b * p.w_b + (int64_t)(p.w_by_head ? p.heads[li] : li) * p.w_h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int a = ta * 64 + ty * 4 + i;
        if (a >= p.nb) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = tc * 64 + tx * 4 + j;
            if (c <= a) W[(int64_t)a * p.nb + c] = acc[i][j] * p.scale;
        }
    }
}

constexpr int kSelNT = 256;

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
    const int t = threadIdx.x;
    red[t] = v;
    __syncthreads();
    for (int s = kSelNT / 2; s > 0; s >>= 1) {
        if (t < s) red[t] = is_max ? fmaxf(red[t], red[t + s]) : red[t] + red[t + s];
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

// Per (batch, listed head, query block a): softmax of z[a][0..a], written
// back as w (zeros for c > a), then top-k with blocks 0 and a forced.
__global__ void __launch_bounds__(kSelNT) bs_select(BsP p) {
    extern __shared__ float row[];  // nb floats
    __shared__ SelectSmem sm;
    __shared__ float red[kSelNT];
    const int a = blockIdx.x % p.nb;
    const int bl = blockIdx.x / p.nb;
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int h = p.heads[li];
    float* W = p.w + b * p.w_b + (int64_t)(p.w_by_head ? h : li) * p.w_h + (int64_t)a * p.nb;
    const int n = a + 1;
    float mx = -INFINITY;
    for (int c = threadIdx.x; c < n; c += kSelNT) {
        const float z = W[c];
        row[c] = z;
        mx = fmaxf(mx, z);
    }
    mx = block_reduce(mx, red, true);
    float sum = 0.f;
    for (int c = threadIdx.x; c < n; c += kSelNT) {
        const float e = fast_exp2((row[c] - mx) * kLog2e);
        row[c] = e;
        sum += e;
    }
    sum = block_reduce(sum, red, false);
    for (int c = threadIdx.x; c < p.nb; c += kSelNT) {
        float wv = 0.f;
        if (c < n) {
            wv = row[c] / sum;
            row[c] = wv;
        }
        W[c] = wv;
    }
    __syncthreads();
    auto key = [&](int c) -> uint32_t { return (c == 0 || c == a) ? kForcedKey : order_key(row[c]); };
    const int k = min(p.top, n);
    int32_t* out = p.block_idx + (((int64_t)b * p.Hq + h) * p.nb + a) * p.top;
    select_topk<kSelNT>(key, n, k, p.top, out, sm);
    if (threadIdx.x == 0) p.block_count[((int64_t)b * p.Hq + h) * p.nb + a] = k;
}

// The same step with one wavefront per query block (rows of at most 64 R
// blocks): the row lives in registers (block c = lane + 64 u in slot u), the
// max and sum are butterfly reductions, and the selection is a 4-pass radix
// select over 8-bit digits with a 256-bin LDS histogram per wavefront, then
// one ordered ballot pass (slots in index order).  No workgroup barriers.
constexpr int kWaveRows = 4;  // wavefronts (rows) per workgroup

template <int R>
__global__ void __launch_bounds__(64 * kWaveRows) bs_select_wave(BsP p) {
    __shared__ uint32_t hist[kWaveRows][256];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t rowid = (int64_t)blockIdx.x * kWaveRows + wv;
    if (rowid >= (int64_t)p.B * p.n_heads * p.nb) return;
    const int a = (int)(rowid % p.nb);
    const int bl = (int)(rowid / p.nb);
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int h = p.heads[li];
    float* W = p.w + b * p.w_b + (int64_t)(p.w_by_head ? h : li) * p.w_h + (int64_t)a * p.nb;
    const int n = a + 1;
    float x[R];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int c = lane + 64 * u;
        x[u] = c < n ? W[c] : -INFINITY;
        mx = fmaxf(mx, x[u]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int c = lane + 64 * u;
        x[u] = c < n ? fast_exp2((x[u] - mx) * kLog2e) : 0.f;
        sum += x[u];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    uint32_t key[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int c = lane + 64 * u;
        const float wv = c < n ? x[u] / sum : 0.f;
        if (c < p.nb) W[c] = wv;
        key[u] = c >= n ? 0u : ((c == 0 || c == a) ? kForcedKey : order_key(wv));
    }
    const int k = min(p.top, n);
    int32_t* out = p.block_idx + (((int64_t)b * p.Hq + h) * p.nb + a) * p.top;
    if (lane == 0) p.block_count[((int64_t)b * p.Hq + h) * p.nb + a] = k;
    for (int m = k + lane; m < p.top; m += 64) out[m] = -1;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (k == n) {
        // every causal block is kept
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int c = lane + 64 * u;
            if (c < n) out[c] = c;
        }
        return;
    }
    // radix select: the k-th largest key T and how many keys == T to take
    uint32_t* hw = hist[wv];
    uint32_t prefix = 0, pmask = 0;
    int rem = k;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int i = 0; i < 4; ++i) hw[lane + 64 * i] = 0u;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int c = lane + 64 * u;
            if (c < n && (key[u] & pmask) == prefix) atomicAdd(&hw[(key[u] >> shift) & 255u], 1u);
        }
        __builtin_amdgcn_wave_barrier();
        // lane l owns bins 255-4l .. 252-4l (descending); suffix counts from the top
        int cnt[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cnt[i] = (int)hw[255 - 4 * lane - i];
            local += cnt[i];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        int run = incl - local;  // keys in higher bins than this lane's first
        int found = -1, above = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (found < 0 && run < rem && run + cnt[i] >= rem) {
                found = 255 - 4 * lane - i;
                above = run;
            }
            run += cnt[i];
        }
        const uint64_t hit = __ballot(found >= 0);
        const int src = __ffsll((long long)hit) - 1;  // exactly one lane finds the bin
        const int digit = __shfl(found, src, 64);
        rem -= __shfl(above, src, 64);
        prefix |= (uint32_t)digit << shift;
        pmask |= 255u << shift;
        __builtin_amdgcn_wave_barrier();
    }
    const uint32_t T = prefix;
    const int need = rem;
    // ordered output: keys > T, then keys == T while fewer than `need` taken
    int run_eq = 0, run_sel = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int c = lane + 64 * u;
        const bool g = c < n && key[u] > T;
        const bool e = c < n && key[u] == T;
        const uint64_t me = __ballot(e);
        const bool sel = g || (e && run_eq + __popcll(me & below) < need);
        const uint64_t ms = __ballot(sel);
        if (sel) out[run_sel + __popcll(ms & below)] = c;
        run_eq += __popcll(me);
        run_sel += __popcll(ms);
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t bs_workspace_bytes(int32_t B, int32_t n_heads, int32_t Hkv, int32_t N, int32_t D,
                          bool caller_scores) {
    const size_t nb = N / 64;
    size_t bytes = align256((size_t)B * n_heads * nb * D * sizeof(float));
    bytes += align256((size_t)B * Hkv * nb * D * sizeof(float));
    if (!caller_scores) bytes += align256((size_t)B * n_heads * nb * nb * sizeof(float));
    return bytes;
}

hipError_t launch_block_estimate(const BsArgs& a, hipStream_t s) {
    BsP p{};
    p.q = static_cast<const char*>(a.q);
    p.k = static_cast<const char*>(a.k);
    p.qs0 = a.qs[0]; p.qs1 = a.qs[1]; p.qs2 = a.qs[2];
    p.ks0 = a.ks[0]; p.ks1 = a.ks[1]; p.ks2 = a.ks[2];
    p.B = a.B; p.Hq = a.Hq; p.N = a.N; p.nb = a.N / 64; p.D = a.D;
    p.group = a.Hq / a.Hkv;
    p.n_heads = a.n_heads; p.top = a.top; p.scale = a.scale;
    for (int i = 0; i < MI_MAX_HEADS; ++i) p.kvslot[i] = -1;
    int nkv = 0;
    for (int i = 0; i < a.n_heads; ++i) {
        p.heads[i] = a.heads[i];
        const int kv = a.heads[i] / p.group;
        if (p.kvslot[kv] < 0) {
            p.kvslot[kv] = nkv;
            p.kvlist[nkv++] = kv;
        }
    }
    p.n_kv = nkv;
    char* ws = static_cast<char*>(a.ws);
    size_t off = 0;
    p.qbar = reinterpret_cast<float*>(ws + off);
    off += align256((size_t)a.B * a.n_heads * p.nb * a.D * sizeof(float));
    p.kbar = reinterpret_cast<float*>(ws + off);
    off += align256((size_t)a.B * a.Hkv * p.nb * a.D * sizeof(float));
    const int64_t nb2 = (int64_t)p.nb * p.nb;
    if (a.w != nullptr) {
        p.w = a.w;
        p.w_b = (int64_t)a.Hq * nb2;
        p.w_h = nb2;
        p.w_by_head = 1;
    } else {
        p.w = reinterpret_cast<float*>(ws + off);
        p.w_b = (int64_t)a.n_heads * nb2;
        p.w_h = nb2;
        p.w_by_head = 0;
    }
    p.block_idx = a.block_idx;
    p.block_count = a.block_count;

    const int pool_rows = a.B * (a.n_heads + nkv);
    if (a.dtype == MI_BF16)
        hipLaunchKernelGGL(bs_pool<uint16_t>, dim3(pool_rows * p.nb), dim3(128), 0, s, p);
    else
        hipLaunchKernelGGL(bs_pool<float>, dim3(pool_rows * p.nb), dim3(128), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int T = (p.nb + 63) / 64;
    hipLaunchKernelGGL(bs_scores, dim3(a.B * a.n_heads * (T * (T + 1) / 2)), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t sel_rows = (int64_t)a.B * a.n_heads * p.nb;
    const dim3 wgrid((unsigned)((sel_rows + kWaveRows - 1) / kWaveRows)), wblock(64 * kWaveRows);
    if (p.nb <= 128) {
        hipLaunchKernelGGL(bs_select_wave<2>, wgrid, wblock, 0, s, p);
    } else if (p.nb <= 512) {
        hipLaunchKernelGGL(bs_select_wave<8>, wgrid, wblock, 0, s, p);
    } else if (p.nb <= 1024) {
        hipLaunchKernelGGL(bs_select_wave<16>, wgrid, wblock, 0, s, p);
    } else if (p.nb <= 2048) {
        hipLaunchKernelGGL(bs_select_wave<32>, wgrid, wblock, 0, s, p);
    } else if (p.nb <= 4096) {
        hipLaunchKernelGGL(bs_select_wave<64>, wgrid, wblock, 0, s, p);
    } else {
        // longer rows: one workgroup per row, the row staged in LDS
        const size_t dyn = (size_t)p.nb * sizeof(float);
        if (dyn > 48 * 1024) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(bs_select),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(bs_select, dim3(a.B * a.n_heads * p.nb), dim3(kSelNT), dyn, s, p);
    }
    return hipGetLastError();
}

}  // namespace mi
