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
    const size_t dyn = (size_t)p.nb * sizeof(float);
    if (dyn > 48 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(bs_select),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bs_select, dim3(a.B * a.n_heads * p.nb), dim3(kSelNT), dyn, s, p);
    return hipGetLastError();
}

}  // namespace mi
