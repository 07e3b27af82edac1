// Block-Sparse estimate for gfx950 (hotpaper.ai summary of arXiv 2407.02490,
// key idea: 64-token mean pooling gives block-level attention weights;
// aifetchly guide, "2. The Block-Sparse Kernel Mechanics": mean key per
// 64-token block, dot products with the query block, top-k key blocks).
//
//   1. pool:   fp32 means of the 64 rows of every query block of the listed
//              heads and every key block of their kv heads (HBM-bound read of
//              Q and K once, 16-byte loads);
//   2. scores: z[a][c] = scale * Qbar_a . Kbar_c for c <= a, fp32 matrix-core
//              products;
//   3. select: per query block a, softmax over c <= a (the block-level
//              attention weights, formed in registers or LDS and written out
//              only when the caller asks for them), then the exact top-k by
//              weight with blocks 0 and a forced (mi_select.h).
// Rows of up to 512 blocks fuse 2 and 3 (bs_fused: the scores stay in LDS);
// longer rows keep the scores in the workspace between two kernels.
#include "mi_device.h"
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

// One workgroup per (pooled row set, block): lane group g of D/8 lanes
// reads rows g, g + G, ... of the block (G = 256 / (D/8) row groups), each
// lane 8 consecutive elements (16-byte loads for bf16), then the G partial
// sums of each column are added in group order through LDS.
constexpr int kPoolNT = 256;

template <typename T>
__device__ __forceinline__ void load8(const T* src, float (&x)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* src, float (&x)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float* src, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(src);
    const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(kPoolNT) bs_pool(BsP p) {
    constexpr int LPR = D / 8;            // lanes per row
    constexpr int G = kPoolNT / LPR;      // row groups
    __shared__ float part[G][D + 1];
    const int a = blockIdx.x % p.nb;
    const int r = blockIdx.x / p.nb;  // [0, B*n_heads) queries, then [.., + B*n_kv) keys
    const T* src;
    float* dst;
    int64_t rs;
    if (r < p.B * p.n_heads) {
        const int b = r / p.n_heads, li = r % p.n_heads;
        src = reinterpret_cast<const T*>(p.q) + b * p.qs0 + p.heads[li] * p.qs1 + (int64_t)a * 64 * p.qs2;
        dst = p.qbar + ((int64_t)r * p.nb + a) * D;
        rs = p.qs2;
    } else {
        const int rk = r - p.B * p.n_heads;
        const int b = rk / p.n_kv, ki = rk % p.n_kv;
        src = reinterpret_cast<const T*>(p.k) + b * p.ks0 + p.kvlist[ki] * p.ks1 + (int64_t)a * 64 * p.ks2;
        dst = p.kbar + ((int64_t)rk * p.nb + a) * D;
        rs = p.ks2;
    }
    const int g = threadIdx.x / LPR, c8 = threadIdx.x % LPR;
    float x[64 / G][8];
#pragma unroll
    for (int u = 0; u < 64 / G; ++u) load8<T>(src + (int64_t)(g + G * u) * rs + 8 * c8, x[u]);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc[i] = x[0][i];
#pragma unroll
        for (int u = 1; u < 64 / G; ++u) acc[i] += x[u][i];
        part[g][8 * c8 + i] = acc[i];
    }
    __syncthreads();
    if (threadIdx.x < D) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < G; ++q) sum += part[q][threadIdx.x];
        dst[threadIdx.x] = sum * (1.0f / 64.0f);
    }
}

// Lower-triangle 128x128 tiles of z.  Each of the four wavefronts computes a
// 64x64 quarter (wavefront w: rows 64 (w/2), columns 64 (w%2); the quarter
// above the diagonal of a diagonal tile is skipped) as 4x4 blocks of
// v_mfma_f32_16x16x4_f32 products (lane l: A = pooled query row l%16 of its
// block, B = pooled key row l%16, D[4 (l/16) + r][l%16]) with operands read
// straight from the pooled rows, which stay in L2.  The dimensions are summed
// in a permuted order so that a lane's operands of four consecutive products
// are one 16-byte load: product s of dimension group m takes dimension
// 16 m + 4 (l/16) + s, for A and B alike.  The next group's operands are
// loaded while the current group's 64 products run.
constexpr int kScTile = 128;

template <int D>
__global__ void __launch_bounds__(256) bs_scores(BsP p) {
    const int T = (p.nb + kScTile - 1) / kScTile;
    const int per = T * (T + 1) / 2;
    const int bl = blockIdx.x / per;
    int x = blockIdx.x % per;
    int ta = 0;
    while (x >= ta + 1) { x -= ta + 1; ++ta; }
    const int tc = x;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wv >> 1, wc = wv & 1;
    if (ta == tc && wc > wr) return;  // every entry above the diagonal
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int kslot = p.kvslot[p.heads[li] / p.group];
    const float* Q = p.qbar + (int64_t)bl * p.nb * D;
    const float* K = p.kbar + ((int64_t)b * p.n_kv + kslot) * p.nb * D;
    const int r16 = lane & 15, g = lane >> 4;
    const int row0 = ta * kScTile + 64 * wr, col0 = tc * kScTile + 64 * wc;
    const float* qp[4];
    const float* kp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // rows past nb read the last row; their products are not stored
        qp[i] = Q + (int64_t)min(row0 + 16 * i + r16, p.nb - 1) * D + 4 * g;
        kp[i] = K + (int64_t)min(col0 + 16 * i + r16, p.nb - 1) * D + 4 * g;
    }
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 qa[4], kb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qa[i] = *reinterpret_cast<const f32x4*>(qp[i]);
        kb[i] = *reinterpret_cast<const f32x4*>(kp[i]);
    }
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        f32x4 qn[4], kn[4];
        if (m + 1 < D / 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qn[i] = *reinterpret_cast<const f32x4*>(qp[i] + 16 * (m + 1));
                kn[i] = *reinterpret_cast<const f32x4*>(kp[i] + 16 * (m + 1));
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][s], kb[j][s], acc[i][j], 0, 0, 0);
        if (m + 1 < D / 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qa[i] = qn[i];
                kb[i] = kn[i];
            }
        }
    }
    float* W = p.w + b * p.w_b + (int64_t)(p.w_by_head ? p.heads[li] : li) * p.w_h;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int a = row0 + 16 * i + 4 * g + r;
            if (a >= p.nb) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = col0 + 16 * j + r16;
                if (c <= a) W[(int64_t)a * p.nb + c] = acc[i][j][r] * p.scale;
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

// Selection key of block c of row a: the weight's order key, forced blocks
// 0 and a above every weight.
__device__ __forceinline__ uint32_t block_key(float w, int c, int a) {
    return (c == 0 || c == a) ? kForcedKey : order_key(w);
}

// Per (batch, listed head, query block a), rows longer than the wavefront
// form holds: the row staged in LDS, its softmax w over c <= a, top-k by w
// with blocks 0 and a forced, and (WEIGHTS) w written back over z (zeros for
// c > a).
template <bool WEIGHTS>
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
    const float inv = 1.f / sum;
    for (int c = threadIdx.x; c < p.nb; c += kSelNT) {
        float wv = 0.f;
        if (c < n) {
            wv = row[c] * inv;
            row[c] = wv;
        }
        if constexpr (WEIGHTS) W[c] = wv;
    }
    __syncthreads();
    auto key = [&](int c) -> uint32_t { return block_key(row[c], c, a); };
    const int k = min(p.top, n);
    int32_t* out = p.block_idx + (((int64_t)b * p.Hq + h) * p.nb + a) * p.top;
    select_topk<kSelNT>(key, n, k, p.top, out, sm);
    if (threadIdx.x == 0) p.block_count[((int64_t)b * p.Hq + h) * p.nb + a] = k;
}

// Top-k of one row held by a wavefront: key[u] belongs to block
// c = lane + 64 u (blocks c >= n absent, key 0).  Writes the count and the
// ascending list padded with -1.  The k-th largest key T and how many keys
// equal to T to take (the lowest blocks first) come from a bisection over
// the key bits for rows of up to 512 blocks (the weights of a row share
// their leading bits, which would put every key of a radix digit into one
// bin), else from a 4-pass radix select over 8-bit digits with the
// wavefront's 256-bin LDS histogram `hw`; then one ordered ballot pass
// (slots in index order) writes the list.  No workgroup barriers.
//
// Longer rows with k <= kFilterK first filter: the k-th largest T' of the
// 128 per-lane top-2 keys has at least k keys of the row at or above it (they
// come from distinct slots), so T >= T'; the keys >= T' (about 120-170 on rows
// of thousands of blocks) are compacted in index order into the wavefront's
// LDS buffer `cb` (kSurvCap keys, then their blocks), where the bisection and
// the ordered pass run over at most kSurvCap / 64 slots.  More survivors
// (heavy exact ties) take the radix select.
constexpr int kFilterK = 128;
constexpr int kSurvCap = 512;

template <int R>
__device__ __forceinline__ void wave_select(const uint32_t (&key)[R], int n, int top, int32_t* out,
                                            int32_t* count, uint32_t* hw, int lane, uint32_t* cb = nullptr) {
    const int k = min(top, n);
    if (lane == 0) *count = k;
    for (int m = k + lane; m < top; m += 64) out[m] = -1;
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
    uint32_t T;
    int need;
    if constexpr (R <= 8) {
        // short rows: the k-th largest key by bisection, one key bit per step
        // (a compare and a ballot per slot), no LDS
        T = 0u;
#pragma unroll 1
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int ge = 0;
#pragma unroll
            for (int u = 0; u < R; ++u) ge += __popcll(__ballot(key[u] >= cand));  // absent keys are 0
            if (ge >= k) T = cand;
        }
        int gt = 0;
#pragma unroll
        for (int u = 0; u < R; ++u) gt += __popcll(__ballot(key[u] > T));
        need = k - gt;
    } else {
    if (k <= kFilterK) {
        uint32_t m1 = 0u, m2 = 0u;  // the lane's two largest keys (absent keys are 0)
#pragma unroll
        for (int u = 0; u < R; ++u) {
            m2 = max(m2, min(m1, key[u]));
            m1 = max(m1, key[u]);
        }
        uint32_t t = 0u;
#pragma unroll 1
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            if (__popcll(__ballot(m1 >= cand)) + __popcll(__ballot(m2 >= cand)) >= k) t = cand;
        }
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int c = lane + 64 * u;
            const bool sv = c < n && key[u] >= t;
            const uint64_t m = __ballot(sv);
            const int pos = cnt + __popcll(m & below);
            if (sv && pos < kSurvCap) {
                cb[pos] = key[u];
                cb[kSurvCap + pos] = (uint32_t)c;
            }
            cnt += __popcll(m);
        }
        if (cnt <= kSurvCap) {
            __builtin_amdgcn_wave_barrier();
            constexpr int V = kSurvCap / 64;
            uint32_t y[V];
#pragma unroll
            for (int v = 0; v < V; ++v) y[v] = lane + 64 * v < cnt ? cb[lane + 64 * v] : 0u;
            uint32_t T = 0u;
#pragma unroll 1
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                int ge = 0;
#pragma unroll
                for (int v = 0; v < V; ++v) ge += __popcll(__ballot(y[v] >= cand));  // absent slots are 0
                if (ge >= k) T = cand;
            }
            int gt = 0;
#pragma unroll
            for (int v = 0; v < V; ++v) gt += __popcll(__ballot(y[v] > T));
            const int need = k - gt;
            // ordered output over the survivors (their positions follow the blocks' order)
            int run_eq = 0, run_sel = 0;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int j = lane + 64 * v;
                const bool g = j < cnt && y[v] > T;
                const bool e = j < cnt && y[v] == T;
                const uint64_t me = __ballot(e);
                const bool sel = g || (e && run_eq + __popcll(me & below) < need);
                const uint64_t ms = __ballot(sel);
                if (sel) out[run_sel + __popcll(ms & below)] = (int32_t)cb[kSurvCap + j];
                run_eq += __popcll(me);
                run_sel += __popcll(ms);
            }
            return;
        }
    }
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
    T = prefix;
    need = rem;
    }
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

// Softmax of a row held by a wavefront, in place (slot u of block
// c = lane + 64 u, blocks c >= n get 0); with WEIGHTS also stored to W[c]
// for every c < nb.
template <int R, bool WEIGHTS>
__device__ __forceinline__ void wave_weights(float (&x)[R], int n, int nb, float* W, int lane) {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < R; ++u) mx = fmaxf(mx, lane + 64 * u < n ? x[u] : -INFINITY);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        x[u] = lane + 64 * u < n ? fast_exp2((x[u] - mx) * kLog2e) : 0.f;
        sum += x[u];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    const float inv = 1.f / sum;  // one division per row; weights within an ulp of x / sum
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int c = lane + 64 * u;
        x[u] = c < n ? x[u] * inv : 0.f;
        if constexpr (WEIGHTS) {
            if (c < nb) W[c] = x[u];
        }
    }
}

// The selection with one wavefront per query block (rows of at most 64 R
// blocks), the row in registers (block c = lane + 64 u in slot u).
constexpr int kWaveRows = 4;  // wavefronts (rows) per workgroup

template <int R, bool WEIGHTS>
__global__ void __launch_bounds__(64 * kWaveRows) bs_select_wave(BsP p) {
    __shared__ uint32_t hist[kWaveRows][256];
    __shared__ uint32_t surv[kWaveRows][R > 8 ? 2 * kSurvCap : 1];
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
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int c = lane + 64 * u;
        x[u] = c < n ? W[c] : -INFINITY;
    }
    wave_weights<R, WEIGHTS>(x, n, p.nb, W, lane);
    uint32_t key[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int c = lane + 64 * u;
        key[u] = c < n ? block_key(x[u], c, a) : 0u;
    }
    const int64_t row = ((int64_t)b * p.Hq + h) * p.nb + a;
    wave_select<R>(key, n, p.top, p.block_idx + row * p.top, p.block_count + row, hist[wv], lane, surv[wv]);
}

// Fused scores and selection for rows of at most kFusedMaxNb blocks: one
// workgroup of eight wavefronts per (batch, listed head, strip of kStrip
// query blocks) forms the strip's scores z[a][c] = scale * Qbar_a . Kbar_c
// for every causal column in LDS, then each wavefront takes two rows from
// LDS: softmax, top-k by weight.  The scores never reach memory; the weights
// are written only when the caller asks.
//
// The scores are fp32 matrix-core products (v_mfma_f32_16x16x4_f32, A = the
// strip's 16 query rows x 4 dimensions, B = 4 dimensions x 16 key blocks),
// 256 columns at a time: wavefront w owns the 16-column blocks 2w, 2w+1 and
// skips those past the strip's last causal column.  Kbar is staged in LDS in
// chunks of kKc dimensions (row pitch 36 floats: the B reads of 16 rows x 4
// dimensions hit distinct banks), the next chunk loaded while the current
// one is used.  Lane l holds A[l % 16][l / 16], B[l / 16][l % 16] and
// D[4 (l / 16) + r][l % 16], r < 4.
constexpr int kStrip = 16;
constexpr int kFusedMaxNb = 512;
constexpr int kKc = 32;
constexpr int kFusedNT = 512;
constexpr int kKsPitch = 36;

template <int D, bool WEIGHTS>
__global__ void __launch_bounds__(kFusedNT) bs_fused(BsP p) {
    constexpr int ZS = kFusedMaxNb + 4;
    constexpr int R = kFusedMaxNb / 64;
    constexpr int NW = kFusedNT / 64;
    constexpr int RPW = kStrip / NW;  // rows selected per wavefront
    __shared__ float zs[kStrip][ZS];
    __shared__ __attribute__((aligned(16))) float qt[D][kStrip];  // Qbar^T of the strip
    __shared__ __attribute__((aligned(16))) float ks[256][kKsPitch];
    // the selection's histograms reuse the Kbar staging buffer, dead by then
    static_assert(sizeof(ks) >= NW * 256 * sizeof(uint32_t), "histograms fit in the staging buffer");
    uint32_t(*hist)[256] = reinterpret_cast<uint32_t(*)[256]>(&ks[0][0]);
    const int nstrip = (p.nb + kStrip - 1) / kStrip;
    const int bl = blockIdx.x / nstrip, strip = blockIdx.x % nstrip;
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int h = p.heads[li];
    const float* Q = p.qbar + (int64_t)bl * p.nb * D;
    const float* K = p.kbar + ((int64_t)b * p.n_kv + p.kvslot[h / p.group]) * p.nb * D;
    const int a0 = strip * kStrip;
    const int rows = min(kStrip, p.nb - a0);
    const int t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    {
        // the strip's rows: all loads issued first (rows past nb read row 0)
        float qv[kStrip * D / kFusedNT];
#pragma unroll
        for (int u = 0; u < kStrip * D / kFusedNT; ++u) {
            const int e = u * kFusedNT + t;
            const int r = e / D, d = e % D;
            qv[u] = Q[(int64_t)(r < rows ? a0 + r : 0) * D + d];
        }
#pragma unroll
        for (int u = 0; u < kStrip * D / kFusedNT; ++u) {
            const int e = u * kFusedNT + t;
            const int r = e / D, d = e % D;
            qt[d][r] = r < rows ? qv[u] : 0.f;
        }
    }
    const int ncol = a0 + rows;
    // Kbar chunks: 256 rows x kKc floats, one row per 8 lanes (float4 along
    // d); all loads of a chunk are in flight together, rows past nb read row
    // 0 and are zeroed when stored
    constexpr int kLd = 256 * kKc / 4 / kFusedNT;
    const int nchunk = (ncol + 255) / 256 * (D / kKc);
    auto load_chunk = [&](int ci, f32x4 (&x)[kLd]) {
        const int c0 = (ci / (D / kKc)) * 256, k0 = (ci % (D / kKc)) * kKc;
#pragma unroll
        for (int u = 0; u < kLd; ++u) {
            const int e = u * kFusedNT + t;
            const int c = c0 + e / (kKc / 4);
            x[u] = *reinterpret_cast<const f32x4*>(K + (int64_t)(c < p.nb ? c : 0) * D + k0 + 4 * (e % (kKc / 4)));
        }
    };
    f32x4 xb[kLd];
    load_chunk(0, xb);
    f32x4 acc[2];
    const int ri = lane & 15, kq = lane >> 4;
    for (int ci = 0; ci < nchunk; ++ci) {
        const int c0 = (ci / (D / kKc)) * 256, k0 = (ci % (D / kKc)) * kKc;
        if (k0 == 0) acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();  // the previous chunk's reads are done
#pragma unroll
        for (int u = 0; u < kLd; ++u) {
            const int e = u * kFusedNT + t;
            const int r = e / (kKc / 4), q4 = e % (kKc / 4);
            const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(&ks[r][4 * q4]) = c0 + r < p.nb ? xb[u] : z0;
        }
        __syncthreads();
        if (ci + 1 < nchunk) load_chunk(ci + 1, xb);
        // the wavefront's column blocks that hold causal columns (uniform)
        const int cb0 = 2 * wv;
        const int nblk = min(2, max(0, (ncol - c0 - 16 * cb0 + 15) / 16));
        if (nblk > 0) {
#pragma unroll
            for (int ks4 = 0; ks4 < kKc / 4; ++ks4) {
                const float av = qt[k0 + 4 * ks4 + kq][ri];
                const float b0 = ks[16 * cb0 + ri][4 * ks4 + kq];
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b0, acc[0], 0, 0, 0);
                if (nblk > 1) {
                    const float b1 = ks[16 * (cb0 + 1) + ri][4 * ks4 + kq];
                    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b1, acc[1], 0, 0, 0);
                }
            }
        }
        if (k0 + kKc < D) continue;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = c0 + 16 * (cb0 + q) + ri;
                if (c < ZS) zs[4 * kq + r][c] = acc[q][r] * p.scale;
            }
    }
    __syncthreads();
    for (int rr = RPW * wv; rr < RPW * wv + RPW && rr < rows; ++rr) {
        const int a = a0 + rr, n = a + 1;
        float x[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int c = lane + 64 * u;
            x[u] = c < n ? zs[rr][c] : -INFINITY;
        }
        wave_weights<R, WEIGHTS>(x, n, p.nb, p.w + b * p.w_b + (int64_t)h * p.w_h + (int64_t)a * p.nb, lane);
        uint32_t key[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int c = lane + 64 * u;
            key[u] = c < n ? block_key(x[u], c, a) : 0u;
        }
        const int64_t row = ((int64_t)b * p.Hq + h) * p.nb + a;
        wave_select<R>(key, n, p.top, p.block_idx + row * p.top, p.block_count + row, hist[wv], lane);
    }
}

// Antidiagonal block scores (hysenlabs review, "How MInference differs from
// xAttention, FlexPrefill and RetrievalAttention": blocks scored by
// antidiagonal sums):
//     x[a][c] = scale * sum_r q[64a + r] . k[64c + 63 - r],   c <= a,
// over the causal half r >= 32 only for c = a.  As a matrix, X = Qt . Kt^T
// with Qt[a] the 64 rows of query block a laid end to end and Kt[c] those of
// key block c in reverse order: a dense contraction over 64 d, so on MFMA.
// One wavefront per 32x32 tile of X (query blocks 32 ta + i, key blocks
// 32 tc + j, tc <= ta): for each r it reads query row 64a + r and key row
// 64c + 63 - r as operand fragments (transposed form, as the Vertical-Slash
// estimate: lane l holds query block l % 32 and key blocks
// 8 (e/4) + 4 (l/32) + e % 4 of acc[e]).  On a diagonal tile the lane whose
// key block equals its query block keeps the sum after r = 31 and subtracts
// it at the end.  The scores go to the score rows that the selection kernels
// then turn into weights and lists.  Used for fp32 inputs.
constexpr int kAdWaves = 4;

template <typename T, int D>
__global__ void __launch_bounds__(64 * kAdWaves) ad_scores(BsP p) {
    typedef typename Elem<T>::frag Frag;
    const int T32 = (p.nb + 31) / 32;
    const int per = T32 * (T32 + 1) / 2;  // lower-triangle tiles per listed head
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * kAdWaves + wv;
    if (item >= (int64_t)p.B * p.n_heads * per) return;
    const int bl = (int)(item / per);
    int x = (int)(item % per);
    int ta = 0;
    while (x >= ta + 1) {
        x -= ta + 1;
        ++ta;
    }
    const int tc = x;
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int h = p.heads[li];
    const int rl = lane & 31, hl = lane >> 5;
    const int a = 32 * ta + rl;             // this lane's query block
    const int ca = a < p.nb ? a : p.nb - 1;  // rows read for blocks past nb (not written)
    const int cb = min(32 * tc + rl, p.nb - 1);
    const T* qrow0 = reinterpret_cast<const T*>(p.q) + b * p.qs0 + h * p.qs1 + (int64_t)ca * 64 * p.qs2 + 8 * hl;
    const T* krow0 = reinterpret_cast<const T*>(p.k) + b * p.ks0 + (h / p.group) * p.ks1 +
                     ((int64_t)cb * 64 + 63) * p.ks2 + 8 * hl;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    // the diagonal entry of this lane (key block == query block), if any
    const bool diag_tile = ta == tc;
    const int e_d = ((rl >> 3) << 2) | (rl & 3);
    const bool has_d = diag_tile && ((rl >> 2) & 1) == hl;
    float d_low = 0.f;
#pragma unroll 2
    for (int r = 0; r < 64; ++r) {
        Frag qf[D / 16], kf[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            qf[s] = load_frag(qrow0 + (int64_t)r * p.qs2 + 16 * s);
            kf[s] = load_frag(krow0 - (int64_t)r * p.ks2 + 16 * s);
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) mma32(acc, kf[s], qf[s]);
        if (r == 31 && has_d) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (e == e_d) d_low = acc[e];
        }
    }
    if (a >= p.nb) return;
    float* W = p.w + b * p.w_b + (int64_t)(p.w_by_head ? h : li) * p.w_h + (int64_t)a * p.nb;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int c = 32 * tc + 8 * (e >> 2) + 4 * hl + (e & 3);
        if (c > a || c >= p.nb) continue;
        const float v = (c == a) ? acc[e] - d_low : acc[e];
        W[c] = v * p.scale;
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// bf16: one workgroup of eight wavefronts per 256 x 256 tile of X (query
// blocks 256 ta + i, key blocks 256 tc + j, tc <= ta), which reads 16 times
// fewer operand rows per product than a wavefront per 32 x 32 tile.  Each step
// stages 64 dimensions of one row of each of the tile's 256 query blocks
// (row r) and 256 key blocks (row 63 - r): 2 x 256 rows of 128 bytes,
// global -> LDS, double-buffered; 16-byte chunk c of row y sits at c ^
// ((y / 2) % 8), so that 16 lanes reading one chunk of 16 consecutive rows
// hit all 64 banks once.  Wavefront w computes query blocks 64 (w / 2) ..
// + 63 against key blocks 128 (w % 2) .. + 127: eight 32 x 32 MFMA tiles, the
// four K operands of a slice used twice and the two Q operands four times.
constexpr int kAdlWaves = 8;
struct AdTile {
    static constexpr int kRowBytes = 128;  // 64 bf16 dimensions
    static constexpr int kRows = 256;
    static constexpr int kBytes = kRows * kRowBytes;  // one side
    __device__ static int offset(int y, int c) { return y * kRowBytes + ((c ^ ((y >> 1) & 7)) << 4); }
};

// Copies of step (r, half) into `dst`: 2 sides x 256 rows x 8 chunks, one
// 16-byte chunk per lane per instruction; rows past nb read block nb - 1
// (their scores are not written).
__device__ __forceinline__ void ad_issue(char* dst, const uint16_t* qb, const uint16_t* kb, int64_t qs2, int64_t ks2,
                                          int qrow0, int krow0, int nb, int r, int half, int wv, int lane) {
    constexpr int kChunks = 2 * AdTile::kRows * 8;
    constexpr int kIters = kChunks / (64 * kAdlWaves);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int idx = it * kAdlWaves + wv;  // wave instruction index
        const int cidx = idx * 64 + lane;     // chunk slot
        const int side = cidx / (AdTile::kRows * 8);
        const int rem = cidx % (AdTile::kRows * 8);
        const int y = rem >> 3, pos = rem & 7;
        const int blk = min((side ? krow0 : qrow0) + y, nb - 1);
        const uint16_t* src = side ? kb + ((int64_t)blk * 64 + 63 - r) * ks2 : qb + ((int64_t)blk * 64 + r) * qs2;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + 128 * half + 16 * (pos ^ ((y >> 1) & 7)),
                                         (lds_void*)(dst + idx * 1024), 16, 0, 0);
    }
}

template <int D>
__global__ void __launch_bounds__(64 * kAdlWaves) ad_scores_lds(BsP p) {
    constexpr int H = D / 64;  // steps per antidiagonal row
    __shared__ __attribute__((aligned(16))) char buf[2][2][AdTile::kBytes];  // [buffer][q, k]
    const int T256 = (p.nb + 255) / 256;
    const int per = T256 * (T256 + 1) / 2;
    // consecutive tiles (of one head, sharing query and key rows) on one XCD:
    // the hardware deals workgroups to the eight XCDs in turn
    const int G = gridDim.x;
    const int L = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int bl = L / per;
    int x = L % per;
    int ta = 0;
    while (x >= ta + 1) {
        x -= ta + 1;
        ++ta;
    }
    const int tc = x;
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int h = p.heads[li];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int rl = lane & 31, hl = lane >> 5;
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + b * p.qs0 + h * p.qs1;
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + b * p.ks0 + (h / p.group) * p.ks1;
    const int qrow0 = 256 * ta, krow0 = 256 * tc;
    const int qsub = wv >> 1, khalf = wv & 1;
    f32x16 acc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;
    // diagonal entries (ta == tc): query sub-tile j meets key sub-tile i on
    // the diagonal when 64 qsub + 32 j == 128 khalf + 32 i
    const int e_d = ((rl >> 3) << 2) | (rl & 3);
    const bool lane_d = ((rl >> 2) & 1) == hl;
    float d_low[2] = {0.f, 0.f};
    ad_issue(&buf[0][0][0], qb, kb, p.qs2, p.ks2, qrow0, krow0, p.nb, 0, 0, wv, lane);
#pragma unroll 1
    for (int st = 0; st < 64 * H; ++st) {
        __syncthreads();  // copies of st have landed (each wave waited for its own); st-1 is read
        if (st + 1 < 64 * H)
            ad_issue(&buf[(st + 1) & 1][0][0], qb, kb, p.qs2, p.ks2, qrow0, krow0, p.nb, (st + 1) / H, (st + 1) % H,
                      wv, lane);
        const char* qs = &buf[st & 1][0][0];
        const char* ks = &buf[st & 1][1][0];
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            bf16x8 kf[4], qf[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kf[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                        ks + AdTile::offset(128 * khalf + 32 * i + rl, 2 * sl + hl)));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                qf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                        qs + AdTile::offset(64 * qsub + 32 * j + rl, 2 * sl + hl)));
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) mma32(acc[j][i], kf[i], qf[j]);
        }
        if (st == 32 * H - 1 && ta == tc && lane_d) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (64 * qsub + 32 * j == 128 * khalf + 32 * i) {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            if (e == e_d) d_low[j] = acc[j][i][e];
                    }
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int a = 256 * ta + 64 * qsub + 32 * j + rl;
        if (a >= p.nb) continue;
        float* W = p.w + b * p.w_b + (int64_t)(p.w_by_head ? h : li) * p.w_h + (int64_t)a * p.nb;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = 256 * tc + 128 * khalf + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
                if (c > a || c >= p.nb) continue;
                const float v = (c == a) ? acc[j][i][e] - d_low[j] : acc[j][i][e];
                W[c] = v * p.scale;
            }
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Softmax and top-k of the score rows p.w (weights written back when asked).
hipError_t launch_select(BsP& p, bool weights, hipStream_t s) {
    hipError_t e = hipSuccess;
    const int64_t sel_rows = (int64_t)p.B * p.n_heads * p.nb;
    const dim3 wgrid((unsigned)((sel_rows + kWaveRows - 1) / kWaveRows)), wblock(64 * kWaveRows);
#define MI_SEL_WAVE(R)                                                                   \
    if (weights) hipLaunchKernelGGL((bs_select_wave<R, true>), wgrid, wblock, 0, s, p); \
    else hipLaunchKernelGGL((bs_select_wave<R, false>), wgrid, wblock, 0, s, p);
    if (p.nb <= 128) {
        MI_SEL_WAVE(2)
    } else if (p.nb <= 512) {
        MI_SEL_WAVE(8)
    } else if (p.nb <= 1024) {
        MI_SEL_WAVE(16)
    } else if (p.nb <= 2048) {
        MI_SEL_WAVE(32)
    } else if (p.nb <= 4096) {
        MI_SEL_WAVE(64)
    } else {
        // longer rows: one workgroup per row, the row staged in LDS
        const size_t dyn = (size_t)p.nb * sizeof(float);
        const void* fn = weights ? reinterpret_cast<const void*>(bs_select<true>)
                                 : reinterpret_cast<const void*>(bs_select<false>);
        if (dyn > 48 * 1024) {
            e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
            if (e != hipSuccess) return e;
        }
        if (weights) hipLaunchKernelGGL(bs_select<true>, dim3(p.B * p.n_heads * p.nb), dim3(kSelNT), dyn, s, p);
        else hipLaunchKernelGGL(bs_select<false>, dim3(p.B * p.n_heads * p.nb), dim3(kSelNT), dyn, s, p);
    }
#undef MI_SEL_WAVE
    return hipGetLastError();
}


}  // namespace

size_t bs_workspace_bytes(int32_t B, int32_t n_heads, int32_t Hkv, int32_t N, int32_t D,
                          bool caller_scores) {
    const size_t nb = N / 64;
    size_t bytes = align256((size_t)B * n_heads * nb * D * sizeof(float));
    bytes += align256((size_t)B * Hkv * nb * D * sizeof(float));
    // scores between the two kernels of rows longer than the fused kernel takes
    if (!caller_scores && nb > (size_t)kFusedMaxNb) bytes += align256((size_t)B * n_heads * nb * nb * sizeof(float));
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
    const dim3 pgrid((unsigned)(pool_rows * p.nb)), pblock(kPoolNT);
    if (a.dtype == MI_BF16) {
        if (a.D == 64) hipLaunchKernelGGL((bs_pool<uint16_t, 64>), pgrid, pblock, 0, s, p);
        else hipLaunchKernelGGL((bs_pool<uint16_t, 128>), pgrid, pblock, 0, s, p);
    } else {
        if (a.D == 64) hipLaunchKernelGGL((bs_pool<float, 64>), pgrid, pblock, 0, s, p);
        else hipLaunchKernelGGL((bs_pool<float, 128>), pgrid, pblock, 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool weights = a.w != nullptr;
    if (p.nb <= kFusedMaxNb) {
        const dim3 grid((unsigned)(a.B * a.n_heads * ((p.nb + kStrip - 1) / kStrip))), block(kFusedNT);
        if (a.D == 64) {
            if (weights) hipLaunchKernelGGL((bs_fused<64, true>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((bs_fused<64, false>), grid, block, 0, s, p);
        } else {
            if (weights) hipLaunchKernelGGL((bs_fused<128, true>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((bs_fused<128, false>), grid, block, 0, s, p);
        }
        return hipGetLastError();
    }
    const int T = (p.nb + kScTile - 1) / kScTile;
    const dim3 sgrid((unsigned)(a.B * a.n_heads * (T * (T + 1) / 2))), sblock(256);
    if (a.D == 64) hipLaunchKernelGGL((bs_scores<64>), sgrid, sblock, 0, s, p);
    else hipLaunchKernelGGL((bs_scores<128>), sgrid, sblock, 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_select(p, weights, s);
}

size_t ad_workspace_bytes(int32_t B, int32_t n_heads, int32_t N, bool caller_scores) {
    const size_t nb = N / 64;
    return caller_scores ? 256 : align256((size_t)B * n_heads * nb * nb * sizeof(float));
}

hipError_t launch_antidiag_estimate(const BsArgs& a, hipStream_t s) {
    BsP p{};
    p.q = static_cast<const char*>(a.q);
    p.k = static_cast<const char*>(a.k);
    p.qs0 = a.qs[0]; p.qs1 = a.qs[1]; p.qs2 = a.qs[2];
    p.ks0 = a.ks[0]; p.ks1 = a.ks[1]; p.ks2 = a.ks[2];
    p.B = a.B; p.Hq = a.Hq; p.N = a.N; p.nb = a.N / 64; p.D = a.D;
    p.group = a.Hq / a.Hkv;
    p.n_heads = a.n_heads; p.top = a.top; p.scale = a.scale;
    for (int i = 0; i < a.n_heads; ++i) p.heads[i] = a.heads[i];
    const int64_t nb2 = (int64_t)p.nb * p.nb;
    const bool weights = a.w != nullptr;
    if (weights) {
        p.w = a.w;
        p.w_b = (int64_t)a.Hq * nb2;
        p.w_h = nb2;
        p.w_by_head = 1;
    } else {
        p.w = static_cast<float*>(a.ws);
        p.w_b = (int64_t)a.n_heads * nb2;
        p.w_h = nb2;
        p.w_by_head = 0;
    }
    p.block_idx = a.block_idx;
    p.block_count = a.block_count;
    const int T32 = (p.nb + 31) / 32;
    const int64_t tiles = (int64_t)a.B * a.n_heads * (T32 * (T32 + 1) / 2);
    const dim3 grid((unsigned)((tiles + kAdWaves - 1) / kAdWaves)), block(64 * kAdWaves);
    if (a.dtype == MI_BF16) {
        const int T256 = (p.nb + 255) / 256;
        const dim3 lgrid((unsigned)(a.B * a.n_heads * (T256 * (T256 + 1) / 2))), lblock(64 * kAdlWaves);
        if (a.D == 64) hipLaunchKernelGGL((ad_scores_lds<64>), lgrid, lblock, 0, s, p);
        else hipLaunchKernelGGL((ad_scores_lds<128>), lgrid, lblock, 0, s, p);
    } else {
        if (a.D == 64) hipLaunchKernelGGL((ad_scores<float, 64>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((ad_scores<float, 128>), grid, block, 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_select(p, weights, s);
}

}  // namespace mi
