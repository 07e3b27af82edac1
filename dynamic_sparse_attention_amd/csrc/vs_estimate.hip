// Vertical-Slash estimate for gfx950: the last last_q queries of a head
// against every key, causal softmax per row, then column sums (vertical
// scores) and diagonal sums (slash scores).  hotpaper.ai summary of arXiv
// 2407.02490, key idea: Vertical-Slash heads estimate their important
// positions from the last last_q queries.
//
// Four launches:
//   1. rowstat_partial (batch, set of up to four listed heads of one kv head,
//      key chunk): each row's running max and normaliser (log2 domain) with
//      bf16/fp32 MFMA scores, the K tiles staged once per set in LDS;
//   2. rowstat_combine: merges the chunk partials of each row in a fixed
//      order;
//   3. scores (batch, listed head, group of sixteen 128-key chunks; chunk c =
//      keys [J0, J0+128), J0 = N-(c+1)*128): recomputes the chunk's scores,
//      normalises them with the row statistics and stores them in LDS
//      skewed by row: with
//      L = last_q, P[r][j] (query i_r = N-L+r) sits at column
//      (j - J0) + L-1 - r, so that a diagonal of the score matrix (offset
//      o = i_r - j) is one column, x = N-1-J0-o.  Columns give the chunk's
//      part of the slash sums of offsets [128c-(L-1), 128c+127]; the
//      anti-diagonals give the complete vertical sums of its keys.  Offsets
//      [128c, 128c+127] are written as partial sums; the offsets below go to
//      the workspace (63 slots, L-1 of them non-zero);
//   4. slash_combine adds those values of chunk c+1 into the top offsets of
//      chunk c.
// Every output is summed by one thread in a fixed order (deterministic).
// The top-k that follows (topk.hip) takes its first radix histogram from
// these kernels: rowstat_partial clears the top-k scratch, and each score
// reaches the histogram of its row where it becomes final (in scores, or in
// slash_combine for the offsets that receive a spill), so the top-k reads
// the rows three times instead of five.
//
// Score layout (MFMA result, transposed): S^T (32 keys x 32 rows) = K . Q^T.
// Lane l holds query row (l%32) of row block rb and keys
// 8*(e/4) + 4*(l/32) + (e%4) of the 32-key unit.
#include <algorithm>

#include "mi_device.h"
#include "mi_internal.h"
#include "mi_topk.h"

namespace mi {
namespace {

// Row-statistics workgroups in flight (three per compute unit); the key
// range of each set of heads is cut into about kRowstatWGs / sets chunks.
constexpr int kRowstatWGs = 768;
constexpr int kChunk2 = 128;   // keys per score work item (one 32-key unit per wavefront)
constexpr int kSpill = 63;     // slash offsets a chunk contributes below its own range
constexpr int kChunksPerItem = 16;  // score chunks per workgroup (the Q rows are loaded once)
// LDS row pitch of the skewed probability tile (floats): 191 columns used; a
// pitch of 194 puts the column of consecutive rows on consecutive banks.
constexpr int kPitch2 = 194;

typedef __attribute__((address_space(3))) void lds_void;

struct VsP {
    const char* q;
    const char* k;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2;
    int32_t B, Hq, N, group, n_heads, last_q;
    float c;  // scale * log2(e)
    int32_t heads[MI_MAX_HEADS];
    float* stats;    // [B*n_heads][nchunk1][64] x (m, l)
    float* rowstat;  // [B*n_heads][64] x (m, l)
    int32_t nchunk1, nchunk2;
    int32_t chunk1;  // keys per row-statistics chunk (a multiple of 64)
    int32_t nsets;   // sets of listed heads that share a kv head (at most 4 each)
    uint8_t set_n[MI_MAX_HEADS];
    uint8_t set_li[MI_MAX_HEADS][4];  // list positions of each set's heads
    float* vscore;
    float* sscore;
    int64_t srow_b, srow_h;  // score row strides (elements)
    int32_t score_by_head;   // 1: row index is the head id, 0: the list position
    float* spill;            // [B*n_heads][nchunk2][kSpill] slash partials below each chunk's range
    uint32_t* topk;          // top-k scratch, kTopkRowWords per score row (mi_topk.h)
    int32_t topk_rows;       // 2 * B * n_heads
    int32_t force_v, force_s;
};

// First-digit histograms of a head's two score rows: the keys are those the
// top-k ranks (mi_topk.h), taken from the final score values.
__device__ __forceinline__ uint32_t* topk_row(const VsP& p, int bl, int which) {
    return p.topk + (int64_t)(2 * bl + which) * kTopkRowWords;
}

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    l = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
    m = M;
}

// Q fragments of the estimate rows: row slot r = 32*rb + (l%32) holds query
// i_r = N - last_q + r (zero for r >= last_q).
template <typename T, int D>
__device__ __forceinline__ void load_q_rows(const VsP& p, const T* qbase, int rl, int hl,
                                            typename Elem<T>::frag (&qf)[2][D / 16]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = rb * 32 + rl;
        if (r < p.last_q) {
            const T* qrow = qbase + (int64_t)(p.N - p.last_q + r) * p.qs2;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) qf[rb][s] = load_frag(qrow + 16 * s + 8 * hl);
        } else {
#pragma unroll
            for (int s = 0; s < D / 16; ++s) qf[rb][s] = typename Elem<T>::frag{};
        }
    }
}

// K fragments of the 32 keys [key0, key0+32): every lane loads (a clamped,
// valid row) so that the loads issue together; lanes whose key lies outside
// [0, N) get zero fragments in unit_mma.
template <typename T, int D>
__device__ __forceinline__ void unit_load(const VsP& p, const T* kbase, int key0, int rl, int hl,
                                          typename Elem<T>::frag (&kf)[D / 16]) {
    const int key = key0 + rl;
    const bool ok = key >= 0 && key < p.N;
    const T* krow = kbase + (int64_t)(ok ? key : 0) * p.ks2 + 8 * hl;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[s] = load_frag(krow + 16 * s);
}

// Scores of those 32 keys against the 64 row slots (out-of-range keys score
// zero; the caller masks them).
template <typename T, int D>
__device__ __forceinline__ void unit_mma(const VsP& p, int key0, int rl, const typename Elem<T>::frag (&kf)[D / 16],
                                         const typename Elem<T>::frag (&qf)[2][D / 16], f32x16 (&acc)[2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][e] = 0.f;
    const int key = key0 + rl;
    const bool ok = key >= 0 && key < p.N;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const typename Elem<T>::frag a = ok ? kf[s] : typename Elem<T>::frag{};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) mma32(acc[rb], a, qf[rb][s]);
    }
}

// Row statistics over one key chunk for a set of up to four listed heads
// that read the same kv head: the workgroup stages each 64-key K tile once
// in LDS (global -> LDS copies, double-buffered) and wavefront w scores it
// against the 64 estimate rows of the set's head w.  LDS rows are 16-byte
// chunks, chunk c of key row r stored at c ^ (r & 15), so the fragment reads
// of 16 consecutive rows hit distinct banks.
template <typename T, int D>
struct KTile {
    static constexpr int kRowBytes = D * (int)sizeof(T);
    static constexpr int kCpr = kRowBytes / 16;           // 16-byte chunks per key row
    static constexpr int kSwz = kCpr < 16 ? kCpr - 1 : 15;
    static constexpr int kBytes = 64 * kRowBytes;
    __device__ static int offset(int r, int c) { return r * kRowBytes + ((c ^ (r & kSwz)) << 4); }
};

template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag tile_frag(const char* tile, int r, int s, int hl) {
    typedef KTile<T, D> Kt;
    if constexpr (sizeof(T) == 2) {
        // slots 16s + 8hl .. +8 of key row r: chunk 2s + hl
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + Kt::offset(r, 2 * s + hl)));
    } else {
        // slots 16s + 8hl .. +8 (32 bytes): chunks 4s + 2hl, +1
        const f32x4 a = *reinterpret_cast<const f32x4*>(tile + Kt::offset(r, 4 * s + 2 * hl));
        const f32x4 b = *reinterpret_cast<const f32x4*>(tile + Kt::offset(r, 4 * s + 2 * hl + 1));
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(256) vs_rowstat_partial(VsP p) {
    typedef KTile<T, D> Kt;
    typedef typename Elem<T>::frag Frag;
    __shared__ __attribute__((aligned(16))) char tiles[2][Kt::kBytes];
    const int nitems = p.B * p.nsets * p.nchunk1;
    const int L = blockIdx.x;
    // the top-k histograms start at zero: cleared here, filled by the score
    // kernels that follow on the stream
    for (int64_t i = (int64_t)L * 256 + threadIdx.x; i < (int64_t)p.topk_rows * kTopkClearWords;
         i += (int64_t)gridDim.x * 256)
        p.topk[(i / kTopkClearWords) * kTopkRowWords + i % kTopkClearWords] = 0u;
    if (L >= nitems) return;
    const int chunk = L % p.nchunk1;
    const int bs = L / p.nchunk1;
    const int b = bs / p.nsets, set = bs % p.nsets;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 31, hl = lane >> 5;
    // list position of this wavefront's head (-1: the set has fewer heads)
    const int li = wave < p.set_n[set] ? (int)p.set_li[set][wave] : -1;
    const int kvh = p.heads[p.set_li[set][0]] / p.group;
    const T* kbase = reinterpret_cast<const T*>(p.k) + b * p.ks0 + kvh * p.ks1;

    Frag qf[2][D / 16];
    if (li >= 0) {
        const int h = p.heads[li];
        load_q_rows<T, D>(p, reinterpret_cast<const T*>(p.q) + b * p.qs0 + h * p.qs1, rl, hl, qf);
    }
    const int k_begin = chunk * p.chunk1;
    const int k_end = min(p.N, k_begin + p.chunk1);
    const int ntiles = (k_end - k_begin + 63) / 64;

    // staging: global -> LDS copies (16 bytes per lane, 1 KiB of consecutive
    // LDS per wavefront instruction); lane slot (row, pos) takes source chunk
    // pos ^ (row & kSwz), which realises the swizzled layout
    auto fetch = [&](char* tile, int ti) {
        const int key0 = k_begin + 64 * ti;
#pragma unroll
        for (int i = 0; i < Kt::kCpr / 4; ++i) {
            const int idx = i * 4 + wave;
            const int cidx = idx * 64 + lane;
            const int r = cidx / Kt::kCpr, pos = cidx % Kt::kCpr;
            const int key = min(key0 + r, p.N - 1);  // rows past N are masked below
            const char* src = reinterpret_cast<const char*>(kbase + (int64_t)key * p.ks2) + 16 * (pos ^ (r & Kt::kSwz));
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(tile + idx * 1024), 16, 0, 0);
        }
    };

    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    fetch(tiles[0], 0);
    __syncthreads();
#pragma unroll 1
    for (int ti = 0; ti < ntiles; ++ti) {
        if (ti + 1 < ntiles) fetch(tiles[(ti + 1) & 1], ti + 1);
        const char* tile = tiles[ti & 1];
        if (li >= 0) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int key0 = k_begin + 64 * ti + 32 * u;
                f32x16 acc[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[rb][e] = 0.f;
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    const Frag a = tile_frag<T, D>(tile, 32 * u + rl, s, hl);
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) mma32(acc[rb], a, qf[rb][s]);
                }
                // units that end before the first estimate row's position need
                // no mask (wave-uniform); the scale is positive, so the raw
                // maximum scales to the scaled one
                const bool open = key0 + 31 <= p.N - p.last_q;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const int r = rb * 32 + rl;
                    const int ir = p.N - p.last_q + r;
                    if (open && rb * 32 + 31 < p.last_q) {
                        float mx = acc[rb][0];
#pragma unroll
                        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, acc[rb][e]);
                        const float M = fmaxf(m[rb], mx * p.c);
                        float sum = 0.f;
#pragma unroll
                        for (int e = 0; e < 16; ++e) sum += fast_exp2(fmaf(acc[rb][e], p.c, -M));
                        l[rb] = l[rb] * fast_exp2(m[rb] - M) + sum;
                        m[rb] = M;
                        continue;
                    }
                    float mx = -INFINITY;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = key0 + 8 * (e >> 2) + 4 * hl + (e & 3);
                        const float sc = (r < p.last_q && j <= ir && j < k_end) ? acc[rb][e] * p.c : -INFINITY;
                        acc[rb][e] = sc;
                        mx = fmaxf(mx, sc);
                    }
                    const float M = fmaxf(m[rb], mx);
                    if (M == -INFINITY) continue;
                    float sum = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) sum += fast_exp2(acc[rb][e] - M);
                    l[rb] = l[rb] * fast_exp2(m[rb] - M) + sum;
                    m[rb] = M;
                }
            }
        }
        __syncthreads();  // waits for this wavefront's copies, then for all
    }
    if (li < 0) return;
    // lanes l and l^32 hold the same row
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        merge_ml(m[rb], l[rb], swap32(m[rb]), swap32(l[rb]));
        if (hl == 0) {
            const int bl = b * p.n_heads + li;
            float* out = p.stats + (((int64_t)bl * p.nchunk1 + chunk) * 64 + rb * 32 + rl) * 2;
            out[0] = m[rb];
            out[1] = l[rb];
        }
    }
}

// Four threads per row: thread q merges chunks q, q+4, q+8, ... in order,
// then the four partials are merged in the order q = 0..3 (deterministic).
__global__ void __launch_bounds__(256) vs_rowstat_combine(VsP p) {
    __shared__ float sm[4][64][2];
    const int bl = blockIdx.x;
    const int r = threadIdx.x & 63, q = threadIdx.x >> 6;
    float M = -INFINITY, Ls = 0.f;
    const float* in = p.stats + ((int64_t)bl * p.nchunk1 * 64 + r) * 2;
    for (int c = q; c < p.nchunk1; c += 4) merge_ml(M, Ls, in[(int64_t)c * 128], in[(int64_t)c * 128 + 1]);
    sm[q][r][0] = M;
    sm[q][r][1] = Ls;
    __syncthreads();
    if (q == 0) {
        for (int k = 1; k < 4; ++k) merge_ml(M, Ls, sm[k][r][0], sm[k][r][1]);
        p.rowstat[((int64_t)bl * 64 + r) * 2] = M;
        p.rowstat[((int64_t)bl * 64 + r) * 2 + 1] = Ls;
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(256) vs_scores(VsP p) {
    __shared__ float P[64 * kPitch2];
    // first-digit histograms of the item's final scores: vertical counts in
    // the low 16 bits, slash counts in the high 16 (at most 2048 each)
    __shared__ uint32_t h1[kTopkH1];
    const int ngroups = (p.nchunk2 + kChunksPerItem - 1) / kChunksPerItem;
    const int nitems = p.B * p.n_heads * ngroups;
    const int L = chunked_xcd_remap(blockIdx.x, gridDim.x, p.group);
    if (L >= nitems) return;
    const int cg = L / (p.B * p.n_heads);
    const int bl = L % (p.B * p.n_heads);
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int h = p.heads[li], kvh = h / p.group;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 31, hl = lane >> 5;
    const T* qbase = reinterpret_cast<const T*>(p.q) + b * p.qs0 + h * p.qs1;
    const T* kbase = reinterpret_cast<const T*>(p.k) + b * p.ks0 + kvh * p.ks1;

    typename Elem<T>::frag qf[2][D / 16];
    load_q_rows<T, D>(p, qbase, rl, hl, qf);
    // p = 2^(s*c - m) / l = 2^(s*c - (m + log2 l)); l >= 1 for every real row
    float mrow[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float* rs = p.rowstat + ((int64_t)bl * 64 + rb * 32 + rl) * 2;
        mrow[rb] = rs[1] > 0.f ? rs[0] + __log2f(rs[1]) : 0.f;
    }
    const int t = threadIdx.x;
    const int Lq = p.last_q;
    const int64_t row_off = b * p.srow_b + (int64_t)(p.score_by_head ? h : li) * p.srow_h;
    // Every chunk writes the same band of the tile (rows r < L, columns
    // [L-1-r, L-1-r+128)); the rest is cleared once and stays zero, so the
    // sums below run over all 64 rows without conditions.
    for (int i = t; i < 64 * kPitch2; i += 256) P[i] = 0.f;
    for (int i = t; i < kTopkH1; i += 256) h1[i] = 0u;
    __syncthreads();

    // the K rows of a chunk are loaded while the previous chunk's
    // probabilities and sums run (into the registers its MFMAs just read)
    typename Elem<T>::frag kf[D / 16];
    if (cg * kChunksPerItem < p.nchunk2)
        unit_load<T, D>(p, kbase, p.N - (cg * kChunksPerItem + 1) * kChunk2 + wave * 32, rl, hl, kf);
#pragma unroll 1
    for (int ci = 0; ci < kChunksPerItem; ++ci) {
        const int chunk = cg * kChunksPerItem + ci;
        if (chunk >= p.nchunk2) break;
        // wavefront w: keys [J0 + 32w, J0 + 32w + 32); J0 < 0 only in the last
        // chunk when N % 128 == 64 (those keys score zero)
        const int J0 = p.N - (chunk + 1) * kChunk2;
        const int key0 = J0 + wave * 32;
        f32x16 acc[2];
        unit_mma<T, D>(p, key0, rl, kf, qf, acc);
        if (ci + 1 < kChunksPerItem && chunk + 1 < p.nchunk2)
            unit_load<T, D>(p, kbase, key0 - kChunk2, rl, hl, kf);
        if (ci > 0) __syncthreads();  // the previous chunk's sums have read the tile
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int r = rb * 32 + rl;
            if (r >= Lq) continue;  // rows past last_q are not queries
            const int ir = p.N - Lq + r;
            float* prow = &P[r * kPitch2 + Lq - 1 - r];
            if (key0 >= 0 && key0 + 31 <= p.N - Lq) {  // wave-uniform: no masked key
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jl = wave * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);  // key - J0
                    prow[jl] = fast_exp2(fmaf(acc[rb][e], p.c, -mrow[rb]));
                }
                continue;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int jl = wave * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);  // key - J0
                const int j = J0 + jl;
                const bool ok = (j >= 0) && (j <= ir);
                prow[jl] = ok ? fast_exp2(fmaf(acc[rb][e], p.c, -mrow[rb])) : 0.f;
            }
        }
        __syncthreads();
        if (t < kChunk2) {
            // vertical sum of key J0 + t: the anti-diagonal (r, t + L-1 - r);
            // for rows r >= L the address falls on cleared cells (of row r, or
            // for r > t + L-1 past the band of row r-1), all inside the tile
            const int j = J0 + t;
            if (j >= 0) {
                float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
                for (int r = 0; r < 64; ++r) a[r & 3] += P[r * kPitch2 + t + Lq - 1 - r];
                const float vs = (a[0] + a[1]) + (a[2] + a[3]);
                p.vscore[row_off + j] = vs;
                atomicAdd(&h1[topk_digit1(topk_key(vs, j, p.force_v))], 1u);
            }
        } else {
            // slash partials: column x holds offset o = N - 1 - J0 - x
            for (int x = t - kChunk2; x < kChunk2 + kSpill; x += 256 - kChunk2) {
                // cells of column x outside the band are cleared
                float ap[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
                for (int r = 0; r < 64; ++r) ap[r & 3] += P[r * kPitch2 + x];
                const float a = (ap[0] + ap[1]) + (ap[2] + ap[3]);
                const int o = p.N - 1 - J0 - x;
                if (x < kChunk2) {
                    if (o < p.N) {
                        p.sscore[row_off + o] = a;
                        // final unless the chunk above spills into it
                        if (x >= kSpill || chunk == p.nchunk2 - 1)
                            atomicAdd(&h1[topk_digit1(topk_key(a, o, p.force_s))], 1u << 16);
                    }
                } else {
                    p.spill[((int64_t)bl * p.nchunk2 + chunk) * kSpill + (x - kChunk2)] = a;
                }
            }
        }
    }
    __syncthreads();
    uint32_t* hv = topk_row(p, bl, 0);
    uint32_t* hs = topk_row(p, bl, 1);
    for (int i = t; i < kTopkH1; i += 256) {
        const uint32_t c = h1[i];
        if (c & 0xFFFFu) atomicAdd(&hv[i], c & 0xFFFFu);
        if (c >> 16) atomicAdd(&hs[i], c >> 16);
    }
}

// Adds the spill of chunk c+1 (offsets [128c+65, 128c+127]) into chunk c's
// partial slash sums, which makes them final, and counts their first
// digits.  One workgroup per (batch, listed head, kCombineChunks spilling
// chunks), one thread per (chunk, offset).
constexpr int kCombineChunks = 64;

__global__ void __launch_bounds__(256) vs_slash_combine(VsP p) {
    __shared__ uint32_t h1[kTopkH1];
    const int nseg = (p.nchunk2 + kCombineChunks - 1) / kCombineChunks;
    const int bl = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int b = bl / p.n_heads, li = bl % p.n_heads;
    const int h = p.heads[li];
    const int64_t row_off = b * p.srow_b + (int64_t)(p.score_by_head ? h : li) * p.srow_h;
    for (int i = threadIdx.x; i < kTopkH1; i += 256) h1[i] = 0u;
    __syncthreads();
    const int c0 = seg * kCombineChunks;
    const int c1 = min(p.nchunk2, c0 + kCombineChunks);
    for (int e = threadIdx.x; e < (c1 - c0) * kSpill; e += 256) {
        const int chunk = c0 + e / kSpill;  // the spilling chunk c+1
        const int k = e % kSpill;
        if (chunk == 0) continue;  // offsets below 0 do not exist
        const int J0 = p.N - (chunk + 1) * kChunk2;
        const int o = p.N - 1 - J0 - (kChunk2 + k);
        const float val = p.sscore[row_off + o] + p.spill[((int64_t)bl * p.nchunk2 + chunk) * kSpill + k];
        p.sscore[row_off + o] = val;
        atomicAdd(&h1[topk_digit1(topk_key(val, o, p.force_s))], 1u);
    }
    __syncthreads();
    uint32_t* hs = topk_row(p, bl, 1);
    for (int i = threadIdx.x; i < kTopkH1; i += 256)
        if (h1[i]) atomicAdd(&hs[i], h1[i]);
}

template <typename T, int D>
hipError_t launch_t(VsP& p, hipStream_t s) {
    const int n1 = p.B * p.nsets * p.nchunk1;
    hipLaunchKernelGGL((vs_rowstat_partial<T, D>), dim3(n1), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(vs_rowstat_combine, dim3(p.B * p.n_heads), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n2 = p.B * p.n_heads * ((p.nchunk2 + kChunksPerItem - 1) / kChunksPerItem);
    hipLaunchKernelGGL((vs_scores<T, D>), dim3(n2), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n3 = p.B * p.n_heads * ((p.nchunk2 + kCombineChunks - 1) / kCombineChunks);
    hipLaunchKernelGGL(vs_slash_combine, dim3(n3), dim3(256), 0, s, p);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t vs_workspace_bytes(int32_t B, int32_t n_heads, int32_t N, bool caller_scores) {
    const size_t nchunk1 = std::min<size_t>(N / 64, kRowstatWGs);  // bound of the launcher's count
    const size_t nchunk2 = (N + kChunk2 - 1) / kChunk2;
    size_t bytes = align256((size_t)B * n_heads * nchunk1 * 64 * 2 * sizeof(float));
    bytes += align256((size_t)B * n_heads * 64 * 2 * sizeof(float));
    bytes += align256((size_t)B * n_heads * nchunk2 * kSpill * sizeof(float));
    bytes += align256(topk_scratch_bytes(2 * B * n_heads));
    if (!caller_scores) bytes += 2 * align256((size_t)B * n_heads * N * sizeof(float));
    return bytes;
}

hipError_t launch_vs_estimate(const VsArgs& a, hipStream_t s) {
    VsP p{};
    p.q = static_cast<const char*>(a.q);
    p.k = static_cast<const char*>(a.k);
    p.qs0 = a.qs[0]; p.qs1 = a.qs[1]; p.qs2 = a.qs[2];
    p.ks0 = a.ks[0]; p.ks1 = a.ks[1]; p.ks2 = a.ks[2];
    p.B = a.B; p.Hq = a.Hq; p.N = a.N; p.group = a.Hq / a.Hkv;
    p.n_heads = a.n_heads; p.last_q = a.last_q;
    p.c = a.scale * kLog2e;
    for (int i = 0; i < a.n_heads; ++i) p.heads[i] = a.heads[i];
    // sets of up to four listed heads per kv head, in list order
    {
        int open_set[MI_MAX_HEADS];
        for (int g = 0; g < a.Hkv; ++g) open_set[g] = -1;
        p.nsets = 0;
        for (int li = 0; li < a.n_heads; ++li) {
            const int g = a.heads[li] / p.group;
            int& st = open_set[g];
            if (st < 0 || p.set_n[st] == 4) {
                st = p.nsets++;
                p.set_n[st] = 0;
            }
            p.set_li[st][p.set_n[st]++] = (uint8_t)li;
        }
    }
    {
        const int nb = a.N / 64;
        int want = (kRowstatWGs + a.B * p.nsets - 1) / (a.B * p.nsets);
        want = std::max(1, std::min(want, nb));
        p.chunk1 = (nb + want - 1) / want * 64;
        p.nchunk1 = (a.N + p.chunk1 - 1) / p.chunk1;
    }
    p.nchunk2 = (a.N + kChunk2 - 1) / kChunk2;
    char* ws = static_cast<char*>(a.ws);
    size_t off = 0;
    p.stats = reinterpret_cast<float*>(ws + off);
    off += align256((size_t)a.B * a.n_heads * p.nchunk1 * 64 * 2 * sizeof(float));
    p.rowstat = reinterpret_cast<float*>(ws + off);
    off += align256((size_t)a.B * a.n_heads * 64 * 2 * sizeof(float));
    p.spill = reinterpret_cast<float*>(ws + off);
    off += align256((size_t)a.B * a.n_heads * p.nchunk2 * kSpill * sizeof(float));
    uint32_t* topk_scratch = reinterpret_cast<uint32_t*>(ws + off);
    off += align256(topk_scratch_bytes(2 * a.B * a.n_heads));
    p.topk = topk_scratch;
    p.topk_rows = 2 * a.B * a.n_heads;
    p.force_v = a.force_vertical;
    p.force_s = a.force_slash;
    if (a.vscore != nullptr) {
        // caller rows [B, Hq, N], indexed by head id
        p.vscore = a.vscore;
        p.sscore = a.sscore;
        p.srow_b = (int64_t)a.Hq * a.N;
        p.srow_h = a.N;
        p.score_by_head = 1;
    } else {
        // workspace rows [B, n_heads, N], indexed by list position
        p.vscore = reinterpret_cast<float*>(ws + off);
        off += align256((size_t)a.B * a.n_heads * a.N * sizeof(float));
        p.sscore = reinterpret_cast<float*>(ws + off);
        p.srow_b = (int64_t)a.n_heads * a.N;
        p.srow_h = a.N;
        p.score_by_head = 0;
    }
    hipError_t e;
    if (a.dtype == MI_BF16)
        e = a.D == 128 ? launch_t<uint16_t, 128>(p, s) : launch_t<uint16_t, 64>(p, s);
    else
        e = a.D == 128 ? launch_t<float, 128>(p, s) : launch_t<float, 64>(p, s);
    if (e != hipSuccess) return e;
    // top-k over both score rows of every listed head
    TopkRows t{};
    t.B = a.B; t.Hq = a.Hq; t.n_heads = a.n_heads; t.n = a.N;
    for (int i = 0; i < a.n_heads; ++i) t.heads[i] = a.heads[i];
    t.score_by_head = p.score_by_head;
    t.srow_b = p.srow_b; t.srow_h = p.srow_h;
    t.list[0] = {p.vscore, a.vertical_idx, a.n_vertical, a.force_vertical};
    t.list[1] = {p.sscore, a.slash_idx, a.n_slash, a.force_slash};
    t.scratch = topk_scratch;
    return launch_topk_rows(t, s);
}

}  // namespace mi
