// Block + column sparse flash attention for gfx950 (and its dense-causal
// comparator).
//
// Work item: one (batch, query head, 64-row query block a).  The item walks
// its key-block list (64x64 tiles) and then its gathered column list in
// chunks of 64 keys, keeping an online softmax (running max m and
// normaliser l per row, fp32), as in the aifetchly guide's section
// "1. The Vertical-Slash Kernel Mechanics".  Non-listed tiles are never
// touched ("2. The Block-Sparse Kernel Mechanics").
//
// Workgroup: 2 wavefronts; wavefront w owns query rows [32w, 32w+32) of the
// block.  Both MFMA stages are computed transposed so that one lane owns one
// query row from the scores to the output:
//     S^T (64 keys x 32 rows)  = K_tile (64 x D) . Q^T (D x 32)
//     O^T (D x 32 rows)       += V^T (D x 64)    . P^T (64 x 32)
// With the 32x32 MFMA result layout, lane l holds query row l%32 and 16 of
// the keys of each 32-key half; the same registers are the B operand of the
// P.V product without any cross-lane move, and the row statistics live on
// the lane pair (l, l^32).
//
// K is staged in LDS row-major (padded rows); V is staged transposed
// (V^T[d][key]) so that both MFMA A-operands read contiguous bytes.
#include "mi_device.h"
#include "mi_internal.h"

namespace mi {
namespace {

enum MaskMode { kMaskNone = 0, kMaskCausal = 1, kMaskAShape = 2, kMaskColumns = 3 };

struct Params {
    const char* q;
    const char* k;
    const char* v;
    char* o;
    float* lse;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;  // element strides
    int32_t B, Hq, Hkv, N, nb, group;
    float c;  // scale * log2(e)
    const int32_t* block_count;
    const int32_t* block_idx;
    const int32_t* col_count;
    const int32_t* col_idx;
    int32_t block_cap, col_cap;
    int32_t sink, local;
    int32_t all_dense;
    int32_t xcd_chunk;
    uint8_t pattern[MI_MAX_HEADS];
};

template <typename T, int D>
struct Smem {
    static constexpr int KP = D + Elem<T>::kKPad;    // K row pitch (elements)
    static constexpr int VP = 64 + Elem<T>::kVPad;   // V^T row pitch (elements)
    T ks[64 * KP];
    T vt[D * VP];
    int32_t colpos[64];
};

// Stage 64 keys of K and V into LDS.  rows[] gives the token of each key slot
// (-1: zero fill).  For a tile, rows are consecutive and `tile_base` >= 0.
template <typename T, int D>
__device__ __forceinline__ void stage_kv(Smem<T, D>& sm, const T* kbase, const T* vbase,
                                         int64_t kstride, int64_t vstride, int tile_base,
                                         bool use_colpos) {
    constexpr int ES = Elem<T>::kSize;
    constexpr int EPC = 16 / ES;           // elements per 16-byte chunk
    constexpr int CPR = D / EPC;           // chunks per row
    const int t = threadIdx.x;
    // K: row-major copy, one 16-byte chunk per thread per step.
#pragma unroll
    for (int it = 0; it < (64 * CPR) / 128; ++it) {
        const int c = it * 128 + t;
        const int key = c / CPR, part = c % CPR;
        const int tok = use_colpos ? sm.colpos[key] : tile_base + key;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (tok >= 0) val = *reinterpret_cast<const u32x4*>(kbase + (int64_t)tok * kstride + part * EPC);
        *reinterpret_cast<u32x4*>(&sm.ks[key * Smem<T, D>::KP + part * EPC]) = val;
    }
    // V: transposed store V^T[d][key].
    if constexpr (ES == 2) {
        // units of (key pair, 8 d-values): two 16-byte loads, eight 4-byte LDS writes
#pragma unroll
        for (int it = 0; it < (32 * CPR) / 128; ++it) {
            const int u = it * 128 + t;
            const int kp = u / CPR, part = u % CPR;
            const int k0 = 2 * kp;
            const int tok0 = use_colpos ? sm.colpos[k0] : tile_base + k0;
            const int tok1 = use_colpos ? sm.colpos[k0 + 1] : tile_base + k0 + 1;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (tok0 >= 0) a = *reinterpret_cast<const u32x4*>(vbase + (int64_t)tok0 * vstride + part * 8);
            if (tok1 >= 0) b = *reinterpret_cast<const u32x4*>(vbase + (int64_t)tok1 * vstride + part * 8);
            uint32_t* dst = reinterpret_cast<uint32_t*>(&sm.vt[(part * 8) * Smem<T, D>::VP + k0]);
            constexpr int W = Smem<T, D>::VP / 2;  // row pitch in 32-bit words
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // element 2e (low half) and 2e+1 (high half) of each key row
                const uint32_t lo = (a[e] & 0xFFFFu) | (b[e] << 16);
                const uint32_t hi = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
                dst[(2 * e) * W] = lo;
                dst[(2 * e + 1) * W] = hi;
            }
        }
    } else {
#pragma unroll
        for (int it = 0; it < (64 * CPR) / 128; ++it) {
            const int u = it * 128 + t;
            const int key = u / CPR, part = u % CPR;
            const int tok = use_colpos ? sm.colpos[key] : tile_base + key;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            if (tok >= 0) a = *reinterpret_cast<const f32x4*>(vbase + (int64_t)tok * vstride + part * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.vt[(part * 4 + e) * Smem<T, D>::VP + key] = a[e];
        }
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(128) sparse_attn_kernel(Params p) {
    __shared__ Smem<T, D> sm;
    typedef typename Elem<T>::frag Frag;
    constexpr int NKS = D / 16;   // contraction steps of S
    constexpr int NDB = D / 32;   // 32-wide d blocks of O

    const int items = p.B * p.Hq * p.nb;
    const int L = chunked_xcd_remap(blockIdx.x, gridDim.x, p.xcd_chunk);
    if (L >= items) return;
    // longest items first: query blocks in descending order
    const int a = p.nb - 1 - L / (p.B * p.Hq);
    const int bh = L % (p.B * p.Hq);
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int kvh = h / p.group;
    const int pattern = p.all_dense ? MI_DENSE : p.pattern[h];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hl = lane >> 5;          // lane half
    const int rl = lane & 31;          // row within the wave
    const int row_local = wave * 32 + rl;
    const int i_row = a * 64 + row_local;

    const T* qbase = reinterpret_cast<const T*>(p.q) + b * p.qs0 + h * p.qs1;
    const T* kbase = reinterpret_cast<const T*>(p.k) + b * p.ks0 + kvh * p.ks1;
    const T* vbase = reinterpret_cast<const T*>(p.v) + b * p.vs0 + kvh * p.vs1;

    // Q fragments of this lane's row: slots 16*ks + 8*hl .. +8
    Frag qf[NKS];
    {
        const T* qrow = qbase + (int64_t)i_row * p.qs2;
#pragma unroll
        for (int s = 0; s < NKS; ++s) qf[s] = load_frag(qrow + 16 * s + 8 * hl);
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY;
    float l_part = 0.f;  // this lane's share of the normaliser (combined at the end)

    const int64_t list_row = ((int64_t)bh * p.nb + a);
    int ntiles, ncols = 0;
    const int32_t* tiles = nullptr;
    const int32_t* cols = nullptr;
    if (pattern == MI_DENSE) {
        ntiles = a + 1;
    } else {
        // counts are clamped to the list capacity so a bad index cannot read past its row
        ntiles = min(max(p.block_count[list_row], 0), p.block_cap);
        tiles = p.block_idx + list_row * p.block_cap;
        if (pattern == MI_VSLASH) {
            ncols = min(max(p.col_count[list_row], 0), p.col_cap);
            cols = p.col_idx + list_row * p.col_cap;
        }
    }
    const int nchunks = (ncols + 63) / 64;
    const int nsteps = ntiles + nchunks;

    for (int step = 0; step < nsteps; ++step) {
        int mode;
        int kb = 0;
        const bool is_col = step >= ntiles;
        if (!is_col) {
            kb = (pattern == MI_DENSE) ? step : tiles[step];
            // key blocks outside [0, a] hold no causal key of this query block
            if (kb < 0 || kb > a) continue;
            if (kb >= a) {
                mode = kMaskCausal;
            } else if (pattern == MI_ASHAPE) {
                const bool full = (kb * 64 + 63 < p.sink) || ((a - kb) * 64 + 63 < p.local);
                mode = full ? kMaskNone : kMaskAShape;
            } else {
                mode = kMaskNone;
            }
            if (pattern == MI_ASHAPE && kb >= a) mode = kMaskAShape;
        } else {
            mode = kMaskColumns;
        }

        __syncthreads();  // previous step's LDS reads are done
        if (is_col) {
            const int c0 = (step - ntiles) * 64;
            if (threadIdx.x < 64) {
                const int cidx = c0 + threadIdx.x;
                const int j = (cidx < ncols) ? cols[cidx] : -1;
                sm.colpos[threadIdx.x] = (j >= 0 && j < p.N) ? j : -1;
            }
            __syncthreads();
            stage_kv<T, D>(sm, kbase, vbase, p.ks2, p.vs2, 0, true);
        } else {
            stage_kv<T, D>(sm, kbase, vbase, p.ks2, p.vs2, kb * 64, false);
        }
        __syncthreads();

        // ---- S^T = K . Q^T : two 32-key halves
        f32x16 s[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s[kh][e] = 0.f;
            const T* krow = &sm.ks[(kh * 32 + rl) * Smem<T, D>::KP + 8 * hl];
#pragma unroll
            for (int st = 0; st < NKS; ++st) {
                Frag kf = load_frag(krow + 16 * st);
                mma32(s[kh], kf, qf[st]);
            }
        }

        // ---- masks: element e of half kh is key 32*kh + 8*(e/4) + 4*hl + (e%4)
        if (mode != kMaskNone) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int kl = kh * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
                    int j;
                    bool keep;
                    if (mode == kMaskColumns) {
                        j = sm.colpos[kl];
                        keep = (j >= 0) && (j <= i_row);
                    } else {
                        j = kb * 64 + kl;
                        keep = j <= i_row;
                        if (mode == kMaskAShape) keep = keep && ((j < p.sink) || (i_row - j < p.local));
                    }
                    if (!keep) s[kh][e] = -INFINITY;
                }
        }

        // ---- online softmax (log2 domain)
        float mx = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kh][e]);
        mx = fmaxf(mx, swap32(mx));
        const float m_new = fmaxf(m_run, mx * p.c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pv = fast_exp2(fmaf(s[kh][e], p.c, -m_use));
                s[kh][e] = pv;
                rs += pv;
            }
        l_part = fmaf(l_part, alpha, rs);
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;

        // ---- O^T += V^T . P^T : 16-key chunks (half kh, part pp) -> s[kh][8pp..8pp+7]
        Frag pf[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) pf[kh][pp] = make_p_frag(s[kh], 8 * pp, (Frag*)nullptr);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const T* vrow = &sm.vt[(db * 32 + rl) * Smem<T, D>::VP + 4 * hl];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    Frag vf = load_vt_frag(vrow + kh * 32 + pp * 16);
                    mma32(oacc[db], vf, pf[kh][pp]);
                }
        }
    }

    // ---- epilogue: O = O^T / l, lse = (m + log2 l) * ln 2
    const float l = l_part + swap32(l_part);
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    T* orow = reinterpret_cast<T*>(p.o) + b * p.os0 + h * p.os1 + (int64_t)i_row * p.os2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d0 = db * 32 + 8 * qd + 4 * hl;
            const float o0 = oacc[db][4 * qd + 0] * inv, o1 = oacc[db][4 * qd + 1] * inv;
            const float o2 = oacc[db][4 * qd + 2] * inv, o3 = oacc[db][4 * qd + 3] * inv;
            if constexpr (sizeof(T) == 2) {
                u32x2 w = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                *reinterpret_cast<u32x2*>(orow + d0) = w;
            } else {
                *reinterpret_cast<f32x4*>(orow + d0) = f32x4{o0, o1, o2, o3};
            }
        }
    if (p.lse && hl == 0) {
        p.lse[(int64_t)bh * p.N + i_row] = (l > 0.f) ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
    }
}

template <typename T, int D>
hipError_t launch_t(const Params& p, hipStream_t s) {
    const int items = p.B * p.Hq * p.nb;
    hipLaunchKernelGGL((sparse_attn_kernel<T, D>), dim3(items), dim3(128), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s) {
    Params p{};
    p.q = static_cast<const char*>(a.q);
    p.k = static_cast<const char*>(a.k);
    p.v = static_cast<const char*>(a.v);
    p.o = static_cast<char*>(a.o);
    p.lse = a.lse;
    p.qs0 = a.qs[0]; p.qs1 = a.qs[1]; p.qs2 = a.qs[2];
    p.ks0 = a.ks[0]; p.ks1 = a.ks[1]; p.ks2 = a.ks[2];
    p.vs0 = a.vs[0]; p.vs1 = a.vs[1]; p.vs2 = a.vs[2];
    p.os0 = a.os[0]; p.os1 = a.os[1]; p.os2 = a.os[2];
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N; p.nb = a.N / 64;
    p.group = a.Hq / a.Hkv;
    p.c = a.scale * kLog2e;
    p.block_count = a.block_count; p.block_idx = a.block_idx;
    p.col_count = a.col_count; p.col_idx = a.col_idx;
    p.block_cap = a.block_cap; p.col_cap = a.col_cap;
    p.sink = a.sink; p.local = a.local;
    p.all_dense = a.all_dense;
    p.xcd_chunk = p.group;
    for (int i = 0; i < MI_MAX_HEADS; ++i) p.pattern[i] = a.pattern[i];
    if (a.dtype == MI_BF16) {
        return a.D == 128 ? launch_t<uint16_t, 128>(p, s) : launch_t<uint16_t, 64>(p, s);
    }
    return a.D == 128 ? launch_t<float, 128>(p, s) : launch_t<float, 64>(p, s);
}

}  // namespace mi
