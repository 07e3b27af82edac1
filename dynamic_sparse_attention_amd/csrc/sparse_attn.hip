// Block + column sparse flash attention for gfx950 (and its dense-causal
// comparator).
//
// Work item: one (batch, query head, pair of 64-row query blocks a0 = 2p,
// a1 = 2p+1).  The two blocks share every staged K/V tile: the item walks the
// ascending merge of their key-block lists; a tile listed by only one block
// is computed only by that block's wavefronts.  Then each block's gathered
// column list is walked in chunks of 64 keys.  An online softmax keeps a
// running max and normaliser per row in fp32 (aifetchly guide, "1. The
// Vertical-Slash Kernel Mechanics"); tiles not listed are never touched
// ("2. The Block-Sparse Kernel Mechanics").
//
// Workgroup: 4 wavefronts; wavefront w owns rows [32(w%2), 32(w%2)+32) of
// block a_{w/2}.  Both MFMA stages are computed transposed so that one lane
// owns one query row from the scores to the output:
//     S^T (64 keys x 32 rows)  = K_tile (64 x D) . Q^T (D x 32)
//     O^T (D x 32 rows)       += V^T (D x 64)    . P^T (64 x 32)
// With the 32x32 MFMA result layout, lane l holds query row l%32 and 16 of
// the keys of each 32-key half; those registers are the B operand of the P.V
// product without any cross-lane move, and each row's statistics live on the
// lane pair (l, l^32).
//
// Staging: K and V rows go from global memory straight into LDS
// (global_load_lds_dwordx4, 16 bytes per lane, a wave writes 1 KiB of
// consecutive LDS per instruction) into two buffers: the loads of step t+1
// are in flight while step t is computed, with one barrier per step.  Rows
// are stored unpadded; 16-byte chunk c of row r sits at position c ^ f(r),
// f(r) = 4(r%4) + (r/4)%4 (16-chunk rows), so that a K operand read (16 lanes
// per LDS cycle: 16 consecutive rows, same chunk) and a V transposed read
// (32 lanes per cycle: 4 rows x 4 chunks) each hit all 64 banks once.
// bf16: the V^T operand is read with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16), which hands lane i of a 16-lane group element (i%4)
// of the 8-byte rows addressed by lanes 4j + i/4, j = 0..3.  fp32: V^T
// elements are read one by one.
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
    int32_t B, Hq, Hkv, N, nb, npairs, group;
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

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// The running max is only raised when a row's new max exceeds it by more
// than this (log2 units); probabilities then stay below 2^kLazy, and the
// result is unchanged because numerator and normaliser share the same max.
constexpr float kLazy = 8.0f;

template <typename T, int D>
struct Layout {
    static constexpr int ES = sizeof(T);
    static constexpr int EPC = 16 / ES;    // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;    // chunks per key row
    static constexpr int ROWB = CPR * 16;  // bytes per key row
    static constexpr int TILEB = 64 * ROWB;
};

// One LDS staging buffer: a 64-key tile (or column chunk) of K and V.
template <typename T, int D>
struct Buf {
    char k[Layout<T, D>::TILEB];
    char v[Layout<T, D>::TILEB];
    int32_t colpos[64];
};

// Chunk swizzle of a staged row (see the header comment); rows of 8 chunks
// (bf16, d = 64) use 4((r/2)%2) + (r/4)%4.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    if constexpr (CPR == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    return ((row & 3) << 2) | ((row >> 2) & 3);
}

// One step of the item: a merged key tile or a chunk of one block's columns.
struct Step {
    int kind;   // 0 tile, 1 column chunk, -1 none
    int kb;     // tile: key block
    int need;   // bit 0: block a0 computes, bit 1: block a1 computes
    int blk;    // column chunk: owning block (0 / 1)
    int c0;     // column chunk: first list position
};

// Wave-uniform read of an index list entry through the constant address
// space, which the backend issues as a scalar (s_load) read: the lists are
// not written while the kernel runs.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int ld_uniform(const int32_t* p) {
    return *reinterpret_cast<const_i32*>(reinterpret_cast<uintptr_t>(p));
}

struct Walker {
    int dense, a0, a1, has1;
    const int32_t* L0;
    const int32_t* L1;
    int n0, n1, p0, p1, dk;
    const int32_t* C0;
    const int32_t* C1;
    int m0, m1, cpos, cblk;

    __device__ __forceinline__ Step next() {
        Step s{-1, 0, 0, 0, 0};
        if (dense) {
            const int lim = has1 ? a1 : a0;
            if (dk <= lim) {
                s.kind = 0;
                s.kb = dk;
                s.need = (dk <= a0 ? 1 : 0) | (has1 ? 2 : 0);
                ++dk;
                return s;
            }
        } else {
            // ascending merge of the two lists; entries outside [0, a] are
            // skipped.  All walker state is wave-uniform: readfirstlane keeps
            // the list reads on the scalar unit (scalar cache) instead of
            // per-lane memory loads with a full wait each.
            while (p0 < n0 && (unsigned)ld_uniform(L0 + p0) > (unsigned)a0) ++p0;
            while (p1 < n1 && (unsigned)ld_uniform(L1 + p1) > (unsigned)a1) ++p1;
            if (p0 < n0 || p1 < n1) {
                const int k0 = p0 < n0 ? ld_uniform(L0 + p0) : 0x7FFFFFFF;
                const int k1 = p1 < n1 ? ld_uniform(L1 + p1) : 0x7FFFFFFF;
                const int kb = k0 < k1 ? k0 : k1;
                s.kind = 0;
                s.kb = kb;
                s.need = (k0 == kb ? 1 : 0) | (k1 == kb ? 2 : 0);
                if (k0 == kb) ++p0;
                if (k1 == kb) ++p1;
                return s;
            }
        }
        // column chunks of block a0, then of block a1
        if (cblk == 0 && cpos >= m0) { cblk = 1; cpos = 0; }
        if (cblk == 0) {
            s.kind = 1; s.blk = 0; s.c0 = cpos; s.need = 1; cpos += 64;
            return s;
        }
        if (cblk == 1 && cpos < m1) {
            s.kind = 1; s.blk = 1; s.c0 = cpos; s.need = 2; cpos += 64;
            return s;
        }
        return s;
    }
};

typedef __attribute__((address_space(3))) void lds_void;

// Issues the global->LDS copies of one step into `buf`.  Wave-instruction
// `idx` fills LDS chunks [64 idx, 64 idx + 64) of a tensor: lane l writes
// chunk 64 idx + l, i.e. row (64 idx + l) / CPR at position (64 idx + l) % CPR,
// which holds source chunk position ^ f(row).
template <typename T, int D>
__device__ __forceinline__ void issue_step(Buf<T, D>& buf, const Step& s, const Walker& w,
                                           const T* kbase, const T* vbase, int64_t kstride,
                                           int64_t vstride, int N) {
    typedef Layout<T, D> Ly;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int it = 0; it < Ly::CPR / kWaves; ++it) {
        const int idx = it * kWaves + wave;
        const int cidx = idx * 64 + lane;
        const int row = cidx / Ly::CPR, pos = cidx % Ly::CPR;
        const int chunk = pos ^ swz<Ly::CPR>(row);
        int tok;
        if (s.kind == 0) {
            tok = s.kb * 64 + row;
        } else {
            const int li = s.c0 + row;
            const int32_t* C = s.blk == 0 ? w.C0 : w.C1;
            const int m = s.blk == 0 ? w.m0 : w.m1;
            tok = li < m ? C[li] : -1;
            if (tok >= N) tok = -1;
            if (pos == 0) buf.colpos[row] = tok;
            if (tok < 0) tok = 0;  // any valid row: the column is masked out
        }
        __builtin_amdgcn_global_load_lds(kbase + (int64_t)tok * kstride + chunk * Ly::EPC,
                                         (lds_void*)(buf.k + idx * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + (int64_t)tok * vstride + chunk * Ly::EPC,
                                         (lds_void*)(buf.v + idx * 1024), 16, 0, 0);
    }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Per-lane LDS byte offsets that do not depend on the step.
template <typename T, int D>
struct LaneOffsets {
    int krow;          // row part of the K operand address: (kh*32 + rl) handled by + kh*32*ROWB
    int kpos[D / 16];  // chunk part for contraction step ks
    int vrow;              // V operand: row part (keys base + 4hl + j)
    int vpos[D / 32][2];   // chunk part for d block db, rows +0 / +8
};

template <typename T, int D>
__device__ __forceinline__ void lane_offsets(LaneOffsets<T, D>& o, int lane) {
    typedef Layout<T, D> Ly;
    const int rl = lane & 31, hl = lane >> 5;
    // row kh*32 + rl has the swizzle of rl (kh*32 leaves the low 4 bits alone)
    const int f = swz<Ly::CPR>(rl);
    o.krow = rl * Ly::ROWB;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) o.kpos[ks] = ((2 * ks + hl) ^ f) * 16;
        const int g16 = (lane >> 4) & 1, s = lane & 15, j = s >> 2, qd = s & 3;
        o.vrow = (4 * hl + j) * Ly::ROWB;
        // rows base + 4hl + j and base + 8 + 4hl + j, base a multiple of 16
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) {
            const int fv = swz<Ly::CPR>(8 * sec + 4 * hl + j);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                o.vpos[db][sec] = ((4 * db + 2 * g16 + (qd >> 1)) ^ fv) * 16 + (qd & 1) * 8;
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) o.kpos[ks] = ((4 * ks + 2 * hl) ^ f) * 16;
        o.vrow = 0;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o.vpos[db][0] = o.vpos[db][1] = 0;
    }
}

// K operand (8 elements of key row kh*32 + rl, slots 16 ks + 8 hl ..).
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const char* kb, const LaneOffsets<uint16_t, D>& o, int kh, int ks) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                          kb + kh * 32 * Layout<uint16_t, D>::ROWB + o.krow + o.kpos[ks]));
}
template <int D>
__device__ __forceinline__ f32x8 k_frag(const char* kb, const LaneOffsets<float, D>& o, int kh, int ks) {
    const int rl = threadIdx.x & 31, hl = (threadIdx.x >> 5) & 1;
    const char* row = kb + kh * 32 * Layout<float, D>::ROWB + o.krow;
    const int f = swz<Layout<float, D>::CPR>(rl);
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + o.kpos[ks]);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + (((4 * ks + 2 * hl + 1) ^ f) * 16));
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// V^T operand for d block db over keys [base, base+16): lane (d = 32 db + l%32,
// half hl) gets keys base+4hl+{0..3} and base+8+4hl+{0..3}.
template <int D>
__device__ __forceinline__ bf16x8 v_frag(const char* vb, const LaneOffsets<uint16_t, D>& o, int db, int base) {
    constexpr int RB = Layout<uint16_t, D>::ROWB;
    const char* p0 = vb + base * RB + o.vrow + o.vpos[db][0];
    const char* p1 = vb + (base + 8) * RB + o.vrow + o.vpos[db][1];
    const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
    const i16x8 r = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    return __builtin_bit_cast(bf16x8, r);
}
template <int D>
__device__ __forceinline__ f32x8 v_frag(const char* vb, const LaneOffsets<float, D>&, int db, int base) {
    constexpr int RB = Layout<float, D>::ROWB;
    const int rl = threadIdx.x & 31, hl = (threadIdx.x >> 5) & 1;
    const int d = db * 32 + rl;
    f32x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int key = base + (e >> 2) * 8 + 4 * hl + (e & 3);
        r[e] = *reinterpret_cast<const float*>(vb + key * RB + (((d >> 2) ^ swz<Layout<float, D>::CPR>(key)) * 16) +
                                               (d & 3) * 4);
    }
    return r;
}

__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-wave running state.
template <typename T, int D>
struct RowState {
    f32x16 oacc[D / 32];
    float m_run;   // running max (log2 units, scaled)
    float l_part;  // this lane's share of the normaliser
};

template <typename T, int D>
__device__ __forceinline__ void compute_step(const Buf<T, D>& buf, const Step& cur, const Params& p,
                                             const LaneOffsets<T, D>& lo,
                                             const typename Elem<T>::frag (&qf)[D / 16],
                                             RowState<T, D>& rs, int pattern, int my_a, int i_row) {
    typedef typename Elem<T>::frag Frag;
    constexpr int NKS = D / 16;
    constexpr int NDB = D / 32;
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;

    int mode;
    if (cur.kind == 1) {
        mode = kMaskColumns;
    } else if (pattern == MI_ASHAPE) {
        const bool full = cur.kb < my_a &&
                          ((cur.kb * 64 + 63 < p.sink) || ((my_a - cur.kb) * 64 + 63 < p.local));
        mode = full ? kMaskNone : kMaskAShape;
    } else {
        mode = cur.kb >= my_a ? kMaskCausal : kMaskNone;
    }

    // ---- S^T = K . Q^T, the two 32-key halves interleaved
    f32x16 s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kh][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) mma32(s[kh], k_frag<D>(buf.k, lo, kh, ks), qf[ks]);

    // ---- masks (element e of half kh is key 32 kh + 8 (e/4) + 4 hl + e%4)
    if (mode == kMaskCausal) {
        const int lim = i_row - cur.kb * 64 - 4 * hl;  // keep key-local kl iff kl - 4hl <= lim
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int klc = kh * 32 + 8 * (e >> 2) + (e & 3);
                s[kh][e] = (klc <= lim) ? s[kh][e] : -INFINITY;
            }
    } else if (mode == kMaskAShape) {
        const int j0 = cur.kb * 64 + 4 * hl;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = j0 + kh * 32 + 8 * (e >> 2) + (e & 3);
                const bool keep = (j <= i_row) && ((j < p.sink) || (i_row - j < p.local));
                s[kh][e] = keep ? s[kh][e] : -INFINITY;
            }
    } else if (mode == kMaskColumns) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int4 j4 = *reinterpret_cast<const int4*>(&buf.colpos[kh * 32 + 8 * q4 + 4 * hl]);
                const int jj[4] = {j4.x, j4.y, j4.z, j4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = (jj[r] >= 0) && (jj[r] <= i_row);
                    s[kh][4 * q4 + r] = keep ? s[kh][4 * q4 + r] : -INFINITY;
                }
            }
    }

    // ---- online softmax (log2 domain, lazily raised max)
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kh][e]);
    mx = pair_max(mx) * p.c;
    const bool raise = mx > rs.m_run + kLazy;
    if (__ballot(raise)) {
        const float alpha = raise ? fast_exp2(rs.m_run - mx) : 1.f;  // 0 when m_run = -inf
        rs.m_run = raise ? mx : rs.m_run;
        rs.l_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) rs.oacc[db][e] *= alpha;
    }
    const float m_use = (rs.m_run == -INFINITY) ? 0.f : rs.m_run;
    float sum = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float pv = fast_exp2(fmaf(s[kh][e], p.c, -m_use));
            s[kh][e] = pv;
            sum += pv;
        }
    rs.l_part += sum;

    // ---- O^T += V^T . P^T over 16-key chunks (half kh, part pp)
    Frag pf[2][2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) pf[kh][pp] = make_p_frag(s[kh], 8 * pp, (Frag*)nullptr);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                mma32(rs.oacc[db], v_frag<D>(buf.v, lo, db, kh * 32 + pp * 16), pf[kh][pp]);
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads) sparse_attn_kernel(Params p) {
    typedef typename Elem<T>::frag Frag;
    constexpr int NKS = D / 16;
    constexpr int NDB = D / 32;
    __shared__ Buf<T, D> buf0;
    __shared__ Buf<T, D> buf1;

    const int items = p.B * p.Hq * p.npairs;
    const int L = chunked_xcd_remap(blockIdx.x, gridDim.x, p.xcd_chunk);
    if (L >= items) return;
    // longest items first: query-block pairs in descending order
    const int pair = p.npairs - 1 - L / (p.B * p.Hq);
    const int bh = L % (p.B * p.Hq);
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int kvh = h / p.group;
    const int pattern = p.all_dense ? MI_DENSE : p.pattern[h];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int blk = wave >> 1;  // 0: block a0, 1: block a1
    const int hl = lane >> 5;
    const int rl = lane & 31;
    const int a0 = 2 * pair, a1 = a0 + 1;
    const int has1 = a1 < p.nb;
    const int my_a = a0 + blk;
    const bool active = blk == 0 || has1;
    const int i_row = my_a * 64 + (wave & 1) * 32 + rl;

    const T* qbase = reinterpret_cast<const T*>(p.q) + b * p.qs0 + h * p.qs1;
    const T* kbase = reinterpret_cast<const T*>(p.k) + b * p.ks0 + kvh * p.ks1;
    const T* vbase = reinterpret_cast<const T*>(p.v) + b * p.vs0 + kvh * p.vs1;

    Frag qf[NKS];
    if (active) {
        const T* qrow = qbase + (int64_t)i_row * p.qs2;
#pragma unroll
        for (int s = 0; s < NKS; ++s) qf[s] = load_frag(qrow + 16 * s + 8 * hl);
    } else {
#pragma unroll
        for (int s = 0; s < NKS; ++s) qf[s] = Frag{};
    }
    LaneOffsets<T, D> lo;
    lane_offsets<T, D>(lo, lane);

    Walker wk{};
    wk.a0 = a0; wk.a1 = a1; wk.has1 = has1;
    if (pattern == MI_DENSE) {
        wk.dense = 1;
    } else {
        const int64_t r0 = (int64_t)bh * p.nb + a0;
        wk.L0 = p.block_idx + r0 * p.block_cap;
        wk.n0 = min(max(p.block_count[r0], 0), p.block_cap);
        if (has1) {
            wk.L1 = p.block_idx + (r0 + 1) * p.block_cap;
            wk.n1 = min(max(p.block_count[r0 + 1], 0), p.block_cap);
        }
        if (pattern == MI_VSLASH) {
            wk.C0 = p.col_idx + r0 * p.col_cap;
            wk.m0 = min(max(p.col_count[r0], 0), p.col_cap);
            if (has1) {
                wk.C1 = p.col_idx + (r0 + 1) * p.col_cap;
                wk.m1 = min(max(p.col_count[r0 + 1], 0), p.col_cap);
            }
        }
    }

    RowState<T, D> rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) rs.oacc[db][e] = 0.f;
    rs.m_run = -INFINITY;
    rs.l_part = 0.f;
    const bool mine0 = active;

    // Two buffers, used alternately; the loop body is written out for each so
    // that the LDS reads of one never wait on the copies into the other.
    Step cur = wk.next();
    if (cur.kind >= 0) issue_step<T, D>(buf0, cur, wk, kbase, vbase, p.ks2, p.vs2, p.N);
    while (cur.kind >= 0) {
        Step nxt = wk.next();
        __syncthreads();  // buf0 landed for every wave; buf1 is no longer read
        if (nxt.kind >= 0) issue_step<T, D>(buf1, nxt, wk, kbase, vbase, p.ks2, p.vs2, p.N);
        if (mine0 && ((cur.need >> blk) & 1))
            compute_step<T, D>(buf0, cur, p, lo, qf, rs, pattern, my_a, i_row);
        if (nxt.kind < 0) break;
        cur = wk.next();
        __syncthreads();  // buf1 landed; buf0 is no longer read
        if (cur.kind >= 0) issue_step<T, D>(buf0, cur, wk, kbase, vbase, p.ks2, p.vs2, p.N);
        if (mine0 && ((nxt.need >> blk) & 1))
            compute_step<T, D>(buf1, nxt, p, lo, qf, rs, pattern, my_a, i_row);
    }

    if (!active) return;
    // ---- epilogue: O = O^T / l, lse = (m + log2 l) * ln 2
    const float l = pair_sum(rs.l_part);
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    T* orow = reinterpret_cast<T*>(p.o) + b * p.os0 + h * p.os1 + (int64_t)i_row * p.os2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d0 = db * 32 + 8 * qd + 4 * hl;
            const float o0 = rs.oacc[db][4 * qd + 0] * inv, o1 = rs.oacc[db][4 * qd + 1] * inv;
            const float o2 = rs.oacc[db][4 * qd + 2] * inv, o3 = rs.oacc[db][4 * qd + 3] * inv;
            if constexpr (sizeof(T) == 2) {
                u32x2 w2 = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                *reinterpret_cast<u32x2*>(orow + d0) = w2;
            } else {
                *reinterpret_cast<f32x4*>(orow + d0) = f32x4{o0, o1, o2, o3};
            }
        }
    if (p.lse && hl == 0) {
        const float m_use = (rs.m_run == -INFINITY) ? 0.f : rs.m_run;
        p.lse[(int64_t)bh * p.N + i_row] = (l > 0.f) ? (m_use + __log2f(l)) * kLn2 : -INFINITY;
    }
    (void)rl;
}

template <typename T, int D>
hipError_t launch_t(const Params& p, hipStream_t s) {
    const int items = p.B * p.Hq * p.npairs;
    hipLaunchKernelGGL((sparse_attn_kernel<T, D>), dim3(items), dim3(kThreads), 0, s, p);
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
    p.npairs = (p.nb + 1) / 2;
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
