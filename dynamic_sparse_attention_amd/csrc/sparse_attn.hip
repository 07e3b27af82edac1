// Block + column sparse flash attention for gfx950 (and its dense-causal
// comparator).  An online softmax keeps a running max and normaliser per row
// in fp32 (aifetchly guide, "1. The Vertical-Slash Kernel Mechanics"); tiles
// that no index list names are never touched ("2. The Block-Sparse Kernel
// Mechanics").
//
// Work item: one (batch, query head, run of four 64-row query blocks
// a_i = 4r + i).  The four blocks share every staged K/V tile.  At the start
// of an item the workgroup writes the item's step list to LDS: the ascending
// merge of the four key-block lists, each entry carrying a 4-bit mask of the
// blocks that list it, followed by the column chunks (64 gathered keys) of
// blocks a_0..a_3; the four column lists themselves are copied to LDS too.
//
// Workgroup: 8 wavefronts in two groups of four (one wavefront of each group
// per SIMD).  Group g owns blocks a_{2g}, a_{2g+1}; each wavefront owns 32
// rows.  Both MFMA stages are computed transposed so that one lane owns one
// query row from the scores to the output:
//     S^T (64 keys x 32 rows)  = K_tile (64 x D) . Q^T (D x 32)
//     O^T (D x 32 rows)       += V^T (D x 64)    . P^T (64 x 32)
// With the 32x32 MFMA result layout, lane l holds query row l%32 and 16 of
// the keys of each 32-key half; those registers are the B operand of the P.V
// product without any cross-lane move, and each row's statistics live on the
// lane pair (l, l^32).
//
// Ping-pong schedule.  A wavefront's work on step t is split into an MFMA
// phase M(t) = {P.V of step t-1, S of step t and its mask} and a vector
// phase V(t) = {row max, running-max update, exponentials, P}.  Phases are
// separated by workgroup barriers; group 0 runs M(t) while group 1 runs
// V(t-1), then group 0 runs V(t) while group 1 runs M(t), so the two
// wavefronts sharing a SIMD keep the matrix cores and the vector ALUs busy
// at the same time.
//
// Split schedule (launches whose heads are all Block-Sparse, when two lists
// per item fit the step area): the four blocks of an item share few key
// blocks, so each group walks the union of its own two blocks' lists with
// its own K and V buffer; the phases stay paired by the same barriers.
//
// Staging: K and V rows go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds, 16 bytes per lane, 1 KiB of consecutive LDS
// per wave instruction; the head's rows are one raw buffer, the tile's first
// row a uniform offset, so a tile copy takes no per-lane address
// arithmetic).  K and V each have two buffers.  A group issues copies at
// the start of its vector phase, while the other group's MFMA phase keeps
// the matrix cores busy: group 1 the copy of K(t+1) in phase 2t, group 0
// that of V(t) in phase 2t+1; both are waited for at the end of phase 2t+1.
// Rows are stored unpadded; 16-byte chunk c of row r sits
// at position c ^ f(r), f(r) = 4(r%4) + (r/4)%4 (16-chunk rows), so that a K
// operand read (16 lanes per LDS cycle: 16 consecutive rows, same chunk) and
// a V transposed read (32 lanes per cycle: 4 rows x 4 chunks) each hit all 64
// banks once.  bf16: the V^T operand is read with the gfx950 LDS transpose
// read (ds_read_b64_tr_b16), which hands lane i of a 16-lane group element
// (i%4) of the 8-byte rows addressed by lanes 4j + i/4, j = 0..3.  fp32: V^T
// elements are read one by one.
#include "mi_device.h"
#include "mi_internal.h"

namespace mi {
namespace {

enum MaskMode { kMaskNone = 0, kMaskCausal = 1, kMaskAShape = 2, kMaskColumns = 3, kMaskExact = 4 };

struct Params {
    const char* q;
    const char* k;
    const char* v;
    char* o;
    float* lse;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;  // element strides
    int32_t B, Hq, Hkv, N, nb, nruns, group;
    float c;  // scale * log2(e)
    const int32_t* block_count;
    const int32_t* block_idx;
    const int32_t* col_count;
    const int32_t* col_idx;
    int32_t block_cap, col_cap;
    int32_t cstride;  // LDS entries per block column list (col_cap rounded up to 64; 0 without VS heads)
    int32_t sink, local;
    int32_t all_dense;
    int32_t xcd_chunk;
    const int32_t* sched;  // item schedule: packed (b * Hq + h) * nruns + run, -1 = none
    int32_t sched_len;
    const uint32_t* vs_bits;  // exact Vertical-Slash heads: [B, Hq, 2, bits_words] membership maps
    int32_t bits_words;
    uint8_t pattern[MI_MAX_HEADS];
};

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;  // 8 wavefronts, two groups of 4
constexpr int kBlocks = 4;             // query blocks per work item
constexpr int kIssueWaves = 4;         // wavefronts that issue a step's copies (one group)
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

// LDS of a work item.  Static: four staging tiles of TILEB bytes, K buffers
// 0/1 and V buffers 0/1 (step t uses buffer t % 2), and the key positions of
// a column step's 64 slots per K buffer; separate objects, so that the
// compiler can tell an operand read from the copies still in flight into the
// other buffers.  Dynamic LDS (byte offsets):
//   [0, 16 cstride)   column lists of the four blocks (-1 past the end)
//   then the packed step list (nb + 4 cstride / 64 entries), then 8 scan
//   slots.  While the step list is built, its first nb bytes hold the
//   per-key-block need masks.
template <typename T, int D>
struct Arena {
    static constexpr int kTile = Layout<T, D>::TILEB;
    static constexpr int kStatic = 4 * kTile + 2 * 64 * 4;  // + the two column-slot position arrays
    __host__ __device__ static int steps(int cstride) { return 16 * cstride; }
    __host__ __device__ static int scan(int nb, int cstride) { return steps(cstride) + 4 * (nb + 4 * (cstride / 64)); }
    __host__ __device__ static int bytes(int nb, int cstride) { return scan(nb, cstride) + 4 * kWaves; }
};

// Packed step: bits 0-19 key block (tile) or first list position (column
// chunk), 20-23 mask of the blocks that compute it, 24-25 owning block of a
// column chunk, 26 column chunk.
constexpr uint32_t kNoStep = 0xffffffffu;
__device__ __forceinline__ uint32_t pack_step(int kb, int need, int blk, int col) {
    return (uint32_t)kb | ((uint32_t)need << 20) | ((uint32_t)blk << 24) | ((uint32_t)col << 26);
}
__device__ __forceinline__ int step_kb(uint32_t w) { return (int)(w & 0xfffffu); }
__device__ __forceinline__ int step_need(uint32_t w) { return (int)((w >> 20) & 15u); }
__device__ __forceinline__ int step_blk(uint32_t w) { return (int)((w >> 24) & 3u); }
__device__ __forceinline__ bool step_col(uint32_t w) { return (w >> 26) & 1u; }

// Chunk swizzle of a staged row (see the header comment); rows of 8 chunks
// (bf16, d = 64) use 4((r/2)%2) + (r/4)%4.  Rows of 32 chunks (fp32,
// d = 128) use the 16-chunk form, which permutes their positions too.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    if constexpr (CPR == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    return ((row & 3) << 2) | ((row >> 2) & 3);
}

// Wave-uniform read of an index list entry through the constant address
// space, which the backend issues as a scalar (s_load) read: the lists are
// not written while the kernel runs.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int ld_uniform(const int32_t* p) {
    return *reinterpret_cast<const_i32*>(reinterpret_cast<uintptr_t>(p));
}

typedef __attribute__((address_space(3))) void lds_void;

// Issues wave instructions it0..it1-1 of the global->LDS copy of one step's
// K (or V) rows into the LDS buffer `dst`; the four wavefronts of one group
// (rank 0..3) share the copy, CPR/4 instructions each.  Wave instruction
// `idx` fills LDS chunks [64 idx, 64 idx + 64):
// lane l writes chunk 64 idx + l, i.e. row (64 idx + l) / CPR at position
// (64 idx + l) % CPR, which holds source chunk position ^ f(row).  Tile rows
// are addressed from a uniform base plus a 32-bit lane offset.  Gathered rows
// read their key position from `tok_src` (-1: empty slot, which reads row 0
// and is masked out later); the K copy also records the positions in
// `tok_dst` for the mask and the V copy of the same step.
template <typename T, int D>
__device__ __forceinline__ void issue_rows(char* dst, uint32_t w, const int32_t* tok_src, int32_t* tok_dst,
                                           const char* base, int64_t stride_b, int rank, int it0, int it1) {
    int lane = threadIdx.x & 63;
    // fp32 rows of 128 elements: eight copy instructions per wavefront; an
    // opaque lane id keeps their addresses from being hoisted out of the
    // step loop (they would not fit in registers and would spill)
    if constexpr (sizeof(T) == 4 && D == 128) asm volatile("" : "+v"(lane));
    const bool col = step_col(w);
    // buffer loads: the head's rows as one raw buffer (SGPR descriptor), a
    // uniform offset for the tile and 32-bit per-lane row offsets
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000);
    const uint32_t sb = (uint32_t)stride_b;  // the host keeps seq_len * stride below 2^32
    if (!col) {
        // a whole tile: loop-invariant lane offsets, the tile in the uniform offset
        const uint32_t soff = (uint32_t)step_kb(w) * 64u * sb;
#pragma unroll
        for (int it = it0; it < it1; ++it) {
            const int idx = it * kIssueWaves + rank;
            const int cidx = idx * 64 + lane;
            const int row = cidx / Layout<T, D>::CPR, pos = cidx % Layout<T, D>::CPR;
            const int chunk = pos ^ swz<Layout<T, D>::CPR>(row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + idx * 1024), 16,
                                                     (int)((uint32_t)row * sb + chunk * 16), (int)soff, 0, 0);
        }
    } else {
#pragma unroll
        for (int it = it0; it < it1; ++it) {
            const int idx = it * kIssueWaves + rank;
            const int cidx = idx * 64 + lane;
            const int row = cidx / Layout<T, D>::CPR, pos = cidx % Layout<T, D>::CPR;
            const int chunk = pos ^ swz<Layout<T, D>::CPR>(row);
            const int tok = tok_src[row];
            if (tok_dst && pos == 0) tok_dst[row] = tok;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + idx * 1024), 16,
                                                     (int)((uint32_t)max(tok, 0) * sb + chunk * 16), 0, 0, 0);
        }
    }
}

// Writes the item's step list (and, for Vertical-Slash heads, the four
// column lists) to LDS; returns the number of steps.  Sparse heads: a mask
// byte per key block kb <= a_3 (bit i: block a_i lists kb, kb <= a_i), then
// an ordered compaction of the non-empty masks.  Dense heads: every causal
// key block, computed by the blocks at or after it.  split: two lists, one
// per ping-pong group (key blocks that block 2g or 2g+1 lists, with those
// two mask bits), n0 entries then n1; the caller guarantees n0 + n1 <= nb.
template <typename T, int D>
__device__ int build_steps(char* dyn, const Params& p, int pattern, int64_t r0, int a0, int nblk, bool split,
                           int& n0, int& n1) {
    typedef Arena<T, D> A;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int cstride = p.cstride;
    uint32_t* steps = reinterpret_cast<uint32_t*>(dyn + A::steps(cstride));
    int32_t* scan = reinterpret_cast<int32_t*>(dyn + A::scan(p.nb, cstride));
    const int nkb = a0 + nblk;
    int ntiles;
    if (pattern == MI_DENSE) {
        for (int kb = t; kb < nkb; kb += kThreads) {
            int need = 0;
            for (int w = 0; w < nblk; ++w) need |= (kb <= a0 + w) ? (1 << w) : 0;
            steps[kb] = pack_step(kb, need, 0, 0);
        }
        ntiles = nkb;
    } else {
        uint32_t* mw = steps;  // nkb mask bytes, packed four per word
        const int words = (nkb + 3) / 4;
        for (int i = t; i < words; i += kThreads) mw[i] = 0u;
        __syncthreads();
        for (int w = 0; w < nblk; ++w) {
            const int cnt = min(max(ld_uniform(p.block_count + r0 + w), 0), p.block_cap);
            const int32_t* L = p.block_idx + (r0 + w) * p.block_cap;
            for (int i = t; i < cnt; i += kThreads) {
                const int kb = L[i];
                if (kb >= 0 && kb <= a0 + w) atomicOr(&mw[kb >> 2], (1u << w) << (8 * (kb & 3)));
            }
        }
        __syncthreads();
        // thread t owns mask words [t per, (t + 1) per): read them, count the
        // non-empty masks, scan the counts, then overwrite the region with
        // the steps (entry o <= key block, so only after every read)
        constexpr int kMaxPer = 16;  // words per thread: nkb <= 4 * 16 * 512
        const int per = (words + kThreads - 1) / kThreads;
        uint32_t mine[kMaxPer];
        int c = 0;
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j) {
            const int wi = t * per + j;
            mine[j] = (j < per && wi < words) ? mw[wi] : 0u;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) c += ((mine[j] >> (8 * bb)) & 0xffu) ? 1 : 0;
        }
        if (split) {
            // one list per ping-pong group: key blocks that block 2g or 2g+1
            // lists, with those two mask bits; counts packed (low: group 0)
            c = 0;
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint32_t m = (mine[j] >> (8 * bb)) & 0xffu;
                    c += ((m & 3u) ? 1 : 0) + ((m & 12u) ? 0x10000 : 0);
                }
        }
        int incl = c;  // inclusive scan over the wavefront
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) scan[wv] = incl;
        __syncthreads();
        int before = 0;
        ntiles = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            before += w < wv ? scan[w] : 0;
            ntiles += scan[w];
        }
        if (split) {
            n0 = ntiles & 0xffff;
            n1 = ntiles >> 16;
            ntiles = n0 + n1;
            int o0 = (before + incl - c) & 0xffff, o1 = n0 + ((before + incl - c) >> 16);
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint32_t m = (mine[j] >> (8 * bb)) & 0xffu;
                    const int kb = 4 * (t * per + j) + bb;
                    if (m & 3u) steps[o0++] = pack_step(kb, (int)(m & 3u), 0, 0);
                    if (m & 12u) steps[o1++] = pack_step(kb, (int)(m & 12u), 0, 0);
                }
        } else {
            int o = before + incl - c;
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint32_t m = (mine[j] >> (8 * bb)) & 0xffu;
                    if (m) steps[o++] = pack_step(4 * (t * per + j) + bb, (int)m, 0, 0);
                }
        }
    }
    int nsteps = ntiles;
    if (pattern == MI_VSLASH || pattern == MI_VSLASH_EXACT) {
        int32_t* colsl = reinterpret_cast<int32_t*>(dyn);
        for (int w = 0; w < kBlocks; ++w) {
            const int cnt = w < nblk ? min(max(ld_uniform(p.col_count + r0 + w), 0), p.col_cap) : 0;
            const int32_t* C = p.col_idx + (r0 + w) * p.col_cap;
            for (int i = t; i < cstride; i += kThreads) {
                const int j = i < cnt ? C[i] : -1;
                colsl[w * cstride + i] = (j >= 0 && j < p.N) ? j : -1;
            }
            const int nch = (cnt + 63) / 64;
            for (int c = t; c < nch; c += kThreads) steps[nsteps + c] = pack_step(64 * c, 1 << w, w, 1);
            nsteps += nch;
        }
    }
    __syncthreads();
    return nsteps;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Per-lane LDS byte offsets of the operand reads (bf16), relative to a
// buffer.  With unpadded rows of ROWB >= 128 bytes and the XOR swizzle:
//   K operand (row kh*32 + rl, chunk 2ks + hl):
//       rl*ROWB + 16((2ks + hl) ^ f(rl)) = (kbase ^ 32ks),  kbase = rl*ROWB + 16(hl ^ f(rl));
//   V^T operand (row base + 8sec + 4hl + j, chunk 4db + x, half qd%2), with
//   x = 2((l/16)%2) + (qd/2) and f(r + 8) = f(r) ^ 2:
//       (base + 8sec)*ROWB + (vbase ^ (64db + 32sec)),
//       vbase = (4hl + j)*ROWB + 16(x ^ f(4hl + j)) + 8(qd%2).
// The XOR constants only touch bits 5..7 (below ROWB); the buffers are
// 1 KiB aligned.  Every XORed base is computed once per work item and held
// in a register (k[ks], v[2 db + sec]): the reads then take the rest of
// their address (buffer, row, kh) as the instruction's immediate offset,
// with no address arithmetic in the step loop.
template <typename T, int D>
struct LaneBase {
    static constexpr int NK = sizeof(T) == 2 ? D / 16 : 1;
    static constexpr int NV = sizeof(T) == 2 ? D / 16 : 1;
    int k[NK], v[NV];
};
template <typename T, int D>
__device__ __forceinline__ LaneBase<T, D> lane_base(int lane) {
    typedef Layout<T, D> Ly;
    const int rl = lane & 31, hl = lane >> 5;
    LaneBase<T, D> b;
    if constexpr (sizeof(T) == 2) {
        const int kb = rl * Ly::ROWB + 16 * (hl ^ swz<Ly::CPR>(rl));
        const int g16 = (lane >> 4) & 1, s = lane & 15, j = s >> 2, qd = s & 3;
        const int x = 2 * g16 + (qd >> 1);
        const int vb = (4 * hl + j) * Ly::ROWB + 16 * (x ^ swz<Ly::CPR>(4 * hl + j)) + 8 * (qd & 1);
#pragma unroll
        for (int i = 0; i < LaneBase<T, D>::NK; ++i) {
            b.k[i] = kb ^ (32 * i);
            asm volatile("" : "+v"(b.k[i]));  // materialised once, not recomputed in the loop
        }
#pragma unroll
        for (int i = 0; i < LaneBase<T, D>::NV; ++i) {
            b.v[i] = vb ^ (64 * (i >> 1) + 32 * (i & 1));
            asm volatile("" : "+v"(b.v[i]));
        }
    } else {
        b.k[0] = rl * Ly::ROWB;
        b.v[0] = 0;
    }
    return b;
}

// K operand (8 elements of key row kh*32 + rl, slots 16 ks + 8 hl ..) from
// the K buffer `kbuf`.
template <int D>
__device__ __forceinline__ bf16x8 k_frag_bf16(const char* kbuf, const LaneBase<uint16_t, D>& lb, int kh, int ks) {
    const char* a = kbuf + (lb.k[ks] + kh * 32 * Layout<uint16_t, D>::ROWB);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a));
}
template <int D>
__device__ __forceinline__ f32x8 k_frag_f32(const char* kbuf, const LaneBase<float, D>& lb, int kh, int ks) {
    typedef Layout<float, D> Ly;
    const int rl = threadIdx.x & 31, hl = (threadIdx.x >> 5) & 1;
    const char* row = kbuf + kh * 32 * Ly::ROWB + lb.k[0];
    const int f = swz<Ly::CPR>(rl);
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + (((4 * ks + 2 * hl) ^ f) * 16));
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + (((4 * ks + 2 * hl + 1) ^ f) * 16));
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// V^T operand for d block db over keys [base, base+16) of the V buffer at
// `vbuf`: lane (d = 32 db + l%32, half hl) gets keys base+4hl+{0..3} and
// base+8+4hl+{0..3}.
template <int D>
__device__ __forceinline__ bf16x8 v_frag_bf16(const char* vbuf, const LaneBase<uint16_t, D>& lb, int db, int base) {
    constexpr int RB = Layout<uint16_t, D>::ROWB;
    const char* p0 = vbuf + (lb.v[2 * db] + base * RB);
    const char* p1 = vbuf + (lb.v[2 * db + 1] + (base + 8) * RB);
    const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
    const i16x8 r = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    return __builtin_bit_cast(bf16x8, r);
}
template <int D>
__device__ __forceinline__ f32x8 v_frag_f32(const char* vbuf, const LaneBase<float, D>&, int db, int base) {
    typedef Layout<float, D> Ly;
    const int rl = threadIdx.x & 31, hl = (threadIdx.x >> 5) & 1;
    const int d = db * 32 + rl;
    f32x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int key = base + (e >> 2) * 8 + 4 * hl + (e & 3);
        r[e] = *reinterpret_cast<const float*>(vbuf + key * Ly::ROWB +
                                               (((d >> 2) ^ swz<Ly::CPR>(key)) * 16) + (d & 3) * 4);
    }
    return r;
}

template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag k_frag(const char* kbuf, const LaneBase<T, D>& lb, int kh, int ks) {
    if constexpr (sizeof(T) == 2) return k_frag_bf16<D>(kbuf, lb, kh, ks);
    else return k_frag_f32<D>(kbuf, lb, kh, ks);
}
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag v_frag(const char* vbuf, const LaneBase<T, D>& lb, int db, int base) {
    if constexpr (sizeof(T) == 2) return v_frag_bf16<D>(vbuf, lb, db, base);
    else return v_frag_f32<D>(vbuf, lb, db, base);
}

__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-wave running state (32 rows).
template <typename T, int D>
struct RowState {
    f32x16 oacc[D / 32];
    float m_run;   // running max (log2 units, scaled)
    float l_part;  // this lane's share of the normaliser
};

// Mask mode of a step for the query block `my_a`.
template <bool EXACT>
__device__ __forceinline__ int step_mode(uint32_t w, const Params& p, int pattern, int my_a) {
    if (step_col(w)) return kMaskColumns;
    if (EXACT && pattern == MI_VSLASH_EXACT) return kMaskExact;
    const int kb = step_kb(w);
    if (pattern == MI_ASHAPE) {
        const bool full = kb < my_a && ((kb * 64 + 63 < p.sink) || ((my_a - kb) * 64 + 63 < p.local));
        return full ? kMaskNone : kMaskAShape;
    }
    return kb >= my_a ? kMaskCausal : kMaskNone;
}

// The wavefront's Q^T operand (32 rows x D).  Held in registers, except
// for fp32 rows of 128 elements, whose 64 registers would not fit beside the
// accumulators at two wavefronts per SIMD: those fragments are re-read from
// global memory (the 16 KiB of a wavefront's rows stay in the L1/L2 caches)
// at each use.
template <typename T, int D>
struct QOperand {
    typedef typename Elem<T>::frag Frag;
    static constexpr bool kRegs = !(sizeof(T) == 4 && D == 128);
    Frag f[kRegs ? D / 16 : 1];
    const T* row;  // this lane's row, offset by its contraction half (8 hl)
    __device__ __forceinline__ void init(const T* qrow, bool active) {
        row = qrow;
        if constexpr (kRegs) {
            if (active) {
#pragma unroll
                for (int s = 0; s < D / 16; ++s) f[s] = load_frag(qrow + 16 * s);
            } else {
#pragma unroll
                for (int s = 0; s < D / 16; ++s) f[s] = Frag{};
            }
        }
    }
    __device__ __forceinline__ Frag get(int ks) const {
        if constexpr (kRegs) return f[ks];
        else return load_frag(row + 16 * ks);
    }
};

// S^T = K . Q^T for one step (the two 32-key halves interleaved).
template <typename T, int D>
__device__ __forceinline__ void s_compute(f32x16 (&s)[2], const char* kbuf, const LaneBase<T, D>& lb,
                                          const QOperand<T, D>& qf) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kh][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const typename Elem<T>::frag qk = qf.get(ks);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) mma32(s[kh], k_frag<T, D>(kbuf, lb, kh, ks), qk);
        // fp32: keep each slice's operand reads next to its MFMAs (hoisting
        // them all would need more registers than two wavefronts per SIMD have)
        if constexpr (sizeof(T) == 4) __builtin_amdgcn_sched_barrier(0);
    }
    // bf16 schedule: four operand reads ahead, then one MFMA per read, so
    // that LDS latency hides behind the MFMA chain
    if constexpr (sizeof(T) == 2) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
}

// S^T = K . Q^T with the K operands of the first two 16-dimension slices
// already read (kpre[ks][kh]); bf16 only.
template <typename T, int D>
__device__ __forceinline__ void s_compute_pre(f32x16 (&s)[2], const char* kbuf, const LaneBase<T, D>& lb,
                                              const QOperand<T, D>& qf,
                                              const typename Elem<T>::frag (&kpre)[2][2]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kh][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const typename Elem<T>::frag qk = qf.get(ks);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) mma32(s[kh], ks < 2 ? kpre[ks][kh] : k_frag<T, D>(kbuf, lb, kh, ks), qk);
    }
    constexpr int kReads = (D / 16 - 2) * 2;
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, D / 8 - kReads, 0);
}

typedef __attribute__((address_space(4))) const uint32_t const_u32;
__device__ __forceinline__ uint32_t ld_uniform_u32(const uint32_t* p) {
    return *reinterpret_cast<const_u32*>(reinterpret_cast<uintptr_t>(p));
}

// Exact Vertical-Slash mask of a tile step (key block kb): row i keeps key
// j = 64 kb + c iff j <= i and (j is a vertical key or i - j a slash offset).
// The maps hold bit x for key / offset x - 64 (64 leading zero bits, so the
// offsets of keys above the diagonal, down to -63, read as absent).  The
// wavefront's 32 rows i0 .. i0+31 need the slash offsets
// [i0 - 64kb - 63, i0 - 64kb + 31]: four words read on the scalar unit, from
// which each lane funnel-shifts its 64-bit window (bit t <-> offset
// i - 64kb - 63 + t <-> key c = 63 - t) and bit-reverses it into key order.
// The vertical bits of the tile's 64 keys are two uniform words.
__device__ __forceinline__ void mask_exact(f32x16 (&s)[2], const uint32_t* vbits, const uint32_t* sbits, int kb,
                                           int i0, int i_row) {
    const int hl = (threadIdx.x >> 5) & 1;
    const uint32_t v0 = ld_uniform_u32(vbits + 2 * kb + 2), v1 = ld_uniform_u32(vbits + 2 * kb + 3);
    const int bit0 = i0 - 64 * kb + 1;  // map bit of offset i0 - 64kb - 63 (>= 1 for kb <= the row's block)
    const int w0 = bit0 >> 5;
    const uint32_t x0 = ld_uniform_u32(sbits + w0), x1 = ld_uniform_u32(sbits + w0 + 1);
    const uint32_t x2 = ld_uniform_u32(sbits + w0 + 2), x3 = ld_uniform_u32(sbits + w0 + 3);
    const int sh = (bit0 & 31) + (i_row - i0);  // 0 .. 62
    const bool up = sh >= 32;
    const uint32_t a0 = up ? x1 : x0, a1 = up ? x2 : x1, a2 = up ? x3 : x2;
    const uint32_t lo = __builtin_amdgcn_alignbit(a1, a0, sh & 31);
    const uint32_t hi = __builtin_amdgcn_alignbit(a2, a1, sh & 31);
    uint32_t k_lo = __builtin_bitreverse32(hi) | v0;  // keys 0..31 of the tile
    uint32_t k_hi = __builtin_bitreverse32(lo) | v1;  // keys 32..63
    const int lim = i_row - 64 * kb;                  // causal: keys c <= lim (lim < 63 only on the diagonal)
    if (lim < 63) {
        k_lo &= lim >= 31 ? ~0u : ((2u << lim) - 1u);
        k_hi &= lim >= 32 ? ((2u << (lim - 32)) - 1u) : 0u;
    }
    // lane half hl holds keys 4 hl + {0..3} of each group of 8
    const uint32_t m_lo = hl ? (k_lo >> 4) | (k_hi << 28) : k_lo;
    const uint32_t m_hi = hl ? (k_hi >> 4) : k_hi;
    const uint32_t ninf = 0xff800000u;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
        const uint32_t m = kh ? m_hi : m_lo;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int bit = 8 * (e >> 2) + (e & 3);
            const uint32_t keep = (uint32_t)((int32_t)(m << (31 - bit)) >> 31);  // all ones iff the bit is set
            s[kh][e] = __uint_as_float((__float_as_uint(s[kh][e]) & keep) | (ninf & ~keep));
        }
    }
}

// Masks one row block's scores (element e of half kh is key 32 kh + 8 (e/4) +
// 4 hl + e%4 of the step).
// Column steps read each slot's key position from `cl`.
template <bool EXACT>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int mode, int kb, const int32_t* cl,
                                            const Params& p, int i_row, const uint32_t* ex_bits, int ex_i0) {
    const int hl = (threadIdx.x >> 5) & 1;
    // Opaque copies: the phase code appears once per group, and without
    // these the compiler merges the two copies' comparisons and hoists them
    // to the top of the step, holding 32+ lane masks in scalar registers.
    asm volatile("" : "+v"(i_row));
    int hl4 = 4 * hl;
    asm volatile("" : "+v"(hl4));
    (void)hl;
    if (mode == kMaskCausal) {
        const int lim = i_row - kb * 64 - hl4;  // keep key-local kl iff kl - 4hl <= lim
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int klc = kh * 32 + 8 * (e >> 2) + (e & 3);
                s[kh][e] = (klc <= lim) ? s[kh][e] : -INFINITY;
            }
    } else if (mode == kMaskAShape) {
        // key j = kb*64 + 4hl + klc: keep iff j <= i_row and (j < sink or i_row - j < local)
        const int j0 = kb * 64 + hl4;
        const int lim = i_row - j0, sl = p.sink - j0, ll = i_row - p.local - j0;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int klc = kh * 32 + 8 * (e >> 2) + (e & 3);
                const bool keep = (klc <= lim) && ((klc < sl) || (klc > ll));
                s[kh][e] = keep ? s[kh][e] : -INFINITY;
            }
    } else if (EXACT && mode == kMaskExact) {
        if constexpr (EXACT) mask_exact(s, ex_bits, ex_bits + p.bits_words, kb, ex_i0, i_row);
    } else if (mode == kMaskColumns) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int4 j4 = *reinterpret_cast<const int4*>(&cl[kh * 32 + 8 * q4 + hl4]);
                const int jj[4] = {j4.x, j4.y, j4.z, j4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = (jj[r] >= 0) && (jj[r] <= i_row);
                    s[kh][4 * q4 + r] = keep ? s[kh][4 * q4 + r] : -INFINITY;
                }
            }
    }
}

// The row's max over a step's scores, scaled to log2 units.
__device__ __forceinline__ float row_max(const f32x16 (&s)[2], float c) {
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kh][e]);
    return pair_max(mx) * c;
}

// Raises the running max if the step's max exceeds it by more than 2^kLazy
// (rare after the first steps).  The accumulator factor `alpha` is applied
// in the next MFMA phase, before the step's P.V is added, so that the vector
// phase never rewrites the accumulators.  Returns whether any row raised.
template <typename T, int D>
__device__ __forceinline__ bool raise_max(RowState<T, D>& rs, float mx, float& alpha) {
    const bool raise = mx > rs.m_run + kLazy;
    alpha = raise ? fast_exp2(rs.m_run - mx) : 1.f;  // 0 when m_run = -inf
    rs.m_run = raise ? mx : rs.m_run;
    rs.l_part *= alpha;
    return __ballot(raise) != 0;
}

// O^T += V^T . P^T over 16-key chunks (half kh, part pp).
template <typename T, int D>
__device__ __forceinline__ void pv_accumulate(RowState<T, D>& rs, const char* vbuf, const LaneBase<T, D>& lb,
                                              const typename Elem<T>::frag (&pf)[2][2]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                mma32(rs.oacc[db], v_frag<T, D>(vbuf, lb, db, kh * 32 + pp * 16), pf[kh][pp]);
                if constexpr (sizeof(T) == 4) __builtin_amdgcn_sched_barrier(0);
            }
    // bf16 schedule: eight transposed reads (four operands) ahead, then one
    // MFMA per operand
    if constexpr (sizeof(T) == 2) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // DS reads
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    }
}

// bf16: the probabilities of a step as P.V operands: pf[kh][pp] holds keys
// 16 pp .. 16 pp + 15 of half kh (8 per lane) as bf16 pairs; returns their
// fp32 sum (before rounding).
__device__ __forceinline__ float probs_bf16(bf16x8 (&pf)[2][2], const f32x16 (&s)[2], float m_use, float c) {
    float sum = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            u32x4 u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(s[kh][8 * pp + 2 * e], c, -m_use));
                const float p1 = fast_exp2(fmaf(s[kh][8 * pp + 2 * e + 1], c, -m_use));
                u[e] = pack_bf16x2(p0, p1);
                sum += p0 + p1;
            }
            pf[kh][pp] = __builtin_bit_cast(bf16x8, u);
        }
    return sum;
}

// fp32: the probabilities overwrite the scores (an fp32 P operand is the
// score registers themselves); returns their sum.
__device__ __forceinline__ float probs_in_place(f32x16 (&s)[2], float m_use, float c) {
    float sum = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s[kh][e] = fast_exp2(fmaf(s[kh][e], c, -m_use));
            sum += s[kh][e];
        }
    return sum;
}

// fp32 O^T += V^T . P^T with P read straight from the score registers
// (16-key chunk pp of half kh is elements 8 pp .. 8 pp + 7 of s[kh]).
template <int D>
__device__ __forceinline__ void pv_accumulate_f32(RowState<float, D>& rs, const char* vbuf, const LaneBase<float, D>& lb,
                                                  const f32x16 (&s)[2]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const f32x8 pf = {s[kh][8 * pp + 0], s[kh][8 * pp + 1], s[kh][8 * pp + 2], s[kh][8 * pp + 3],
                              s[kh][8 * pp + 4], s[kh][8 * pp + 5], s[kh][8 * pp + 6], s[kh][8 * pp + 7]};
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                mma32(rs.oacc[db], v_frag<float, D>(vbuf, lb, db, kh * 32 + pp * 16), pf);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
}

// Barrier that does not wait for outstanding global->LDS copies.
__device__ __forceinline__ void phase_barrier() { __builtin_amdgcn_s_barrier(); }

// EXACT: the instantiation launched when some head is MI_VSLASH_EXACT (its
// tile steps take the per-element Vertical-Slash mask); the other
// instantiation carries no code for it.
template <typename T, int D, bool EXACT, bool SPLIT>
__global__ void __launch_bounds__(kThreads) sparse_attn_kernel(Params p) {
    typedef typename Elem<T>::frag Frag;
    typedef Layout<T, D> Ly;
    typedef Arena<T, D> Ar;
    constexpr int NDB = D / 32;
    __shared__ __attribute__((aligned(1024))) char kbuf0[Ly::TILEB];
    __shared__ __attribute__((aligned(1024))) char kbuf1[Ly::TILEB];
    __shared__ __attribute__((aligned(1024))) char vbuf0[Ly::TILEB];
    __shared__ __attribute__((aligned(1024))) char vbuf1[Ly::TILEB];
    __shared__ __attribute__((aligned(16))) int32_t cpos0[64];  // key positions of a column step's slots
    __shared__ __attribute__((aligned(16))) int32_t cpos1[64];
    extern __shared__ __attribute__((aligned(16))) char dyn[];

    const int items = p.B * p.Hq * p.nruns;
    const int L = rotated_xcd_remap(blockIdx.x, gridDim.x, p.sched ? 4 : p.xcd_chunk);
    int run, bh;
    if (p.sched) {
        // scheduled order: chunks of four items of one kv group and pattern
        // class, longest first
        if (L >= p.sched_len) return;
        const int it = ld_uniform(p.sched + L);
        if (it < 0 || it >= items) return;
        run = it % p.nruns;
        bh = it / p.nruns;
    } else {
        if (L >= items) return;
        // longest items first: runs of query blocks in descending order
        run = p.nruns - 1 - L / (p.B * p.Hq);
        bh = L % (p.B * p.Hq);
    }
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int kvh = h / p.group;
    const int pattern = p.all_dense ? MI_DENSE : p.pattern[h];
    const uint32_t* ex_bits = EXACT ? p.vs_bits + (int64_t)(b * p.Hq + h) * 2 * p.bits_words : nullptr;

    const int lane = threadIdx.x & 63;
    // wave-uniform: lets all per-wave control live in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;                    // ping-pong group
    const int blk = 2 * grp + ((wave >> 1) & 1);  // query block of this wave in the run
    const int hl = lane >> 5;
    const int rl = lane & 31;
    const int a0 = run * kBlocks;
    const int nblk = min(kBlocks, p.nb - a0);
    const int my_a = a0 + blk;
    const bool active = blk < nblk;
    const int i_row = my_a * 64 + (wave & 1) * 32 + rl;

    const T* qbase = reinterpret_cast<const T*>(p.q) + b * p.qs0 + h * p.qs1;
    const char* kbase = p.k + (b * p.ks0 + kvh * p.ks1) * (int64_t)sizeof(T);
    const char* vbase = p.v + (b * p.vs0 + kvh * p.vs1) * (int64_t)sizeof(T);
    const int64_t kstride = p.ks2 * (int64_t)sizeof(T), vstride = p.vs2 * (int64_t)sizeof(T);

    const int64_t r0 = (int64_t)bh * p.nb + a0;
    // Block-Sparse items whose four lists hold at most nb entries run in
    // split mode: each ping-pong group walks the union of its own two
    // blocks' lists with its own K and V buffer (the four blocks' lists share
    // few key blocks, so one common step list would leave most of its steps
    // to a single block).
    const bool split = SPLIT && pattern == MI_BSPARSE && 4 * p.block_cap <= p.nb;
    int n0 = 0, n1 = 0;
    const int nsteps = build_steps<T, D>(dyn, p, pattern, r0, a0, nblk, split, n0, n1);
    const int32_t* colsl = reinterpret_cast<const int32_t*>(dyn);
    const uint32_t* steps = reinterpret_cast<const uint32_t*>(dyn + Ar::steps(p.cstride));
    const int cstride = p.cstride;
    const uint32_t* my_steps = (split && grp == 1) ? steps + n0 : steps;
    const int my_n = split ? (grp == 1 ? n1 : n0) : nsteps;
    auto fetch = [&](int t) -> uint32_t {
        return t < my_n ? (uint32_t)__builtin_amdgcn_readfirstlane(my_steps[t]) : kNoStep;
    };

    QOperand<T, D> qf;
    qf.init(qbase + (int64_t)i_row * p.qs2 + 8 * hl, active);
    const LaneBase<T, D> lb = lane_base<T, D>(lane);

    RowState<T, D> rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) rs.oacc[db][e] = 0.f;
    rs.m_run = -INFINITY;
    rs.l_part = 0.f;

    auto needs = [&](uint32_t w) { return active && w != kNoStep && ((step_need(w) >> blk) & 1); };
    // The scores of a step live from its MFMA phase to its vector phase
    // only (fp32: then its probabilities, in place, up to the next MFMA
    // phase); bf16 P operands are carried to the next MFMA phase in pfr.
    Frag pfr[2][2];
    f32x16 s_keep[2];  // the scores (fp32: then the parked probabilities)
    float alpha = 1.f;     // accumulator factor of the last vector phase
    bool rescale = false;  // some row of the wavefront raised its max

    // Step t = 0..nsteps-1 (and one drain step); phase 2t: group 0 runs M(t),
    // group 1 runs V(t-1); phase 2t+1: group 1 runs M(t), group 0 runs V(t).
    // K(t) sits in K buffer t%2, V(t) in V buffer t%2.  Group 1 issues the
    // copy of K(t+1) at the start of phase 2t and group 0 that of V(t) at the
    // start of phase 2t+1 (the buffers' last readers finished in phase
    // 2t-1); every wave waits for its own copies at the end of phase 2t+1.
    uint32_t wprev = kNoStep, wcur = fetch(0), wnext = fetch(1);
    // M(t) on this wavefront: P.V of step t-1 (V buffer vprev), then S of
    // step t (K buffer kcur) and its mask.
    auto m_phase = [&](const char* kcur, const char* vprev, const int32_t* cpcur, bool pv_need, bool s_need,
                       f32x16 (&s)[2]) __attribute__((always_inline)) {
        // bf16: the first S operands are read before the P.V chain (the K
        // buffer is complete since the phase began), so that S starts
        // without waiting on LDS
        Frag kpre[2][2];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) kpre[ks][kh] = k_frag<T, D>(kcur, lb, kh, ks);
        }
        if (pv_need) {
            if (rescale) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) rs.oacc[db][e] *= alpha;
            }
            if constexpr (sizeof(T) == 2) {
                pv_accumulate<T, D>(rs, vprev, lb, pfr);
            } else {
                pv_accumulate_f32<D>(rs, vprev, lb, s);
            }
        }
        if (s_need) {
            if constexpr (sizeof(T) == 2) s_compute_pre<T, D>(s, kcur, lb, qf, kpre);
            else s_compute<T, D>(s, kcur, lb, qf);
            mask_scores<EXACT>(s, step_mode<EXACT>(wcur, p, pattern, my_a), step_kb(wcur), cpcur, p, i_row, ex_bits,
                               my_a * 64 + (wave & 1) * 32);
        }
    };
    // Vector phase on this wavefront: row max, running-max update,
    // probabilities (parked as P operands over the scores).
    auto v_phase = [&](bool need, f32x16 (&s)[2]) __attribute__((always_inline)) {
        if (need) {
            rescale = raise_max<T, D>(rs, row_max(s, p.c), alpha);
            const float m_use = (rs.m_run == -INFINITY) ? 0.f : rs.m_run;
            if constexpr (sizeof(T) == 2) {
                rs.l_part += probs_bf16(pfr, s, m_use, p.c);
            } else {
                rs.l_part += probs_in_place(s, m_use, p.c);
            }
        }
    };
    constexpr int NI = Ly::CPR / kIssueWaves;
    // Each group runs its steps in a loop of its own (the two loops meet at
    // the same barriers): phase 2t: group 0 runs M(t) while group 1 issues
    // the copy of K(t+1) and runs V(t-1); phase 2t+1: group 1 runs M(t)
    // while group 0 issues the copy of V(t) and runs V(t).  K(t) sits in K
    // buffer t%2, V(t) in V buffer t%2; the loops unroll two steps so that
    // every buffer is a fixed LDS object in each copy.  Every wave waits for
    // its own copies at the end of phase 2t+1.  A group-1 step is (copy of
    // K(t+1), V(t-1), barrier, M(t)): the scores of step t-1 cross from one
    // iteration into the next in s_keep.
    auto advance = [&](int t) __attribute__((always_inline)) {
        wprev = wcur;
        wcur = wnext;
        wnext = fetch(t + 2);
    };
    // The scores of a step sit in s_keep from its MFMA phase to its vector
    // phase (for group 1 across an iteration); fp32 then keeps its
    // probabilities there up to the next MFMA phase, bf16 moves them to pfr.
    auto step0 = [&](int t, const char* kcur, char* vcur, const char* vprev, const int32_t* cpcur)
        __attribute__((always_inline)) {
        const bool pv_need = needs(wprev), s_need = needs(wcur);
        f32x16 (&s)[2] = s_keep;
        m_phase(kcur, vprev, cpcur, pv_need, s_need, s);
        phase_barrier();
        if (wcur != kNoStep) issue_rows<T, D>(vcur, wcur, cpcur, nullptr, vbase, vstride, wave & 3, 0, NI);
        v_phase(s_need, s);
        if (wcur == kNoStep) return false;
        __syncthreads();  // K(t+1) and V(t) have landed; phase 2t+2 begins
        advance(t);
        return true;
    };
    auto step1 = [&](int t, const char* kcur, char* knext, const char* vprev, const int32_t* cpcur, int32_t* cpnext)
        __attribute__((always_inline)) {
        const bool pv_need = needs(wprev), s_need = needs(wcur);
        f32x16 (&s)[2] = s_keep;
        if (wnext != kNoStep)
            issue_rows<T, D>(knext, wnext, colsl + step_blk(wnext) * cstride + step_kb(wnext), cpnext, kbase,
                             kstride, wave & 3, 0, NI);
        v_phase(pv_need, s);
        phase_barrier();
        m_phase(kcur, vprev, cpcur, pv_need, s_need, s);
        if (wcur == kNoStep) return false;
        __syncthreads();
        advance(t);
        return true;
    };
    if (split) {
        // Phase 2t: group 0 runs M(t) on its step t, group 1 copies K of its
        // step t and V of its step t-1, then runs V(t-1); phase 2t+1: group 0
        // copies V of its step t and K of its step t+1, then runs V(t), group
        // 1 runs M(t).  Group g stages into K buffer g and V buffer g only
        // (each buffer's last reader finished in the phase before the copy)
        // and waits for its copies at the end of the phase that issued them.
        // Both loops run max(n0, n1) + 1 iterations of two barriers.
        const int T2 = max(n0, n1);
        if (wcur != kNoStep && grp == 0)
            issue_rows<T, D>(kbuf0, wcur, nullptr, nullptr, kbase, kstride, wave & 3, 0, NI);
        __syncthreads();
        if (grp == 0) {
            for (int t = 0; t <= T2; ++t) {
                const bool pv_need = needs(wprev), s_need = needs(wcur);
                m_phase(kbuf0, vbuf0, cpos0, pv_need, s_need, s_keep);
                __syncthreads();
                if (wcur != kNoStep) issue_rows<T, D>(vbuf0, wcur, nullptr, nullptr, vbase, vstride, wave & 3, 0, NI);
                if (wnext != kNoStep)
                    issue_rows<T, D>(kbuf0, wnext, nullptr, nullptr, kbase, kstride, wave & 3, 0, NI);
                v_phase(s_need, s_keep);
                __syncthreads();
                advance(t);
            }
        } else {
            for (int t = 0; t <= T2; ++t) {
                const bool pv_need = needs(wprev), s_need = needs(wcur);
                if (wcur != kNoStep) issue_rows<T, D>(kbuf1, wcur, nullptr, nullptr, kbase, kstride, wave & 3, 0, NI);
                if (wprev != kNoStep)
                    issue_rows<T, D>(vbuf1, wprev, nullptr, nullptr, vbase, vstride, wave & 3, 0, NI);
                v_phase(pv_need, s_keep);
                __syncthreads();
                m_phase(kbuf1, vbuf1, cpos1, pv_need, s_need, s_keep);
                __syncthreads();
                advance(t);
            }
        }
    } else {
    if (wcur != kNoStep && grp == 1)
        issue_rows<T, D>(kbuf0, wcur, colsl + step_blk(wcur) * cstride + step_kb(wcur), cpos0, kbase, kstride,
                         wave & 3, 0, NI);
    __syncthreads();
    if (grp == 0) {
        for (int t = 0;; t += 2) {
            if (!step0(t, kbuf0, vbuf0, vbuf1, cpos0)) break;
            if (!step0(t + 1, kbuf1, vbuf1, vbuf0, cpos1)) break;
        }
    } else {
        for (int t = 0;; t += 2) {
            if (!step1(t, kbuf0, kbuf1, vbuf1, cpos0, cpos1)) break;
            if (!step1(t + 1, kbuf1, kbuf0, vbuf0, cpos1, cpos0)) break;
        }
    }
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
    (void)Ly::ROWB;
}

template <typename T, int D>
size_t lds_bytes_t(int nb, int cstride) {
    return (size_t)Arena<T, D>::kStatic + (size_t)Arena<T, D>::bytes(nb, cstride);
}

template <typename T, int D, bool EXACT, bool SPLIT = false>
hipError_t launch_t(const Params& p, hipStream_t s) {
    const int items = p.sched ? p.sched_len : p.B * p.Hq * p.nruns;
    const size_t dyn = lds_bytes_t<T, D>(p.nb, p.cstride) - Arena<T, D>::kStatic;
    if (dyn + Arena<T, D>::kStatic > kAttnMaxLds) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_kernel<T, D, EXACT, SPLIT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sparse_attn_kernel<T, D, EXACT, SPLIT>), dim3(items), dim3(kThreads), dyn, s, p);
    return hipGetLastError();
}

}  // namespace

int attn_col_stride(const AttnArgs& a) {
    bool any_vs = false;
    for (int h = 0; h < a.Hq; ++h)
        any_vs |= !a.all_dense && (a.pattern[h] == MI_VSLASH || a.pattern[h] == MI_VSLASH_EXACT);
    return any_vs ? (a.col_cap + 63) / 64 * 64 : 0;
}

size_t sparse_attn_lds_bytes(const AttnArgs& a) {
    const int nb = a.N / 64, cs = attn_col_stride(a);
    if (a.dtype == MI_BF16) return a.D == 128 ? lds_bytes_t<uint16_t, 128>(nb, cs) : lds_bytes_t<uint16_t, 64>(nb, cs);
    return a.D == 128 ? lds_bytes_t<float, 128>(nb, cs) : lds_bytes_t<float, 64>(nb, cs);
}

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
    p.nruns = (p.nb + kBlocks - 1) / kBlocks;
    p.group = a.Hq / a.Hkv;
    p.c = a.scale * kLog2e;
    p.block_count = a.block_count; p.block_idx = a.block_idx;
    p.col_count = a.col_count; p.col_idx = a.col_idx;
    p.block_cap = a.block_cap; p.col_cap = a.col_cap;
    p.cstride = attn_col_stride(a);
    p.sink = a.sink; p.local = a.local;
    p.all_dense = a.all_dense;
    p.xcd_chunk = p.group;
    p.sched = a.sched;
    p.sched_len = a.sched_len;
    bool any_exact = false;
    for (int i = 0; i < MI_MAX_HEADS; ++i) p.pattern[i] = a.pattern[i];
    for (int h = 0; h < a.Hq; ++h) any_exact |= !a.all_dense && a.pattern[h] == MI_VSLASH_EXACT;
    p.vs_bits = a.vs_bits;
    p.bits_words = a.N / 32 + 4;
    // layers whose heads are all Block-Sparse take the split schedule
    bool all_bs = !a.all_dense;
    for (int h = 0; h < a.Hq; ++h) all_bs &= !a.all_dense && a.pattern[h] == MI_BSPARSE;
    const bool split = all_bs && 4 * a.block_cap <= p.nb;
    if (a.dtype == MI_BF16) {
        if (split) return a.D == 128 ? launch_t<uint16_t, 128, false, true>(p, s) : launch_t<uint16_t, 64, false, true>(p, s);
        if (any_exact) return a.D == 128 ? launch_t<uint16_t, 128, true>(p, s) : launch_t<uint16_t, 64, true>(p, s);
        return a.D == 128 ? launch_t<uint16_t, 128, false>(p, s) : launch_t<uint16_t, 64, false>(p, s);
    }
    if (split) return a.D == 128 ? launch_t<float, 128, false, true>(p, s) : launch_t<float, 64, false, true>(p, s);
    if (any_exact) return a.D == 128 ? launch_t<float, 128, true>(p, s) : launch_t<float, 64, true>(p, s);
    return a.D == 128 ? launch_t<float, 128, false>(p, s) : launch_t<float, 64, false>(p, s);
}

}  // namespace mi
