// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, the two MFMA shapes used, cross-lane reductions and the
// XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;   // token block (query block and key block) size
constexpr int kWave = 64;    // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct bf16_t { uint16_t bits; };  // storage type of bf16 tensors

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 32x32 MFMA over a 16-deep slice of the contraction dimension.
//
// Lane l supplies 8 consecutive contraction elements: A row (l % 32),
// B column (l % 32), contraction slots 8*(l/32) .. 8*(l/32)+7.  The result
// block is 32x32 fp32: lane l holds column (l % 32) and rows
// 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15.
//   bf16: one v_mfma_f32_32x32x16_bf16.
//   fp32: eight v_mfma_f32_32x32x2_f32, the e-th taking element e of each
//         lane's 8-vector (slot 8*(l/32)+e); the slot order is immaterial to
//         the contraction as long as A and B agree, which they do.
// ---------------------------------------------------------------------------
struct Frag8bf { bf16x8 v; };
struct Frag8f { f32x8 v; };

__device__ __forceinline__ void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_shfl(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}

// Exchange with the lane 32 positions away (rows l and l^32 of the MFMA
// result hold the same column).
__device__ __forceinline__ float swap32(float x) { return __shfl_xor(x, 32, 64); }

// ---------------------------------------------------------------------------
// XCD-aware remap.  Workgroups are dispatched round-robin over the 8 XCDs of
// the chip (workgroup w -> XCD w % 8).  Remapping so that logical work items
// k, k+1, ... land on the same XCD lets neighbouring items share that XCD's L2.
// The first 8*floor(G/8) workgroups are permuted among themselves; the tail
// keeps its ids.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int pid, int grid) {
    const int per = grid >> 3;
    if (pid >= (per << 3)) return pid;
    return (pid & 7) * per + (pid >> 3);
}

// ---------------------------------------------------------------------------
// Element traits and MFMA operand loaders shared by the kernels.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kSize = 4;
    static constexpr int kKPad = 4;   // K row pad (elements)
    static constexpr int kVPad = 4;   // V^T row pad (elements)
    typedef f32x8 frag;
};
template <> struct Elem<uint16_t> {
    static constexpr int kSize = 2;
    static constexpr int kKPad = 8;
    static constexpr int kVPad = 8;
    typedef bf16x8 frag;
};

__device__ __forceinline__ int chunked_xcd_remap(int w, int grid, int chunk) {
    const int span = 8 * chunk;
    const int full = (grid / span) * span;
    if (w >= full) return w;
    const int t = w >> 3, x = w & 7;
    return (t / chunk) * span + x * chunk + (t % chunk);
}

// As chunked_xcd_remap, but the chunk an XCD takes from a span rotates every
// 8 spans: span s gives XCD x its chunk (x - s/8) mod 8.  Chunks of a span
// that differ in work (query heads of different patterns) then spread over
// all XCDs, while runs of 8 spans keep a chunk on one XCD (its L2).
__device__ __forceinline__ int rotated_xcd_remap(int w, int grid, int chunk) {
    const int span = 8 * chunk;
    const int full = (grid / span) * span;
    if (w >= full) return w;
    const int t = w >> 3, x = w & 7;
    const int s = t / chunk;
    const int c = (x - (s >> 3)) & 7;
    return s * span + c * chunk + (t % chunk);
}

// Load 8 consecutive elements (16 or 32 bytes) as an MFMA operand fragment.
__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f32x8 load_frag(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// Two 4-element runs (keys base+4h.., base+8+4h..) of a V^T row.
__device__ __forceinline__ bf16x8 load_vt_frag(const uint16_t* p) {
    u32x2 a = *reinterpret_cast<const u32x2*>(p);
    u32x2 b = *reinterpret_cast<const u32x2*>(p + 8);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}
__device__ __forceinline__ f32x8 load_vt_frag(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 8);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// P fragment for the P.V product from 8 fp32 probabilities.
__device__ __forceinline__ bf16x8 make_p_frag(const f32x16& s, int base, bf16x8*) {
    u32x4 u;
    u[0] = pack_bf16x2(s[base + 0], s[base + 1]);
    u[1] = pack_bf16x2(s[base + 2], s[base + 3]);
    u[2] = pack_bf16x2(s[base + 4], s[base + 5]);
    u[3] = pack_bf16x2(s[base + 6], s[base + 7]);
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x8 make_p_frag(const f32x16& s, int base, f32x8*) {
    return f32x8{s[base + 0], s[base + 1], s[base + 2], s[base + 3],
                 s[base + 4], s[base + 5], s[base + 6], s[base + 7]};
}

}  // namespace mi
