// Scratch layout and keys of the Vertical-Slash top-k, shared by the score
// kernels (which build the first radix histogram while they hold the scores)
// and the top-k kernels.
//
// Selection is by (key desc, index asc), key = order_key(score), the first
// `forced` indices of a row keyed above every score.  The 32-bit key is
// resolved in three digits: bits 31..22 (1024 bins), 21..11 and 10..0 (2048
// bins each).
//
// Per score row (row = 2 (b n_heads + list position) + which, which 0 for the
// vertical row and 1 for the slash row), in uint32 words:
//   [0, 1024)        histogram of digit 1, filled by the score kernels
//   [1024, 3072)     histogram of digit 2
//   [3072, 5120)     histogram of digit 3
//   [5120, 5128)     state: (prefix, rank left) after digit 1 and digit 2
//   [5128, ...)      per wavefront slice of the row (segment-major): keys
//                    above the 22-bit prefix of the k-th key, keys sharing
//                    that prefix, and the digit-3 values of the first four of
//                    those (16 bits each, index order)
// Everything but the slice records accumulates and is cleared before the
// score kernels run.
#pragma once
#include "mi_select.h"

namespace mi {

constexpr int kTopkH1 = 1024;
constexpr int kTopkH2 = 2048;
constexpr int kTopkH3 = 2048;
constexpr int kTopkOffH2 = kTopkH1;
constexpr int kTopkOffH3 = kTopkOffH2 + kTopkH2;
constexpr int kTopkOffState = kTopkOffH3 + kTopkH3;
constexpr int kTopkOffSlices = kTopkOffState + 8;
constexpr int kTopkMaxSeg = 64;   // segments per row
constexpr int kTopkNW = 4;        // wavefront slices per segment
constexpr int kTopkSliceWords = 4;
constexpr int kTopkSliceList = 4;  // digit-3 values kept per slice
constexpr int kTopkRowWords = kTopkOffSlices + kTopkSliceWords * kTopkMaxSeg * kTopkNW;
constexpr int kTopkClearWords = kTopkOffSlices;  // words that must start at zero

__device__ __forceinline__ uint32_t topk_key(float score, int i, int forced) {
    return i < forced ? kForcedKey : order_key(score);
}

__device__ __forceinline__ uint32_t topk_digit1(uint32_t key) { return key >> 22; }

}  // namespace mi
