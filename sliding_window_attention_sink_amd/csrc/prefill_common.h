// Device helpers shared by the prefill kernels (gfx950).
#pragma once

#include "swa_internal.h"

namespace swa {
namespace pf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 64;               // key positions per LDS tile
constexpr int WROWS = 32;            // query rows per wave
constexpr float RESCALE_TH = 8.0f;   // log2 units: raise the running max only past 2^8
constexpr int NO_BAND = 0x7fffffff;

// MFMA row rho of a 32-key block holds key swap23(rho) (bits 2 and 3 swapped).
// With that order the 32x32 accumulator element i of lane group g holds key
// 16*(i/8) + 8*g + (i%8): eight consecutive keys per PV k-step.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
__device__ __forceinline__ constexpr int keyoff(int i, int g) { return 16 * (i / 8) + 8 * g + (i % 8); }

// A range of key tiles visited with one mask rule:
//   key i is valid for row t iff i <= t and (i < sink_hi or i >= max(band_lo, t - r + 1)).
struct Phase {
    int first, last;     // tile indices, inclusive
    int sink_hi;         // keys < sink_hi are sinks
    int band_lo;         // band keys are >= max(band_lo, t - r + 1)
    int use_qs;          // read the sink queries
};

// The phases of a block of query rows at positions t0..t1: the sink block
// (keys < s, visited once) and the band (keys >= max(s, t - r + 1)); they
// merge into one phase with the single rule "i < s or i >= t - r + 1" when
// they touch and the same queries serve both (no RoPE).
__device__ __forceinline__ int make_phases(int t0, int t1, int s, int r, bool merge, Phase& ph0, Phase& ph1) {
    const int sink_end = s < t1 + 1 ? s : t1 + 1;
    const int band_lo = s > t0 - r + 1 ? s : t0 - r + 1;
    const bool has_sink = sink_end > 0, has_band = band_lo <= t1;
    const int st_last = has_sink ? (sink_end - 1) / BN : -1;
    const int bt_first = band_lo / BN, bt_last = t1 / BN;
    const Phase sink_ph = {0, st_last, s, NO_BAND, 1};
    const Phase band_ph = {bt_first, bt_last, 0, s, 0};
    if (merge && has_sink && has_band && bt_first <= st_last + 1) {
        ph0 = Phase{0, bt_last, s, s, 0};
        return 1;
    }
    if (has_sink) {
        ph0 = sink_ph;
        ph1 = band_ph;
        return has_band ? 2 : 1;
    }
    if (has_band) {
        ph0 = band_ph;
        return 1;
    }
    return 0;
}

// Maps blockIdx to a work item so that each XCD (blocks are dealt to the 8
// XCDs round-robin) gets one contiguous run of work items: neighbouring query
// tiles of a head, which read overlapping key tiles, then share that XCD's L2.
__device__ __forceinline__ int xcd_work_item(int bid, int nblk) {
    const int x = bid & 7, k = bid >> 3;
    const int per = nblk >> 3, rem = nblk & 7;
    return x * per + (x < rem ? x : rem) + k;
}

__device__ __forceinline__ float max_pair_lanes(float x) {
    // max of lanes l and l^32 (v_permlane32_swap hands each lane both halves)
    const uint32_t xb = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
    const uint32_t lo = sw[0], hi = sw[1];
    return fmaxf(x, fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi)));
}

}  // namespace pf
}  // namespace swa
