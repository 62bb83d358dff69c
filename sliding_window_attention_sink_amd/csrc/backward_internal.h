// Private declarations of the backward kernels, shared with the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

// Backward (bf16 inputs, fp32 gradients).  Row (b, h, t) of q/o/dout and
// lse2/dd is (b * Hq + h) * L + t; key (b, kvh, i) of k/v/dk/dv is
// (b * Hkv + kvh) * L + i.
struct BackwardArgs {
    const void* q;      // [B, Hq, L, d] bf16
    const void* k;      // [B, Hkv, L, d] bf16
    const void* v;
    const void* o;      // forward output [B, Hq, L, d] bf16
    const void* dout;   // upstream gradient [B, Hq, L, d] bf16
    float* dq;          // [B, Hq, L, d]
    float* dk;          // [B, Hkv, L, d]
    float* dv;
    float* lse2;        // workspace [B, Hq, L] (+ padding): log2-sum-exp of each row's scaled scores
    float* dd;          // workspace [B, Hq, L] (+ padding): dout . o of each row
    float* part;        // workspace: partial dK, dV of key-tile segments 1 ..
    int64_t L;
    int32_t B, Hq, Hkv, s, r;
    float scale;
    float scale_log2e;
};

// Work items of the dK/dV kernel: per (batch, kv-head) and key tile of 128
// keys, segments of segb query blocks (32 rows, every q-head of the group).
// Tiles 0 .. tiles_sink-1 hold sink keys (queries to the end of the
// sequence, nseg_sink segments at most); the others nseg_band at most.
// Segments after the first write partial sums to `part`, 2 * 128 * d
// floats per slot: slots_band slots for the band tiles, then slots_sink.
struct BwdGrid {
    int32_t bhkv, tiles, tiles_sink, segb, nseg_band, nseg_sink;
    int64_t slots_band, slots_sink;
};

// Rows of padding after each of lse2 and dd (a query block reads 32 rows).
constexpr int kBwdStatPad = 64;
// Query-block iterations (blocks x q-heads) per dK/dV work item.
constexpr int kBwdSegIters = 256;

// Work-item layout for these shapes (host side).
inline BwdGrid bwd_grid(int B, int Hq, int Hkv, int s, int r, int64_t L) {
    BwdGrid g{};
    const int G = Hq / Hkv;
    g.bhkv = B * Hkv;
    g.tiles = (int)((L + 127) / 128);
    const int ts = (int)(((int64_t)s + 127) / 128);
    g.tiles_sink = ts < g.tiles ? ts : g.tiles;
    g.segb = kBwdSegIters / G > 0 ? kBwdSegIters / G : 1;
    // a full band tile's query blocks: keys i0 .. i0+127 are seen by queries
    // up to i0 + 127 + r - 1
    const int64_t band_blocks = (126 + (int64_t)r) / 32 + 1;
    const int64_t lb = (L - 1) / 32 + 1;
    const int64_t bb = band_blocks < lb ? band_blocks : lb;
    g.nseg_band = (int)((bb + g.segb - 1) / g.segb);
    g.nseg_sink = (int)((lb + g.segb - 1) / g.segb);
    g.slots_band = (int64_t)g.bhkv * (g.tiles - g.tiles_sink) * (g.nseg_band - 1);
    g.slots_sink = (int64_t)g.bhkv * g.tiles_sink * (g.nseg_sink - 1);
    return g;
}

hipError_t launch_backward_bf16(const BackwardArgs& a, const BwdGrid& gr, int d, hipStream_t st);

}  // namespace swa
