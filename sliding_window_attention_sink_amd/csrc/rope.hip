// Keys rotated once, at their token's absolute position, gfx950.
//
// StreamingLLM keeps the cache's keys and, for every query, places the keys
// of U(t) at consecutive positions 0 .. |U(t)|-1 with the query at
// |U(t)|-1 (the paragraph after eq:attn-fixed-streaming on the t6page page
// "滑窗与固定稀疏").  Rotary scores depend only on the difference of the two
// positions, so with U(t) in temporal order a window key i >= s sits
// t - i before the query (its true distance) and sink j sits
// min(t, s+r-1) - j before it.  Both hold with every key rotated at its own
// absolute position (window key i at i, sink j at j) and the query rotated
// at t for window keys and at min(t, s+r-1) for sinks.  A key's rotation
// therefore never changes: swa_rope_keys applies it once, when the key
// enters the library, and the attention kernels rotate only the queries.
//
// A thread rotates one 16-byte chunk of a row's first half together with
// its partner chunk d/2 further (dims j and j + d/2 form a rotation pair).
#include "rope_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void rope_keys_kernel(RopeKeysArgs a, int64_t total) {
    constexpr int HC = D / 16;     // chunk pairs per row
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = idx / HC;              // (b * Hkv + h) * n + i
        const int c = (int)(idx - row * HC);
        const int64_t p = a.pos0 + row % a.n;
        // each source row is read once: non-temporal
        const __bf16* src = (const __bf16*)a.k + (size_t)row * D;
        u32x4 lo = __builtin_nontemporal_load((const u32x4*)(src + 8 * c));
        u32x4 hi = __builtin_nontemporal_load((const u32x4*)(src + 8 * c + D / 2));
        rope::rot_chunk_pair(lo, hi, 8 * c, (double)p, a.rope_rr);
        __bf16* dst = (__bf16*)a.kr + (size_t)row * D;
        *(u32x4*)(dst + 8 * c) = lo;
        *(u32x4*)(dst + 8 * c + D / 2) = hi;
    }
}

}  // namespace

hipError_t launch_rope_keys_bf16(const RopeKeysArgs& a, int d, hipStream_t st) {
    const int64_t total = a.rows * (d / 16);
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (d == 128) {
        hipLaunchKernelGGL(rope_keys_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, st, a, total);
    } else if (d == 64) {
        hipLaunchKernelGGL(rope_keys_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, st, a, total);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace swa
