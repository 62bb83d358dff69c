// Dilated sliding window: layout passes around the banded prefill, gfx950.
//
// With a dilation delta the window of query t is t, t - delta, ..., t -
// (r-1) delta (the glossary entry on dilated SWA and the Longformer section
// of the t6page page "滑窗与固定稀疏": attended positions skip delta-1
// tokens, as many keys, a delta times wider reach), next to the s sinks.
// Every window key of t has t's residue mod delta, so the positions of one
// residue class c form an ordinary sliding-window problem: the sequence
//     sinks 0 .. s'-1, then the positions p >= s' with p = c (mod delta)
// (s' = min(s, L)) run through the plain banded prefill gives every row of
// class c its dilated key set, and the sink rows their own (keys 0 .. t).
// The gather pass builds these delta sequences as extra batch entries
// ([B * delta, H, Lc, d], padded with zero rows to one length Lc); the
// scatter pass writes each output row back to its position, the sink rows
// from class p mod delta.  The work of the attention itself is that of the
// undilated window.
#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// first position >= s1 of residue class c
__device__ __forceinline__ int64_t class_first(int64_t c, int64_t s1, int64_t dil) {
    return s1 + ((c - s1) % dil + dil) % dil;
}

__global__ __launch_bounds__(256) void dilate_gather_kernel(DilateArgs a, const void* src, void* dst, int32_t H) {
    const int64_t chunks = (int64_t)a.row_bytes / 16;
    const int64_t total = (int64_t)a.B * a.dil * H * a.Lc * chunks;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ch = x % chunks;
        int64_t rest = x / chunks;
        const int64_t i = rest % a.Lc;
        rest /= a.Lc;
        const int64_t h = rest % H;
        rest /= H;
        const int64_t c = rest % a.dil, b = rest / a.dil;
        const int64_t p = i < a.s1 ? i : class_first(c, a.s1, a.dil) + a.dil * (i - a.s1);
        u32x4 val = {0, 0, 0, 0};
        if (p < a.L) val = ((const u32x4*)((const char*)src + ((b * H + h) * a.L + p) * a.row_bytes))[ch];
        ((u32x4*)((char*)dst + x / chunks * a.row_bytes))[ch] = val;
    }
}

__global__ __launch_bounds__(256) void dilate_scatter_kernel(DilateArgs a, const void* src, void* dst, int32_t H) {
    const int64_t chunks = (int64_t)a.row_bytes / 16;
    const int64_t total = (int64_t)a.B * H * a.L * chunks;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ch = x % chunks;
        int64_t rest = x / chunks;
        const int64_t p = rest % a.L;
        rest /= a.L;
        const int64_t h = rest % H, b = rest / H;
        const int64_t c = p % a.dil;
        const int64_t i = p < a.s1 ? p : a.s1 + (p - class_first(c, a.s1, a.dil)) / a.dil;
        const int64_t row = ((b * a.dil + c) * H + h) * a.Lc + i;
        ((u32x4*)((char*)dst + x / chunks * a.row_bytes))[ch] =
            ((const u32x4*)((const char*)src + row * a.row_bytes))[ch];
    }
}

unsigned grid_for(int64_t total) {
    int64_t blocks = (total + 255) / 256;
    return (unsigned)(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192);
}

}  // namespace

hipError_t launch_dilate_gather(const DilateArgs& a, const void* src, void* dst, int32_t H, hipStream_t st) {
    const int64_t total = (int64_t)a.B * a.dil * H * a.Lc * (a.row_bytes / 16);
    hipLaunchKernelGGL(dilate_gather_kernel, dim3(grid_for(total)), dim3(256), 0, st, a, src, dst, H);
    return hipGetLastError();
}

hipError_t launch_dilate_scatter(const DilateArgs& a, const void* src, void* dst, int32_t H, hipStream_t st) {
    const int64_t total = (int64_t)a.B * H * a.L * (a.row_bytes / 16);
    hipLaunchKernelGGL(dilate_scatter_kernel, dim3(grid_for(total)), dim3(256), 0, st, a, src, dst, H);
    return hipGetLastError();
}

}  // namespace swa
