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
    float* lse2;        // workspace [B, Hq, L]: log2-sum-exp of each row's scaled scores (log2 units)
    float* dd;          // workspace [B, Hq, L]: dout . o of each row
    int64_t L;
    int32_t B, Hq, Hkv, s, r;
    float scale;
    float scale_log2e;
};

// Queries per work item of the sink keys' backward beyond their first r.
constexpr int kSinkSeg = 1024;

hipError_t launch_backward_bf16(const BackwardArgs& a, int d, hipStream_t st);

}  // namespace swa
