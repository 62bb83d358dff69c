// Private declarations shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

// Query rows per workgroup of the fp32 prefill kernel (4 waves x 32 rows).
constexpr int kPrefillF32RowsPerBlock = 128;

// Plain-old-data arguments of the prefill kernel.  Positions: query row i of
// the call is token pos0 + i.  Key position p lives at
//   kc/vc + slot(p) * d   if p < pos0   (rolling cache: slot p if p < s, else s + p mod r)
//   kn/vn + (p - pos0) * d otherwise (the call's own tokens)
// per (b, kv-head); q/o per (b, q-head) hold L rows.
struct PrefillArgs {
    const void* q;      // queries (before rotation with RoPE)
    const void* kn;
    const void* vn;
    const void* kc;
    const void* vc;
    void* o;
    int64_t L;          // own rows per (b, head); with dil > 1 see Lp
    int64_t pos0;
    // Element strides: own row i of (b, head) sits at (b H + head) q_bh +
    // i rs in q and o, and at (b Hkv + kvh) kv_bh + i rs in kn and vn;
    // cache slot j at (b Hkv + kvh) c_bh + j d.  Dense calls: rs = d,
    // q_bh = kv_bh = L d, c_bh = (s + r) d.
    int64_t rs, q_bh, kv_bh, c_bh;
    // Residue classes (dil > 1; with pos0 <= s and rs = dil d): the grid's
    // batch index is b dil + c, and the own rows of class c are the
    // positions first(c), first(c) + dil, ... below Lp, with first(c) the
    // first position >= pos0 that is c mod dil (row i at element offset
    // first(c) d + i rs).  Cache slots 0 .. pos0-1 hold the sinks.
    int32_t dil;
    int64_t Lp;
    int32_t B, Hq, Hkv, s, r;
    int32_t n_mtiles;   // query tiles per (b, q-head)
    int32_t merge_sink; // 1: sinks may share tiles with the band (same queries for both)
    int32_t pair_mode;  // bf16 kernel: workgroup = two q-heads of one kv-head (else 256 rows of one head)
    float scale_log2e;  // scale * log2(e)
    // RoPE (rope_rr > 0): every key, own and cached, comes rotated at its
    // token's position; the kernel rotates the queries, at t for window keys
    // and at min(t, s+r-1) for sinks.  rope_rr = base^(-2/d).
    double rope_rr;
    // Task-bound global tokens (ng > 0; bf16 kernel, no RoPE; kc / vc then
    // point at the [B Hkv, 64, d] blocks, c_bh = 64 d, pos0 = 0): the keys
    // and values of the global positions g >= s, in order, form one more key
    // tile after the band, and row t keeps rows 0 .. gjb[t]-1 of it, the
    // globals below its window (gjb[t] = #{g : s <= g < t - r + 1}; the
    // globals below s are sinks already, those from t - r + 1 on are in the
    // window or in the future).
    const uint8_t* gjb;   // [L]
    int32_t ng;
    // Fused append (kc_next set; bf16 kernel, dense call, L >= r): the cache
    // after this call, written to a second cache: the own rows that survive
    // (positions >= pos0 + L - r, and those below s) at their slots, the
    // sink slots below pos0 copied from kc / vc.  Every rolling slot is
    // rewritten (L >= r), so nothing of kc_next is read.
    void* kc_next;
    void* vc_next;
};

struct AppendArgs {
    const void* kn;     // [B, Hkv, n, d]
    const void* vn;
    void* kc;           // [B, Hkv, s + r, d]
    void* vc;
    int64_t n;
    int64_t pos0;
    int64_t first;      // first token of the call that survives (tokens before it are superseded)
    int32_t B, Hkv, s, r, d;
    int32_t elem_bytes;
};

struct DecodeArgs {
    const void* q;      // [B, Hq, d]
    const void* kc;     // [B, Hkv, s + r, d]
    const void* vc;
    void* o;            // [B, Hq, d]
    float* ws;          // [B, Hq, n_split, d + 2]: m (log2 units), l, o[d]
    const void* kn;     // null, or token T-1's K [B, Hkv, d], written to slot j_new first
    const void* vn;     // same for V
    int64_t T;          // tokens in the cache including the current one
    int32_t j_new;      // cache slot of token T-1 with kn/vn, else -1
    double rope_rr;     // RoPE: base^(-2/d) (cache keys stored rotated at their position); 0 = no RoPE
    int64_t qo_stride;  // elements between the (batch, q-head) rows of q and of o (d for [B, Hq, d])
    int32_t B, Hq, Hkv, s, r;
    int32_t n_split;
    int32_t slots_per_split;
    float scale_log2e;
    // npos > 0: the query rows of npos positions at once (G * npos <= 16, no
    // RoPE): row (b, h, pos[pi]) of q and o sits at (b Hq + h) qo_stride +
    // pos[pi] d and sees keys (slots) 0 .. pos[pi]; pos ascending, T =
    // pos[npos-1] + 1; ws is [B, Hq, npos, n_split, d + 2]
    int32_t npos;
    int32_t pos[16];
};

// Rows [rows, d] of keys for positions pos0 + (row mod n) (the rows of
// each (batch, kv-head) hold tokens pos0 .. pos0+n-1), rotated into kr.
struct RopeKeysArgs {
    const void* k;
    void* kr;
    int64_t rows, n, pos0;
    double rope_rr;     // base^(-2/d)
};

// Task-bound global tokens (swa_prefill_global): at most kMaxGlobals sorted
// positions, passed by value.
constexpr int kMaxGlobals = 64;
struct GlobalArgs {
    const void* k;      // [B, Hkv, L, d]
    const void* v;
    void* kg;           // workspace [B * Hkv, kMaxGlobals, d]: keys of the global positions
    void* vg;           // ... values
    uint8_t* gjb;       // workspace [L]: gjb[t] = #{j : pos[j] < t - r + 1}
    int64_t L;
    int32_t B, Hkv, r, ng;   // pos[0 .. ng-1]: the global positions >= s, ascending
    int32_t pos[kMaxGlobals];
};
hipError_t launch_global_gather_bf16(const GlobalArgs& a, int d, hipStream_t st);

// Query rows per workgroup of the bf16 prefill kernel for this head layout.
int prefill_bf16_rows_per_block(int Hq, int Hkv);

// Launchers (return hipError_t of the launch).  `d` selects the instantiation.
hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, hipStream_t st);
hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, hipStream_t st);
hipError_t launch_decode_bf16(const DecodeArgs& a, int d, hipStream_t st);

// Bytes of the static device scratch behind swa_decode_step_noalloc, and
// its address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t decode_noalloc_scratch(void** out);
hipError_t launch_rope_keys_bf16(const RopeKeysArgs& a, int d, hipStream_t st);

}  // namespace swa
