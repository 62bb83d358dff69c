// C ABI of the gfx950 sliding-window attention library (see include/swa.h).
// Validates every argument on the host before any HIP call, then enqueues the
// kernels on the caller's stream.  Never allocates, frees or synchronises.
#include "swa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "swa_internal.h"
#include "backward_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = '\0'; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int64_t kMaxPos = (int64_t)1 << 30;    // positions and slot counts stay in int32 arithmetic
constexpr int32_t kMaxDilation = 65536;         // a 64-row tile of one residue class spans < 2^31 bytes

// Shared descriptor checks; `need_bf16` for entry points built for bf16 only.
int check_desc(const swa_desc* d, const char* fn) {
    if (!d) return fail(SWA_ERR_INVALID_ARG, "%s: desc is NULL", fn);
    if (d->B < 1 || d->Hq < 1 || d->Hkv < 1)
        return fail(SWA_ERR_INVALID_ARG, "%s: B, Hq, Hkv must be >= 1 (got %d, %d, %d)", fn, d->B, d->Hq, d->Hkv);
    if (d->Hq % d->Hkv)
        return fail(SWA_ERR_INVALID_ARG, "%s: Hq (%d) must be a multiple of Hkv (%d)", fn, d->Hq, d->Hkv);
    if (d->s < 0) return fail(SWA_ERR_INVALID_ARG, "%s: s must be >= 0 (got %d)", fn, d->s);
    if (d->r < 1) return fail(SWA_ERR_INVALID_ARG, "%s: r must be >= 1 (got %d)", fn, d->r);
    if ((int64_t)d->s + d->r > kMaxPos)
        return fail(SWA_ERR_INVALID_ARG, "%s: s + r too large (%lld)", fn, (long long)d->s + d->r);
    if (!(d->scale > 0.0f) || !std::isfinite(d->scale))
        return fail(SWA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
    if (!(d->rope_base >= 0.0f) || !std::isfinite(d->rope_base))
        return fail(SWA_ERR_INVALID_ARG, "%s: rope_base must be finite and >= 0", fn);
    if (d->dtype != SWA_F32 && d->dtype != SWA_BF16)
        return fail(SWA_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, d->dtype);
    if (d->d != 64 && d->d != 128) return fail(SWA_ERR_UNSUPPORTED, "%s: head dim %d not built (64, 128)", fn, d->d);
    if (d->rope_base > 0.0f && d->dtype != SWA_BF16)
        return fail(SWA_ERR_UNSUPPORTED, "%s: RoPE is built for bf16 only", fn);
    return SWA_OK;
}

int check_ptr(const void* p, const char* fn, const char* name) {
    if (!p) return fail(SWA_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
    if (!aligned16(p)) return fail(SWA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);
    return SWA_OK;
}

int hip_status(hipError_t e, const char* fn) {
    if (e == hipSuccess) return SWA_OK;
    return fail(SWA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
}

size_t elem_bytes(const swa_desc* d) { return d->dtype == SWA_BF16 ? 2 : 4; }

// Rotation frequencies theta_j = base^(-2j/d) = rope_rr(desc)^j.
double rope_rr(const swa_desc* d) { return std::pow((double)d->rope_base, -2.0 / (double)d->d); }

// Splits per (batch, kv-head) unit: enough workgroups for two per compute
// unit (512 on 256 CUs), each over at least 256 slots; one split when the
// units alone fill the chip (the split kernel then writes the output).
int32_t default_splits(const swa_desc* d) {
    const int64_t S = (int64_t)d->s + d->r;
    const int64_t units = (int64_t)d->B * d->Hkv;
    int64_t n = (512 + units - 1) / units;
    int64_t cap = S / 256;
    if (cap < 1) cap = 1;
    if (n > cap) n = cap;
    if (n > 64) n = 64;
    if (n < 1) n = 1;
    return (int32_t)n;
}

// Backward workspace: per-row log-sum-exp and D (each padded by a query
// block's rows), then the partial dK/dV slots of split key tiles.
struct BackwardLayout {
    swa::BwdGrid grid{};
    size_t lse2 = 0, dd = 0, part = 0, total = 0;
};

BackwardLayout backward_layout(const swa_desc* d, int64_t L) {
    BackwardLayout x;
    x.grid = swa::bwd_grid(d->B, d->Hq, d->Hkv, d->s, d->r, L);
    const size_t rows = (size_t)d->B * d->Hq * (size_t)L + swa::kBwdStatPad;
    x.lse2 = 0;
    x.dd = round_up(rows * sizeof(float), 256);
    x.part = x.dd + round_up(rows * sizeof(float), 256);
    const size_t slots = (size_t)(x.grid.slots_band + x.grid.slots_sink);
    x.total = x.part + round_up(slots * 2 * 128 * (size_t)d->d * sizeof(float), 256);
    return x;
}

// Per-split partial results (max, sum, unnormalised O) per query head; one
// split writes the output directly and needs none.
size_t decode_ws_bytes(const swa_desc* desc, int32_t n_split) {
    if (n_split == 1) return 0;
    return (size_t)desc->B * desc->Hq * n_split * (desc->d + 2) * sizeof(float);
}

}  // namespace

extern "C" {

int swa_abi_version(void) { return SWA_ABI_VERSION; }

const char* swa_last_error(void) { return g_last_error; }

const char* swa_status_str(int status) {
    switch (status) {
        case SWA_OK: return "ok";
        case SWA_ERR_INVALID_ARG: return "invalid argument";
        case SWA_ERR_UNSUPPORTED: return "unsupported configuration";
        case SWA_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

size_t swa_prefill_workspace_bytes(const swa_desc* desc, int64_t L) {
    if (check_desc(desc, "swa_prefill_workspace_bytes") != SWA_OK || L < 1) return 0;
    return 0;
}

}  // extern "C"

namespace {

// Query tiles per (batch, q-head) for L rows
int64_t prefill_mtiles(const swa_desc* desc, int64_t L) {
    const int64_t rows_per_block = desc->dtype == SWA_BF16 ? swa::prefill_bf16_rows_per_block(desc->Hq, desc->Hkv)
                                                           : swa::kPrefillF32RowsPerBlock;
    return (L + rows_per_block - 1) / rows_per_block;
}

// Kernel arguments of a call on dense [B, H, L, d] tensors (and a cache of
// s + r slots per (batch, kv-head), or none)
swa::PrefillArgs dense_prefill_args(const swa_desc* desc, const void* q, const void* k, const void* v, void* o,
                                    int64_t L, const void* k_cache, const void* v_cache, int64_t pos0) {
    swa::PrefillArgs a{};
    a.q = q;
    a.kn = k;
    a.vn = v;
    a.kc = k_cache;
    a.vc = v_cache;
    a.o = o;
    a.L = L;
    a.pos0 = pos0;
    a.rs = desc->d;
    a.q_bh = L * desc->d;
    a.kv_bh = L * desc->d;
    a.c_bh = ((int64_t)desc->s + desc->r) * desc->d;
    a.dil = 1;
    a.Lp = L;
    a.B = desc->B;
    a.Hq = desc->Hq;
    a.Hkv = desc->Hkv;
    a.s = desc->s;
    a.r = desc->r;
    a.n_mtiles = (int32_t)prefill_mtiles(desc, L);
    a.merge_sink = 1;
    a.pair_mode = (desc->dtype == SWA_BF16 && (desc->Hq / desc->Hkv) % 2 == 0) ? 1 : 0;
    a.scale_log2e = (float)((double)desc->scale * 1.4426950408889634);
    return a;
}

hipError_t launch_prefill(const swa_desc* desc, const swa::PrefillArgs& a, hipStream_t hs) {
    return desc->dtype == SWA_BF16 ? swa::launch_prefill_bf16(a, desc->d, hs) : swa::launch_prefill_f32(a, desc->d, hs);
}

// swa_prefill
// swa_prefill, and with k_next / v_next swa_prefill_append
int prefill_impl(const char* fn, const swa_desc* desc, const void* q, const void* k, const void* v, void* o,
                 int64_t L, const void* k_cache, const void* v_cache, int64_t pos0, void* stream,
                 void* k_next = nullptr, void* v_next = nullptr, bool fused = false) {
    clear_error();
    int st = check_desc(desc, fn);
    if (st) return st;
    if ((st = check_ptr(q, fn, "q")) || (st = check_ptr(k, fn, "k")) || (st = check_ptr(v, fn, "v")) ||
        (st = check_ptr(o, fn, "o")))
        return st;
    if (L < 1) return fail(SWA_ERR_INVALID_ARG, "%s: L must be >= 1 (got %lld)", fn, (long long)L);
    if (pos0 < 0) return fail(SWA_ERR_INVALID_ARG, "%s: pos0 must be >= 0", fn);
    if (pos0 + L > kMaxPos) return fail(SWA_ERR_INVALID_ARG, "%s: positions beyond 2^30", fn);
    const bool has_cache = k_cache || v_cache;
    if (has_cache) {
        if ((st = check_ptr(k_cache, fn, "k_cache")) || (st = check_ptr(v_cache, fn, "v_cache"))) return st;
    } else if (pos0 != 0) {
        return fail(SWA_ERR_INVALID_ARG, "%s: pos0 > 0 needs the rolling cache", fn);
    }
    const bool rope = desc->rope_base > 0.0f;
    if ((int64_t)desc->B * desc->Hq * prefill_mtiles(desc, L) > 0x7fffffffLL)
        return fail(SWA_ERR_INVALID_ARG, "%s: grid too large", fn);
    if (fused) {
        if (desc->dtype != SWA_BF16) return fail(SWA_ERR_UNSUPPORTED, "%s: the fused append is built for bf16", fn);
        if ((st = check_ptr(k_next, fn, "k_next")) || (st = check_ptr(v_next, fn, "v_next"))) return st;
        if (k_next == k_cache || v_next == v_cache || k_next == v_next || k_next == v_cache || v_next == k_cache)
            return fail(SWA_ERR_INVALID_ARG, "%s: the next cache must be another buffer pair", fn);
        // every rolling slot that holds a token afterwards comes from the chunk
        if (L < desc->r && pos0 > desc->s)
            return fail(SWA_ERR_INVALID_ARG, "%s: needs L >= r or pos0 <= s (L %lld, r %d, pos0 %lld, s %d)", fn,
                        (long long)L, desc->r, (long long)pos0, desc->s);
    }

    swa::PrefillArgs a = dense_prefill_args(desc, q, k, v, o, L, has_cache ? k_cache : nullptr,
                                            has_cache ? v_cache : nullptr, pos0);
    a.kc_next = k_next;
    a.vc_next = v_next;
    if (rope) {
        // the keys (own and cached) come rotated; the kernel turns the queries
        a.merge_sink = 0;
        a.rope_rr = rope_rr(desc);
    }
    return hip_status(launch_prefill(desc, a, reinterpret_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

int swa_prefill(const swa_desc* desc, const void* q, const void* k, const void* v, void* o, int64_t L,
                const void* k_cache, const void* v_cache, int64_t pos0, void* workspace, size_t workspace_bytes,
                void* stream) {
    (void)workspace;         // no prefill kernel uses one (swa_prefill_workspace_bytes is 0)
    (void)workspace_bytes;
    return prefill_impl("swa_prefill", desc, q, k, v, o, L, k_cache, v_cache, pos0, stream);
}

int swa_prefill_append(const swa_desc* desc, const void* q, const void* k, const void* v, void* o, int64_t L,
                       const void* k_cache, const void* v_cache, int64_t pos0, void* k_next, void* v_next,
                       void* stream) {
    return prefill_impl("swa_prefill_append", desc, q, k, v, o, L, k_cache, v_cache, pos0, stream, k_next, v_next,
                        true);
}

int swa_cache_append(const swa_desc* desc, const void* k_new, const void* v_new, int64_t n, int64_t pos0,
                     void* k_cache, void* v_cache, void* stream) {
    static const char* fn = "swa_cache_append";
    clear_error();
    int st = check_desc(desc, fn);
    if (st) return st;
    if ((st = check_ptr(k_new, fn, "k_new")) || (st = check_ptr(v_new, fn, "v_new")) ||
        (st = check_ptr(k_cache, fn, "k_cache")) || (st = check_ptr(v_cache, fn, "v_cache")))
        return st;
    if (n < 1) return fail(SWA_ERR_INVALID_ARG, "%s: n must be >= 1 (got %lld)", fn, (long long)n);
    if (pos0 < 0) return fail(SWA_ERR_INVALID_ARG, "%s: pos0 must be >= 0", fn);
    if (pos0 + n > kMaxPos) return fail(SWA_ERR_INVALID_ARG, "%s: positions beyond 2^30", fn);
    swa::AppendArgs a{};
    a.kn = k_new;
    a.vn = v_new;
    a.kc = k_cache;
    a.vc = v_cache;
    a.n = n;
    a.pos0 = pos0;
    int64_t first = pos0 + n - desc->r;      // recent tokens before this one are overwritten within the call
    if (first < pos0) first = pos0;
    if (first < desc->s) first = desc->s;
    if (first > pos0 + n) first = pos0 + n;
    a.first = first;
    a.B = desc->B;
    a.Hkv = desc->Hkv;
    a.s = desc->s;
    a.r = desc->r;
    a.d = desc->d;
    a.elem_bytes = (int32_t)elem_bytes(desc);
    return hip_status(swa::launch_append(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

int swa_rope_keys(const swa_desc* desc, const void* k, int64_t n, int64_t pos0, void* k_rot, void* stream) {
    static const char* fn = "swa_rope_keys";
    clear_error();
    int st = check_desc(desc, fn);
    if (st) return st;
    if (!(desc->rope_base > 0.0f)) return fail(SWA_ERR_INVALID_ARG, "%s: rope_base must be > 0", fn);
    if ((st = check_ptr(k, fn, "k")) || (st = check_ptr(k_rot, fn, "k_rot"))) return st;
    if (n < 1) return fail(SWA_ERR_INVALID_ARG, "%s: n must be >= 1 (got %lld)", fn, (long long)n);
    if (pos0 < 0) return fail(SWA_ERR_INVALID_ARG, "%s: pos0 must be >= 0", fn);
    if (pos0 + n > kMaxPos) return fail(SWA_ERR_INVALID_ARG, "%s: positions beyond 2^30", fn);
    swa::RopeKeysArgs a{};
    a.k = k;
    a.kr = k_rot;
    a.rows = (int64_t)desc->B * desc->Hkv * n;
    a.n = n;
    a.pos0 = pos0;
    a.rope_rr = rope_rr(desc);
    return hip_status(swa::launch_rope_keys_bf16(a, desc->d, reinterpret_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"

namespace {

// Workspace of swa_prefill_global: gathered global keys and values, each
// position's count of globals below its window, and the split partials of
// the dense global rows.
struct GlobalLayout {
    swa_desc dense{};
    int32_t n_split = 1;
    size_t kg = 0, vg = 0, jb = 0, part = 0, total = 0;
};

GlobalLayout global_layout(const swa_desc* d, int64_t L) {
    GlobalLayout x;
    // the rows in G attend keys 0 .. t: the decode over a "cache" of L slots
    // with L-1 sink slots and one rolling slot, which holds exactly keys
    // 0 .. T-1 for T <= L
    x.dense = *d;
    x.dense.s = (int32_t)(L - 1);
    x.dense.r = 1;
    x.n_split = default_splits(&x.dense);
    const size_t kgb = (size_t)d->B * d->Hkv * swa::kMaxGlobals * d->d * 2;
    x.kg = 0;
    x.vg = round_up(kgb, 256);
    x.jb = x.vg + round_up(kgb, 256);
    x.part = x.jb + round_up((size_t)L, 256);
    // partial results of the batched dense rows: up to 16 positions a launch
    x.total = x.part + round_up(16 * decode_ws_bytes(&x.dense, x.n_split), 256);
    return x;
}

}  // namespace

extern "C" {

size_t swa_prefill_global_workspace_bytes(const swa_desc* desc, int64_t L, int32_t ng) {
    if (check_desc(desc, "swa_prefill_global_workspace_bytes") != SWA_OK || L < 1 || L > kMaxPos) return 0;
    if (ng < 1 || ng > swa::kMaxGlobals) return 0;
    return global_layout(desc, L).total;
}

int swa_prefill_global(const swa_desc* desc, const void* q, const void* k, const void* v, void* o, int64_t L,
                       const int32_t* globals, int32_t ng, void* workspace, size_t workspace_bytes, void* stream) {
    static const char* fn = "swa_prefill_global";
    clear_error();
    int st = check_desc(desc, fn);
    if (st) return st;
    if (desc->dtype != SWA_BF16) return fail(SWA_ERR_UNSUPPORTED, "%s: global tokens are built for bf16", fn);
    if (desc->rope_base > 0.0f) return fail(SWA_ERR_UNSUPPORTED, "%s: global tokens with RoPE are not built", fn);
    if (desc->Hq / desc->Hkv > 16) return fail(SWA_ERR_UNSUPPORTED, "%s: more than 16 q-heads per kv-head", fn);
    if ((st = check_ptr(q, fn, "q")) || (st = check_ptr(k, fn, "k")) || (st = check_ptr(v, fn, "v")) ||
        (st = check_ptr(o, fn, "o")))
        return st;
    if (L < 1) return fail(SWA_ERR_INVALID_ARG, "%s: L must be >= 1 (got %lld)", fn, (long long)L);
    if (L > kMaxPos) return fail(SWA_ERR_INVALID_ARG, "%s: positions beyond 2^30", fn);
    if (ng < 0 || ng > swa::kMaxGlobals)
        return fail(SWA_ERR_INVALID_ARG, "%s: %d global tokens (0 .. %d)", fn, ng, swa::kMaxGlobals);
    if (ng > 0 && globals == nullptr) return fail(SWA_ERR_INVALID_ARG, "%s: globals is NULL", fn);
    for (int32_t j = 0; j < ng; ++j) {
        if (globals[j] < 0 || globals[j] >= L)
            return fail(SWA_ERR_INVALID_ARG, "%s: global position %d outside 0 .. L-1", fn, globals[j]);
        if (j > 0 && globals[j] <= globals[j - 1])
            return fail(SWA_ERR_INVALID_ARG, "%s: global positions must increase strictly", fn);
    }
    if (ng == 0) return swa_prefill(desc, q, k, v, o, L, nullptr, nullptr, 0, nullptr, 0, stream);
    const GlobalLayout lay = global_layout(desc, L);
    if ((st = check_ptr(workspace, fn, "workspace"))) return st;
    if (workspace_bytes < lay.total)
        return fail(SWA_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, lay.total);
    if ((int64_t)desc->B * desc->Hq * ((L + 127) / 128) > 0x7fffffffLL) return fail(SWA_ERR_INVALID_ARG, "%s: grid too large", fn);

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    // the globals at or past s, gathered into one 64-key block per (batch,
    // kv-head), with each row's count of them below its window
    swa::GlobalArgs ga{};
    ga.k = k;
    ga.v = v;
    ga.kg = ws + lay.kg;
    ga.vg = ws + lay.vg;
    ga.gjb = reinterpret_cast<uint8_t*>(ws + lay.jb);
    ga.L = L;
    ga.B = desc->B;
    ga.Hkv = desc->Hkv;
    ga.r = desc->r;
    for (int32_t j = 0; j < ng; ++j)
        if (globals[j] >= desc->s) ga.pos[ga.ng++] = globals[j];
    if ((st = hip_status(swa::launch_global_gather_bf16(ga, desc->d, hs), fn))) return st;
    // the banded rows, with those globals as one more key tile
    swa::PrefillArgs pa = dense_prefill_args(desc, q, k, v, o, L, ws + lay.kg, ws + lay.vg, 0);
    pa.c_bh = (int64_t)swa::kMaxGlobals * desc->d;
    pa.gjb = reinterpret_cast<const uint8_t*>(ws + lay.jb);
    pa.ng = ga.ng;
    if (ga.ng > 0 && (st = hip_status(launch_prefill(desc, pa, hs), fn))) return st;
    if (ga.ng == 0 && (st = prefill_impl(fn, desc, q, k, v, o, L, nullptr, nullptr, 0, stream))) return st;
    // the global rows: dense causal rows over keys 0 .. t, 16 / G positions
    // a launch as extra query columns (each K/V byte read once per launch)
    const int S = (int)L;
    int sps = (S + lay.n_split - 1) / lay.n_split;
    sps = (sps + 31) / 32 * 32;
    const int per = 16 / (desc->Hq / desc->Hkv);
    for (int32_t j0 = 0; j0 < ng; j0 += per) {
        const int np = (ng - j0) < per ? (ng - j0) : per;
        swa::DecodeArgs da{};
        da.q = q;
        da.kc = k;
        da.vc = v;
        da.o = o;
        da.ws = reinterpret_cast<float*>(ws + lay.part);
        da.kn = nullptr;
        da.vn = nullptr;
        da.T = (int64_t)globals[j0 + np - 1] + 1;
        da.j_new = -1;
        da.rope_rr = 0.0;
        da.qo_stride = L * desc->d;
        da.B = desc->B;
        da.Hq = desc->Hq;
        da.Hkv = desc->Hkv;
        da.s = lay.dense.s;
        da.r = lay.dense.r;
        da.n_split = lay.n_split;
        da.slots_per_split = sps;
        da.scale_log2e = pa.scale_log2e;
        da.npos = np;
        for (int i = 0; i < np; ++i) da.pos[i] = globals[j0 + i];
        if ((st = hip_status(swa::launch_decode_bf16(da, desc->d, hs), fn))) return st;
    }
    return SWA_OK;
}

size_t swa_prefill_dilated_workspace_bytes(const swa_desc* desc, int64_t L, int32_t dilation) {
    (void)desc;
    (void)L;
    (void)dilation;
    return 0;
}

int swa_prefill_dilated(const swa_desc* desc, int32_t dilation, const void* q, const void* k, const void* v, void* o,
                        int64_t L, void* workspace, size_t workspace_bytes, void* stream) {
    static const char* fn = "swa_prefill_dilated";
    (void)workspace;
    (void)workspace_bytes;
    clear_error();
    int st = check_desc(desc, fn);
    if (st) return st;
    if (dilation < 1) return fail(SWA_ERR_INVALID_ARG, "%s: dilation must be >= 1 (got %d)", fn, dilation);
    if (dilation > kMaxDilation)
        return fail(SWA_ERR_INVALID_ARG, "%s: dilation must be <= %d (got %d)", fn, kMaxDilation, dilation);
    if (desc->rope_base > 0.0f) return fail(SWA_ERR_UNSUPPORTED, "%s: dilation with RoPE is not built", fn);
    // with L <= s every row is a sink row (keys 0 .. t), the plain window's rows
    if (dilation == 1 || L <= desc->s)
        return prefill_impl(fn, desc, q, k, v, o, L, nullptr, nullptr, 0, stream);
    if ((st = check_ptr(q, fn, "q")) || (st = check_ptr(k, fn, "k")) || (st = check_ptr(v, fn, "v")) ||
        (st = check_ptr(o, fn, "o")))
        return st;
    if (L > kMaxPos) return fail(SWA_ERR_INVALID_ARG, "%s: positions beyond 2^30", fn);
    const int64_t s = desc->s, d = desc->d;
    const int64_t n_max = (L - s + dilation - 1) / dilation;   // rows of the longest class
    if ((int64_t)desc->B * dilation * desc->Hq * prefill_mtiles(desc, n_max) > 0x7fffffffLL)
        return fail(SWA_ERR_INVALID_ARG, "%s: grid too large", fn);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);

    // 1. the sink rows 0 .. s-1 (keys 0 .. t): the plain window on the first
    //    s rows of each (batch, head)
    if (s > 0) {
        swa::PrefillArgs a = dense_prefill_args(desc, q, k, v, o, s, nullptr, nullptr, 0);
        a.q_bh = a.kv_bh = L * d;
        if ((st = hip_status(launch_prefill(desc, a, hs), fn))) return st;
    }
    // 2. every residue class mod dilation in one launch, read and written in
    //    place: class c's rows p >= s, p = c (mod dilation), are the own rows
    //    of a call at pos0 = s with row stride dilation * d, and its sinks are
    //    the cache slots 0 .. s-1, i.e. the first s rows of K and V
    swa::PrefillArgs a = dense_prefill_args(desc, q, k, v, o, n_max, s > 0 ? k : nullptr, s > 0 ? v : nullptr, s);
    a.rs = (int64_t)dilation * d;
    a.q_bh = a.kv_bh = a.c_bh = L * d;
    a.dil = dilation;
    a.Lp = L;
    a.B = (int32_t)(desc->B * dilation);
    return hip_status(launch_prefill(desc, a, hs), fn);
}

int32_t swa_decode_default_splits(const swa_desc* desc) {
    if (check_desc(desc, "swa_decode_default_splits") != SWA_OK) return 0;
    return default_splits(desc);
}

size_t swa_decode_workspace_bytes(const swa_desc* desc, int32_t n_split) {
    if (check_desc(desc, "swa_decode_workspace_bytes") != SWA_OK) return 0;
    if (n_split == 0) n_split = default_splits(desc);
    if (n_split < 1 || n_split > 64) return 0;
    return decode_ws_bytes(desc, n_split);
}

}  // extern "C"

namespace {

// swa_decode, and with k_new/v_new swa_decode_step (append fused in).
// validate_only: check the arguments (the workspace aside) and launch nothing.
int decode_impl(const char* fn, const swa_desc* desc, const void* q, const void* k_new, const void* v_new,
                const void* k_cache, const void* v_cache, int64_t T, void* o, int32_t n_split, void* workspace,
                size_t workspace_bytes, void* stream, bool validate_only = false) {
    clear_error();
    int st = check_desc(desc, fn);
    if (st) return st;
    if (desc->dtype != SWA_BF16) return fail(SWA_ERR_UNSUPPORTED, "%s: decode is built for bf16 only", fn);
    if (desc->Hq / desc->Hkv > 16)
        return fail(SWA_ERR_UNSUPPORTED, "%s: more than 16 q-heads per kv-head", fn);
    if (desc->rope_base > 0.0f && desc->Hq / desc->Hkv > 8)
        return fail(SWA_ERR_UNSUPPORTED, "%s: RoPE decode is built for up to 8 q-heads per kv-head", fn);
    if ((st = check_ptr(q, fn, "q")) || (st = check_ptr(k_cache, fn, "k_cache")) ||
        (st = check_ptr(v_cache, fn, "v_cache")) || (st = check_ptr(o, fn, "o")))
        return st;
    const bool fused = k_new != nullptr || v_new != nullptr;
    if (fused && ((st = check_ptr(k_new, fn, "k_new")) || (st = check_ptr(v_new, fn, "v_new")))) return st;
    if (T < 1) return fail(SWA_ERR_INVALID_ARG, "%s: T must be >= 1", fn);
    if (T > kMaxPos) return fail(SWA_ERR_INVALID_ARG, "%s: T beyond 2^30", fn);
    if (n_split == 0) n_split = default_splits(desc);
    if (n_split < 1 || n_split > 64) return fail(SWA_ERR_INVALID_ARG, "%s: n_split %d outside 1..64", fn, n_split);
    if ((int64_t)desc->B * desc->Hkv * n_split > 0x7fffffffLL) return fail(SWA_ERR_INVALID_ARG, "%s: grid too large", fn);
    if (validate_only) return SWA_OK;
    const size_t need = decode_ws_bytes(desc, n_split);
    if (need > 0 && (st = check_ptr(workspace, fn, "workspace"))) return st;
    if (workspace_bytes < need)
        return fail(SWA_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);

    const int S = desc->s + desc->r;
    int sps = (S + n_split - 1) / n_split;
    sps = (sps + 31) / 32 * 32;
    swa::DecodeArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.o = o;
    a.ws = static_cast<float*>(workspace);
    a.kn = fused ? k_new : nullptr;
    a.vn = fused ? v_new : nullptr;
    a.T = T;
    a.j_new = !fused ? -1 : (T - 1 < desc->s) ? (int32_t)(T - 1) : desc->s + (int32_t)((T - 1) % desc->r);
    a.B = desc->B;
    a.Hq = desc->Hq;
    a.Hkv = desc->Hkv;
    a.s = desc->s;
    a.r = desc->r;
    a.n_split = n_split;
    a.slots_per_split = sps;
    a.scale_log2e = (float)((double)desc->scale * 1.4426950408889634);
    a.rope_rr = desc->rope_base > 0.0f ? rope_rr(desc) : 0.0;
    a.qo_stride = desc->d;
    return hip_status(swa::launch_decode_bf16(a, desc->d, reinterpret_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

int swa_decode(const swa_desc* desc, const void* q, const void* k_cache, const void* v_cache, int64_t T, void* o,
               int32_t n_split, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl("swa_decode", desc, q, nullptr, nullptr, k_cache, v_cache, T, o, n_split, workspace,
                       workspace_bytes, stream);
}

int swa_decode_step(const swa_desc* desc, const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, int64_t T, void* o, int32_t n_split, void* workspace, size_t workspace_bytes,
                    void* stream) {
    if (k_new == nullptr || v_new == nullptr) {
        clear_error();
        return fail(SWA_ERR_INVALID_ARG, "swa_decode_step: k_new and v_new are required");
    }
    return decode_impl("swa_decode_step", desc, q, k_new, v_new, k_cache, v_cache, T, o, n_split, workspace,
                       workspace_bytes, stream);
}

int swa_decode_step_noalloc(const swa_desc* desc, const void* q, const void* k_new, const void* v_new, void* k_cache,
                            void* v_cache, int64_t T, void* o, int32_t n_split, void* stream) {
    static const char* fn = "swa_decode_step_noalloc";
    clear_error();
    if (k_new == nullptr || v_new == nullptr) return fail(SWA_ERR_INVALID_ARG, "%s: k_new and v_new are required", fn);
    int st = check_desc(desc, fn);
    if (st) return st;
    const int32_t ns = n_split == 0 ? default_splits(desc) : n_split;
    if (ns < 1 || ns > 64) return fail(SWA_ERR_INVALID_ARG, "%s: n_split %d outside 1..64", fn, n_split);
    const size_t need = decode_ws_bytes(desc, ns);
    if (need > swa::kNoAllocScratchBytes)
        return fail(SWA_ERR_INVALID_ARG,
                    "%s: %d splits of B=%d, Hq=%d, d=%d need %zu bytes of scratch, more than the %zu built in "
                    "(fewer splits or a smaller batch, or swa_decode_step with a workspace)",
                    fn, ns, desc->B, desc->Hq, desc->d, need, (size_t)swa::kNoAllocScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        // argument checks of decode_impl first, so a rejected call touches no HIP state
        st = decode_impl(fn, desc, q, k_new, v_new, k_cache, v_cache, T, o, ns, nullptr, 0, nullptr, true);
        if (st) return st;
        if ((st = hip_status(swa::decode_noalloc_scratch(&ws), fn))) return st;
    }
    return decode_impl(fn, desc, q, k_new, v_new, k_cache, v_cache, T, o, ns, ws, need, stream);
}

}  // extern "C"

extern "C" {

size_t swa_backward_workspace_bytes(const swa_desc* desc, int64_t L) {
    if (check_desc(desc, "swa_backward_workspace_bytes") != SWA_OK || L < 1 || L > kMaxPos) return 0;
    return backward_layout(desc, L).total;
}

int swa_backward(const swa_desc* desc, const void* q, const void* k, const void* v, const void* o, const void* dout,
                 float* dq, float* dk, float* dv, int64_t L, void* workspace, size_t workspace_bytes, void* stream) {
    static const char* fn = "swa_backward";
    clear_error();
    int st = check_desc(desc, fn);
    if (st) return st;
    if (desc->dtype != SWA_BF16) return fail(SWA_ERR_UNSUPPORTED, "%s: the backward is built for bf16 inputs", fn);
    if (desc->rope_base > 0.0f) return fail(SWA_ERR_UNSUPPORTED, "%s: the backward with RoPE is not built", fn);
    if ((st = check_ptr(q, fn, "q")) || (st = check_ptr(k, fn, "k")) || (st = check_ptr(v, fn, "v")) ||
        (st = check_ptr(o, fn, "o")) || (st = check_ptr(dout, fn, "dout")) || (st = check_ptr(dq, fn, "dq")) ||
        (st = check_ptr(dk, fn, "dk")) || (st = check_ptr(dv, fn, "dv")) ||
        (st = check_ptr(workspace, fn, "workspace")))
        return st;
    if (L < 1) return fail(SWA_ERR_INVALID_ARG, "%s: L must be >= 1 (got %lld)", fn, (long long)L);
    if (L > kMaxPos) return fail(SWA_ERR_INVALID_ARG, "%s: positions beyond 2^30", fn);
    const BackwardLayout lay = backward_layout(desc, L);
    if (workspace_bytes < lay.total)
        return fail(SWA_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, lay.total);
    // grids: query tiles of 128 rows; dK/dV work items; 4-value groups of every key
    const int64_t nqt = (L + 127) / 128;
    const int64_t items = (int64_t)lay.grid.bhkv * ((int64_t)lay.grid.tiles_sink * lay.grid.nseg_sink +
                                                    (int64_t)(lay.grid.tiles - lay.grid.tiles_sink) * lay.grid.nseg_band);
    if ((int64_t)desc->B * desc->Hq * nqt > 0x7fffffffLL || items > 0x7fffffffLL ||
        ((int64_t)lay.grid.bhkv * L * (desc->d / 4) + 255) / 256 > 0x7fffffffLL)
        return fail(SWA_ERR_INVALID_ARG, "%s: grid too large", fn);

    char* ws = static_cast<char*>(workspace);
    swa::BackwardArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.lse2 = reinterpret_cast<float*>(ws + lay.lse2);
    a.dd = reinterpret_cast<float*>(ws + lay.dd);
    a.part = reinterpret_cast<float*>(ws + lay.part);
    a.L = L;
    a.B = desc->B;
    a.Hq = desc->Hq;
    a.Hkv = desc->Hkv;
    a.s = desc->s;
    a.r = desc->r;
    a.scale = desc->scale;
    a.scale_log2e = (float)((double)desc->scale * 1.4426950408889634);
    return hip_status(swa::launch_backward_bf16(a, lay.grid, desc->d, reinterpret_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
