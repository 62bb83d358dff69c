// Split-K single-query decode over the sink + rolling-buffer KV cache, gfx950.
//
// The query of token T-1 attends every slot of the cache that holds a token
// (the cache is the first s tokens plus the r most recent ones,
// eq:attn-fixed-streaming on the t6page page "滑窗与固定稀疏").  Softmax
// attention over a set ignores the order of its members, so slots are read
// in physical order (the permutation-invariance remark in section 3 of the
// Blurry Window Attention page).
//
// Decode is bound by HBM: every cache byte is read once per step.  A
// workgroup takes one (batch, kv-head) and one of n_split slot ranges; its 4
// waves split that range.  The Hq/Hkv query heads of the kv-head share each
// K/V byte:
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 query columns,
//    the group's heads padded to 16); K goes straight from HBM into the MFMA
//    operand registers, rows fed in a permuted order so that every lane's
//    eight scores are eight consecutive keys;
//  * online softmax per query column in fp32 (exp2, scale*log2(e) folded);
//  * O^T += V^T P^T on the same MFMA; V is transposed through a per-wave LDS
//    tile so each lane's eight keys of one dimension are one 16-byte read;
//  * the 4 waves merge in LDS and write (max, sum, unnormalised O) per head
//    and split; a second kernel merges the splits and normalises.  With one
//    split (enough (batch, kv-head) units to fill the chip) the workgroup
//    writes the normalised output itself and the second kernel is skipped.
//  * RoPE re-positioning (rope_rr > 0): U(T-1) sits at consecutive
//    positions in temporal order, the query at the last (the StreamingLLM
//    paragraph after eq:attn-fixed-streaming on the t6page page).  Window
//    keys then sit at their true distance from the query and sink j at
//    min(T-1, s+r-1) - j, so the cache holds every key rotated once at its
//    token's position (swa_rope_keys) and only the query turns: at T-1
//    for window slots, at min(T-1, s+r-1) for sink slots.  The two rotated
//    copies of each q-head take two of the 16 MFMA query columns, so one
//    product scores both; sink slots take the second column's score.
//  * fused step (kn/vn given): the workgroup whose slot range holds the
//    current token's slot first writes the token's K/V row there (then
//    waits for the stores and a barrier), so one launch does the append and
//    the decode.
//  * several query rows at once (npos > 0, the dense rows of task-bound
//    global tokens): the q-heads of npos positions take G * npos <= 16
//    query columns, and column (pi, head) keeps only the keys <= pos[pi],
//    so each K/V byte is read once for all of them.
#include <mutex>

#include "rope_common.h"
#include "swa_internal.h"

// Device scratch of swa_decode_step_noalloc: the per-split partial results
// (max, sum, unnormalised O) go here instead of a caller-provided workspace.
// One copy per GPU, held until the process ends.  In host code this name is
// only a stand-in for the device address: kernels get the address that
// hipGetSymbolAddress returns for the current device (decode_noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[swa::kNoAllocScratchBytes];

namespace swa {

// The address of this device's scratch array, looked up once per device
// with that device current.
hipError_t decode_noalloc_scratch(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int KW = 32;                // keys per wave step
constexpr float RESCALE_TH = 8.0f;

// Row rho (0..15) of MFMA block b (0..1) of a 32-key step holds key
// 8*(rho/4) + 4*b + rho%4, so lane group g (lanes 16g..16g+15) ends up with
// keys 8g .. 8g+7 of the step.
__device__ __forceinline__ int dec_key(int b, int rho) { return 8 * (rho >> 2) + 4 * b + (rho & 3); }

template <int D>
struct DecodeSmem {
    // per wave: V^T tile [dim][8-key chunk ^ vswz(dim)] during the loop, then
    // the wave's unnormalised O [16 columns][D] for the merge (same bytes)
    union {
        u32x4 vt[NW][D * (KW / 8)];
        float o[NW][16][D];
    };
    float m[NW][16];
    float l[NW][16];
};

__device__ __forceinline__ int vswz(int dim) { return ((dim >> 1) ^ (dim >> 3)) & 3; }

template <int D, bool ROPE, bool MULTI>
__global__ __launch_bounds__(NT, 2) void decode_split_kernel(DecodeArgs a) {
    __shared__ DecodeSmem<D> sm;
    constexpr int CH = D / 8;            // 16-byte chunks per row
    constexpr int KSTEPS = D / 32;       // 16x16x32 k-steps over the head dim
    constexpr int DB = D / 16;           // 16-dim blocks of O^T
    constexpr int KPL = KW * CH / 64;    // V keys per lane per step (8 for D=128, 4 for D=64)
    static_assert(KPL == 8 || KPL == 4, "unsupported head dim");

    const int split = blockIdx.x % a.n_split;
    const int bh = blockIdx.x / a.n_split;      // b * Hkv + kvh
    const int b = bh / a.Hkv, kvh = bh % a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int S = a.s + a.r;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g = lane >> 4;
    const int kq = lane / CH, cc = lane % CH;   // V staging: key group, dim chunk

    const int j0 = split * a.slots_per_split;
    const int j1 = (j0 + a.slots_per_split) < S ? (j0 + a.slots_per_split) : S;
    const int nsteps = j1 > j0 ? (j1 - j0 + KW - 1) / KW : 0;
    const int st0 = (nsteps * wave) / NW, st1 = (nsteps * (wave + 1)) / NW;

    const __bf16* kc = (const __bf16*)a.kc + (size_t)bh * S * D;
    const __bf16* vc = (const __bf16*)a.vc + (size_t)bh * S * D;
    if (a.j_new >= 0 && split == a.j_new / a.slots_per_split) {
        // fused append: the workgroup whose slot range holds the current
        // token's slot writes its row there, and every wave reads the slot
        // only after the stores are complete and the workgroup barrier
        if (wave == 0 && lane < 2 * CH) {
            const int c = lane % CH;
            const bool is_v = lane >= CH;
            const u32x4* src = (const u32x4*)((const __bf16*)(is_v ? a.vn : a.kn) + (size_t)bh * D);
            u32x4* dst = (u32x4*)((__bf16*)(is_v ? a.vc : a.kc) + ((size_t)bh * S + a.j_new) * D);
            dst[c] = src[c];
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the stores have completed
        __syncthreads();
    }
    const int64_t T = a.T;
    const bool all_valid = T >= (int64_t)S;
    // slot j holds a token: sinks j < min(s, T); rolling slot s + q holds the
    // tokens p >= s with p mod r == q, so it has been written once the first
    // of them, q + r * ceil((s - q) / r) (or q itself when q >= s), is below T
    auto valid = [&](int j) -> bool {
        if (j >= j1) return false;
        if (all_valid) return true;
        if (j < a.s) return j < T;
        const int64_t q = j - a.s;
        const int64_t first = q >= a.s ? q : q + (int64_t)a.r * ((a.s - q + a.r - 1) / a.r);
        return first <= T - 1;
    };

    // Q^T operand: column col = q-head kvh*G + col (zero past the group);
    // with RoPE columns G .. 2G-1 hold the same heads rotated for the sinks;
    // with several positions column col is head col % G of row pos[col / G]
    constexpr int HK = KSTEPS / 2;
    constexpr bool rope = ROPE;
    const int ncol = MULTI ? G * a.npos : G;
    const int col_pi = MULTI ? col / G : 0;
    const int col_head = MULTI ? col - col_pi * G : col;
    // this lane's column sees keys up to lim (several positions)
    const int lim = MULTI ? (col < ncol ? a.pos[col_pi] : -1) : 0;
    bf16x8 qreg[KSTEPS];
    {
        const bool qband = col < ncol;
        const bool qsink = rope && col >= G && col < 2 * G;
        const int head = qband ? col_head : (qsink ? col - G : 0);
        const __bf16* qrow = (const __bf16*)a.q + ((size_t)b * a.Hq + kvh * G + head) * a.qo_stride +
                             (MULTI && qband ? (size_t)a.pos[col_pi] * D : 0);
        u32x4 x[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            x[ks] = (qband || qsink) ? *(const u32x4*)(qrow + 32 * ks + 8 * g) : u32x4{0, 0, 0, 0};
        if (rope) {
            const int64_t qpos = qband ? T - 1 : (T - 1 < (int64_t)S - 1 ? T - 1 : (int64_t)S - 1);
#pragma unroll
            for (int ks = 0; ks < HK; ++ks) rope::rot_chunk_pair(x[ks], x[ks + HK], 32 * ks + 8 * g, (double)qpos, a.rope_rr);
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, x[ks]);
    }

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};
    float m_c = -__builtin_inff(), l_part = 0.0f;
    const float c = a.scale_log2e;

    // one step's K (MFMA operand order) and V rows in registers; without
    // RoPE two such buffers keep two steps of loads in flight per wave (with
    // RoPE the sink-score exchange, with several positions the per-column
    // limits, need the registers of the second)
    struct StepRegs {
        u32x4 k[2][KSTEPS];
        u32x4 v[KPL];
    };
    constexpr int DEPTH = (ROPE || MULTI) ? 1 : 2;
    // K and V are streamed with the non-temporal hint: every cache byte is
    // read once per step, so keeping it out of the caches leaves them to the
    // reads that do repeat (measured on the 64-sequence workload: 6.7 TB/s
    // against 5.8 with default caching)
    auto load = [&](StepRegs& R, int st) __attribute__((always_inline)) {
        const int kb = j0 + st * KW;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const int j = kb + dec_key(bb, col);
            const bool ok = valid(j);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                R.k[bb][ks] = ok ? __builtin_nontemporal_load((const u32x4*)(kc + (size_t)j * D + 32 * ks + 8 * g))
                                 : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const int j = kb + KPL * kq + e;
            R.v[e] = valid(j) ? __builtin_nontemporal_load((const u32x4*)(vc + (size_t)j * D + 8 * cc))
                              : u32x4{0, 0, 0, 0};
        }
    };

    auto step = [&](StepRegs& R, int st) __attribute__((always_inline)) {
        auto& kr = R.k;
        auto& vr = R.v;
        const int kb = j0 + st * KW;
        f32x4 sacc[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            sacc[bb] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[bb][ks]), qreg[ks],
                                                                   sacc[bb], 0, 0, 0);
        }
        // stage V^T of this step: KPL keys x 8 dims per lane -> 8 dims x KPL keys
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int dim = 8 * cc + e;
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const int w = e >> 1;
            if constexpr (KPL == 8) {
                u32x4 cell;
#pragma unroll
                for (int m2 = 0; m2 < 4; ++m2) cell[m2] = __builtin_amdgcn_perm(vr[2 * m2 + 1][w], vr[2 * m2][w], sel);
                sm.vt[wave][dim * (KW / 8) + (kq ^ vswz(dim))] = cell;
            } else {
                u32x2 cell;
                cell[0] = __builtin_amdgcn_perm(vr[1][w], vr[0][w], sel);
                cell[1] = __builtin_amdgcn_perm(vr[3][w], vr[2][w], sel);
                ((u32x2*)sm.vt[wave])[(dim * (KW / 8) + ((kq >> 1) ^ vswz(dim))) * 2 + (kq & 1)] = cell;
            }
        }
        if (st + DEPTH < st1) load(R, st + DEPTH);

        if (rope && kb < a.s) {
            // sink slots: head col scores with its sink-rotated copy, column col + G
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sk = __shfl(sacc[bb][i], lane + G);
                    if (col < G && kb + 8 * g + 4 * bb + i < a.s) sacc[bb][i] = sk;
                }
        }
        const bool step_full = all_valid && kb + KW <= j1;
        if (!step_full) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!valid(kb + 8 * g + 4 * bb + i)) sacc[bb][i] = -__builtin_inff();
        }
        if (MULTI && kb + KW - 1 > a.pos[0]) {
            // past the first row's limit: each column keeps its own keys
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kb + 8 * g + 4 * bb + i > lim) sacc[bb][i] = -__builtin_inff();
        }
        float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                         fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxc = mx * c;
        const bool upd = mxc > m_c + RESCALE_TH;
        if (__builtin_amdgcn_ballot_w64(upd)) {
            const float alpha = upd ? __builtin_amdgcn_exp2f(m_c - mxc) : 1.0f;
            m_c = upd ? mxc : m_c;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha;
        }
        const float mneg = (m_c == -__builtin_inff()) ? 0.0f : -m_c;
        bf16x8 pb;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[bb][i], c, mneg));
                l_part += p;
                pb[4 * bb + i] = (__bf16)p;
            }
        // O^T += V^T P^T over this lane group's 8 keys
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int dim = 16 * db + col;
            const u32x4 x = sm.vt[wave][dim * (KW / 8) + (g ^ vswz(dim))];
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), pb, oacc[db], 0, 0, 0);
        }
    };

    if constexpr (DEPTH == 1) {
        StepRegs A;
        if (st0 < st1) load(A, st0);
        for (int st = st0; st < st1; ++st) step(A, st);
    } else {
        StepRegs A, Bf;
        if (st0 < st1) load(A, st0);
        if (st0 + 1 < st1) load(Bf, st0 + 1);
        for (int st = st0; st < st1; st += 2) {
            step(A, st);
            if (st + 1 < st1) step(Bf, st + 1);
        }
    }

    // row sums over the 4 lane groups; the wave's O goes to its own LDS region
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
    if (g == 0) {
        sm.m[wave][col] = m_c;
        sm.l[wave][col] = l_part;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.o[wave][col][16 * db + 4 * g + i] = oacc[db][i];
    __syncthreads();

    // merge the 4 waves: thread -> (column, dim)
    for (int idx = tid; idx < ncol * D; idx += NT) {
        const int cl = idx / D, dim = idx % D;
        float M = sm.m[0][cl];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, sm.m[w][cl]);
        const float Mu = (M == -__builtin_inff()) ? 0.0f : M;
        float o = 0.0f, l = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = __builtin_amdgcn_exp2f(sm.m[w][cl] - Mu);
            o += f * sm.o[w][cl][dim];
            l += f * sm.l[w][cl];
        }
        // output row and partial-result row of column cl
        const int cpi = MULTI ? cl / G : 0, chead = MULTI ? cl - cpi * G : cl;
        const size_t bhq = (size_t)b * a.Hq + kvh * G + chead;
        if (a.n_split == 1) {
            // one split: this workgroup saw every slot, so it finishes the head
            ((__bf16*)a.o)[bhq * a.qo_stride + (MULTI ? (size_t)a.pos[cpi] * D : 0) + dim] = (__bf16)(o / l);
            continue;
        }
        float* ws = a.ws + (((MULTI ? bhq * a.npos + cpi : bhq)) * a.n_split + split) * (D + 2);
        if (dim == 0) {
            ws[0] = M;
            ws[1] = l;
        }
        ws[2 + dim] = o;
    }
}

template <int D, bool MULTI>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
    const int bh = blockIdx.x;     // b * Hq + h (with several positions: (b * Hq + h) * npos + pi)
    const int dim = threadIdx.x;
    const float* ws = a.ws + (size_t)bh * a.n_split * (D + 2);
    float M = -__builtin_inff();
    for (int k = 0; k < a.n_split; ++k) M = fmaxf(M, ws[k * (D + 2)]);
    float o = 0.0f, l = 0.0f;
    for (int k = 0; k < a.n_split; ++k) {
        const float mk = ws[k * (D + 2)];
        const float f = (mk == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mk - M);
        l += f * ws[k * (D + 2) + 1];
        o += f * ws[k * (D + 2) + 2 + dim];
    }
    if (MULTI) {
        const int pi = bh % a.npos;
        ((__bf16*)a.o)[(size_t)(bh / a.npos) * a.qo_stride + (size_t)a.pos[pi] * D + dim] = (__bf16)(o / l);
    } else {
        ((__bf16*)a.o)[(size_t)bh * a.qo_stride + dim] = (__bf16)(o / l);
    }
}

template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
    const unsigned nblk = (unsigned)a.B * a.Hkv * a.n_split;
    const bool multi = a.npos > 0;
    if (multi)
        hipLaunchKernelGGL((decode_split_kernel<D, false, true>), dim3(nblk), dim3(NT), 0, st, a);
    else if (a.rope_rr > 0.0)
        hipLaunchKernelGGL((decode_split_kernel<D, true, false>), dim3(nblk), dim3(NT), 0, st, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, false, false>), dim3(nblk), dim3(NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    if (multi)
        hipLaunchKernelGGL((decode_reduce_kernel<D, true>), dim3((unsigned)a.B * a.Hq * a.npos), dim3(D), 0, st, a);
    else
        hipLaunchKernelGGL((decode_reduce_kernel<D, false>), dim3((unsigned)a.B * a.Hq), dim3(D), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int d, hipStream_t st) {
    if (d == 128) return launch<128>(a, st);
    if (d == 64) return launch<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace swa
