// Banded flash-style prefill for sliding-window attention with sinks, gfx950:
// the fp32 kernel (bf16 inputs go to the ping-pong kernel in prefill_bf16.hip,
// which uses the same tiling, masks and accumulator layouts).
//
// Row t attends U(t) = {i <= t : i < s or i >= t - r + 1} (sinks plus the r
// most recent keys, each once; hyper.ai summary of arXiv 2608.28444, section
// "带 Sink 的滑动窗口注意力", and eq:attn-fixed-streaming on the t6page page
// "滑窗与固定稀疏").  The mask is fixed by position, so whole tiles outside
// the band are never loaded (the "zero scoring cost, regular banded access"
// argument of the fixed-sparsity section of that page).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one q-head):
//  * key tiles of 64 positions are staged in LDS; a phase is a range of tiles
//    with a mask rule: the sink phase (keys < s, visited once per query tile)
//    and the band phase (keys >= max(s, t - r + 1)); without RoPE the two
//    merge when they touch, with the single mask "i < s or i >= t - r + 1";
//  * each wave owns 32 query rows and skips 32-key blocks that are masked for
//    all of them;
//  * S^T = K Q^T on v_mfma_f32_32x32x2_f32:
//    the accumulator gives every lane one query row (lanes l and l+32 share
//    it), so the row max needs one cross-lane exchange and the row sum none
//    until the end;
//  * online softmax in fp32 on exp2 with scale*log2(e) folded in; the running
//    max is only raised when a block's max exceeds it by more than 2^8, which
//    keeps O's rescaling rare and the result exact (the same max enters the
//    numerator and the denominator);
//  * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator; with one key per lane per MFMA step, V stays row-major in
//    LDS.
#include "prefill_common.h"

namespace swa {
namespace {

using namespace pf;


constexpr int NW = 4;            // waves per workgroup
constexpr int BM = NW * WROWS;   // query rows per workgroup
static_assert(BM == kPrefillF32RowsPerBlock, "host tiling must match");
constexpr int NT = NW * 64;      // threads per workgroup

template <typename T, int D>
struct Tiles;

// ---------------------------------------------------------------- fp32 tiles
template <int D>
struct Tiles<float, D> {
    static constexpr int CH = D / 4;                    // 16-byte chunks per key row
    static constexpr int LD = BN * CH / NT;             // chunks per thread (K and V each)
    static constexpr int KS = D + 1;                    // padded K row stride (floats)
    static constexpr int QK_STEPS = D / 2;
    struct Smem {
        float k[BN * KS];
        float v[BN * D];
    };
    struct Regs { u32x4 k[LD]; u32x4 v[LD]; };
    typedef float QReg;
    static constexpr int QREGS = QK_STEPS;

    template <class KPtr, class VPtr, class Loadable>
    static __device__ __forceinline__ void load(Regs& R, int kbase, int tid, KPtr kptr, VPtr vptr,
                                                Loadable ok) {
#pragma unroll
        for (int ld = 0; ld < LD; ++ld) {
            int idx = ld * NT + tid;
            int key = idx / CH, c = idx % CH;
            int p = kbase + key;
            bool y = ok(p);
            R.k[ld] = y ? *(const u32x4*)(kptr(p) + c * 4) : u32x4{0, 0, 0, 0};
            R.v[ld] = y ? *(const u32x4*)(vptr(p) + c * 4) : u32x4{0, 0, 0, 0};
        }
    }

    // rows rs elements apart
    static __device__ __forceinline__ void load_contig(Regs& R, const float* kb, const float* vb, int64_t rs,
                                                       int tid) {
        const int64_t ofs = (tid / CH) * rs + (tid % CH) * 4;
#pragma unroll
        for (int ld = 0; ld < LD; ++ld) {
            R.k[ld] = *(const u32x4*)(kb + ofs + ld * (NT / CH) * rs);
            R.v[ld] = *(const u32x4*)(vb + ofs + ld * (NT / CH) * rs);
        }
    }

    static __device__ __forceinline__ void load_ring(Regs& R, const float* kc, const float* vc, int slot0,
                                                     int slot_end, int r, int tid) {
#pragma unroll
        for (int ld = 0; ld < LD; ++ld) {
            int sl = slot0 + ld * (NT / CH) + tid / CH;
            sl = sl >= slot_end ? sl - r : sl;
            R.k[ld] = *(const u32x4*)(kc + (size_t)sl * D + (tid % CH) * 4);
            R.v[ld] = *(const u32x4*)(vc + (size_t)sl * D + (tid % CH) * 4);
        }
    }

    static __device__ __forceinline__ void store(Smem& S, const Regs& R, int tid) {
#pragma unroll
        for (int ld = 0; ld < LD; ++ld) {
            int idx = ld * NT + tid;
            int key = idx / CH, c = idx % CH;
            // bit-cast the whole vector: clang mis-lowers a bit-cast of a single
            // ext-vector element (every element becomes element 0)
            const f32x4 kv = __builtin_bit_cast(f32x4, R.k[ld]);
#pragma unroll
            for (int e = 0; e < 4; ++e) S.k[key * KS + 4 * c + e] = kv[e];
            *(u32x4*)&S.v[key * D + 4 * c] = R.v[ld];
        }
    }

    static __device__ __forceinline__ void load_q(QReg* q, const float* row, bool valid, int g) {
#pragma unroll
        for (int ks = 0; ks < QK_STEPS; ++ks) q[ks] = valid ? row[2 * ks + g] : 0.0f;
    }

    static __device__ __forceinline__ f32x16 qk(const Smem& S, const QReg* q, int hb, int l32, int g) {
        f32x16 acc = {};
        const float* krow = &S.k[(hb * 32 + swap23(l32)) * KS];
#pragma unroll
        for (int ks = 0; ks < QK_STEPS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * ks + g], q[ks], acc, 0, 0, 0);
        return acc;
    }

    static __device__ __forceinline__ void pv(const Smem& S, const float* p, f32x16* o, int hb, int l32, int g) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float* vrow = &S.v[(hb * 32 + keyoff(i, g)) * D];
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db + l32], p[i], o[db], 0, 0, 0);
        }
    }

    static __device__ __forceinline__ void store_o(float* row, const f32x16* o, float inv, int g) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float4 w = make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                                       o[db][4 * q4 + 3] * inv);
                *(float4*)(row + 32 * db + 8 * q4 + 4 * g) = w;
            }
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(NT, 2) void prefill_kernel(PrefillArgs a) {
    typedef Tiles<T, D> TL;
    __shared__ typename TL::Smem smem;

    const int w = xcd_work_item(blockIdx.x, gridDim.x);
    const int mt = a.n_mtiles - 1 - (w % a.n_mtiles);   // late (heavier) query tiles first
    const int bh = w / a.n_mtiles;
    const int h = bh % a.Hq;
    int b = bh / a.Hq;
    const int kvh = h / (a.Hq / a.Hkv);
    const int s = a.s, r = a.r;
    const int pos0 = (int)a.pos0;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: keep it scalar
    const int l32 = lane & 31, g = lane >> 5;

    // residue classes: batch index b dil + c, own rows first(c) + i dil
    int64_t Lown = a.L, own_off = 0;
    if (a.dil > 1) {
        const int c = b % a.dil;
        b /= a.dil;
        const int64_t first = pos0 + ((c - pos0) % a.dil + a.dil) % a.dil;
        Lown = first < a.Lp ? (a.Lp - 1 - first) / a.dil + 1 : 0;
        own_off = first * D;
    }
    const int row0 = mt * BM;                                   // first row of the tile (call-relative)
    if (row0 >= Lown) return;                                   // a shorter class's last tile
    const int nrows = (int)((Lown - row0) < BM ? (Lown - row0) : BM);
    const int t0 = pos0 + row0, t1 = t0 + nrows - 1;            // positions of the tile's rows
    const int tw0 = t0 + wave * WROWS;
    const int tw1 = (tw0 + WROWS - 1) < t1 ? (tw0 + WROWS - 1) : t1;
    const bool wave_active = tw0 <= t1;
    const int my_t = tw0 + l32;
    const bool my_valid = my_t <= t1;

    const int64_t rs = a.rs;
    const size_t qoff = (size_t)(b * a.Hq + h) * a.q_bh + own_off + (size_t)(row0 + wave * WROWS + l32) * rs;
    const T* kn = (const T*)a.kn + (size_t)(b * a.Hkv + kvh) * a.kv_bh + own_off;
    const T* vn = (const T*)a.vn + (size_t)(b * a.Hkv + kvh) * a.kv_bh + own_off;
    const T* kc = a.kc ? (const T*)a.kc + (size_t)(b * a.Hkv + kvh) * a.c_bh : nullptr;
    const T* vc = a.vc ? (const T*)a.vc + (size_t)(b * a.Hkv + kvh) * a.c_bh : nullptr;

    auto kptr = [&](int p) __attribute__((always_inline)) -> const T* {
        if (p >= pos0) return kn + (size_t)(p - pos0) * rs;
        int sl = p < s ? p : s + (int)((unsigned)p % (unsigned)r);
        return kc + (size_t)sl * D;
    };
    auto vptr = [&](int p) __attribute__((always_inline)) -> const T* {
        if (p >= pos0) return vn + (size_t)(p - pos0) * rs;
        int sl = p < s ? p : s + (int)((unsigned)p % (unsigned)r);
        return vc + (size_t)sl * D;
    };

    // ---- phases (uniform over the workgroup)
    Phase ph0 = {0, -1, 0, NO_BAND, 0}, ph1 = {0, -1, 0, NO_BAND, 0};
    const int nph = make_phases(t0, t1, s, r, a.merge_sink != 0, ph0, ph1);

    typename TL::QReg qreg[TL::QREGS];
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_c = -__builtin_inff();   // running max in scale*log2e units
    float l_part = 0.0f;             // this lane's share of the row sum
    const float c = a.scale_log2e;

    typename TL::Regs regs;
    int q_loaded = -1;
    for (int pi = 0; pi < nph; ++pi) {
        const Phase P = pi ? ph1 : ph0;
        // a key position is loaded iff some row of this tile needs it
        const int lo_any = P.band_lo > t0 - r + 1 ? P.band_lo : t0 - r + 1;
        auto loadable = [&](int p) __attribute__((always_inline)) { return p <= t1 && (p < P.sink_hi || p >= lo_any); };

        if (q_loaded < 0) {
            TL::load_q(qreg, (const T*)a.q + qoff, my_valid, g);
            q_loaded = 0;
        }

        // Tile-uniform choice of the load path: rows that every query of the
        // tile may need, all in the call's own tokens or all in the rolling
        // part of the cache, take a fast path; edge tiles check every row.
        auto load_tile = [&](int j) __attribute__((always_inline)) {
            const int kbase = j * BN, klast = kbase + BN - 1;
            const bool all_needed = klast <= t1 && (kbase >= lo_any || klast < P.sink_hi);
            if (all_needed && kbase >= pos0) {
                TL::load_contig(regs, kn + (size_t)(kbase - pos0) * rs, vn + (size_t)(kbase - pos0) * rs, rs, tid);
            } else if (all_needed && kbase >= s && klast < pos0) {
                TL::load_ring(regs, kc, vc, s + kbase % r, s + r, r, tid);
            } else {
                TL::load(regs, kbase, tid, kptr, vptr, loadable);
            }
        };
        load_tile(P.first);
        for (int j = P.first; j <= P.last; ++j) {
            __syncthreads();
            TL::store(smem, regs, tid);
            __syncthreads();
            if (j < P.last) load_tile(j + 1);
            if (!wave_active) continue;

            const int lo_w0 = P.band_lo > tw0 - r + 1 ? P.band_lo : tw0 - r + 1;
            const int lo_w1 = P.band_lo > tw1 - r + 1 ? P.band_lo : tw1 - r + 1;
            const int lo_me = P.band_lo > my_t - r + 1 ? P.band_lo : my_t - r + 1;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int kb = j * BN + hb * 32;
                const bool need = kb <= tw1 && (kb < P.sink_hi || kb + 31 >= lo_w0);
                if (!need) continue;
                const bool full = kb + 31 <= tw0 && (kb >= lo_w1 || kb + 31 < P.sink_hi);

                f32x16 sacc = TL::qk(smem, qreg, hb, l32, g);
                if (!full) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb + keyoff(i, g);
                        const bool ok = key <= my_t && (key < P.sink_hi || key >= lo_me);
                        sacc[i] = ok ? sacc[i] : -__builtin_inff();
                    }
                }
                float mx = sacc[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
                mx = max_pair_lanes(mx);
                const float mxc = mx * c;
                const bool upd = mxc > m_c + RESCALE_TH;
                if (__builtin_amdgcn_ballot_w64(upd)) {
                    const float alpha = upd ? __builtin_amdgcn_exp2f(m_c - mxc) : 1.0f;
                    m_c = upd ? mxc : m_c;
                    l_part *= alpha;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
                }
                const float mneg = (m_c == -__builtin_inff()) ? 0.0f : -m_c;
                float p[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c, mneg));
                    l_part += p[i];
                }
                TL::pv(smem, p, oacc, hb, l32, g);
            }
        }
    }

    if (!wave_active) return;
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (!my_valid) return;
    const float inv = 1.0f / l_tot;
    TL::store_o((T*)a.o + qoff, oacc, inv, g);
}

template <typename T, int D>
hipError_t launch(const PrefillArgs& a, hipStream_t st) {
    const long long nblk = (long long)a.B * a.Hq * a.n_mtiles;
    hipLaunchKernelGGL((prefill_kernel<T, D>), dim3((unsigned)nblk), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t st) {
    if (d == 128) return launch<float, 128>(a, st);
    if (d == 64) return launch<float, 64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace swa
