// Banded flash-style prefill, bf16 inputs, gfx950: the ping-pong kernel.
//
// Row t attends U(t) = {i <= t : i < s or i >= t - r + 1} (sinks plus the r
// most recent keys, each once; hyper.ai summary of arXiv 2608.28444, section
// "带 Sink 的滑动窗口注意力", and eq:attn-fixed-streaming on the t6page page
// "滑窗与固定稀疏").  The mask depends on positions only, so tiles outside
// the band are never loaded (the fixed-sparsity section of that page: no
// scoring cost, regular banded access).
//
// Workgroup = 8 waves = two groups of 4; a SIMD runs one wave of each group.
// Both groups read the same key tiles:
//   * GQA (q-heads per kv-head even): the groups take two q-heads of one
//     kv-head over the same 128 tokens;
//   * otherwise: the groups take the two 128-row halves of 256 tokens of one
//     q-head.
// Each wave owns 32 query rows.  Per 64-key tile a wave does two phases:
//   M: S^T = K Q^T for the tile's two 32-key halves (two independent chains
//      of v_mfma_f32_32x32x16_bf16, 16 MFMAs);
//   S: online softmax of those scores in fp32 (VALU) and O^T += V^T P^T
//      (16 MFMAs).
// Group 1 runs one phase behind group 0 and a workgroup barrier closes every
// phase, so on each SIMD one wave issues QK MFMAs while the other runs the
// softmax and its PV MFMAs: the matrix unit stays busy while the vector unit
// works.  Key tiles are double-buffered in LDS and fetched two phases ahead.
//
// Layout details (see the fp32 kernel in prefill.hip for the same scheme):
// the 32x32 S^T accumulator gives every lane one query row (lanes l and l+32
// share it), so the row max is one v_permlane32_swap exchange; K rows enter
// the MFMA in a permuted order so that each lane's eight P values are eight
// consecutive keys; V is stored transposed in LDS so those eight keys of one
// dimension are a single 16-byte read.  The running max is raised only when a
// tile's max exceeds it by more than 2^8 (exact: the same max scales the
// numerator and the denominator).
#include "prefill_common.h"

namespace swa {
namespace {

using namespace pf;

constexpr int PW = 8;             // waves per workgroup
constexpr int PNT = PW * 64;      // threads per workgroup

template <int D>
struct PP {
    static constexpr int CH = D / 8;                 // 16-byte chunks per key row
    static constexpr int KCH = CH + 1;               // padded K row (chunks)
    static constexpr int VCH = BN / 8 + 1;           // padded V^T row (chunks of 8 keys)
    static constexpr int K_LD = BN * CH / PNT;       // K chunks per thread per tile
    static constexpr int V_TASKS = (BN / 4) * CH;    // blocks of 4 keys x 8 dims per tile
    static constexpr int QK_STEPS = D / 16;
    static_assert(K_LD >= 1 && V_TASKS <= 256, "tile shape");

    // Padded rows keep every operand address affine in the loop indices (one
    // base register per lane plus immediate offsets) and the reads free of
    // bank conflicts: 8 or 16 lanes reading consecutive rows at one column hit
    // distinct banks.
    struct Buf {
        u32x4 k[BN * KCH];         // row = MFMA row order: key 32h + swap23(x) at row 32h + x
        u32x4 vt[D * VCH];         // row = dim, chunk = 8 keys
    };
    struct Regs {
        u32x4 k[K_LD];
        u32x4 v[4];
    };

    static __device__ __forceinline__ int krow(int key) { return (key & ~31) | swap23(key & 31); }
    // V work is spread over waves 0, 1, 4, 5; consecutive lanes take
    // consecutive 4-key groups so the transposed 8-byte writes of 16 lanes
    // cover all banks once.
    static __device__ __forceinline__ int vtask(int tid) { return (tid & 127) | ((tid >> 8) << 7); }
    static __device__ __forceinline__ bool has_v(int tid) {
        return ((tid >> 7) & 1) == 0 && vtask(tid) < V_TASKS;
    }
    static __device__ __forceinline__ int v_kq(int vt) { return vt & 15; }
    static __device__ __forceinline__ int v_dc(int vt) { return vt >> 4; }

    // Per-thread rows of a tile: K chunk ld is row k_row(ld, tid), chunk tid % CH;
    // V rows 4 kq + j (j < 4), chunk dc (threads with has_v only).
    static __device__ __forceinline__ int k_row(int ld, int tid) { return ld * (PNT / CH) + tid / CH; }
    static __device__ __forceinline__ int v_row(int j, int tid) { return 4 * v_kq(vtask(tid)) + j; }

    // One set of loads from per-row pointers (all load paths share it).
    static __device__ __forceinline__ void load_rows(Regs& R, const __bf16* const* kp, const __bf16* const* vp,
                                                     int tid) {
#pragma unroll
        for (int ld = 0; ld < K_LD; ++ld) R.k[ld] = *(const u32x4*)(kp[ld] + (tid % CH) * 8);
        if (has_v(tid)) {
            const int dc = v_dc(vtask(tid));
#pragma unroll
            for (int j = 0; j < 4; ++j) R.v[j] = *(const u32x4*)(vp[j] + dc * 8);
        }
    }

    static __device__ __forceinline__ void store(Buf& S, const Regs& R, int tid) {
#pragma unroll
        for (int ld = 0; ld < K_LD; ++ld) {
            const int idx = ld * PNT + tid;
            const int key = idx / CH, c = idx % CH;
            S.k[krow(key) * KCH + c] = R.k[ld];
        }
        if (has_v(tid)) {
            const int vt = vtask(tid), kq = v_kq(vt), dc = v_dc(vt);
            // 4 keys x 8 dims -> 8 dims x 4 keys (8-byte cells)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const int w = e >> 1;
                u32x2 cell;
                cell[0] = __builtin_amdgcn_perm(R.v[1][w], R.v[0][w], sel);
                cell[1] = __builtin_amdgcn_perm(R.v[3][w], R.v[2][w], sel);
                const int dim = dc * 8 + e;
                ((u32x2*)S.vt)[(dim * VCH + (kq >> 1)) * 2 + (kq & 1)] = cell;
            }
        }
    }

    // A wave's 32 query rows in LDS (padded rows like K): row l32 holds the
    // query of lane l32, read as the B operand of S^T = K Q^T.
    struct QTile {
        u32x4 q[WROWS * KCH];
    };

    // Fill the wave's Q tile: lane l copies row l % 32, half g of its chunks.
    static __device__ __forceinline__ void load_q(QTile& Q, const __bf16* row, bool valid, int l32, int g) {
#pragma unroll
        for (int j = 0; j < CH / 2; ++j) {
            const int c = 2 * j + g;
            Q.q[l32 * KCH + c] = valid ? *(const u32x4*)(row + 8 * c) : u32x4{0, 0, 0, 0};
        }
    }

    // S^T for both 32-key halves as two independent MFMA chains, accumulated
    // onto the seeds already in a0, a1 (0, or -inf on masked elements).
    static __device__ __forceinline__ void qk2(const Buf& S, const QTile& Q, int l32, int g, f32x16& a0, f32x16& a1) {
        const u32x4* k0 = &S.k[l32 * KCH + g];
        const u32x4* k1 = k0 + 32 * KCH;
        const u32x4* qq = &Q.q[l32 * KCH + g];
#pragma unroll
        for (int ks = 0; ks < QK_STEPS; ++ks) {
            const bf16x8 q = __builtin_bit_cast(bf16x8, qq[2 * ks]);
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k0[2 * ks]), q, a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k1[2 * ks]), q, a1, 0, 0, 0);
        }
    }

    // Same with zero-initialised accumulators (the first MFMA takes C = 0).
    static __device__ __forceinline__ void qk2_zero(const Buf& S, const QTile& Q, int l32, int g, f32x16& a0,
                                                    f32x16& a1) {
        const u32x4* k0 = &S.k[l32 * KCH + g];
        const u32x4* k1 = k0 + 32 * KCH;
        const u32x4* qq = &Q.q[l32 * KCH + g];
        const bf16x8 q0 = __builtin_bit_cast(bf16x8, qq[0]);
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k0[0]), q0, f32x16{}, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k1[0]), q0, f32x16{}, 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < QK_STEPS; ++ks) {
            const bf16x8 q = __builtin_bit_cast(bf16x8, qq[2 * ks]);
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k0[2 * ks]), q, a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k1[2 * ks]), q, a1, 0, 0, 0);
        }
    }

    // P of half hb as two bf16x8 operands (accumulator order): exp2 of the
    // scaled, max-shifted scores, packed pairwise as they are produced; the
    // fp32 values only feed this lane's share of the row sum.
    static __device__ __forceinline__ void softmax_pack(const f32x16& sc, float c, float mneg, float& l,
                                                        bf16x8& b0, bf16x8& b1) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c, mneg));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i + 1], c, mneg));
            l += p0 + p1;
            if (i < 8) {
                b0[i] = (__bf16)p0;
                b0[i + 1] = (__bf16)p1;
            } else {
                b1[i - 8] = (__bf16)p0;
                b1[i - 7] = (__bf16)p1;
            }
        }
    }

    // O^T += V^T P^T for half hb.
    static __device__ __forceinline__ void pv(const Buf& S, const bf16x8& b0, const bf16x8& b1, f32x16* o, int hb,
                                              int l32, int g) {
        const u32x4* v = &S.vt[l32 * VCH + g];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 b = kk ? b1 : b0;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const u32x4 x = v[db * 32 * VCH + 4 * hb + 2 * kk];
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), b, o[db], 0, 0, 0);
            }
        }
    }

    static __device__ __forceinline__ void store_o(__bf16* row, const f32x16* o, float inv, int g) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t v0 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 0] * inv));
                const uint32_t v1 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 1] * inv));
                const uint32_t v2 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 2] * inv));
                const uint32_t v3 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 3] * inv));
                u32x2 w;
                w[0] = v0 | (v1 << 16);
                w[1] = v2 | (v3 << 16);
                *(u32x2*)(row + 32 * db + 8 * q4 + 4 * g) = w;
            }
        }
    }
};

template <int D>
__global__ __launch_bounds__(PNT) void prefill_pp_kernel(PrefillArgs a) {
    typedef PP<D> T;
    __shared__ typename T::Buf smem[2];
    __shared__ typename T::QTile qsm[PW];

    const int s = a.s, r = a.r;
    const int pos0 = (int)a.pos0;
    const int G = a.Hq / a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, sub = wave & 3;
    const int l32 = lane & 31, g = lane >> 5;

    // ---- work item
    const int w = xcd_work_item(blockIdx.x, gridDim.x);
    const int mt = a.n_mtiles - 1 - (w % a.n_mtiles);   // late (heavier) query tiles first
    const int rest = w / a.n_mtiles;
    int b, kvh, h, row0, tok;
    if (a.pair_mode) {
        const int npairs = G / 2;
        const int pair = rest % npairs, bk = rest / npairs;
        b = bk / a.Hkv;
        kvh = bk % a.Hkv;
        h = kvh * G + 2 * pair + grp;
        tok = 128;
        row0 = mt * tok;
    } else {
        const int bh = rest;
        b = bh / a.Hq;
        h = bh % a.Hq;
        kvh = h / G;
        tok = 256;
        row0 = mt * tok;
    }
    const int nrows = (int)((a.L - row0) < tok ? (a.L - row0) : tok);
    const int t0 = pos0 + row0, t1 = t0 + nrows - 1;                  // the workgroup's rows
    const int wrow0 = row0 + (a.pair_mode ? 0 : 128 * grp) + WROWS * sub;   // this wave's first row (call-relative)
    const int tw0 = pos0 + wrow0;
    const int tw1 = (tw0 + WROWS - 1) < t1 ? (tw0 + WROWS - 1) : t1;
    const bool wave_active = tw0 <= t1;
    const int my_t = tw0 + l32;
    const bool my_valid = my_t <= t1;

    const size_t qoff = ((size_t)(b * a.Hq + h) * a.L + wrow0 + l32) * D;
    const __bf16* kn = (const __bf16*)a.kn + (size_t)(b * a.Hkv + kvh) * a.L * D;
    const __bf16* vn = (const __bf16*)a.vn + (size_t)(b * a.Hkv + kvh) * a.L * D;
    const __bf16* kc = a.kc ? (const __bf16*)a.kc + (size_t)(b * a.Hkv + kvh) * (s + r) * D : nullptr;
    const __bf16* vc = a.vc ? (const __bf16*)a.vc + (size_t)(b * a.Hkv + kvh) * (s + r) * D : nullptr;
    auto kptr = [&](int p) -> const __bf16* {
        if (p >= pos0) return kn + (size_t)(p - pos0) * D;
        const int sl = p < s ? p : s + (int)((unsigned)p % (unsigned)r);
        return kc + (size_t)sl * D;
    };
    auto vptr = [&](int p) -> const __bf16* {
        if (p >= pos0) return vn + (size_t)(p - pos0) * D;
        const int sl = p < s ? p : s + (int)((unsigned)p % (unsigned)r);
        return vc + (size_t)sl * D;
    };

    // ---- tiles of the workgroup: phase 0 then phase 1, as one list
    Phase ph0 = {0, -1, 0, NO_BAND, 0}, ph1 = {0, -1, 0, NO_BAND, 0};
    const int nph = make_phases(t0, t1, s, r, a.merge_sink != 0, ph0, ph1);
    const int n0 = nph >= 1 ? ph0.last - ph0.first + 1 : 0;
    const int n1 = nph >= 2 ? ph1.last - ph1.first + 1 : 0;
    const int nv = n0 + n1;
    auto phase_of = [&](int v) -> Phase { return v < n0 ? ph0 : ph1; };
    auto tile_of = [&](int v) -> int { return v < n0 ? ph0.first + v : ph1.first + (v - n0); };

    typename T::Regs regs;
    // Rows of tile v: rows every query of the workgroup may need, all in the
    // call's own tokens (contiguous) or all in the rolling part of the cache
    // (slot slot0 + row with one wrap), take a direct formula; other tiles
    // clamp each row to one the tile does need.  A clamped row is real,
    // finite data that the score mask then removes (-inf score, weight 0).
    auto load_tile = [&](int v) {
        const Phase P = phase_of(v);
        const int kbase = tile_of(v) * BN, klast = kbase + BN - 1;
        const int lo_any = P.band_lo > t0 - r + 1 ? P.band_lo : t0 - r + 1;
        const bool all_needed = klast <= t1 && (kbase >= lo_any || klast < P.sink_hi);
        const __bf16* kp[T::K_LD];
        const __bf16* vp[4];
        if (all_needed && kbase >= pos0) {
            const __bf16* kb = kn + (size_t)(kbase - pos0) * D;
            const __bf16* vb = vn + (size_t)(kbase - pos0) * D;
#pragma unroll
            for (int ld = 0; ld < T::K_LD; ++ld) kp[ld] = kb + T::k_row(ld, tid) * D;
#pragma unroll
            for (int j = 0; j < 4; ++j) vp[j] = vb + T::v_row(j, tid) * D;
        } else if (all_needed && kbase >= s && klast < pos0) {
            const int slot0 = s + kbase % r, slot_end = s + r;
#pragma unroll
            for (int ld = 0; ld < T::K_LD; ++ld) {
                int sl = slot0 + T::k_row(ld, tid);
                sl = sl >= slot_end ? sl - r : sl;
                kp[ld] = kc + (size_t)sl * D;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int sl = slot0 + T::v_row(j, tid);
                sl = sl >= slot_end ? sl - r : sl;
                vp[j] = vc + (size_t)sl * D;
            }
        } else {
            // nearest needed row: past t1 -> t1; between the sinks and the
            // band -> the band's first row, or the last sink if the phase has
            // no band rows
            const int gap_to = lo_any <= t1 ? lo_any : P.sink_hi - 1;
            auto clamp = [&](int p) {
                p = (p >= P.sink_hi && p < lo_any) ? gap_to : p;
                return p < t1 ? p : t1;
            };
#pragma unroll
            for (int ld = 0; ld < T::K_LD; ++ld) kp[ld] = kptr(clamp(kbase + T::k_row(ld, tid)));
#pragma unroll
            for (int j = 0; j < 4; ++j) vp[j] = vptr(clamp(kbase + T::v_row(j, tid)));
        }
        T::load_rows(regs, kp, vp, tid);
    };

    // ---- per-wave state
    typename T::QTile& qt = qsm[wave];
    int q_loaded = -1;
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_c = -__builtin_inff();
    float l_part = 0.0f;
    const float c = a.scale_log2e;
    f32x16 sacc0 = {}, sacc1 = {};     // scores of the tile between its M and S phases
    bool need0 = false, need1 = false, full0 = false, full1 = false;

    // M phase: scores of tile v
    auto phase_m = [&](int v) {
        const Phase P = phase_of(v);
        const int kb = tile_of(v) * BN;
        const int lo_w0 = P.band_lo > tw0 - r + 1 ? P.band_lo : tw0 - r + 1;
        const int lo_w1 = P.band_lo > tw1 - r + 1 ? P.band_lo : tw1 - r + 1;
        need0 = kb <= tw1 && (kb < P.sink_hi || kb + 31 >= lo_w0);
        need1 = kb + 32 <= tw1 && (kb + 32 < P.sink_hi || kb + 63 >= lo_w0);
        full0 = kb + 31 <= tw0 && (kb >= lo_w1 || kb + 31 < P.sink_hi);
        full1 = kb + 63 <= tw0 && (kb + 32 >= lo_w1 || kb + 63 < P.sink_hi);
        if (!need0 && !need1) return;   // the whole tile is masked for these rows
        const int want_q = (P.use_qs && a.qs != a.q) ? 1 : 0;
        if (want_q != q_loaded) {
            T::load_q(qt, (const __bf16*)(want_q ? a.qs : a.q) + qoff, my_valid, l32, g);
            q_loaded = want_q;
        }
        if (full0 && full1) {
            T::qk2_zero(smem[v & 1], qt, l32, g, sacc0, sacc1);
            return;
        }
        // seed the score accumulators with the mask: 0 where the key is in
        // U(t), -inf elsewhere (-inf plus any finite product stays -inf).
        // Element i of half hb is key kb + 32 hb + 8 g + k_i, k_i an immediate;
        // a half no row of this wave needs comes out all -inf.
        const int lo_me = P.band_lo > my_t - r + 1 ? P.band_lo : my_t - r + 1;
        const int kbg = kb + 8 * g;
        const int lim_t = my_t - kbg, lim_s = P.sink_hi - kbg, lim_b = lo_me - kbg;
        const float NEG = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k0 = keyoff(i, 0), k1 = 32 + keyoff(i, 0);
            sacc0[i] = (k0 <= lim_t && (k0 < lim_s || k0 >= lim_b)) ? 0.0f : NEG;
            sacc1[i] = (k1 <= lim_t && (k1 < lim_s || k1 >= lim_b)) ? 0.0f : NEG;
        }
        T::qk2(smem[v & 1], qt, l32, g, sacc0, sacc1);
    };

    // S phase: online softmax of tile v's scores, then O^T += V^T P^T
    auto phase_s = [&](int v) {
        if (!need0 && !need1) return;
        const float NEG = -__builtin_inff();
        float mx = NEG;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(sacc0[i], sacc1[i]));
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
        const float mneg = (m_c == NEG) ? 0.0f : -m_c;
        const typename T::Buf& B = smem[v & 1];
        {
            bf16x8 b0, b1;
            T::softmax_pack(sacc0, c, mneg, l_part, b0, b1);
            T::pv(B, b0, b1, oacc, 0, l32, g);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
            bf16x8 b0, b1;
            T::softmax_pack(sacc1, c, mneg, l_part, b0, b1);
            T::pv(B, b0, b1, oacc, 1, l32, g);
        }
    };

    // ---- prologue: tiles 0 and 1 in LDS, tile 2 in flight
    if (nv > 0) {
        load_tile(0);
        T::store(smem[0], regs, tid);
    }
    if (nv > 1) {
        load_tile(1);
        T::store(smem[1], regs, tid);
    }
    if (nv > 2) load_tile(2);
    __syncthreads();

    // ---- slots: group 0 runs M(v) in slot 2v and S(v) in slot 2v+1; group 1
    // one slot later.  Tile k is stored in slot 2k-1 (its buffer was last read
    // by group 1's S(k-2) in slot 2k-2) and fetched from memory in slot 2k-3.
    // Each group runs its own straight-line loop (same barriers in the same
    // order), so no value has to be merged between an M and an S path.
    auto stage = [&](int slot) {
        if ((slot & 1) && slot >= 3) {
            const int k = (slot + 1) >> 1;
            if (k < nv) {
                T::store(smem[k & 1], regs, tid);
                if (k + 1 < nv) load_tile(k + 1);
            }
        }
        __syncthreads();
    };
    if (grp == 0) {
        for (int v = 0; v <= nv; ++v) {
            if (wave_active && v < nv) phase_m(v);
            stage(2 * v);
            if (wave_active && v < nv) phase_s(v);
            stage(2 * v + 1);
        }
    } else {
        for (int v = 0; v <= nv; ++v) {
            if (wave_active && v >= 1) phase_s(v - 1);
            stage(2 * v);
            if (wave_active && v < nv) phase_m(v);
            stage(2 * v + 1);
        }
    }

    if (!wave_active) return;
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (!my_valid) return;
    T::store_o((__bf16*)a.o + qoff, oacc, 1.0f / l_tot, g);
}

template <int D>
hipError_t launch(const PrefillArgs& a, hipStream_t st) {
    const long long G = a.Hq / a.Hkv;
    const long long nblk = a.pair_mode ? (long long)a.B * a.Hkv * (G / 2) * a.n_mtiles
                                       : (long long)a.B * a.Hq * a.n_mtiles;
    hipLaunchKernelGGL((prefill_pp_kernel<D>), dim3((unsigned)nblk), dim3(PNT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int prefill_bf16_rows_per_block(int Hq, int Hkv) { return ((Hq / Hkv) % 2 == 0) ? 128 : 256; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, hipStream_t st) {
    if (d == 128) return launch<128>(a, st);
    if (d == 64) return launch<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace swa
