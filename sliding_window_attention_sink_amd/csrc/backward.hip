// Backward of the windowed rows (training) on the matrix units, bf16 inputs,
// fp32 gradients, gfx950.
//
// The forward row t is softmax over U(t) = {i <= t : i < s or i >= t-r+1}
// of scale * q_t . k_i, weighting v_i (hyper.ai summary of arXiv
// 2608.28444, section "带 Sink 的滑动窗口注意力"; eq:attn-fixed-streaming on
// the t6page page for the key set).  Its gradient for an upstream dO, with
// P the row's softmax weights and D_t = dO_t . O_t:
//   dV_i = sum_{t : i in U(t)} P_ti dO_t
//   dS_ti = P_ti (dO_t . v_i - D_t)
//   dQ_t = scale sum_{i in U(t)} dS_ti k_i,   dK_i = scale sum_t dS_ti q_t
// with dK and dV summed over the q-heads of a kv-head.
//
// Two kernels, both tiled in 32x32 blocks on v_mfma_f32_32x32x16_bf16, with
// the block operands staged in LDS by direct global->LDS loads:
//
//   bwd_dq (query-outer, like the forward; 4 waves, three buffer sets
//     loaded two blocks ahead): a wave owns 32 query rows with q and dO in
//     registers and walks the key blocks of their key sets (the sink
//     block, then the band; blocks outside are never loaded):
//       S^T = K Q^T and dP^T = V dO^T (16 MFMAs), an online softmax over
//       the keys (running max lazily raised, as in the forward), dS^T =
//       P^T (dP^T - D) packed to bf16, dQ^T += K^T dS^T (8 MFMAs, K read
//       transposed from LDS).  It also writes the row's log-sum-exp and
//       D_t for the second kernel.
//   bwd_dkdv (key-outer; 8 waves in two groups that alternate on the
//     SIMDs): a wave owns 32 keys of the tile's 128, whose K and V stay in
//     LDS, and every other 32-row query block of the q-heads of the
//     kv-head that see them: S = Q K^T and dP = dO V^T (16 MFMAs), P from
//     the row's log-sum-exp, dS = P (dP - D), then dV^T += dO^T P and dK^T
//     += Q^T dS (16 MFMAs, Q and dO read transposed from LDS).  A key tile
//     whose queries span more than one segment is split into segments;
//     segment 0 stores its sums, the others store partial sums that
//     bwd_reduce adds in a fixed order (sink keys see every later query,
//     so their tiles take many segments).  No atomics: the gradients are
//     the same on every call.
//
// Rows of an MFMA block enter in the order swap23(m) (bits 2 and 3 of the
// row index swapped), so that each lane's eight accumulator values of one
// half are eight consecutive rows: the score accumulators are then the
// bf16 B operands of the next products as they are.  Block tiles are
// row-major with the 16-byte chunks of row r rotated by sw(r), which keeps
// both the row reads (16 rows x one chunk) and the transposing reads
// (ds_read_b64_tr_b16: 4 rows x 64 bytes per 32 lanes) free of LDS bank
// conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "backward_internal.h"
#include "mfma_tile.h"

namespace swa {
namespace {

using namespace mt;

constexpr float RESCALE_TH = 8.0f; // log2 units: raise the running max only past 2^8

// U(t) membership of key i for query t (bitwise, so it compiles to selects,
// not branches).
__device__ __forceinline__ bool in_set(int t, int i, int s, int r) { return (i <= t) & ((i < s) | (i >= t - r + 1)); }

// ---------------------------------------------------------------------------
// dQ, per-row log-sum-exp and D.
template <int D>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(BackwardArgs a) {
    typedef Tile<D> TT;
    constexpr int KS = TT::KS, NDB = TT::NDB;
    __shared__ __attribute__((aligned(1024))) char smem[NBUF][2][TT::BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int L = (int)a.L, s = a.s, r = a.r;
    const int G = a.Hq / a.Hkv;
    const int nqt = (L + 127) / 128;
    // the q-heads of a kv-head innermost, then the query tiles of that
    // (batch, kv-head), late (heavier) ones first: each XCD runs the query
    // tiles of few kv-heads, whose key blocks its L2 then shares
    const int bid = xcd_item(blockIdx.x, gridDim.x);
    const int hg = bid % G, rest = bid / G;
    const int qt = nqt - 1 - rest % nqt;
    const int bk = rest / nqt;                                   // b * Hkv + kv-head
    const int b = bk / a.Hkv, kvh = bk % a.Hkv, h = kvh * G + hg;
    const int bhq = b * a.Hq + h;
    const int t0 = qt * 128, t1 = (t0 + 127) < (L - 1) ? (t0 + 127) : (L - 1);
    const int tw0 = t0 + 32 * wave, tw1 = (tw0 + 31) < t1 ? (tw0 + 31) : t1;
    const bool wave_active = tw0 <= t1;
    const int my_t = tw0 + l32;
    const bool my_valid = my_t <= t1;
    const size_t rowq = (size_t)bhq * L + (my_valid ? my_t : t1);

    const __bf16* kg = (const __bf16*)a.k + (size_t)(b * a.Hkv + kvh) * L * D;
    const __bf16* vg = (const __bf16*)a.v + (size_t)(b * a.Hkv + kvh) * L * D;

    // q and dO as B operands (lane: its row, dims 16 ks + 8 g .. +7); D_t
    bf16x8 qB[KS], dB[KS];
    float Dt;
    {
        const __bf16* qr = (const __bf16*)a.q + rowq * D;
        const __bf16* dr = (const __bf16*)a.dout + rowq * D;
        const __bf16* orow = (const __bf16*)a.o + rowq * D;
        float part = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qB[ks] = *(const bf16x8*)(qr + 16 * ks + 8 * g);
            dB[ks] = *(const bf16x8*)(dr + 16 * ks + 8 * g);
            const bf16x8 ov = *(const bf16x8*)(orow + 16 * ks + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e) part += (float)dB[ks][e] * (float)ov[e];
        }
        Dt = pair_sum(part);
    }

    // key blocks: the sink block(s) [0, min(s, t1+1)) and the band
    // [max(s, t0-r+1), t1], as one list (merged when they touch)
    const int sink_end = s < t1 + 1 ? s : t1 + 1;
    const int band_lo = s > t0 - r + 1 ? s : t0 - r + 1;
    int n0 = sink_end > 0 ? (sink_end - 1) / BLK + 1 : 0;
    int bf = band_lo <= t1 ? band_lo / BLK : 0;
    int n1 = band_lo <= t1 ? t1 / BLK - bf + 1 : 0;
    if (n0 > 0 && n1 > 0 && bf <= n0) {   // contiguous: one run [0, t1 / BLK]
        n1 = t1 / BLK - n0 + 1;
        bf = n0;
    }
    const int nv = n0 + n1;
    // the band's blocks walked rotated: step v >= n0 takes the band block
    // whose absolute index is congruent to v - n0 modulo the band's block
    // count, so the query tiles of a head (bands of one length a few blocks
    // apart) read the same key block at each step
    int brho = n1 > 0 ? bf % n1 : 0;
    brho = brho == 0 ? 0 : n1 - brho;
    auto blk_of = [&](int v) __attribute__((always_inline)) {
        if (v < n0) return v;
        const int u = v - n0 + brho;
        return bf + (u >= n1 ? u - n1 : u);
    };

    auto issue = [&](int v, int buf) __attribute__((always_inline)) {
        const int kb = blk_of(v) * BLK;
        TT::load(smem[buf][0], kg, kb, 0, L - 1, wave, lane);
        TT::load(smem[buf][1], vg, kb, 0, L - 1, wave, lane);
    };

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_c = -__builtin_inff(), l_part = 0.0f;
    const float c = a.scale_log2e;

    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): q, dO, o are in registers
    if (nv > 0) issue(0, 0);
    if (nv > 1) issue(1, 1);
    int buf = 0;
    for (int v = 0; v < nv; ++v) {
        wait_vm(v + 1 < nv ? 2 * TT::JW : 0);
        wg_barrier();
        if (v + 2 < nv) issue(v + 2, buf == 0 ? 2 : buf - 1);
        const int kb = blk_of(v) * BLK;
        const bool need = wave_active && kb <= tw1 && (kb < s || kb + BLK - 1 >= tw0 - r + 1);
        if (need) {
            const char* Kt = smem[buf][0];
            const char* Vt = smem[buf][1];
            f32x16 sa = {}, pa = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sa = mfma(TT::rowop(Kt, l32, g, ks), qB[ks], sa);
                pa = mfma(TT::rowop(Vt, l32, g, ks), dB[ks], pa);
            }
            const bool full = kb + BLK - 1 <= tw0 && (kb + BLK - 1 < s || kb >= tw1 - r + 1);
            if (!full) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sa[i] = (my_valid & in_set(my_t, kb + crow(i, g), s, r)) ? sa[i] : -__builtin_inff();
            }
            float mx = sa[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sa[i]);
            mx = pair_max(mx);
            const float mxc = mx * c;
            const bool upd = mxc > m_c + RESCALE_TH;
            if (__builtin_amdgcn_ballot_w64(upd)) {
                const float alpha = upd ? __builtin_amdgcn_exp2f(m_c - mxc) : 1.0f;
                m_c = upd ? mxc : m_c;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
            }
            const float mneg = m_c == -__builtin_inff() ? 0.0f : -m_c;
            bf16x8 ds[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, mneg));
                l_part += p;
                ds[i / 8][i % 8] = (__bf16)(p * (pa[i] - Dt));
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int db = 0; db < NDB; ++db) acc[db] = mfma(TT::trop(Kt, lane, db, kk), ds[kk], acc[db]);
        }
        buf = buf == 2 ? 0 : buf + 1;
    }
    if (!my_valid) return;
    const float l_tot = pair_sum(l_part);
    const float inv = a.scale / l_tot;
    float* dq = a.dq + ((size_t)bhq * L + my_t) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = acc[db][4 * q4 + j] * inv;
            *(f32x4*)(dq + 32 * db + 8 * q4 + 4 * g) = x;
        }
    if (g == 0) {
        a.lse2[(size_t)bhq * L + my_t] = m_c + __builtin_amdgcn_logf(l_tot);
        a.dd[(size_t)bhq * L + my_t] = Dt;
    }
}

// ---------------------------------------------------------------------------
// dK and dV.  Work items: (b * Hkv + kvh, key tile of 128 keys, segment);
// first the tiles holding sink keys (their queries run to the end), then
// the others.  Segment seg of a tile walks its query blocks
// [qb_lo + seg * segb, ...) for every q-head of the kv-head: iteration it
// is block qb_lo + seg * segb + qrot(it / G) of q-head kvh * G + it % G
// (the segment's blocks walked rotated, below).
//
// Eight waves in two groups of four share the tile's K and V in LDS; wave
// (grp, sub) owns keys i0 + 32 sub .. +31 and the iterations it = grp (mod
// 2), and the two groups alternate on each compute unit's SIMDs (a
// ping-pong, one barrier per half-slot).  In half-slot h the group with
// h = grp (mod 2) runs C: dV^T += dO^T P and dK^T += Q^T dS of iteration
// h-2 and S = Q K^T, dP = dO V^T of iteration h (32 MFMAs); the other runs
// X: the loads of iteration h+2 and the softmax of iteration h-1 (P from
// the row's log-sum-exp, dS = P (dP - D), packed to bf16).  An iteration's
// Q, dO and statistics stay in one of PB buffers from its loads (half-slot
// it-2) to its transposed reads (half-slot it+2); a wave waits for its own
// loads at the end of its next C half-slot, one barrier before their first
// reader.  At the end group 1 hands its partial sums to group 0 through
// LDS.
constexpr int PB = 5;

template <int D>
__global__ __launch_bounds__(2 * NT, 2) void bwd_dkdv_kernel(BackwardArgs a, BwdGrid gr) {
    typedef Tile<D> TT;
    constexpr int KS = TT::KS, NDB = TT::NDB;
    constexpr int TB = TT::BYTES;
    constexpr int OFF_BUF = 2 * NW * TB;                 // after K and V of the tile
    constexpr int OFF_STAT = OFF_BUF + PB * 2 * TB;
    constexpr int LDS_BYTES = OFF_STAT + PB * 2 * BLK * 4;
    // the final hand-over: 4 waves x (dK, dV) x NDB x 16 values x 64 lanes
    static_assert(4 * 2 * NDB * 16 * 64 * 4 <= OFF_STAT, "hand-over fits the tile buffers");
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
    auto kv_tile = [&](int kv, int w) __attribute__((always_inline)) { return lds + (kv * NW + w) * TB; };
    auto buf_tile = [&](int bi, int x) __attribute__((always_inline)) { return lds + OFF_BUF + (bi * 2 + x) * TB; };
    auto buf_stat = [&](int bi) __attribute__((always_inline)) {
        return (float*)(lds + OFF_STAT) + bi * 2 * BLK;
    };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2, sub = wave & 3;
    const int l32 = lane & 31, g = lane >> 5;
    const int L = (int)a.L, s = a.s, r = a.r;
    const int G = a.Hq / a.Hkv;
    // it / G as a multiply-high (exact for it < 2^16, G < 2^16)
    const uint64_t gmag = (uint64_t)0xFFFFFFFFu / (uint32_t)G + 1;
    auto div_g = [&](int it) __attribute__((always_inline)) { return (int)(((uint64_t)(uint32_t)it * gmag) >> 32); };

    // ---- work item
    int bhk, tile, seg;
    size_t slot_base;
    {
        // sink items (long) first and in their own order, which the
        // round-robin dispatch spreads over the XCDs; the band items in XCD
        // runs, so the key tiles that share query blocks share an L2
        const int n_sink_items = gr.bhkv * gr.tiles_sink * gr.nseg_sink;
        int id = (int)blockIdx.x < n_sink_items
                     ? (int)blockIdx.x
                     : n_sink_items + xcd_item((int)blockIdx.x - n_sink_items, (int)gridDim.x - n_sink_items);
        if (id < n_sink_items) {
            seg = id % gr.nseg_sink;
            tile = (id / gr.nseg_sink) % gr.tiles_sink;
            bhk = id / (gr.nseg_sink * gr.tiles_sink);
            slot_base = gr.slots_band + ((size_t)bhk * gr.tiles_sink + tile) * (gr.nseg_sink - 1);
        } else {
            id -= n_sink_items;
            const int tb = gr.tiles - gr.tiles_sink;
            seg = id % gr.nseg_band;
            tile = gr.tiles_sink + (id / gr.nseg_band) % tb;
            bhk = id / (gr.nseg_band * tb);
            slot_base = ((size_t)bhk * tb + (tile - gr.tiles_sink)) * (gr.nseg_band - 1);
        }
    }
    const int b = bhk / a.Hkv, kvh = bhk % a.Hkv;
    const int i0 = tile * 128, i1 = (i0 + 127) < (L - 1) ? (i0 + 127) : (L - 1);
    // query blocks of the tile: keys i0..i1 are seen by queries i0 .. i1 + r - 1
    // (sink keys: every later query)
    const int q_hi = i0 < s ? L - 1 : ((i1 + r - 1) < (L - 1) ? (i1 + r - 1) : (L - 1));
    const int qb_lo = i0 / BLK, qb_hi = q_hi / BLK;
    const int nb = qb_hi - qb_lo + 1;
    const int sb0 = seg * gr.segb;
    if (sb0 >= nb) return;                                 // an empty segment (all waves leave)
    const int sb1 = (sb0 + gr.segb) < nb ? (sb0 + gr.segb) : nb;
    const int niter = (sb1 - sb0) * G;
    const int qbase = (qb_lo + sb0) * BLK;                 // first query of the segment
    // The segment's query blocks are walked rotated: iteration it takes block
    // qrot(it / G), the one whose absolute index is congruent to it / G
    // modulo the segment's block count.  Items of neighbouring key tiles of a
    // kv-head have segments of one length a few blocks apart, so at each step
    // they read the same Q and dO block (or one of two), which the XCD's L2
    // then serves.
    const int nqb = sb1 - sb0;
    int qrho = (qb_lo + sb0) % nqb;
    qrho = qrho == 0 ? 0 : nqb - qrho;
    auto qrot = [&](int qi) __attribute__((always_inline)) {
        const int u = qi + qrho;
        return u >= nqb ? u - nqb : u;
    };

    const int kw0 = i0 + 32 * sub;                         // this wave's keys kw0 .. kw0 + 31
    const int my_key = kw0 + l32;
    const bool wave_active = kw0 <= i1;
    const __bf16* kg = (const __bf16*)a.k + (size_t)bhk * L * D;
    const __bf16* vg = (const __bf16*)a.v + (size_t)bhk * L * D;

    // K and V of the tile's 128 keys stay in LDS for the whole item (the
    // B operands of S = Q K^T and dP = dO V^T: lane takes its key, dims
    // 16 ks + 8 g .. +7); keys past L are row L-1 (masked).  Group 0
    // loads K, group 1 V.
#pragma unroll
    for (int w = 0; w < NW; ++w) TT::load(kv_tile(grp, w), grp ? vg : kg, i0 + 32 * w, 0, L - 1, sub, lane);
    const char* Kw = kv_tile(0, sub);
    const char* Vw = kv_tile(1, sub);

    // the loads of iteration it into buffer bi, by the four waves of one group
    auto issue = [&](int it, int bi) __attribute__((always_inline)) {
        const int q0 = div_g(it);
        const int qb = qb_lo + sb0 + qrot(q0);
        const int bhq = b * a.Hq + kvh * G + (it - q0 * G);
        const __bf16* qg = (const __bf16*)a.q + (size_t)bhq * L * D;
        const __bf16* dg = (const __bf16*)a.dout + (size_t)bhq * L * D;
        TT::load(buf_tile(bi, 0), qg, qb * BLK, 0, L - 1, sub, lane);
        TT::load(buf_tile(bi, 1), dg, qb * BLK, 0, L - 1, sub, lane);
        // lse and D of the block's 32 rows: 4 lanes of every wave, 16 bytes
        // each (rows past L read the next head's values or the arrays'
        // padding; the masks drop them)
        if (lane < 4) {
            const int x = 4 * sub + lane;                       // 16-byte piece 0..15
            const float* src = (x < 8 ? a.lse2 : a.dd) + (size_t)bhq * L;
            load_lds16(src + qb * BLK + 4 * (x & 7), buf_stat(bi) + 16 * sub);
        }
    };
    // does this wave's key block meet iteration it's query block?
    auto need_of = [&](int it) __attribute__((always_inline)) {
        const int tq0 = qbase + BLK * qrot(div_g(it));
        return wave_active && kw0 <= tq0 + BLK - 1 && tq0 <= L - 1 && (kw0 < s || kw0 + BLK - 1 >= tq0 - r + 1);
    };

    f32x16 dvT[NDB], dkT[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dvT[db] = f32x16{};
        dkT[db] = f32x16{};
    }
    f32x16 sa = {}, pa = {};            // S and dP of an iteration, from its C to its X
    bf16x8 pp[2], ps[2];                // P and dS, from its X to the group's next C
    const float c = a.scale_log2e;

    // iterations 0 and 1 travel with K and V
    if (grp < niter) issue(grp, grp);
    wait_vm(0);
    wg_barrier();

    auto bmod = [](int x) __attribute__((always_inline)) { return x >= PB ? x - PB : x; };
    int bh = 0;                         // h mod PB
    for (int h = 0; h < niter + 2; ++h) {
        if (((h ^ grp) & 1) == 0) {
            // ---- C: dV/dK of iteration h-2, S/dP of iteration h
            const int ip = h - 2;
            if (ip >= 0 && need_of(ip)) {
                const int bp = bmod(bh + PB - 2);
                const char* Qp = buf_tile(bp, 0);
                const char* Op = buf_tile(bp, 1);   // dO
                // transposed operands one step ahead, as above
                bf16x8 ot[2], qt[2];
                auto rdt = [&](int n) __attribute__((always_inline)) {
                    ot[n & 1] = TT::trop(Op, lane, n % NDB, n / NDB);
                    qt[n & 1] = TT::trop(Qp, lane, n % NDB, n / NDB);
                };
                rdt(0);
#pragma unroll
                for (int n = 0; n < 2 * NDB; ++n) {
                    if (n + 1 < 2 * NDB) rdt(n + 1);
                    const int db = n % NDB, kk = n / NDB;
                    dvT[db] = mfma(ot[n & 1], pp[kk], dvT[db]);
                    dkT[db] = mfma(qt[n & 1], ps[kk], dkT[db]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // P and dS die before S and dP are born (registers)
            __builtin_amdgcn_sched_barrier(0);
            if (h < niter && need_of(h)) {
                const char* Qt = buf_tile(bh, 0);
                const char* Ot = buf_tile(bh, 1);
                sa = f32x16{};
                pa = f32x16{};
                // operands one k-step ahead of their products (two register
                // sets), so each product's LDS reads are in flight during
                // the previous step's products
                bf16x8 qa[2], oa[2], ka[2], va[2];
                auto rd = [&](int ks) __attribute__((always_inline)) {
                    const int sl = ks & 1;
                    qa[sl] = TT::rowop(Qt, l32, g, ks);
                    ka[sl] = TT::colop(Kw, l32, g, ks);
                    oa[sl] = TT::rowop(Ot, l32, g, ks);
                    va[sl] = TT::colop(Vw, l32, g, ks);
                };
                rd(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 1 < KS) rd(ks + 1);
                    const int sl = ks & 1;
                    sa = mfma(qa[sl], ka[sl], sa);
                    pa = mfma(oa[sl], va[sl], pa);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // this wave's loads (issued in its last X half-slot) land before
            // the barrier that precedes their first reader
            wait_vm(0);
        } else {
            // ---- X: softmax of iteration h-1, loads of iteration h+2
            const int ix = h - 1;
            if (ix >= 0 && ix < niter && need_of(ix)) {
                const int tq0 = qbase + BLK * qrot(div_g(ix));
                const float* ls = buf_stat(bmod(bh + PB - 1));
                const float* dd = ls + BLK;
                // lse and D of this lane's 16 queries (rows 8g .. 8g+7, 16+8g .. +7)
                auto lq = [&](int i) __attribute__((always_inline)) { return ls[crow(i, g)]; };
                auto dq4 = [&](int i) __attribute__((always_inline)) { return dd[crow(i, g)]; };
                const bool full = kw0 + BLK - 1 <= tq0 && tq0 + BLK - 1 <= L - 1 && kw0 + BLK - 1 <= L - 1 &&
                                  (kw0 + BLK - 1 < s || kw0 >= tq0 + BLK - 1 - r + 1);
                if (full) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, -lq(i)));
                        pp[i / 8][i % 8] = (__bf16)p;
                        ps[i / 8][i % 8] = (__bf16)(p * (pa[i] - dq4(i)));
                    }
                } else {
                    // masked pairs (and rows past L, whose statistics are
                    // not this head's) give P = dS = 0
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = tq0 + crow(i, g);
                        const bool ok = (t <= L - 1) & (my_key <= L - 1) & in_set(t, my_key, s, r);
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, -lq(i)));
                        const float dsv = p * (pa[i] - dq4(i));
                        pp[i / 8][i % 8] = (__bf16)(ok ? p : 0.0f);
                        ps[i / 8][i % 8] = (__bf16)(ok ? dsv : 0.0f);
                    }
                }
            }
            if (h + 2 < niter) issue(h + 2, bmod(bh + 2));
        }
        wg_barrier();
        bh = bmod(bh + 1);
    }

    // group 1 hands its sums to group 0 (the buffers are free: every load
    // landed before the last barrier and every read is behind it)
    float* red = (float*)lds + (size_t)sub * (2 * NDB * 16 * 64) + lane;
    if (grp == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                red[((2 * db) * 16 + i) * 64] = dkT[db][i];
                red[((2 * db + 1) * 16 + i) * 64] = dvT[db][i];
            }
    }
    wg_barrier();
    if (grp == 1 || !wave_active || my_key > L - 1) return;
    // segment 0 stores the sums, the others partial sums for bwd_reduce
    float *dk, *dv;
    if (seg == 0) {
        dk = a.dk + ((size_t)bhk * L + my_key) * D;
        dv = a.dv + ((size_t)bhk * L + my_key) * D;
    } else {
        float* slot = a.part + (slot_base + seg - 1) * (size_t)(2 * 128 * D);
        dk = slot + (size_t)(my_key - i0) * D;
        dv = slot + (size_t)(128 + my_key - i0) * D;
    }
    // one 32-dim block at a time (the partner's values and the sums of one
    // block in registers at once)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 xk, xv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * q4 + j;
                xk[j] = (dkT[db][i] + red[((2 * db) * 16 + i) * 64]) * a.scale;
                xv[j] = dvT[db][i] + red[((2 * db + 1) * 16 + i) * 64];
            }
            *(f32x4*)(dk + 32 * db + 8 * q4 + 4 * g) = xk;
            *(f32x4*)(dv + 32 * db + 8 * q4 + 4 * g) = xv;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Adds the partial sums of segments 1 .. of every split key tile among keys
// key0 .. key0+nkeys-1 (of each (batch, kv-head)) to dK and dV, in segment
// order.  Thread: 4 values of one key.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BackwardArgs a, BwdGrid gr, int key0, int nkeys) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_bh = (int64_t)nkeys * (D / 4);
    if (idx >= (int64_t)gr.bhkv * per_bh) return;
    const int bhk = (int)(idx / per_bh);
    const int key = key0 + (int)((idx % per_bh) / (D / 4));
    const int e4 = (int)(idx % (D / 4)) * 4;
    const int L = (int)a.L;
    const int tile = key / 128, i0 = tile * 128;
    const int i1 = (i0 + 127) < (L - 1) ? (i0 + 127) : (L - 1);
    const bool sink = tile < gr.tiles_sink;
    const int q_hi = sink ? L - 1 : ((i1 + a.r - 1) < (L - 1) ? (i1 + a.r - 1) : (L - 1));
    const int nb = q_hi / BLK - i0 / BLK + 1;
    const int nseg = (nb + gr.segb - 1) / gr.segb;
    if (nseg <= 1) return;
    const size_t base = sink ? gr.slots_band + ((size_t)bhk * gr.tiles_sink + tile) * (gr.nseg_sink - 1)
                             : ((size_t)bhk * (gr.tiles - gr.tiles_sink) + (tile - gr.tiles_sink)) * (gr.nseg_band - 1);
    float* dk = a.dk + ((size_t)bhk * L + key) * D + e4;
    float* dv = a.dv + ((size_t)bhk * L + key) * D + e4;
    f32x4 sk = *(const f32x4*)dk, sv = *(const f32x4*)dv;
    for (int sg = 1; sg < nseg; ++sg) {
        const float* slot = a.part + (base + sg - 1) * (size_t)(2 * 128 * D);
        sk += *(const f32x4*)(slot + (size_t)(key - i0) * D + e4);
        sv += *(const f32x4*)(slot + (size_t)(128 + key - i0) * D + e4);
    }
    *(f32x4*)dk = sk;
    *(f32x4*)dv = sv;
}

template <int D>
hipError_t launch(const BackwardArgs& a, const BwdGrid& gr, hipStream_t st) {
    const int nqt = (int)((a.L + 127) / 128);
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)(a.B * a.Hq * nqt)), dim3(NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)gr.bhkv * (gr.tiles_sink * gr.nseg_sink + (gr.tiles - gr.tiles_sink) * gr.nseg_band);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)items), dim3(2 * NT), 0, st, a, gr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // only the key tiles that have partial sums: the sink tiles, the band
    // tiles, or both
    const int ksink = (int)((int64_t)gr.tiles_sink * 128 < a.L ? (int64_t)gr.tiles_sink * 128 : a.L);
    if (gr.slots_sink > 0) {
        const int64_t n = (int64_t)gr.bhkv * ksink * (D / 4);
        hipLaunchKernelGGL((bwd_reduce_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, gr, 0, ksink);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (gr.slots_band > 0) {
        const int nk = (int)(a.L - ksink);
        const int64_t n = (int64_t)gr.bhkv * nk * (D / 4);
        hipLaunchKernelGGL((bwd_reduce_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, gr, ksink, nk);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_backward_bf16(const BackwardArgs& a, const BwdGrid& gr, int d, hipStream_t st) {
    if (d == 128) return launch<128>(a, gr, st);
    if (d == 64) return launch<64>(a, gr, st);
    return hipErrorInvalidValue;
}

}  // namespace swa
