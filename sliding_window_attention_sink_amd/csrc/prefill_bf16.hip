// Banded flash-style prefill, bf16 inputs, gfx950.
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
// Each wave owns 32 query rows and alternates two clusters per 64-key tile:
//   C(v): MFMA only: O^T += V^T P^T for tile v-1 and S^T = K Q^T for tile v
//         (32 v_mfma_f32_32x32x16_bf16 in six independent chains, operands
//         read from LDS a few steps ahead);
//   X(v): VALU only: the online softmax of tile v's scores into bf16 P, and
//         the direct global->LDS loads of a later tile.
// Group 1 runs one cluster behind group 0 and a workgroup barrier closes each
// cluster, so on every SIMD one wave streams MFMAs while the other does the
// exponentials: a wave never waits for the matrix unit with vector work
// queued behind its MFMAs.  K and V tiles rotate through three LDS buffer
// sets and are fetched four clusters before use.  "Tile v" is the tile of
// step v: the band's tiles are walked rotated (the step-v tile is the one
// whose absolute index is congruent to v modulo the band's tile count), so
// the work items that share K/V read the same tile at the same step and
// their XCD's L2 serves it.
//
// The 32x32 S^T accumulator gives every lane one query row (lanes l and l+32
// share it), so the row max is one v_permlane32_swap exchange; K rows enter
// the MFMA in a permuted order so that each lane's eight P values are eight
// consecutive keys, which makes the accumulator itself the P^T operand.  V
// stays row-major in LDS and ds_read_b64_tr_b16 delivers it transposed.  A
// tile's weights are first taken against the running max; only when some
// lane's weights of the tile sum past 2^8 (or a row has no max yet) is the
// exact row max taken and the running state rescaled (exact either way: the
// same max scales the numerator and the denominator).
//
// The call's own rows are addressed through element strides, so a residue
// class of the dilated window (rows dil apart, the sinks as cache slots) runs
// in place.  The GLB instantiation adds, after the band and outside the
// ping-pong, one tile of gathered task-bound global keys (the Longformer
// section and the glossary entry on global tokens of the t6page page).
#include <type_traits>

#include "prefill_common.h"
#include "rope_common.h"

namespace swa {
namespace {

using namespace pf;

constexpr int PW = 8;             // waves per workgroup
constexpr int GW = 4;             // waves per group
constexpr int PNT = PW * 64;      // threads per workgroup
constexpr int NSET = 3;           // LDS buffer sets

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct PP {
    static constexpr int CH = D / 8;                 // 16-byte chunks per key row
    static constexpr int RPB = 64 / CH;              // key rows per 1 KB block: 4 or 8
    static constexpr int NINS = BN * CH / 64;        // direct-load instructions per K (or V) tile
    static constexpr int JN = NINS / GW;             // ... per wave of the loading group
    static constexpr int JSTEP = RPB * GW;           // key rows between a wave's successive instructions
    static constexpr int RB = D * 2;                 // bytes per key row
    static constexpr int QK_STEPS = D / 16;          // k-steps of S^T = K Q^T; also rounds of a cluster
    static constexpr int NDB = D / 32;               // 32-dim blocks of O^T
    static_assert(NINS % GW == 0 && 2 * QK_STEPS == 4 * NDB, "tile shape");

    // K tile: LDS row rho holds key krow(rho) (MFMA row order: key
    // 32h + swap23(x) at row 32h + x), in 1 KB blocks of RPB rows stored
    // chunk-major with a block-dependent swizzle:
    //   chunk c of row rho at  (rho / RPB) KB + (c ^ ksw(rho / RPB)) * 16 RPB + (rho % RPB) * 16,
    // so the MFMA operand reads (16 lanes, 16 consecutive rows, one chunk)
    // cover 16 distinct bank groups.  V tile: rows = keys in order, chunk c
    // of row k at chunk c ^ vsw(k), so the transposing reads (4 rows x 64
    // bytes per 32 lanes) are free of bank conflicts.  Both tiles are written
    // by direct global->LDS loads, one instruction per 1 KB block.
    struct Buf {
        u32x4 k[BN * CH];
        u32x4 v[BN * CH];
    };

    static __device__ __forceinline__ int krow(int key) { return (key & ~31) | swap23(key & 31); }
    static __device__ __forceinline__ int ksw(int blk) { return D == 128 ? (blk & 3) : (blk & 1); }
    static __device__ __forceinline__ int vsw(int k) { return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }

    // Direct-load maps for wave `sub` of the loading group: its instruction
    // j fills block i = sub + GW j.  The lane's key row is key0 + JSTEP j and
    // its byte offset inside the row is chk (both independent of j).
    //   K: lane l -> block position l = (chunk l / RPB, row l % RPB).
    //   V: lane l -> row RPB i + l / CH, physical chunk l % CH.
    static __device__ __forceinline__ void k_map(int sub, int lane, int& key0, int& chk) {
        key0 = krow(RPB * sub + lane % RPB);
        chk = ((lane / RPB) ^ ksw(sub)) * 16;
    }
    static __device__ __forceinline__ void v_map(int sub, int lane, int& key0, int& chk) {
        key0 = RPB * sub + lane / CH;
        chk = ((lane % CH) ^ vsw(lane / CH)) * 16;
    }

    // Per-lane byte offsets of the K operand reads: step ks of half hb reads
    // k_rd(ks) + hb * 32 rows.  D = 128: the swizzle flips chunk bits 0-1, so
    // even and odd steps use two bases; D = 64: one base.
    static __device__ __forceinline__ void k_rd_bases(int l32, int g, int& be, int& bo) {
        const int blk = l32 / RPB, x = ksw(blk);
        const int common = blk * 1024 + (l32 % RPB) * 16;
        if (D == 128) {
            be = common + (g ^ (x & 1)) * 64 + (x >> 1) * 128;
            bo = common + (g ^ (x & 1)) * 64 + ((x >> 1) ^ 1) * 128;
        } else {
            be = bo = common + (g ^ x) * 128;
        }
    }
    static constexpr int k_rd_step(int ks) { return D == 128 ? (ks >> 1) * 256 : ks * 256; }
    static constexpr int K_HALF = 32 * RB;           // bytes between the two 32-row halves (32 rows = 32 / RPB blocks)

    // A wave's 32 query rows in registers, as the B operand of S^T = K Q^T:
    // lane (l32, g) holds row l32, chunks 2 ks + g for ks < D/16.
    struct QRegs {
        u32x4 q[QK_STEPS];
    };

    static __device__ __forceinline__ void load_q(QRegs& Q, const __bf16* row, bool valid, int g) {
#pragma unroll
        for (int ks = 0; ks < QK_STEPS; ++ks)
            Q.q[ks] = valid ? *(const u32x4*)(row + 8 * (2 * ks + g)) : u32x4{0, 0, 0, 0};
    }

    // RoPE: rotate the lane's query row to position pos.  Chunk 2 ks + g
    // (dims 16 ks + 8 g ..) pairs with chunk 2 (ks + QK_STEPS/2) + g, d/2
    // dims further, which the same lane holds.
    static __device__ __forceinline__ void rope_q(QRegs& Q, int pos, double rr, int g) {
#pragma unroll
        for (int ks = 0; ks < QK_STEPS / 2; ++ks)
            rope::rot_chunk_pair(Q.q[ks], Q.q[ks + QK_STEPS / 2], 16 * ks + 8 * g, (double)pos, rr);
    }

    // Byte offset in a V tile of this lane's transposing reads for d-block db.
    // ds_read_b64_tr_b16 hands lane 16q + 4a + j element e of the four
    // 16-bit values lane 16q + a + 4e reads, so lane 16q + a + 4e reads key
    // 8 (q/2) + e (plus the k-step's base) at dims 16 (q&1) + 4a .. +3 of the
    // block, and every lane receives V[key][dim l%32] for four keys.
    static __device__ __forceinline__ int v_base(int lane, int db) {
        const int a = lane & 3, e = (lane >> 2) & 3, q = lane >> 4;
        const int row = 8 * (q >> 1) + e;
        const int chunk = (4 * db + 2 * (q & 1) + (a >> 1)) ^ vsw(e);
        return row * RB + chunk * 16 + 8 * (a & 1);
    }

    // The V^T operand of PV product n of a cluster: half hb = n / (2 NDB),
    // k-step kk = (n / NDB) % 2, d-block db = n % NDB (two transposing reads:
    // keys 8 g' + 0..3 and + 4..7 of the k-step).
    static __device__ __forceinline__ bf16x8 v_op(const Buf& S, const int* vb, int n) {
        const int hb = n / (2 * NDB), kk = (n / NDB) % 2, db = n % NDB;
        const char* p = (const char*)S.v + vb[db] + (32 * hb + 16 * kk) * RB;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * RB));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    }

    // The MFMA cluster C: QK_STEPS rounds, each with one step of both S^T
    // chains (K of tile v, Q; starting from 0) and two PV products of tile
    // v-1 (V, P in pk: half hb, k-step kk at pk[2 hb + kk]).  Operands are
    // read LA rounds ahead; mid() runs once, after the first round's MFMAs
    // are issued.
    template <bool QK, bool PV, class Mid>
    static __device__ __forceinline__ void cluster(const Buf& S, const QRegs& Q, const int* vb, const bf16x8* pk,
                                                   int kbe, int kbo, f32x16& a0, f32x16& a1, f32x16* o, Mid&& mid) {
        constexpr int LA = 1;
        constexpr int R = QK_STEPS;
        const char* kbase = (const char*)S.k;
        u32x4 ka[LA + 1], kb[LA + 1];
        bf16x8 va[LA + 1][2];
        auto rd = [&](int i) __attribute__((always_inline)) {
            const int sl = i % (LA + 1);
            if (QK) {
                const char* p = kbase + ((i & 1) ? kbo : kbe) + k_rd_step(i);
                ka[sl] = *(const u32x4*)p;
                kb[sl] = *(const u32x4*)(p + K_HALF);
            }
            if (PV) {
                va[sl][0] = v_op(S, vb, 2 * i);
                va[sl][1] = v_op(S, vb, 2 * i + 1);
            }
        };
#pragma unroll
        for (int i = 0; i < LA; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if (i + LA < R) rd(i + LA);
            const int sl = i % (LA + 1);
            const bf16x8 q = __builtin_bit_cast(bf16x8, Q.q[i]);
            if (QK) a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[sl]), q,
                                                                 i == 0 ? f32x16{} : a0, 0, 0, 0);
            if (PV) {
                const int n = 2 * i;
                o[n % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[sl][0], pk[n / NDB], o[n % NDB], 0, 0, 0);
            }
            if (QK) a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kb[sl]), q,
                                                                 i == 0 ? f32x16{} : a1, 0, 0, 0);
            if (PV) {
                const int n = 2 * i + 1;
                o[n % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[sl][1], pk[n / NDB], o[n % NDB], 0, 0, 0);
            }
            if (i == 0) mid();
            // keep each round's reads ahead of the MFMAs that follow (the
            // scheduler would otherwise sink them next to their uses)
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Eight P values (accumulator elements i0 .. i0+7 of one half) as one
    // bf16x8 operand: exp2 of the scaled, max-shifted scores, packed
    // pairwise; the fp32 values feed this lane's share of the row sum (plain
    // adds: the packed dot-product instructions share the matrix pipe and
    // would stall beside the MFMAs of the other wave).
    static __device__ __forceinline__ bf16x8 pack8(const f32x16& sc, int i0, float c, float mneg, float& l) {
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i0 + i], c, mneg));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i0 + i + 1], c, mneg));
            l += p0 + p1;
            b[i] = (__bf16)p0;
            b[i + 1] = (__bf16)p1;
        }
        return b;
    }

    // Row max over both halves: four independent v_max3 chains of eight
    // values each, then their max (depth 6 instead of 16).
    static __device__ __forceinline__ float max8(const f32x16& x, int i) {
        float m = fmaxf(fmaxf(x[i], x[i + 1]), x[i + 2]);
        m = fmaxf(fmaxf(m, x[i + 3]), x[i + 4]);
        m = fmaxf(fmaxf(m, x[i + 5]), x[i + 6]);
        return fmaxf(m, x[i + 7]);
    }
    static __device__ __forceinline__ float max2x16(const f32x16& x, const f32x16& y) {
        const float m0 = max8(x, 0), m1 = max8(x, 8), m2 = max8(y, 0), m3 = max8(y, 8);
        return fmaxf(fmaxf(fmaxf(m0, m1), m2), m3);
    }

    // Epilogue of one wave: its 32 normalised output rows go to LDS as bf16
    // (row stride RB + 16 bytes, so the 32 rows of one write start in
    // different banks), then to HBM as whole rows, 16 bytes per lane and
    // 64 / (RB / 16) rows per instruction (scattered 8-byte writes of the
    // O^T accumulator layout straight to HBM cost several microseconds per
    // workgroup).  Rows from nvalid on are not stored.
    static constexpr int ORS = RB + 16;
    static __device__ __forceinline__ void store_o(char* lds, __bf16* orow0, uint32_t orsb, const f32x16* o,
                                                   float inv, int lane, int nvalid) {
        const int row = lane & 31, g = lane >> 5;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t v0 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 0] * inv));
                const uint32_t v1 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 1] * inv));
                const uint32_t v2 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 2] * inv));
                const uint32_t v3 = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * q4 + 3] * inv));
                u32x2 w;
                w[0] = v0 | (v1 << 16);
                w[1] = v2 | (v3 << 16);
                *(u32x2*)(lds + row * ORS + 2 * (32 * db + 8 * q4 + 4 * g)) = w;
            }
        }
        // LDS accesses of one wave complete in order; the empty asm keeps
        // the compiler from moving the reads above the writes
        asm volatile("" ::: "memory");
        constexpr int CPR = RB / 16, RPI = 64 / CPR;
        const int rr = lane / CPR, cc = lane % CPR;
#pragma unroll
        for (int i = 0; i < WROWS / RPI; ++i) {
            const int r = RPI * i + rr;
            const u32x4 x = *(const u32x4*)(lds + r * ORS + 16 * cc);
            if (r < nvalid) *(u32x4*)((char*)orow0 + (size_t)r * orsb + 16 * cc) = x;
        }
    }
};

// One 16-byte direct global->LDS load per lane: lane l's chunk lands at
// lds + 16 l (lds is wave-uniform).  Written as inline asm so that the
// compiler, which cannot tell which LDS bytes the load writes, does not make
// every later LDS read wait for it; the kernel waits for these loads itself
// (wait_vm) before the barrier that publishes the tile.
__device__ __forceinline__ void load_lds16(const void* gp, void* lds) {
    const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gp), "s"(la) : "m0");
}

// Same from a wave-uniform base plus a per-lane unsigned byte offset.
__device__ __forceinline__ void load_lds16_off(const void* base, uint32_t off, void* lds) {
    const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(la) : "m0");
}

// Wait until at most n of this wave's vector-memory operations (loads, and
// the fused copy's stores, which this GPU family counts alike and completes
// in issue order) are outstanding.
__device__ __forceinline__ void wait_vm(int n) {
    if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (n == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (n == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else if (n == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// Workgroup barrier without a memory fence (the direct loads are waited
// for explicitly); the empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// What the fused append of a work item needs during the band and at its end
// (see below).
struct FuseInfo {
    __bf16* dst[2];            // the next cache's K and V of the item's (batch, kv-head)
    const __bf16* src[2];      // the item's own K and V rows (row 0 = position pos0)
    const __bf16* csrc[2];     // the current cache's K and V (sink slots below pos0), or null
    int32_t write;             // this item writes the next cache
    int32_t keep_lo;           // first surviving position past the sinks
    int32_t f0, f1;            // the own survivors' full tiles: positions f0 .. f1
    int32_t pz, row0, s, r;
};

template <int D, bool GLB, bool FUSE>
__global__ __launch_bounds__(PNT) void prefill_pp_kernel(PrefillArgs a) {
    typedef PP<D> T;
    __shared__ typename T::Buf smem[NSET];
    __shared__ FuseInfo finfo;

    const int s = a.s, r = a.r;
    const int pos0 = (int)a.pos0;
    const int G = a.Hq / a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, sub = wave & 3;
    const int l32 = lane & 31, g = lane >> 5;

    // ---- work item
    const int w = xcd_work_item(blockIdx.x, gridDim.x);
    // Late (heavier) query tiles first.  In pair mode the q-head pairs of a
    // kv-head are the innermost index: the pairs of one query tile read the
    // same K/V tiles, so running them side by side halves the key range in
    // flight on an XCD and its L2 keeps the tiles for their second reader.
    int mt, b, kvh, h, row0, tok;
    if (a.pair_mode) {
        const int npairs = G / 2;
        const int pair = w % npairs, rest = w / npairs;
        mt = a.n_mtiles - 1 - (rest % a.n_mtiles);
        const int bk = rest / a.n_mtiles;
        b = bk / a.Hkv;
        kvh = bk % a.Hkv;
        h = kvh * G + 2 * pair + grp;
        tok = 128;
        row0 = mt * tok;
    } else {
        mt = a.n_mtiles - 1 - (w % a.n_mtiles);
        const int bh = w / a.n_mtiles;
        b = bh / a.Hq;
        h = bh % a.Hq;
        kvh = h / G;
        tok = 256;
        row0 = mt * tok;
    }
    // Residue classes: the item's batch index is b * dil + c, and the own
    // rows of class c are the positions first(c), first(c) + dil, ... below
    // Lp (first(c) the first position >= pos0 in the class).
    int64_t Lown = a.L, own_off = 0;
    if (a.dil > 1) {
        const int c = b % a.dil;
        b /= a.dil;
        const int64_t first = pos0 + ((c - pos0) % a.dil + a.dil) % a.dil;
        Lown = first < a.Lp ? (a.Lp - 1 - first) / a.dil + 1 : 0;
        own_off = first * D;
    }
    if (row0 >= Lown) return;   // a shorter class's last tile (workgroup-uniform, before any barrier)
    const int nrows = (int)((Lown - row0) < tok ? (Lown - row0) : tok);
    const int t0 = pos0 + row0, t1 = t0 + nrows - 1;                  // the workgroup's rows
    const int wrow0 = row0 + (a.pair_mode ? 0 : 128 * grp) + WROWS * sub;   // this wave's first row (call-relative)
    const int tw0 = pos0 + wrow0;
    const int tw1 = (tw0 + WROWS - 1) < t1 ? (tw0 + WROWS - 1) : t1;
    const bool wave_active = tw0 <= t1;
    const int my_t = tw0 + l32;
    const bool my_valid = my_t <= t1;

    const int64_t rs = a.rs;                                           // elements between own rows
    const size_t qoff = (size_t)(b * a.Hq + h) * a.q_bh + own_off + (size_t)(wrow0 + l32) * rs;
    const __bf16* kn = (const __bf16*)a.kn + (size_t)(b * a.Hkv + kvh) * a.kv_bh + own_off;
    const __bf16* vn = (const __bf16*)a.vn + (size_t)(b * a.Hkv + kvh) * a.kv_bh + own_off;
    const __bf16* kc = a.kc ? (const __bf16*)a.kc + (size_t)(b * a.Hkv + kvh) * a.c_bh : nullptr;
    const __bf16* vc = a.vc ? (const __bf16*)a.vc + (size_t)(b * a.Hkv + kvh) * a.c_bh : nullptr;

    // ---- tiles of the workgroup: phase 0 then phase 1, as one list
    Phase ph0 = {0, -1, 0, NO_BAND, 0}, ph1 = {0, -1, 0, NO_BAND, 0};
    int nph = make_phases(t0, t1, s, r, a.merge_sink != 0, ph0, ph1);
    // Sink packing.  When the sinks would take a tile of their own (they do
    // not touch the band) and the band's first tile starts with at least s
    // keys that every row of the workgroup masks (the keys below
    // t0 - r + 1), the s sink rows are loaded into those slots and the sink
    // tile is dropped: one phase whose keys kb0 .. kb0+s-1 stand for sinks
    // 0 .. s-1.  Only with one set of queries for both (no RoPE).
    int pack_lo = NO_BAND;
    if (a.merge_sink && nph == 2) {
        const int kb0 = ph1.first * BN;
        const int lo = s > t0 - r + 1 ? s : t0 - r + 1;
        if (lo - kb0 >= s) {
            pack_lo = kb0;
            ph0 = Phase{ph1.first, ph1.last, kb0 + s, s, 0};
            nph = 1;
        }
    }
    const int n0 = nph >= 1 ? ph0.last - ph0.first + 1 : 0;
    const int n1 = nph >= 2 ? ph1.last - ph1.first + 1 : 0;
    const int nv = n0 + n1;
    auto phase_of = [&](int v) __attribute__((always_inline)) -> Phase { return v < n0 ? ph0 : ph1; };
    auto tile_of = [&](int v) __attribute__((always_inline)) -> int { return v < n0 ? ph0.first + v : ph1.first + (v - n0); };
    // The tiles of the last phase are one arithmetic run, key tile vo0 + u
    // for run index u in [vo, nv).  The band walks that run rotated: step v
    // takes run index rot(v), the tile whose absolute index is congruent to
    // v - vo modulo the run's length.  The work items that share K/V (the
    // query tiles of one kv-head) have runs of one length offset by a few
    // tiles, so at each step they read the same tile or one of two, which
    // their XCD's L2 then serves; walked in plain order they would read as
    // many tiles as there are items, each again several tiles later.  It
    // also spreads the items' own (last) tiles over the band.  The
    // global-tile instantiation walks in plain order (one more scalar across
    // its band spills inside the loop there).
    const Phase PL = nph >= 2 ? ph1 : ph0;
    const int vo = nph >= 2 ? n0 : 0;
    const int vo0 = PL.first - vo;
    const int nrun = nv - vo;
    int rho = 0;
    if (!GLB && nrun > 1) {
        rho = PL.first % nrun;
        rho = rho == 0 ? 0 : nrun - rho;
    }
    auto rot = [&](int v) __attribute__((always_inline)) -> int {
        if (GLB || v < vo) return v;
        const int u = v + rho;
        return u >= nv ? u - nrun : u;
    };

    // ---- direct loads: a tile's K (or V) is brought in by the 4 waves of
    // one group; wave `sub` issues instructions sub, sub + 4, ...
    int kkey0, kchk, vkey0, vchk;
    T::k_map(sub, lane, kkey0, kchk);
    T::v_map(sub, lane, vkey0, vchk);
    int kbe, kbo;
    T::k_rd_bases(l32, g, kbe, kbo);

    // Loads of tile v's K (or V) into buffer set `set`.  When every query of
    // the workgroup may need every row of the tile and the rows are all in
    // the call's own tokens (contiguous) or all in the rolling part of the
    // cache (slot s + p mod r, one wrap), a direct formula; otherwise each
    // row is clamped to one the tile does need.  A clamped row is real,
    // finite data that the score mask then removes (-inf score, weight 0).
    // Past the last tile the last tile is read again into the given set (a
    // buffer region no later cluster reads), so every wave always issues
    // the same number of loads.
    // (own rows are rsb bytes apart; a tile of own rows spans 64 rsb bytes,
    // which the host keeps below 2^31)
    const uint32_t rsb = (uint32_t)(2 * rs);
    const uint32_t kloff = (uint32_t)kkey0 * rsb + (uint32_t)kchk, vloff = (uint32_t)vkey0 * rsb + (uint32_t)vchk;
    auto issue = [&](auto is_k_c, int v, int set) __attribute__((always_inline)) {
        constexpr bool is_k = decltype(is_k_c)::value;
        u32x4* dst0 = is_k ? smem[set].k : smem[set].v;
        v = rot(v < nv ? v : nv - 1);
        const Phase P = phase_of(v);
        const int kbase = tile_of(v) * BN, klast = kbase + BN - 1;
        const int lo_any = P.band_lo > t0 - r + 1 ? P.band_lo : t0 - r + 1;
        const bool all_needed = klast <= t1 && (kbase >= lo_any || klast < P.sink_hi);
        const __bf16* own = is_k ? kn : vn;
        const __bf16* cache = is_k ? kc : vc;
        const int key0 = is_k ? kkey0 : vkey0;
        const int chk = is_k ? kchk : vchk;
        if (all_needed && kbase >= pos0) {
            // the call's own rows kbase.. (contiguous)
            const __bf16* base = own + (size_t)(kbase - pos0) * rs;
#pragma unroll
            for (int j = 0; j < T::JN; ++j)
                load_lds16_off(base + (size_t)T::JSTEP * j * rs, is_k ? kloff : vloff, dst0 + 64 * (sub + GW * j));
        } else if (all_needed && kbase >= s && klast < pos0) {
            // rolling cache slots s + (p mod r), at most one wrap in a tile
            const __bf16* base = cache + (size_t)s * D;
            const int rel0 = kbase % r;
#pragma unroll
            for (int j = 0; j < T::JN; ++j) {
                int rel = rel0 + key0 + T::JSTEP * j;
                rel = rel >= r ? rel - r : rel;
                load_lds16_off(base, (uint32_t)(rel * T::RB + chk), dst0 + 64 * (sub + GW * j));
            }
        } else {
            // each row clamped to one the tile needs: past t1 -> t1; between
            // the sinks and the band -> the band's first row, or the last
            // sink if the phase has no band rows
            const int gap_to = lo_any <= t1 ? lo_any : P.sink_hi - 1;
#pragma unroll
            for (int j = 0; j < T::JN; ++j) {
                int p = kbase + key0 + T::JSTEP * j;
                p = (p >= P.sink_hi && p < lo_any) ? gap_to : p;
                p = (p >= pack_lo && p < P.sink_hi) ? p - pack_lo : p;   // packed sink slot -> sink row
                p = p < t1 ? p : t1;
                const __bf16* rowp;
                if (p >= pos0) {
                    rowp = own + (size_t)(p - pos0) * rs;
                } else {
                    const int sl = p < s ? p : s + (int)((unsigned)p % (unsigned)r);
                    rowp = cache + (size_t)sl * D;
                }
                load_lds16((const char*)rowp + chk, dst0 + 64 * (sub + GW * j));
            }
        }
    };
    const std::integral_constant<bool, true> K_;
    const std::integral_constant<bool, false> V_;

    // Sub-runs of the last phase's run (in run indices u, see rot) are fixed
    // once per work item so the steady state spends a range check per tile
    // instead of re-deriving the tile's class:
    //   [vf_lo, vf_hi]: every row of the tile is needed by some query of the
    //     workgroup and lies in the call's own tokens, so a tile is one
    //     contiguous 16 KB read (the first branch of issue());
    //   [vx_lo, vx_hi]: every key of the tile is in U(t) of every row of this
    //     wave, so its scores take no mask (cluster_x's full tile);
    //   [vc_lo, vc_hi] (below): the same as the first for the rolling part
    //     of the cache.
    // Tiles outside them (sinks, band edges, a tile straddling the cache's
    // wrap) take the general code.
    auto cdiv = [](int x) __attribute__((always_inline)) { return x >= 0 ? (x + BN - 1) / BN : -((-x) / BN); };
    auto fdiv = [](int x) __attribute__((always_inline)) { return x >= 0 ? x / BN : -((-x + BN - 1) / BN); };
    int vf_lo = 0, vf_hi = -1, vx_lo = 0, vx_hi = -1;
    if (nph > 0 && PL.band_lo != NO_BAND) {
        const int lo_any = PL.band_lo > t0 - r + 1 ? PL.band_lo : t0 - r + 1;
        const int ca = cdiv(lo_any), cp = cdiv(pos0);
        vf_lo = (ca > cp ? ca : cp) - vo0;
        vf_lo = vf_lo > vo ? vf_lo : vo;
        vf_hi = fdiv(t1 - (BN - 1)) - vo0;
        vf_hi = vf_hi < nv - 1 ? vf_hi : nv - 1;
        const int lo_w1 = PL.band_lo > tw1 - r + 1 ? PL.band_lo : tw1 - r + 1;
        vx_lo = cdiv(lo_w1) - vo0;
        vx_lo = vx_lo > vo ? vx_lo : vo;
        vx_hi = fdiv(tw0 - (BN - 1)) - vo0;
        vx_hi = vx_hi < nv - 1 ? vx_hi : nv - 1;
    }
    // The same for the rolling part of the cache (chunked calls): tiles in
    // [vc_lo, vc_hi] have every row needed and all keys in [s, pos0), so
    // tile v holds slots s + (rel(v) .. rel(v) + 63) with rel(v) = key mod r.
    // A band covers fewer than r cached keys, so the run wraps at most once;
    // a tile that does not straddle the wrap is 64 contiguous slots.
    int vc_lo = 0, vc_hi = -1, relc0 = 0;
    if (kc != nullptr && nph > 0 && PL.band_lo != NO_BAND) {
        const int lo_any = PL.band_lo > t0 - r + 1 ? PL.band_lo : t0 - r + 1;
        const int ca = cdiv(lo_any), cs = cdiv(s);
        vc_lo = (ca > cs ? ca : cs) - vo0;
        vc_lo = vc_lo > vo ? vc_lo : vo;
        vc_hi = fdiv(pos0 - BN) - vo0;
        vc_hi = vc_hi < nv - 1 ? vc_hi : nv - 1;
        if (vc_lo <= vc_hi) relc0 = (BN * (vo0 + vc_lo)) % r;
    }
    // issue() with the contiguous runs taken by a pointer step.  The cache
    // runs share the own rows' lane offsets: a call with a cache run (keys
    // in [s, pos0)) has rs = d.  Residue classes set pos0 <= s, which leaves
    // [vc_lo, vc_hi] empty.
    auto issue_run = [&](auto is_k_c, int v, int set) __attribute__((always_inline)) {
        constexpr bool is_k = decltype(is_k_c)::value;
        const int vv = rot(v < nv ? v : nv - 1);
        const __bf16* base = nullptr;
        if (vv >= vf_lo && vv <= vf_hi) {
            base = (is_k ? kn : vn) + (size_t)(BN * (vo0 + vv) - pos0) * rs;
        } else if (vv >= vc_lo && vv <= vc_hi) {
            int rel = relc0 + BN * (vv - vc_lo);
            rel = rel >= r ? rel - r : rel;
            if (rel + BN <= r) base = (is_k ? kc : vc) + (size_t)(s + rel) * D;
        }
        if (base != nullptr) {
            u32x4* dst0 = is_k ? smem[set].k : smem[set].v;
            const uint32_t off = is_k ? kloff : vloff;
#pragma unroll
            for (int j = 0; j < T::JN; ++j)
                load_lds16_off(base, off + (uint32_t)(T::JSTEP * j) * rsb, dst0 + 64 * (sub + GW * j));
        } else {
            issue(is_k_c, v, set);
        }
    };

    // ---- per-wave state
    typename T::QRegs qr;
    int q_loaded = -1, q_raw = -1;
    f32x16 oacc[T::NDB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) oacc[db] = f32x16{};
    int vb[T::NDB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) vb[db] = T::v_base(lane, db);
    float m_c = -__builtin_inff();
    float l_part = 0.0f;
    const float c = a.scale_log2e;
    f32x16 sacc0 = {}, sacc1 = {};     // scores of a tile, from its C to its X cluster
    bf16x8 pk[4];                      // P of a tile, from its X cluster to the next C

    // The queries tile v is scored with.  With RoPE the band phase takes the
    // query rotated to t and the sink phase the query rotated to
    // min(t, s+r-1) (keys are stored rotated at their own positions); the
    // rotated copy is made when the phase changes, from a fresh read of the
    // row (waited for here so no later instruction waits on it), or from the
    // row the prologue read (q_raw: which copy it is meant for).
    //   With one sink tile and every row of the workgroup at or past s+r-1,
    // the sink phase's query position is s+r-1 for all rows, and
    // (R(s+r-1) q) . k = q . (R(-(s+r-1)) k): the sink keys are turned by
    // -(s+r-1) once in LDS (after the prologue's loads), the sink tile is scored with
    // the unrotated query, and the band's copy is the same registers rotated
    // to t, with no second read of the row.
    const bool rope = a.rope_rr > 0.0;
    const bool sink_turn = rope && nph == 2 && ph0.use_qs && ph0.last == 0 && t0 >= s + r - 1;
    auto ensure_q = [&](int v) __attribute__((always_inline)) {
        const int want_q = (rope && phase_of(v).use_qs) ? 1 : 0;
        if (want_q != q_loaded && sink_turn) {
            if (want_q == 0) T::rope_q(qr, my_t, a.rope_rr, g);
            q_loaded = want_q;
        } else if (want_q != q_loaded) {
            if (q_raw != want_q) {
                T::load_q(qr, (const __bf16*)a.q + qoff, my_valid, g);
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            }
            if (rope) {
                const int cap = s + r - 1;
                T::rope_q(qr, want_q ? (my_t < cap ? my_t : cap) : my_t, a.rope_rr, g);
            }
            q_loaded = want_q;
            q_raw = -1;
        }
    };

    // C(v), 1 <= v < nv: PV of tile v-1 and QK of tile v, both from buffer
    // set v % 3, with this group's loads for a later tile issued after the
    // first round.  A tile the wave does not need is still multiplied (its
    // scores are dropped, its weights are 0), which keeps one code path.
    // X(v): online softmax of tile v's scores into pk (zeros when no row of
    // the wave needs the tile); the mask is applied only to tiles that are
    // not inside every row's key set.
    // online softmax of a tile's (masked) scores sacc0/sacc1 into pk
    auto softmax = [&]() __attribute__((always_inline)) {
        const float NEG = -__builtin_inff();
        // P against the running max first: while this lane's weights of the
        // tile sum to at most 2^8 (so each is at most 2^8, as the lazily
        // raised max allows anyway) they stand and the tile needs no row
        // max.  Otherwise, and while a row has no running max yet, the exact
        // row max is taken, the running state rescaled and P recomputed.
        float t = 0.0f;
        bool slow = __builtin_amdgcn_ballot_w64(m_c == NEG) != 0;
        if (!slow) {
            const float mneg = -m_c;
            pk[0] = T::pack8(sacc0, 0, c, mneg, t);
            pk[1] = T::pack8(sacc0, 8, c, mneg, t);
            pk[2] = T::pack8(sacc1, 0, c, mneg, t);
            pk[3] = T::pack8(sacc1, 8, c, mneg, t);
            slow = __builtin_amdgcn_ballot_w64(!(t <= 256.0f)) != 0;
        }
        if (slow) {
            float mx = T::max2x16(sacc0, sacc1);
            mx = max_pair_lanes(mx);
            const float mxc = mx * c;
            const bool upd = mxc > m_c;
            if (__builtin_amdgcn_ballot_w64(upd)) {
                const float alpha = upd ? __builtin_amdgcn_exp2f(m_c - mxc) : 1.0f;
                m_c = upd ? mxc : m_c;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < T::NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            }
            const float mneg = (m_c == NEG) ? 0.0f : -m_c;
            t = 0.0f;
            pk[0] = T::pack8(sacc0, 0, c, mneg, t);
            pk[1] = T::pack8(sacc0, 8, c, mneg, t);
            pk[2] = T::pack8(sacc1, 0, c, mneg, t);
            pk[3] = T::pack8(sacc1, 8, c, mneg, t);
        }
        l_part += t;
    };
    auto cluster_x = [&](int vs) __attribute__((always_inline)) {
        const float NEG = -__builtin_inff();
        const int v = rot(vs);
        if (v < vx_lo || v > vx_hi) {
            // tiles in [vx_lo, vx_hi] are needed and mask-free for every row
            // of the wave; only the others are classified here (the masks
            // leave the scores of the kept keys; softmax() follows)
            const Phase P = phase_of(v);
            const int kb = tile_of(v) * BN;
            const int lo_w0 = P.band_lo > tw0 - r + 1 ? P.band_lo : tw0 - r + 1;
            const int lo_w1 = P.band_lo > tw1 - r + 1 ? P.band_lo : tw1 - r + 1;
            const bool need = kb <= tw1 && (kb < P.sink_hi || kb + 63 >= lo_w0);
            if (!need) {
#pragma unroll
                for (int i = 0; i < 4; ++i) pk[i] = bf16x8{};
                return;
            }
            const bool full = kb + 63 <= tw0 && (kb >= lo_w1 || kb + 63 < P.sink_hi);
            if (!full) {
                // (with the fused append, r through an empty asm: my_t - r +
                // 1 formed here, not held across the loop)
                int r_ = r;
                if constexpr (FUSE) asm volatile("" : "+s"(r_));
                const int lo_me = P.band_lo > my_t - r_ + 1 ? P.band_lo : my_t - r_ + 1;
                const int kbg = kb + 8 * g;
                const int lim_t = my_t - kbg, lim_s = P.sink_hi - kbg, lim_b = lo_me - kbg;
                // Most cut tiles hold no sinks and cut one edge only: the
                // diagonal (every row's window reaches below the tile: keep
                // k <= t) or the window's lower edge (the tile is below every
                // row: keep k >= t - r + 1); one compare per score there.
                const bool no_sink = kb >= P.sink_hi;
                if (no_sink && kb >= lo_w1) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int k0 = keyoff(i, 0), k1 = 32 + keyoff(i, 0);
                        sacc0[i] = k0 <= lim_t ? sacc0[i] : NEG;
                        sacc1[i] = k1 <= lim_t ? sacc1[i] : NEG;
                    }
                } else if (no_sink && kb + 63 <= tw0) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int k0 = keyoff(i, 0), k1 = 32 + keyoff(i, 0);
                        sacc0[i] = k0 >= lim_b ? sacc0[i] : NEG;
                        sacc1[i] = k1 >= lim_b ? sacc1[i] : NEG;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int k0 = keyoff(i, 0), k1 = 32 + keyoff(i, 0);
                        sacc0[i] = (k0 <= lim_t && (k0 < lim_s || k0 >= lim_b)) ? sacc0[i] : NEG;
                        sacc1[i] = (k1 <= lim_t && (k1 < lim_s || k1 >= lim_b)) ? sacc1[i] : NEG;
                    }
                }
            }
        }
        softmax();
    };

    // ---- schedule.  Half-slot hs: group 0 runs C(v) at hs = 2v and X(v) at
    // 2v+1, group 1 runs X(v-1) at 2v and C(v) at 2v+1; a barrier ends every
    // half-slot.  C(v) reads K of tile v and V of tile v-1 from set v % 3
    // during half-slots 2v and 2v+1.  The softmax half-slots also carry the
    // direct loads (their waves have issue slots to spare): group 1 fetches
    // K of tile v+2 at 2v and group 0 V of tile v+1 at 2v+1, both into set
    // (v+2) % 3 (last read at 2v-1); a wave ends each half-slot waiting for
    // all but its latest batch of loads, so every batch lands at least one
    // barrier before its first reader.  C(0) (no PV) and C(nv) (no QK) are
    // peeled off the loop.
    int n_last = 0;
    if (nv > 0) {
        // the queries of tile 0 travel with the first tiles' loads
        if (wave_active) {
            T::load_q(qr, (const __bf16*)a.q + qoff, my_valid, g);
            if (a.rope_rr > 0.0)
                q_raw = phase_of(0).use_qs ? 1 : 0;   // rotated in ensure_q, after the prologue's wait
            else
                q_loaded = 0;
        }
        if (grp == 0) {
            issue(K_, 0, 0);
            issue(V_, 0, 1);
        } else if (nv > 1) {
            issue(K_, 1, 1);
        }
    }
    wait_vm(0);
    wg_barrier();
    if (sink_turn) {
        // one wave turns the s sink rows of tile 0 (set 0) by -(s+r-1); a
        // lane takes one chunk pair (dims 8 cp .. and their partners d/2
        // further) of one key, at the key's place in the K tile layout
        if (wave == 0) {
            constexpr int NPAIR = T::CH / 2;
            char* kt = (char*)smem[0].k;
            for (int u = lane; u < s * NPAIR; u += 64) {
                const int j = u / NPAIR, cp = u % NPAIR;
                const int rho = T::krow(j), blk = rho / T::RPB;
                char* rowb = kt + blk * 1024 + (rho % T::RPB) * 16;
                u32x4* lo = (u32x4*)(rowb + (cp ^ T::ksw(blk)) * 16 * T::RPB);
                u32x4* hi = (u32x4*)(rowb + ((cp + NPAIR) ^ T::ksw(blk)) * 16 * T::RPB);
                u32x4 x0 = *lo, x1 = *hi;
                rope::rot_chunk_pair(x0, x1, 8 * cp, -(double)(s + r - 1), a.rope_rr);
                *lo = x0;
                *hi = x1;
            }
        }
        __syncthreads();
    }
    // Fused append (the FUSE instantiation, kc_next set): the workgroup's own key and
    // value rows that survive the call (positions from pos0 + L - r on, and
    // those below s) go to their slots of the next cache; the items of the
    // kv-head's first q-head (pair, in pair mode) write them (the other
    // q-heads' items have the same rows).  Tiles of the band whose 64 rows
    // are all own rows that survive are copied from LDS while resident:
    // group 0 takes the K rows of tile v in its X(v) half-slot (K of tile v
    // sits in set v % 3 through half-slot 2v+1), group 1 the V rows in its
    // X(v) (V of tile v sits in set (v+1) % 3 from 2v+2 to 2v+4); the wave
    // issues its NS stores after its tile loads and the half-slot's wait
    // counts them.  The other surviving rows (a partial tile at either end
    // of the item, positions below s, and in the item of the first query
    // tile the cache's sink slots below pos0) are copied from global memory
    // at the end.  What the copy needs is put in LDS by thread 0 before the
    // band (held in scalar registers across it, it would crowd them).
    constexpr int NS = 16 * T::CH / 64;        // stores per lane: 16 rows of a tile per wave
    if constexpr (FUSE) {
        if (tid == 0) {
            // one writer per row: the kv-head's first q-head (pair)
            const bool w = a.kc_next != nullptr && h - kvh * G < (a.pair_mode ? 2 : 1);
            finfo.write = w ? 1 : 0;
            if (w) {
                finfo.dst[0] = (__bf16*)a.kc_next + (size_t)(b * a.Hkv + kvh) * a.c_bh;
                finfo.dst[1] = (__bf16*)a.vc_next + (size_t)(b * a.Hkv + kvh) * a.c_bh;
                finfo.src[0] = kn;
                finfo.src[1] = vn;
                finfo.csrc[0] = kc;
                finfo.csrc[1] = vc;
                const int64_t keep = pos0 + a.L - r;
                const int klo = (int)(keep > s ? keep : s);
                const int a0 = t0 > klo ? t0 : klo;                // first own survivor past the sinks
                finfo.keep_lo = klo;
                finfo.f0 = (a0 + BN - 1) / BN * BN;                 // full tiles: [f0, f1]
                finfo.f1 = (t1 + 1) / BN * BN - 1;
                finfo.pz = pos0;
                finfo.row0 = row0;
                finfo.s = s;
                finfo.r = r;
            }
        }
        // the record is written before the wave's next barrier
        if (wave == 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // X(v)'s copy of tile v (K for group 0, V for group 1) when all its rows
    // are own survivors of the item
    auto copy_own = [&](int vs, int cset) __attribute__((always_inline)) {
        if constexpr (FUSE) {
            const int v = rot(vs);
            const int kb = tile_of(v) * BN;
            if (kb + BN - 1 > t1 || kb < t0 || v < vo) return;       // not all own rows (or a sink-phase tile)
            if (__builtin_amdgcn_readfirstlane(finfo.write) == 0) return;
            if (kb < __builtin_amdgcn_readfirstlane(finfo.f0)) return;
            const int sz = __builtin_amdgcn_readfirstlane(finfo.s), rz = __builtin_amdgcn_readfirstlane(finfo.r);
            // the next cache's base as a wave-uniform global pointer; each
            // half goes through uint32_t (readfirstlane returns int, whose
            // widening would sign-extend the low half into the high one)
            typedef __attribute__((address_space(1))) char gchar;
            typedef __attribute__((address_space(1))) u32x4 gu32x4;
            const uint64_t dp = (uint64_t)(uintptr_t)finfo.dst[grp];
            const uint64_t dlo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)dp);
            const uint64_t dhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(dp >> 32));
            gchar* dstb = (gchar*)(uintptr_t)((dhi << 32) | dlo) + (size_t)sz * T::RB;
            const char* tile = grp == 0 ? (const char*)smem[cset].k : (const char*)smem[cset].v;
            const int rel0 = kb % rz;                                   // slot of row 0 is sz + rel0 (one wrap at most)
#pragma unroll
            for (int it = 0; it < NS; ++it) {
                const int u = lane + 64 * it, ch = u % T::CH;
                const int row = 16 * sub + u / T::CH;                   // key kb + row
                int off;
                if (grp == 0) {
                    const int rho = T::krow(row), blk = rho / T::RPB;
                    off = blk * 1024 + (ch ^ T::ksw(blk)) * 16 * T::RPB + (rho % T::RPB) * 16;
                } else {
                    off = row * T::RB + (ch ^ T::vsw(row)) * 16;
                }
                const u32x4 x = *(const u32x4*)(tile + off);
                int rel = rel0 + row;
                rel = rel >= rz ? rel - rz : rel;
                // a uniform base and a 32-bit lane offset (one address register)
                *(gu32x4*)(dstb + (uint32_t)(rel * T::RB + 16 * ch)) = x;
                // one chunk in registers at a time (the softmax's values are live)
                __builtin_amdgcn_sched_barrier(0);
            }
            n_last += NS;
        }
    };
    // the rest at the end, from global memory: own survivors outside the
    // full tiles, own positions below s, the cache's sinks below pos0
    auto fuse_tail = [&]() __attribute__((always_inline)) {
        if constexpr (FUSE) {
            if (__builtin_amdgcn_readfirstlane(finfo.write) == 0) return;
            const int sz = finfo.s, rz = finfo.r, pz = finfo.pz, row0f = finfo.row0;
            const int t0f = pz + row0f, t1f = t1;
            const int a0 = t0f > finfo.keep_lo ? t0f : finfo.keep_lo, f0 = finfo.f0, f1 = finfo.f1;
            __bf16* dst = finfo.dst[grp];
            const __bf16* src = finfo.src[grp];
            const int gt = tid & 255;
            auto rows = [&](int p0, int p1, bool sink) __attribute__((always_inline)) {
                for (int u = gt; u < (p1 - p0 + 1) * T::CH; u += 256) {
                    const int p = p0 + u / T::CH, ch = u % T::CH;
                    const int slot = sink ? p : sz + p % rz;
                    *(u32x4*)(dst + (size_t)slot * D + 8 * ch) = *(const u32x4*)(src + (size_t)(p - pz) * D + 8 * ch);
                }
            };
            if (f0 > f1) {
                rows(a0, t1f, false);                                   // no full tile
            } else {
                rows(a0, f0 - 1, false);
                rows(f1 + 1, t1f, false);
            }
            if (t0f < sz) rows(t0f, (sz - 1) < t1f ? sz - 1 : t1f, true);
            const __bf16* cs = finfo.csrc[grp];
            if (row0f == 0 && cs != nullptr) {
                const int ns = sz < pz ? sz : pz;
                for (int u = gt; u < ns * T::CH; u += 256) {
                    const int j = u / T::CH, ch = u % T::CH;
                    *(u32x4*)(dst + j * D + 8 * ch) = *(const u32x4*)(cs + j * D + 8 * ch);
                }
            }
        }
    };

    auto end_half = [&]() __attribute__((always_inline)) {
        wait_vm(n_last);
        wg_barrier();
    };
    // this group's X half-slot: its loads (group 1 at hs = 2v: K of tile
    // v+2; group 0 at hs = 2v+1: V of tile v+1; both into set (v+2) % 3),
    // then the softmax of tile vx
    auto x_half = [&](auto is_k_c, int vx, int v, int nset, int cset) __attribute__((always_inline)) {
        n_last = T::JN;
        issue_run(is_k_c, decltype(is_k_c)::value ? v + 2 : v + 1, nset);
        if (wave_active && vx >= 0) cluster_x(vx);
        if (FUSE && vx >= 0) copy_own(vx, cset);
    };

    // Whether some row of this wave has a key of tile v in its key set.  The
    // products of a tile no row needs are skipped (its scores would be
    // dropped and its weights are zero): the workgroup visits the union of
    // its waves' tiles, and the matrix work saved also lets the clock run
    // higher.
    auto wave_needs = [&](int vs) __attribute__((always_inline)) -> bool {
        const int v = rot(vs);
        if (v >= vx_lo && v <= vx_hi) return true;
        const Phase P = phase_of(v);
        const int kb = tile_of(v) * BN;
        const int lo_w0 = P.band_lo > tw0 - r + 1 ? P.band_lo : tw0 - r + 1;
        return kb <= tw1 && (kb < P.sink_hi || kb + BN - 1 >= lo_w0);
    };
    auto c_first = [&]() __attribute__((always_inline)) {
        if (wave_active && wave_needs(0)) {
            ensure_q(0);
            T::template cluster<true, false>(smem[0], qr, vb, pk, kbe, kbo, sacc0, sacc1, oacc, [] {});
        }
    };
    auto c_mid = [&](int v, int set) __attribute__((always_inline)) {
        if (wave_active && (wave_needs(v) || wave_needs(v - 1))) {
            ensure_q(v);
            T::template cluster<true, true>(smem[set], qr, vb, pk, kbe, kbo, sacc0, sacc1, oacc, [] {});
        }
    };
    auto c_last = [&](int set) __attribute__((always_inline)) {
        if (wave_active && wave_needs(nv - 1))
            T::template cluster<false, true>(smem[set], qr, vb, pk, kbe, kbo, sacc0, sacc1, oacc, [] {});
    };
    if (nv > 0) {
        if (grp == 0) {
            c_first();
            end_half();
            x_half(V_, 0, 0, 2, 0);
            end_half();
            int set = 1;                       // v % 3
            for (int v = 1; v < nv; ++v) {
                const int nset = set == 0 ? 2 : set - 1;   // (v + 2) % 3
                c_mid(v, set);
                end_half();
                x_half(V_, v, v, nset, set);
                end_half();
                set = set == 2 ? 0 : set + 1;
            }
            n_last = 0;
            c_last(set);
            end_half();
            end_half();
        } else {
            x_half(K_, -1, 0, 2, 0);
            end_half();
            c_first();
            end_half();
            int set = 1;
            for (int v = 1; v < nv; ++v) {
                const int nset = set == 0 ? 2 : set - 1;
                x_half(K_, v - 1, v, nset, set);
                end_half();
                c_mid(v, set);
                end_half();
                set = set == 2 ? 0 : set + 1;
            }
            x_half(K_, nv - 1, nv, set == 0 ? 2 : set - 1, set);
            end_half();
            c_last(set);
            end_half();
        }
    }

    // Task-bound global tokens: the gathered global keys at or past s (kc /
    // vc point at the [64, d] blocks in calls with globals) as one more tile
    // after the band, once per item with no ping-pong: row t keeps rows 0 ..
    // gjb[t]-1 of the block, the globals below its window.
    if constexpr (GLB) {
        if (nv > 0 && __builtin_amdgcn_readfirstlane((int)a.gjb[t1]) > 0) {
            wait_vm(0);
            wg_barrier();                  // every tile read is done: set 0 is free
            {
                // group 0 loads K, group 1 V (rows 0 .. 63, contiguous; a
                // call with globals has rs = d, so the own-row offsets fit)
                const bool is_k = grp == 0;
                const __bf16* base = is_k ? kc : vc;
                u32x4* dst0 = is_k ? smem[0].k : smem[0].v;
#pragma unroll
                for (int j = 0; j < T::JN; ++j)
                    load_lds16_off(base + (size_t)T::JSTEP * j * D, is_k ? kloff : vloff, dst0 + 64 * (sub + GW * j));
            }
            wait_vm(0);
            wg_barrier();
            if (wave_active && __builtin_amdgcn_readfirstlane((int)a.gjb[tw1]) > 0) {
                // lane-derived offsets formed again here (held across the
                // band's last products they would cost registers there)
                int ln = (int)threadIdx.x & 63;
                asm volatile("" : "+v"(ln));
                int gbe, gbo;
                T::k_rd_bases(ln & 31, ln >> 5, gbe, gbo);
                T::template cluster<true, false>(smem[0], qr, vb, pk, gbe, gbo, sacc0, sacc1, oacc, [] {});
                const int tt = tw0 + (ln & 31);
                const int lim = (int)a.gjb[tt < t1 ? tt : t1] - 8 * (ln >> 5);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int k0 = keyoff(i, 0), k1 = 32 + keyoff(i, 0);
                    sacc0[i] = k0 < lim ? sacc0[i] : -__builtin_inff();
                    sacc1[i] = k1 < lim ? sacc1[i] : -__builtin_inff();
                }
                softmax();
                T::template cluster<false, true>(smem[0], qr, vb, pk, kbe, kbo, sacc0, sacc1, oacc, [] {});
            }
        }
    }

    // the buffers take the output rows once every load has landed and every
    // wave is past its last read
    wait_vm(0);
    wg_barrier();
    if (wave_active) {
        const float l_tot = l_part + __shfl_xor(l_part, 32);
        static_assert(PW * WROWS * T::ORS <= (int)sizeof(smem), "output staging fits the tile buffers");
        T::store_o((char*)smem + wave * WROWS * T::ORS, (__bf16*)a.o + qoff - (size_t)l32 * rs, rsb, oacc,
                   my_valid ? 1.0f / l_tot : 0.0f, lane, tw1 - tw0 + 1);
    }
    if constexpr (FUSE) fuse_tail();
}
template <int D>
hipError_t launch(const PrefillArgs& a, hipStream_t st) {
    const long long G = a.Hq / a.Hkv;
    const long long nblk = a.pair_mode ? (long long)a.B * a.Hkv * (G / 2) * a.n_mtiles
                                       : (long long)a.B * a.Hq * a.n_mtiles;
    if (a.ng > 0)
        hipLaunchKernelGGL((prefill_pp_kernel<D, true, false>), dim3((unsigned)nblk), dim3(PNT), 0, st, a);
    else if (a.kc_next != nullptr)
        hipLaunchKernelGGL((prefill_pp_kernel<D, false, true>), dim3((unsigned)nblk), dim3(PNT), 0, st, a);
    else
        hipLaunchKernelGGL((prefill_pp_kernel<D, false, false>), dim3((unsigned)nblk), dim3(PNT), 0, st, a);
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
