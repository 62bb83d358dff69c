// 32x32 MFMA block tiles in LDS and their operand reads, shared by the
// gfx950 backward kernels, which tile on v_mfma_f32_32x32x16_bf16.
//
// Rows of an MFMA block enter in the order swap23(m) (bits 2 and 3 of the
// row index swapped), so that each lane's eight accumulator values of one
// half are eight consecutive rows: the score accumulators are then the bf16
// B operands of the next products as they are.  Block tiles are row-major
// with the 16-byte chunks of row r rotated by sw(r), which keeps both the
// row reads (16 rows x one chunk) and the transposing reads
// (ds_read_b64_tr_b16: 4 rows x 64 bytes per 32 lanes) free of LDS bank
// conflicts; they are filled by direct global->LDS loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {
namespace mt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int NW = 4;              // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int BLK = 32;            // rows of an MFMA block
constexpr int NBUF = 3;            // LDS buffer sets

__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
// Block row held by accumulator element i of lane group g (rows fed in swap23 order).
__device__ __forceinline__ constexpr int crow(int i, int g) { return 16 * (i / 8) + 8 * g + (i % 8); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float pair_max(float x) {
    // max of lanes l and l^32 (v_permlane32_swap hands each lane both halves)
    const uint32_t xb = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
    return fmaxf(x, fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1])));
}
__device__ __forceinline__ float pair_sum(float x) {
    // x of lane l plus x of lane l^32 (the swap hands each lane both)
    const uint32_t xb = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
    return __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
}

// Maps blockIdx to a work item so that each XCD (blocks are dealt to the 8
// XCDs round-robin) gets one contiguous run of work items, whose operand
// tiles then share that XCD's L2.
__device__ __forceinline__ int xcd_item(int bid, int nblk) {
    const int x = bid & 7, k = bid >> 3;
    const int per = nblk >> 3, rem = nblk & 7;
    return x * per + (x < rem ? x : rem) + k;
}

// One 16-byte direct global->LDS load per active lane: lane l's chunk lands
// at lds + 16 l (lds is wave-uniform).  The kernels wait for these loads
// themselves (wait_vm) before the barrier that publishes a block.
__device__ __forceinline__ void load_lds16(const void* gp, void* lds) {
    const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gp), "s"(la) : "m0");
}

// Wait until at most n of this wave's vector-memory loads are outstanding.
__device__ __forceinline__ void wait_vm(int n) {
    if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (n == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (n == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
}

__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A block tile: 32 rows of D bf16 values, row-major, the 16-byte chunk c of
// row r stored at chunk c ^ sw(r).
template <int D>
struct Tile {
    static constexpr int CH = D / 8;         // chunks per row
    static constexpr int KS = D / 16;        // k-steps over the head dim
    static constexpr int NDB = D / 32;       // 32-dim blocks
    static constexpr int RB = D * 2;         // bytes per row
    static constexpr int BYTES = BLK * RB;
    static constexpr int NINS = BYTES / 1024;  // direct-load instructions per tile
    static constexpr int JW = NINS / NW;       // ... per wave
    static_assert(JW >= 1 && NINS % NW == 0, "tile shape");

    static __device__ __forceinline__ int sw(int r) {
        return D == 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
    }
    static __device__ __forceinline__ int off(int r, int c) { return r * RB + ((c ^ sw(r)) << 4); }

    // Row operand of k-step ks for MFMA row l32 (tile row swap23(l32), dims
    // 16 ks + 8 g .. +7): the A operand of a product over the head dim.
    static __device__ __forceinline__ bf16x8 rowop(const char* t, int l32, int g, int ks) {
        return *(const bf16x8*)(t + off(swap23(l32), 2 * ks + g));
    }

    // Column operand of k-step ks for MFMA column l32 (tile row l32, dims
    // 16 ks + 8 g .. +7): the B operand of a product over the head dim.
    static __device__ __forceinline__ bf16x8 colop(const char* t, int l32, int g, int ks) {
        return *(const bf16x8*)(t + off(l32, 2 * ks + g));
    }

    // Transposed operand [dim x row] of d-block db, k-step kk: lane (l32, g)
    // gets dim 32 db + l32 of tile rows 16 kk + 8 g .. +7.  ds_read_b64_tr_b16
    // hands lane 16q + 4a + j element e of the four values lane 16q + a + 4e
    // reads; that lane reads row 16 kk + 8 (q / 2) + e (+4 for the second
    // read), dims 32 db + 16 (q & 1) + 4a .. +3.
    static __device__ __forceinline__ bf16x8 trop(const char* t, int lane, int db, int kk) {
        const int a = lane & 3, e = (lane >> 2) & 3, q = lane >> 4;
        const int row = 16 * kk + 8 * (q >> 1) + e;
        const int c = 4 * db + 2 * (q & 1) + (a >> 1);
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + off(row, c) + 8 * (a & 1)));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + off(row + 4, c) + 8 * (a & 1)));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    }

    // This wave's share of the direct loads of a tile whose row x is global
    // row base + clamp(row0 + x) (clamped into [lo, hi]; a clamped row is
    // real data the masks then drop).
    static __device__ __forceinline__ void load(char* t, const __bf16* base, int row0, int lo, int hi, int wave,
                                                int lane) {
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int ins = wave + NW * j;
            const int x = 64 * ins + lane;
            const int r = x / CH, phys = x % CH;
            int gr = row0 + r;
            gr = gr < lo ? lo : (gr > hi ? hi : gr);
            load_lds16(base + (size_t)gr * D + 8 * (phys ^ sw(r)), t + 1024 * ins);
        }
    }
};

}  // namespace mt
}  // namespace swa
