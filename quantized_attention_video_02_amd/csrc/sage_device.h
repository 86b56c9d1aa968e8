// Device helpers shared by the attention kernels (forward and backward):
// the XCD-aware workgroup order, the direct global -> LDS tile copies and the
// lane-pair reductions of the 32x32 accumulator layout.
#pragma once

#include "sage_common.h"

namespace sage {

// The hardware hands workgroup IDs to the 8 XCDs round-robin (bid % 8).
// Renumber so that XCD x runs a contiguous range of logical workgroups:
// consecutive Q tiles of one head then share that XCD's L2 for K and V.
__device__ inline int xcd_remap(int bid, int total) {
    constexpr int nx = 8;
    const int q = total / nx, r = total % nx, x = bid % nx, s = bid / nx;
    return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

typedef __attribute__((address_space(3))) void lds_void;

// Source offset (bytes, inside the HBM tile) of the 16-byte chunk that lands in
// LDS slot P of a padded tile: LDS row P / (STR/16), chunk P % (STR/16); the
// pad chunk of each row takes a duplicate of the row's first chunk.
template <int ROW, int STR>
__device__ inline int slot_src(int P) {
    constexpr int CPR = STR / 16;
    const int row = P / CPR, c = P % CPR;
    return row * ROW + (c < ROW / 16 ? 16 * c : 0);
}

// One 1 KB piece of a tile, global -> LDS: global_load_lds_dwordx4 with the LDS
// destination in M0, lane i filling bytes [16 i, 16 i + 16) of the piece.
// Issued from asm: the compiler cannot tell these in-flight writes from the
// other LDS buffer's reads and would otherwise wait for every copy before the
// next LDS read.  Completion is awaited explicitly (wait_vmem before the
// barrier that publishes the buffer).  The asm has no register outputs.
__device__ inline void dma_piece(const uint8_t* gbase, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(gbase), "s"(lds)
        : "memory", "m0");
}

// This wave's pieces of a tile: piece J = wave + NW j.  g and l are uniform.
template <int NPIECES, int MAXP, int NW>
__device__ inline void tile_to_lds(const uint8_t* g, uint32_t l, int wave, const int* off) {
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        const int J = wave + NW * j;
        if (J < NPIECES) dma_piece(g, (uint32_t)off[j], l + 1024u * J);
    }
}

__device__ inline void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// An empty use of x at this point of the program: everything that computes x
// happens before it.  (In a __device__ function: the host pass never
// generates code for it.)
__device__ inline void consume(const v16f& x) { asm volatile("" ::"v"(x)); }

// Value of lane ^ 32 combined with this lane's (v_permlane32_swap: the two
// halves of the wave exchange registers; both results hold one value from
// each half, so max/sum of the pair is the same on both lanes).
__device__ inline int pair_max(int x) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ inline float pair_fmax(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace sage
