// Operand fragments of v_mfma_f32_32x32x16_bf16 loaded in 64-byte runs.
//
// Either operand of the 32x32x16 MFMA gives lane l the 8 bf16 of row (l & 31)
// at k-chunk (l >> 5) of the step: a load in that layout reads 32 rows, 16
// bytes from each, and the address unit takes it as 64 separate pieces. The
// kernels that load their operands from global memory straight into
// registers (the small-T projections, with W and x rows kept in registers
// for a whole k range) spent microseconds of address-unit time on such
// loads: 80 blocks loading a 160 KB W slice each, in 160 loads per block,
// took about 4.4 us, and the same bytes in 64-byte runs about 1.2 us.
//
// Run layout. For a wave's k range of 8 n-element chunks (chunk c holds k
// elements 8c .. 8c+7 of the range) and 32 rows, register q, lane l loads row
// run_row(q, l) = (q & 3) + (l & 28) at chunk run_chunk(q, l) =
// (l >> 5) + 2 (l & 3) + 8 (q >> 2): four neighbouring lanes read one 64-byte
// run of one row. In bits (rows r0..r4, chunks c0..), the run layout has
// lane bits l0, l1 = c1, c2 and register bits q0, q1 = r0, r1, where the MFMA
// layout has l0, l1 = r0, r1 and q0, q1 = c1, c2; everything else agrees.
// Two exchanges of a lane bit with a register bit (l0 with q0, l1 with q1)
// turn one into the other: afterwards register q, lane l holds row (l & 31),
// chunk 2q + (l >> 5), the fragment of k-step q.
//
// One exchange of lane bit b between registers x (register bit 0) and y
// (register bit 1): on lanes with bit b set, x takes y from lane l ^ b and y
// keeps its value; on the others, y takes x from lane l ^ b and x keeps its
// value. Each output is one v_cndmask_b32 with a DPP quad_perm source
// (swapping lanes l and l ^ 1, or l and l ^ 2) under a lane mask in VCC.
// It is written as inline assembly: the compiler selects with a 64-bit
// SGPR mask, the VOP3 form, which takes no DPP operand, and so spends a
// separate DPP move on every value. The s_nop gives the two wait states a
// DPP read needs after a VALU write of the same register.
#pragma once

#include "ple_kernels.h"

namespace ple {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int run_row(int q, int lane) { return (q & 3) + (lane & 28); }
__device__ __forceinline__ int run_chunk(int q, int lane) { return (lane >> 5) + 2 * (lane & 3) + 8 * (q >> 2); }

#define PLE_LANE_SWAP_ASM(QP)                                                                        \
    asm volatile("s_nop 1\n\t"                                                                        \
                 "s_mov_b64 vcc, %16\n\t"                                                             \
                 "v_cndmask_b32_dpp %4, %8, %12, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_cndmask_b32_dpp %5, %9, %13, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_cndmask_b32_dpp %6, %10, %14, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_cndmask_b32_dpp %7, %11, %15, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "s_mov_b64 vcc, %17\n\t"                                                             \
                 "v_cndmask_b32_dpp %0, %12, %8, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_cndmask_b32_dpp %1, %13, %9, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_cndmask_b32_dpp %2, %14, %10, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_cndmask_b32_dpp %3, %15, %11, vcc " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1"      \
                 : "=&v"(nx[0]), "=&v"(nx[1]), "=&v"(nx[2]), "=&v"(nx[3]),                                \
                   "=&v"(ny[0]), "=&v"(ny[1]), "=&v"(ny[2]), "=&v"(ny[3])                                 \
                 : "v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]),                                        \
                   "v"(yv[0]), "v"(yv[1]), "v"(yv[2]), "v"(yv[3]), "s"(m), "s"(~m)                        \
                 : "vcc")

// exchange lane bit BIT (1 or 2) with the register bit that tells x from y;
// m has bit l set for the lanes l with that lane bit set
template <int BIT>
__device__ __forceinline__ void lane_swap(bf16x8& x, bf16x8& y, uint64_t m) {
    static_assert(BIT == 1 || BIT == 2, "lane bit 0 or 1");
    const u32x4 xv = __builtin_bit_cast(u32x4, x), yv = __builtin_bit_cast(u32x4, y);
    u32x4 nx, ny;
    if (BIT == 1) PLE_LANE_SWAP_ASM("quad_perm:[1,0,3,2]");
    else PLE_LANE_SWAP_ASM("quad_perm:[2,3,0,1]");
    x = __builtin_bit_cast(bf16x8, nx);
    y = __builtin_bit_cast(bf16x8, ny);
}
#undef PLE_LANE_SWAP_ASM

// N registers loaded in the run layout -> the MFMA fragments of k-steps
// 0 .. N-1 (128 VALU instructions per 16 registers)
template <int N>
__device__ __forceinline__ void runs_to_fragments(bf16x8 (&f)[N]) {
    static_assert(N % 4 == 0, "register bits 0 and 1 pair the registers in groups of four");
#pragma unroll
    for (int q = 0; q < N; q += 2) lane_swap<1>(f[q], f[q + 1], 0xAAAAAAAAAAAAAAAAull);
#pragma unroll
    for (int q = 0; q < N; ++q)
        if (!(q & 2)) lane_swap<2>(f[q], f[q + 2], 0xCCCCCCCCCCCCCCCCull);
}

}  // namespace ple
