// MFMA building blocks for the attention kernels (gfx950 wave64).
//
// Lane layouts (checked on the device by a layout probe):
//  v_mfma_f32_32x32x16_bf16: A[m][k] in lane (m = l%32), k = 8*(l/32) + e,
//    e = 0..7; B[k][n] in lane (n = l%32), k = 8*(l/32) + e; C[m][n] in lane
//    (n = l%32), register i holds m = 8*(i/4) + 4*(l/32) + i%4.
//  v_mfma_f32_32x32x2_f32: as above with one k per lane, k = l/32.
//
// Scores are formed transposed (S^T = K Q^T), so the C layout puts one query
// per lane column: the softmax row statistics of a query live in one lane
// pair (l, l^32).  P^T in C layout is then directly the B operand of
// O^T = V^T P^T, with the contraction over the keys taken in the order the
// C layout holds them; the A operand (V^T) is read in the same order.
// Operands that run down the columns of a row-major tile (V^T, Q^T, dO^T,
// K^T) are read from that same tile with the LDS transpose read
// ds_read_b64_tr_b16 (layout below), so every tile is staged once,
// row-major.
//
//  ds_read_b64_tr_b16 (checked on the device; independent of the addresses):
//    in each group of 16 lanes, lane i receives element i%4 of the 8-byte
//    chunks fetched by lanes i/4 + 4j of its group, j = 0..3, as its
//    elements j.  So if lane c + 4j of a group fetches 4 columns starting at
//    4c of row j, lane i ends up with column i of rows 0..3.
//
// LDS tiles are unpadded and XOR-swizzled in 16-byte slots (Swz), and are
// filled by the memory unit straight from global memory (global_load_lds, 16
// bytes per lane): a wave instruction writes 1 KB of contiguous LDS, so the
// swizzle is applied by choosing which global slot each lane fetches.
#pragma once

#include "zz_device.h"

namespace zz {

// Key offset (inside a 32-key score block) of C register i in lane half hh.
__device__ __forceinline__ constexpr int c_row(int i, int hh) { return 8 * (i / 4) + 4 * hh + (i % 4); }

// c_row(i, hh) = c_row0(i) + 4*hh.
__device__ __forceinline__ constexpr int c_row0(int i) { return 8 * (i / 4) + (i % 4); }

// Masks on a 32-row block in C layout, with a per-lane bound already shifted
// by the lane half (bound - 4*hh): one compare with an immediate per register,
// so nothing per register stays live across a loop.
// Rows c_row(i, hh) > bound get -inf.
__device__ __forceinline__ void mask_rows_above(f32x16 &x, int bound_hh) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (c_row0(i) > bound_hh) x[i] = -INFINITY;
}
// Rows c_row(i, hh) < bound get -inf.
__device__ __forceinline__ void mask_rows_below(f32x16 &x, int bound_hh) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (c_row0(i) < bound_hh) x[i] = -INFINITY;
}

// Exchange a value with lane l^32.
__device__ __forceinline__ float swap_halves(float x, int lane) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// Tile rows of W 16-byte slots, unpadded: logical slot s of row r sits at
// slot r*W + (s ^ key(r)).  The key is chosen so that both read patterns of
// the kernels touch each 16-byte group of a 256-byte bank window once:
//  - row reads: 16 consecutive rows (aligned to 16) at one logical slot;
//  - transpose reads: 4 consecutive rows (aligned to 4) x 4 consecutive
//    slots (aligned to 4).
// For W <= 16 a row covers W groups of the window and 16/W rows share one
// window; key = 4 * ((r / (16/W)) % (W/4)) + (r/4) % 4 puts the rows of an
// aligned 4-row set on distinct 4-slot quarters and 16 aligned rows on
// distinct groups.  Wider rows (fp32 with D = 128) use key = r % 16.
template <int W> struct Swz {
    static_assert(W == 4 || W == 8 || W == 16 || W == 32, "row width in 16-byte slots");
    static __device__ __forceinline__ constexpr int key(int r) {
        return W > 16 ? r % 16 : 4 * ((r / (16 / W)) % (W / 4)) + (r / 4) % 4;
    }
    static __device__ __forceinline__ constexpr int slot(int r, int s) { return r * W + (s ^ key(r)); }
};

typedef __attribute__((address_space(3))) char lds_char;

// One 1 KB block of a global -> LDS copy: lane l's 16 bytes at
// base + off[l] land at LDS byte lds + 16*l (base wave-uniform, in SGPRs).
// Written as inline asm so the compiler's counter bookkeeping does not see an
// LDS write in flight (it cannot tell the two buffers apart and would wait
// for the copy before every LDS read of the other buffer); the issuing wave
// orders it with s_waitcnt vmcnt(0) and a barrier before any wave reads the
// block.  M0 is named as clobbered; the kernels give the compiler no other
// use of it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The LDS destination is lds + IMM: the per-instruction part is an immediate,
// so the kernels keep one scalar register per tile buffer, not one per block.
template <uint32_t IMM>
__device__ __forceinline__ void dma_block(const char *base, uint32_t off, uint32_t lds) {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds), "i"(IMM) : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(lds_char *)p; }

// Global -> LDS copy of a tile of ROWS rows x W 16-byte slots into the Swz<W>
// image, by NW waves (wave w issues instructions w, w+NW, ...; each moves
// 64 slots = 1 KB).  Row r of the tile is global row min(r, nrows-1) at
// base + row * gstride bytes (rows past a ragged tile re-read its last row;
// the kernels give them zero weight).  A lane's byte offsets for a whole
// tile are computed once; only ragged tiles recompute them.
// Completion: s_waitcnt vmcnt(0) in the issuing wave, then a barrier.
template <int ROWS, int W, int NW> struct Dma {
    static constexpr int INSTR = ROWS * W / 64;
    static constexpr int PER = (INSTR + NW - 1) / NW;   // instructions per wave
    static_assert((ROWS * W) % 64 == 0, "a tile is a whole number of 1 KB blocks");
    uint32_t off[PER];
    uint32_t gstride;
    int w, lane;

    __device__ __forceinline__ Dma(uint32_t gstride_, int wave, int lane_) : gstride(gstride_), lane(lane_) {
        w = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int j = 0; j < PER; ++j) off[j] = offset(j, ROWS);
    }
    __device__ __forceinline__ uint32_t offset(int j, int nrows) const {
        const int pu = (j * NW + w) * 64 + lane;
        const int r = pu / W;
        const int sl = (pu % W) ^ Swz<W>::key(r);
        return (uint32_t)min(r, nrows - 1) * gstride + (uint32_t)(sl * 16);
    }
    template <int J, bool FULL>
    __device__ __forceinline__ void issue_from(const char *base, int nrows, uint32_t l0) const {
        if constexpr (J < PER) {
            if (INSTR % NW == 0 || J * NW + w < INSTR)
                dma_block<(uint32_t)(J * NW * 1024)>(base, FULL ? off[J] : offset(J, nrows), l0);
            issue_from<J + 1, FULL>(base, nrows, l0);
        }
    }
    __device__ __forceinline__ void issue(const char *base, int nrows, const void *lds) const {
        const uint32_t l0 = lds_addr(lds) + (uint32_t)w * 1024u;
        if (nrows >= ROWS) issue_from<0, true>(base, nrows, l0);
        else issue_from<0, false>(base, nrows, l0);
    }
};

template <typename T, int D> struct Mfma;

// bf16 operands, v_mfma_f32_32x32x16_bf16.  Row-major LDS tiles hold D
// elements (W = D/8 slots) per row in the Swz layout.
template <int D> struct Mfma<bf16, D> {
    static constexpr int KS = D / 16;   // contraction steps over the head dim
    static constexpr int W = D / 8;     // slots per row-major tile row
    typedef bf16x8 Op;

    // Row-major operand of one lane: 8 consecutive values at column 16*ks + 8*hh.
    static __device__ __forceinline__ void load_row_op(Op (&op)[KS], const bf16 *row, int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) op[ks] = *reinterpret_cast<const bf16x8 *>(row + 16 * ks + 8 * hh);
    }
    static __device__ __forceinline__ void zero_op(Op (&op)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) op[ks][e] = bf16(0.0f);
    }
    // A operand of step ks from row `row` of a row-major tile.
    static __device__ __forceinline__ bf16x8 row_frag(const bf16 *tile, int row, int ks, int hh) {
        return *reinterpret_cast<const bf16x8 *>(tile + 8 * Swz<W>::slot(row, 2 * ks + hh));
    }
    // acc += A x B(op), A = row `row` of a row-major LDS tile (one row per
    // lane: row = r0 + l%32), contraction over D.
    static __device__ __forceinline__ void gemm_rows_lds(f32x16 &acc, const bf16 *tile, int row, const Op (&op)[KS],
                                                         int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(tile, row, ks, hh), op[ks], acc, 0, 0, 0);
    }
    // Two chains over the same operand op: acc0 += rows row0.. x op and
    // acc1 += rows row1.. x op.  The LDS operands of a step are read one step
    // ahead, and the two chains alternate, so neither the LDS latency nor the
    // accumulator dependency stalls the matrix unit.
    static __device__ __forceinline__ void gemm_rows_lds2(f32x16 &acc0, f32x16 &acc1, const bf16 *tile, int row0,
                                                          int row1, const Op (&op)[KS], int hh) {
        // operands of step ks + PF are read while step ks multiplies
        constexpr int PF = KS >= 4 ? 2 : 1;
        bf16x8 a0[PF + 1], a1[PF + 1];
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            a0[j] = row_frag(tile, row0, j, hh);
            a1[j] = row_frag(tile, row1, j, hh);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + PF < KS) {
                a0[(ks + PF) % (PF + 1)] = row_frag(tile, row0, ks + PF, hh);
                a1[(ks + PF) % (PF + 1)] = row_frag(tile, row1, ks + PF, hh);
            }
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[ks % (PF + 1)], op[ks], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[ks % (PF + 1)], op[ks], acc1, 0, 0, 0);
        }
    }
    // Two chains with their own tiles and operands (same rows).
    static __device__ __forceinline__ void gemm_rows_lds_pair(f32x16 &acc0, const bf16 *tile0, const Op (&op0)[KS],
                                                              f32x16 &acc1, const bf16 *tile1, const Op (&op1)[KS],
                                                              int row, int hh) {
        constexpr int PF = KS >= 4 ? 2 : 1;
        bf16x8 a0[PF + 1], a1[PF + 1];
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            a0[j] = row_frag(tile0, row, j, hh);
            a1[j] = row_frag(tile1, row, j, hh);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + PF < KS) {
                a0[(ks + PF) % (PF + 1)] = row_frag(tile0, row, ks + PF, hh);
                a1[(ks + PF) % (PF + 1)] = row_frag(tile1, row, ks + PF, hh);
            }
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[ks % (PF + 1)], op0[ks], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[ks % (PF + 1)], op1[ks], acc1, 0, 0, 0);
        }
    }
    // A operand of X^T for one 32x32x16 step over 16 contraction rows of a
    // row-major Swz<W> tile X, taken in the order the C layout holds them:
    // lane l gets X[r0 + 8*(e/4) + 4*hh + e%4][32*cb + l%32], e = 0..7
    // (r0 % 16 == 0), from two transpose reads (e = 0..3 and 4..7).  For a
    // read, lane c + 4j of group g fetches 4 columns from
    // 32*cb + 16*(g%2) + 4c of row r0 + 4*(g/2) + j (+8).
    static __device__ __forceinline__ bf16x8 col_frag(const bf16 *tile, int r0, int cb, int lane) {
        const int g = lane >> 4, i = lane & 15;
        const int row = r0 + 4 * (g >> 1) + (i >> 2);
        const int col = 32 * cb + 16 * (g & 1) + 4 * (i & 3);
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(tile + 8 * Swz<W>::slot(row, col / 8) + col % 8));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(tile + 8 * Swz<W>::slot(row + 8, col / 8) + col % 8));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // acc[cb] += X^T * P for rows r0..r0+31 of a row-major Swz<W> tile X
    // against a 32 x 32 block P in C layout (columns of X as the MFMA rows).
    // The contraction runs over the rows in C-layout order: registers
    // 8*half .. 8*half+7 of a lane half are its B operand of step `half`
    // as they stand, and col_frag reads X's rows in the same order.  All LDS
    // operands of the block are read before the first MFMA, so only the
    // first read's latency shows.
    static __device__ __forceinline__ void gemm_t_c(f32x16 (&acc)[D / 32], const bf16 *tile, int r0,
                                                    const f32x16 &p, int lane) {
        bf16x8 a[2][D / 32];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) a[half][cb] = col_frag(tile, r0 + 16 * half, cb, lane);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = to_bf16(p[8 * half + e]);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[half][cb], b, acc[cb], 0, 0, 0);
        }
    }
};

// fp32 operands, v_mfma_f32_32x32x2_f32 (W = D/4 slots per row-major row).
template <int D> struct Mfma<float, D> {
    static constexpr int KS = D / 2;
    static constexpr int W = D / 4;
    typedef float Op;

    static __device__ __forceinline__ void load_row_op(Op (&op)[KS], const float *row, int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) op[ks] = row[2 * ks + hh];
    }
    static __device__ __forceinline__ void zero_op(Op (&op)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) op[ks] = 0.0f;
    }
    // Element (row, col) of a Swz<WS> tile of 4-element slots.
    template <int WS>
    static __device__ __forceinline__ float at(const float *tile, int row, int col) {
        return tile[4 * Swz<WS>::slot(row, col / 4) + col % 4];
    }
    static __device__ __forceinline__ void gemm_rows_lds(f32x16 &acc, const float *tile, int row, const Op (&op)[KS],
                                                         int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(at<W>(tile, row, 2 * ks + hh), op[ks], acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void gemm_rows_lds2(f32x16 &acc0, f32x16 &acc1, const float *tile, int row0,
                                                          int row1, const Op (&op)[KS], int hh) {
        gemm_rows_lds(acc0, tile, row0, op, hh);
        gemm_rows_lds(acc1, tile, row1, op, hh);
    }
    static __device__ __forceinline__ void gemm_rows_lds_pair(f32x16 &acc0, const float *tile0, const Op (&op0)[KS],
                                                              f32x16 &acc1, const float *tile1, const Op (&op1)[KS],
                                                              int row, int hh) {
        gemm_rows_lds(acc0, tile0, row, op0, hh);
        gemm_rows_lds(acc1, tile1, row, op1, hh);
    }
    // acc[cb] += X^T * P for rows r0..r0+31 of a row-major tile X against a
    // 32 x 32 block P in C layout: one contraction row per MFMA, the lanes
    // of a half reading 32 consecutive columns of it.
    static __device__ __forceinline__ void gemm_t_c(f32x16 (&acc)[D / 32], const float *tile, int r0,
                                                    const f32x16 &p, int lane) {
        const int hh = lane >> 5;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pos = r0 + c_row(i, hh);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(at<W>(tile, pos, 32 * cb + (lane & 31)), p[i],
                                                                acc[cb], 0, 0, 0);
        }
    }
};

// Address of row `row0` of head h in a [*, heads, D] tensor: the tile base
// every thread adds its own loop-invariant byte offset to (the base is
// wave-uniform, so loads take the scalar-base + 32-bit-offset form).
template <typename T, int D>
__device__ __forceinline__ const char *tile_base(const T *g, int64_t row0, int heads, int h) {
    return reinterpret_cast<const char *>(g + (row0 * heads + h) * D);
}

}  // namespace zz
