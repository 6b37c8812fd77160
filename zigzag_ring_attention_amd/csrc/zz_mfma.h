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
// pair (l, l^32).  P^T in C layout becomes the B operand of O^T = V^T P^T
// after one exchange between the lane halves (order_for_b), which puts the
// keys of a lane half in natural order; the A operand (V^T) is read from a
// transposed LDS copy whose rows hold the keys in natural order.
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

// Reorder a 32-row block in C layout into B-operand order: afterwards lane
// half hh holds rows 16*h + 8*hh + e in register 8*h + e (h = 0, 1; e = 0..7),
// the contraction order of a 32x32x16 MFMA over natural rows.  In C layout
// half hh holds rows 16*h + 4*hh + {0..3, 8..11}; one permlane32 swap per
// register pair (j, j+4) exchanges rows 4..7 of half 0 with rows 8..11 of
// half 1.
__device__ __forceinline__ void order_for_b(f32x16 &x) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[8 * h + j]), __float_as_uint(x[8 * h + 4 + j]),
                                                      false, false);
            x[8 * h + j] = __uint_as_float(r[0]);       // lanes 0-31 keep, 32-63 get rows 8..11 of half 0
            x[8 * h + 4 + j] = __uint_as_float(r[1]);   // lanes 0-31 get rows 4..7 of half 1, 32-63 keep
        }
}

// Exchange a value with lane l^32.
__device__ __forceinline__ float swap_halves(float x, int lane) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

template <typename T, int D> struct Mfma;

// bf16 operands, v_mfma_f32_32x32x16_bf16.
// Row-major LDS tiles: 16 bytes of padding per row, so the 16 rows read by
// 16 lanes (one row per lane, same column) start on 16 different bank
// groups.
template <typename T, int D> struct RowLayout {
    static constexpr int EPV = 16 / sizeof(T);
    static constexpr int LD = D + EPV;   // row stride (elements)
    static __device__ __forceinline__ int at(int r, int e) { return r * LD + e; }
};

template <int D> struct Mfma<bf16, D> {
    static constexpr int KS = D / 16;   // contraction steps over the head dim
    using RL = RowLayout<bf16, D>;
    static constexpr int LD = RL::LD;   // row-major LDS row stride (elements)
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
    // acc += A x B(op), A = row `row` of a row-major LDS tile (one row per
    // lane: row = r0 + l%32), contraction over D.
    static __device__ __forceinline__ void gemm_rows_lds(f32x16 &acc, const bf16 *tile, int row, const Op (&op)[KS],
                                                         int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(tile + RL::at(row, 16 * ks + 8 * hh));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op[ks], acc, 0, 0, 0);
        }
    }
    // Two chains over the same operand op: acc0 += rows row0.. x op and
    // acc1 += rows row1.. x op.  The LDS operands of a step are read one step
    // ahead, and the two chains alternate, so neither the LDS latency nor the
    // accumulator dependency stalls the matrix unit.
    static __device__ __forceinline__ void gemm_rows_lds2(f32x16 &acc0, f32x16 &acc1, const bf16 *tile, int row0,
                                                          int row1, const Op (&op)[KS], int hh) {
        bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(tile + RL::at(row0, 8 * hh));
        bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(tile + RL::at(row1, 8 * hh));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 n0 = a0, n1 = a1;
            if (ks + 1 < KS) {
                n0 = *reinterpret_cast<const bf16x8 *>(tile + RL::at(row0, 16 * (ks + 1) + 8 * hh));
                n1 = *reinterpret_cast<const bf16x8 *>(tile + RL::at(row1, 16 * (ks + 1) + 8 * hh));
            }
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, op[ks], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, op[ks], acc1, 0, 0, 0);
            a0 = n0;
            a1 = n1;
        }
    }
    // Two chains with their own tiles and operands (same rows).
    static __device__ __forceinline__ void gemm_rows_lds_pair(f32x16 &acc0, const bf16 *tile0, const Op (&op0)[KS],
                                                              f32x16 &acc1, const bf16 *tile1, const Op (&op1)[KS],
                                                              int row, int hh) {
        bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(tile0 + RL::at(row, 8 * hh));
        bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(tile1 + RL::at(row, 8 * hh));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 n0 = a0, n1 = a1;
            if (ks + 1 < KS) {
                n0 = *reinterpret_cast<const bf16x8 *>(tile0 + RL::at(row, 16 * (ks + 1) + 8 * hh));
                n1 = *reinterpret_cast<const bf16x8 *>(tile1 + RL::at(row, 16 * (ks + 1) + 8 * hh));
            }
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, op0[ks], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, op1[ks], acc1, 0, 0, 0);
            a0 = n0;
            a1 = n1;
        }
    }
    // acc[cb] += X^T * P for a tile X stored transposed in LDS (row = column
    // of X, LDT elements per row, X rows in natural order): X rows r0..r0+31
    // against a 32 x 32 block P in C layout.  16-byte reads, two MFMAs per 32
    // contraction rows and 32 columns; all LDS operands of the block are read
    // before the first MFMA, so only the first read's latency shows.
    // The transposed tile is a TileStageT copy: SLOTS 16-byte slots per row,
    // swizzled by TileStageT::tpos.
    template <int LDT, int SLOTS>
    static __device__ __forceinline__ void gemm_t_c(f32x16 (&acc)[D / 32], const bf16 *tileT, int r0,
                                                    const f32x16 &p, int lane) {
        const int hh = lane >> 5;
        bf16x8 a[2][D / 32];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int row = 32 * cb + (lane & 31);
                const int slot = ((r0 + 16 * half + 8 * hh) / 8) ^ ((row >> 4) & (SLOTS - 1));
                a[half][cb] = *reinterpret_cast<const bf16x8 *>(tileT + row * LDT + 8 * slot);
            }
        f32x16 pb = p;
        order_for_b(pb);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = to_bf16(pb[8 * half + e]);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[half][cb], b, acc[cb], 0, 0, 0);
        }
    }
};

// fp32 operands, v_mfma_f32_32x32x2_f32.
template <int D> struct Mfma<float, D> {
    static constexpr int KS = D / 2;
    using RL = RowLayout<float, D>;
    static constexpr int LD = RL::LD;
    typedef float Op;

    static __device__ __forceinline__ void load_row_op(Op (&op)[KS], const float *row, int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) op[ks] = row[2 * ks + hh];
    }
    static __device__ __forceinline__ void zero_op(Op (&op)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) op[ks] = 0.0f;
    }
    static __device__ __forceinline__ void gemm_rows_lds(f32x16 &acc, const float *tile, int row, const Op (&op)[KS],
                                                         int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(tile[RL::at(row, 2 * ks + hh)], op[ks], acc, 0, 0, 0);
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
    template <int LDT, int SLOTS>
    static __device__ __forceinline__ void gemm_t_c(f32x16 (&acc)[D / 32], const float *tileT, int r0,
                                                    const f32x16 &p, int lane) {
        const int hh = lane >> 5;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pos = r0 + c_row(i, hh);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int row = 32 * cb + (lane & 31);
                const int at = (((pos / 4) ^ ((row >> 4) & (SLOTS - 1))) * 4) + pos % 4;
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(tileT[row * LDT + at], p[i], acc[cb], 0, 0, 0);
            }
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

// A tile of ROWS rows x D columns of a [*, H, D] tensor (one head), staged
// global -> registers -> LDS by NT threads.  Issuing the global loads for the
// next tile before computing on the current one hides their latency.
// Rows past nrows (a ragged tile) re-read row nrows-1, so every load stays
// inside the tile's chunk and the code has no branch; the kernels give those
// rows zero weight (masked scores, or an infinite LSE).
template <typename T, int D, int ROWS, int NT> struct TileStage {
    static constexpr int EPV = 16 / sizeof(T);   // elements per 16-byte chunk
    static constexpr int CPR = D / EPV;          // chunks per row
    static constexpr int N = ROWS * CPR / NT;    // chunks per thread
    static_assert(N >= 1 && (ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
    static constexpr int LD = RowLayout<T, D>::LD;
    i32x4 r[N];
    uint32_t rstride;   // bytes between consecutive rows (wave-uniform)

    // Chunk c = tid + i*NT is row c / CPR, elements (c % CPR)*EPV.. of it.
    __device__ __forceinline__ void init(int heads, int tid) { rstride = (uint32_t)(heads * D * sizeof(T)); }
    __device__ __forceinline__ void load(const char *base, int nrows, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int c = tid + i * NT;
            const uint32_t rr = (uint32_t)min(c / CPR, nrows - 1);
            r[i] = *reinterpret_cast<const i32x4 *>(base + rr * rstride + (uint32_t)((c % CPR) * 16));
        }
    }
    __device__ __forceinline__ void store(T *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int c = tid + i * NT, e = (c % CPR) * EPV;
            *reinterpret_cast<i32x4 *>(lds + (c / CPR) * LD + e) = r[i];
        }
    }
};

// A tile of ROWS rows x D columns of a [*, H, D] tensor (one head), staged
// global -> registers -> LDS as a row-major copy (RowLayout) and a transposed
// copy: LDS row c holds column c of the tile, the tile rows in natural order
// in 16-byte groups whose slots are XOR-swizzled by the row (tpos), with
// LDT = ROWS + 16 bytes of padding per row.  A unit is RU = 16/sizeof(T)
// consecutive rows x one 16-byte column group; its RU x RU block is
// transposed in registers, so both copies are written with 16-byte stores
// (narrower LDS stores run far below the 16-byte ones).  Units are dealt to
// the NT staging threads column-group first, so each global load of a wave
// reads whole rows and the row-major stores of 16 lanes fill consecutive
// 16-byte slots; the swizzle does the same for the transposed stores, whose
// 16 lanes would otherwise land on two bank groups.  Rows past nrows re-read
// row nrows-1 (see TileStage).
template <typename T, int D, int ROWS, int NT> struct TileStageT {
    static constexpr int EPV = 16 / sizeof(T);   // elements per 16-byte chunk
    static constexpr int RU = EPV;               // rows per unit
    static constexpr int CPR = D / EPV;          // 16-byte column groups
    static constexpr int NQ = ROWS / RU;         // row units
    static constexpr int UNITS = NQ * CPR;
    static constexpr int N = (UNITS + NT - 1) / NT;
    static constexpr int LDT = ROWS + EPV;       // transposed row stride (elements)
    static_assert(ROWS % RU == 0, "rows must split into units");
    static_assert((NQ & (NQ - 1)) == 0, "row units must be a power of two");
    i32x4 r[N][RU];
    uint32_t rstride;   // bytes between consecutive rows (wave-uniform)

    // unit -> (row unit m, column group cg)
    static __device__ __forceinline__ void unit(int u, int &m, int &cg) {
        m = u / CPR;
        cg = u % CPR;
    }
    // Element offset of tile row `pos` inside transposed LDS row `row`: the
    // 16-byte slot is XOR-ed with bits 4.. of the row, so 16 consecutive
    // rows read the same slot conflict-free (odd row stride in slots) and the
    // 16 rows cg*EPV + c written by 16 lanes spread over all slots.
    static __device__ __forceinline__ constexpr int tpos(int row, int pos) {
        return (((pos / EPV) ^ ((row >> 4) & (NQ - 1))) * EPV) + pos % EPV;
    }
    __device__ __forceinline__ void init(int heads) { rstride = (uint32_t)(heads * D * sizeof(T)); }
    // t: this thread's index among the NT staging threads.
    __device__ __forceinline__ void load(const char *base, int nrows, int t) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = t + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            int m, cg;
            unit(u, m, cg);
#pragma unroll
            for (int j = 0; j < RU; ++j) {
                const uint32_t rr = (uint32_t)min(RU * m + j, nrows - 1);
                r[i][j] = *reinterpret_cast<const i32x4 *>(base + rr * rstride + (uint32_t)(cg * 16));
            }
        }
    }
    // Row-major copy (the layout of RowLayout).
    __device__ __forceinline__ void store_rows(T *lds, int t) const {
        using RL = RowLayout<T, D>;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = t + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            int m, cg;
            unit(u, m, cg);
#pragma unroll
            for (int j = 0; j < RU; ++j) *reinterpret_cast<i32x4 *>(lds + (RU * m + j) * RL::LD + cg * EPV) = r[i][j];
        }
    }
    // Element c (0..EPV-1) of row j of unit i, as the low bits of a word.
    __device__ __forceinline__ uint32_t half_of(int i, int j, int c) const {
        const uint32_t w = (uint32_t)r[i][j][c / 2];
        return (c & 1) ? (w >> 16) : (w & 0xffffu);
    }
    // Transposed copy: column c of the unit's column group is LDS row
    // cg*EPV + c, the unit's RU rows at positions RU*m .. RU*m+RU-1.
    __device__ __forceinline__ void store(T *ldsT, int t) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = t + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            int m, cg;
            unit(u, m, cg);
#pragma unroll
            for (int c = 0; c < EPV; ++c) {
                u32x4 col;
                if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) col[k] = half_of(i, 2 * k, c) | (half_of(i, 2 * k + 1, c) << 16);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) col[k] = (uint32_t)r[i][k][c];
                }
                const int row = cg * EPV + c;
                *reinterpret_cast<u32x4 *>(ldsT + row * LDT + tpos(row, RU * m)) = col;
            }
        }
    }
};

}  // namespace zz
