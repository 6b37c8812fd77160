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
// pair (l, l^32), and P^T in C layout is already the B operand of O^T = V^T P^T
// when the contraction runs over the keys in the order k(e) = 8*(e/4) +
// 4*(l/32) + e%4 -- the A operand (V^T) is then read from a transposed LDS
// copy whose rows hold the keys in that order (tperm).
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

// Position of row k of a tile inside a transposed LDS row: bits 2 and 3 of k
// swapped.  With it, the 8 contraction values a lane half needs for one
// 32x32x16 MFMA (rows 4h..4h+3 and 8+4h..8+4h+3 of a 16-row block, the order
// c_row produces) sit in 16 contiguous bytes.
__device__ __forceinline__ constexpr int tperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

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
    // acc[cb] += X^T * P for a tile X stored transposed in LDS (row = column of
    // X, LDT elements per row, X rows permuted by tperm): X rows r0..r0+31
    // against a 32 x 32 block P in C layout.  16-byte reads, two MFMAs per
    // 32 contraction rows and 32 columns.
    template <int LDT>
    static __device__ __forceinline__ void gemm_t_c(f32x16 (&acc)[D / 32], const bf16 *tileT, int r0,
                                                    const f32x16 &p, int lane) {
        const int hh = lane >> 5;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = to_bf16(p[8 * half + e]);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(tileT + (32 * cb + (lane & 31)) * LDT + r0 +
                                                                   16 * half + 8 * hh);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[cb], 0, 0, 0);
            }
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
    template <int LDT>
    static __device__ __forceinline__ void gemm_t_c(f32x16 (&acc)[D / 32], const float *tileT, int r0,
                                                    const f32x16 &p, int lane) {
        const int hh = lane >> 5;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pos = r0 + tperm(c_row(i, hh));
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(tileT[(32 * cb + (lane & 31)) * LDT + pos], p[i],
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
// into LDS transposed: LDS row c holds column c of the tile, the tile rows
// placed at tperm(row).  Each thread gathers RPU (4 or 2) consecutive rows x
// one 16-byte column group, regroups them in registers, and writes RPU
// consecutive rows per LDS column.  The same registers also give the
// row-major copy (store_rows).  Lanes are laid out as 4 column groups x the
// row units x the rest of the column groups, which keeps the stores of 16
// lanes on distinct (RPU 4) or at most two-way shared (RPU 2) bank groups.
template <typename T, int D, int ROWS, int NT, int RPU = 4> struct TileStageT {
    static constexpr int EPV = 16 / sizeof(T);
    static constexpr int CPR = D / EPV;          // 16-byte column groups
    static constexpr int NQ = ROWS / RPU;        // row units
    static constexpr int UNITS = NQ * CPR;
    static constexpr int N = (UNITS + NT - 1) / NT;
    static constexpr int PADT = 16 / sizeof(T);  // 16 bytes of padding per LDS row
    static constexpr int LDT = ROWS + PADT;
    static_assert(ROWS % 16 == 0, "row count must be a multiple of 16");
    static_assert(CPR % 4 == 0, "column groups must come in fours");
    static_assert(RPU == 4 || RPU == 2, "2 or 4 rows per unit");
    i32x4 r[N][RPU];
    uint32_t rstride;   // bytes between consecutive rows (wave-uniform)

    // unit -> (row unit m, column group cg)
    static __device__ __forceinline__ void unit(int u, int &m, int &cg) {
        m = (u / 4) % NQ;
        cg = (u / (4 * NQ)) * 4 + u % 4;
    }
    __device__ __forceinline__ void init(int heads, int tid) { rstride = (uint32_t)(heads * D * sizeof(T)); }
    // Rows past nrows re-read row nrows-1 (see TileStage).
    __device__ __forceinline__ void load(const char *base, int nrows, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            int m, cg;
            unit(u, m, cg);
#pragma unroll
            for (int j = 0; j < RPU; ++j) {
                const uint32_t rr = (uint32_t)min(RPU * m + j, nrows - 1);
                r[i][j] = *reinterpret_cast<const i32x4 *>(base + rr * rstride + (uint32_t)(cg * 16));
            }
        }
    }
    // Row-major copy of the same rows (the layout of RowLayout).
    __device__ __forceinline__ void store_rows(T *lds, int tid) const {
        using RL = RowLayout<T, D>;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            int m, cg;
            unit(u, m, cg);
#pragma unroll
            for (int j = 0; j < RPU; ++j) *reinterpret_cast<i32x4 *>(lds + (RPU * m + j) * RL::LD + cg * EPV) = r[i][j];
        }
    }
    // 32-bit word d of a 16-byte chunk (d is a compile-time constant after
    // unrolling; no address is taken, so the chunk stays in registers).
    static __device__ __forceinline__ uint32_t word(const i32x4 &v, int d) { return (uint32_t)v[d]; }
    __device__ __forceinline__ void store(T *ldsT, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            int m, cg;
            unit(u, m, cg);
            const int pos = tperm(RPU * m);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t w0 = word(r[i][0], d), w1 = word(r[i][1], d);
                if constexpr (sizeof(T) == 2 && RPU == 4) {
                    const uint32_t w2 = word(r[i][2], d), w3 = word(r[i][3], d);
                    u32x2 lo, hi;   // column 2d (low halves) and 2d+1 (high halves), rows 4m..4m+3
                    lo[0] = (w0 & 0xffffu) | (w1 << 16);
                    lo[1] = (w2 & 0xffffu) | (w3 << 16);
                    hi[0] = (w0 >> 16) | (w1 & 0xffff0000u);
                    hi[1] = (w2 >> 16) | (w3 & 0xffff0000u);
                    *reinterpret_cast<u32x2 *>(ldsT + (cg * EPV + 2 * d) * LDT + pos) = lo;
                    *reinterpret_cast<u32x2 *>(ldsT + (cg * EPV + 2 * d + 1) * LDT + pos) = hi;
                } else if constexpr (sizeof(T) == 2) {
                    const uint32_t lo = (w0 & 0xffffu) | (w1 << 16);
                    const uint32_t hi = (w0 >> 16) | (w1 & 0xffff0000u);
                    *reinterpret_cast<uint32_t *>(ldsT + (cg * EPV + 2 * d) * LDT + pos) = lo;
                    *reinterpret_cast<uint32_t *>(ldsT + (cg * EPV + 2 * d + 1) * LDT + pos) = hi;
                } else if constexpr (RPU == 4) {
                    const u32x4 col = {w0, w1, word(r[i][2], d), word(r[i][3], d)};
                    *reinterpret_cast<u32x4 *>(ldsT + (cg * EPV + d) * LDT + pos) = col;
                } else {
                    const u32x2 col = {w0, w1};
                    *reinterpret_cast<u32x2 *>(ldsT + (cg * EPV + d) * LDT + pos) = col;
                }
            }
        }
    }
};

}  // namespace zz
