// MFMA building blocks for the attention kernels (gfx950 wave64).
//
// Lane layouts (checked on the device by a layout probe):
//  v_mfma_f32_32x32x16_bf16: A[m][k] in lane (m = l%32), k = 8*(l/32) + e,
//    e = 0..7; B[k][n] in lane (n = l%32), k = 8*(l/32) + e; C[m][n] in lane
//    (n = l%32), register i holds m = 8*(i/4) + 4*(l/32) + i%4.
//  v_mfma_f32_32x32x2_f32: as above with one k per lane, k = l/32.
//  ds_read_b64_tr_b16: in each group of 16 lanes, lane t supplies the address
//    of 4 consecutive 16-bit values; lane t of the group then receives the
//    values at positions t, 16+t, 32+t, 48+t of the 64 values the group
//    loaded (in lane order).  Pointing lane t at row (k0 + t/4), column
//    (n0 + 4*(t%4)) of a row-major tile therefore hands lane t the column
//    n0 + t, rows k0..k0+3: a transposed operand read.
//
// Scores are formed transposed (S^T = K Q^T), so the C layout puts one query
// per lane column: the softmax row statistics of a query live in one lane
// pair (l, l^32), and P^T in C layout is already the B operand of O^T = V^T P^T
// when the contraction runs over the keys in the order k(e) = 8*(e/4) +
// 4*(l/32) + e%4 -- the A operand (V^T) is then read with that same order.
#pragma once

#include "zz_device.h"

namespace zz {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Key offset (inside a 32-key score block) of C register i in lane half hh.
__device__ __forceinline__ constexpr int c_row(int i, int hh) { return 8 * (i / 4) + 4 * hh + (i % 4); }

// Exchange a value with lane l^32.
__device__ __forceinline__ float swap_halves(float x, int lane) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

template <typename T, int D> struct Mfma;

// bf16 operands, v_mfma_f32_32x32x16_bf16.
template <int D> struct Mfma<bf16, D> {
    static constexpr int KS = D / 16;   // contraction steps over the head dim
    static constexpr int PAD = 8;       // LDS row padding (elements)
    static constexpr int LD = D + PAD;  // LDS row stride (elements)
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
    // acc += A(rows of lds tile, row = row0 + l%32) x B(op), contraction over D.
    static __device__ __forceinline__ void gemm_rows_lds(f32x16 &acc, const bf16 *lds_row, const Op (&op)[KS], int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(lds_row + 16 * ks + 8 * hh);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op[ks], acc, 0, 0, 0);
        }
    }
    // Transposed read of a row-major LDS tile: lane gets column (n0 + l%16 within
    // its 16-lane group), rows k0..k0+3, from lane-supplied addresses.
    static __device__ __forceinline__ s16x4 tr4(const bf16 *tile, int k0, int n0, int lane) {
        const int t = lane & 15;
        const bf16 *p = tile + (k0 + t / 4) * LD + n0 + 4 * (t % 4);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    }
    // A operand (8 values along the contraction) of X^T where X is a row-major
    // LDS tile [rows][D]: lane (col = 32*cb + l%32) reads rows
    // r0 + 4*(l/32) + {0..3} and r0 + 8 + 4*(l/32) + {0..3}.
    static __device__ __forceinline__ bf16x8 tr_op(const bf16 *tile, int r0, int cb, int lane) {
        const int g = lane >> 4;
        const int n0 = 32 * cb + 16 * (g & 1);
        const int hh = g >> 1;
        const s16x4 x = tr4(tile, r0 + 4 * hh, n0, lane);
        const s16x4 y = tr4(tile, r0 + 8 + 4 * hh, n0, lane);
        // Join as whole vectors: building the result element by element through
        // scalar 16-bit bit casts was miscompiled (lanes duplicated) by hipcc 7.2.
        const s16x8 xy = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, xy);
    }
    // acc[cb] += X^T(LDS tile rows r0.. r0+31 of a 32-row block) * P where P is a
    // 32(contraction) x 32 block in C layout (register i = contraction index
    // c_row(i, l/32)).  Two MFMAs per 32 contraction rows.
    static __device__ __forceinline__ void gemm_tr_c(f32x16 (&acc)[D / 32], const bf16 *tile, int r0,
                                                     const f32x16 &p, int lane) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = to_bf16(p[8 * half + e]);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const bf16x8 a = tr_op(tile, r0 + 16 * half, cb, lane);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[cb], 0, 0, 0);
            }
        }
    }
};

// fp32 operands, v_mfma_f32_32x32x2_f32.
template <int D> struct Mfma<float, D> {
    static constexpr int KS = D / 2;
    static constexpr int PAD = 4;
    static constexpr int LD = D + PAD;
    typedef float Op;

    static __device__ __forceinline__ void load_row_op(Op (&op)[KS], const float *row, int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) op[ks] = row[2 * ks + hh];
    }
    static __device__ __forceinline__ void zero_op(Op (&op)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) op[ks] = 0.0f;
    }
    static __device__ __forceinline__ void gemm_rows_lds(f32x16 &acc, const float *lds_row, const Op (&op)[KS], int hh) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_row[2 * ks + hh], op[ks], acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void gemm_tr_c(f32x16 (&acc)[D / 32], const float *tile, int r0,
                                                     const f32x16 &p, int lane) {
        const int hh = lane >> 5;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = r0 + c_row(i, hh);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(tile[row * LD + 32 * cb + (lane & 31)], p[i],
                                                                acc[cb], 0, 0, 0);
        }
    }
};

// A tile of ROWS rows x D columns of a [*, H, D] tensor (one head), staged
// global -> registers -> LDS by NT threads.  Issuing the global loads for the
// next tile before computing on the current one hides their latency.
// Rows past nrows are zero-filled (no read past the end of a chunk).
template <typename T, int D, int ROWS, int NT> struct TileStage {
    static constexpr int EPV = 16 / sizeof(T);   // elements per 16-byte chunk
    static constexpr int CPR = D / EPV;          // chunks per row
    static constexpr int N = ROWS * CPR / NT;    // chunks per thread
    static_assert(N >= 1 && (ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
    static constexpr int LD = Mfma<T, D>::LD;
    int4 r[N];

    __device__ __forceinline__ void load(const T *__restrict__ g, int64_t row0, int nrows, int heads, int h,
                                         int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int c = tid + i * NT, row = c / CPR, e = (c % CPR) * EPV;
            r[i] = row < nrows ? *reinterpret_cast<const int4 *>(g + ((row0 + row) * heads + h) * D + e)
                               : int4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(T *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int c = tid + i * NT, row = c / CPR, e = (c % CPR) * EPV;
            *reinterpret_cast<int4 *>(lds + row * LD + e) = r[i];
        }
    }
};

}  // namespace zz
