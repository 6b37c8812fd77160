// Backward ring step of zigzag varlen attention (FlagScale PR #910: the
// per-step backward of a ring driver).  With the global LSE of the merged
// forward, a step's contribution is a plain sum:
//   P = exp(S - LSE), dP = dO V^T, dS = P (dP - delta), delta = rowsum(dO O)
//   dQ_r += scale dS K_j,  dK_j += scale dS^T Q_r,  dV_j += P^T dO_r
// summed over the query heads of each key/value group.
//
// Two kernels per step, neither uses atomics:
//  * dkv (key-major): a workgroup owns up to 128 keys of shard j and one
//    key/value head.  It walks every query head of the group and every listed
//    query tile (up to 64 rows, staged in LDS with its LSE and delta), forming
//    S and dP with the keys in the lane dimension, so that P and dS are
//    directly the operands of dV^T += dO^T P and dK^T += Q^T dS.
//  * dq (query-major, zz_bwd_dq.hip): like the forward step, S^T and dP^T
//    with the queries in the lane dimension, then dQ^T += K^T dS^T.
// Fully masked tiles are never visited (tile lists from the planner).

#include <type_traits>

#include "zz_bwd.h"

namespace zz {
namespace {

// ---------------------------------------------------------------- dK, dV

// Query rows per streamed tile (must match the planner's dK/dV tile).
template <typename T, int D> constexpr int q_tile() { return (sizeof(T) == 4 && D >= 64) ? 32 : 64; }

constexpr int kDkvThreads = 512;

// Eight waves own 128 keys as four pairs of 32 keys.  In a pair, wave A
// (waves 0-3) forms S = Q K^T and P = exp(S - LSE), hands P to its partner
// through LDS and accumulates dV^T += dO^T P; wave B (waves 4-7) forms
// dP = dO V^T, takes P, forms dS = P (dP - delta) and accumulates
// dK^T += Q^T dS.  Each wave keeps one key-side operand and one accumulator
// (half of what one wave doing everything would hold), so two waves fit per
// SIMD, and the two roles of a pair share a SIMD and overlap their matrix
// and vector work.  Q and dO tiles are staged once, row-major, in double
// buffers filled by the memory unit while the previous tile is computed; S
// and dP read their rows, dK^T and dV^T read them transposed.
template <typename T, int D>
__global__ void __launch_bounds__(kDkvThreads) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dkv_kernel(BwdArgs a) {
    constexpr int kQT = q_tile<T, D>();
    constexpr int NQB = kQT / 32;
    using M = Mfma<T, D>;
    constexpr int NW = kDkvThreads / 64;
    using DmaRows = Dma<kQT, M::W, NW>;
    constexpr int NB = D / 32;
    // Three buffers per tile operand: tile k is formed while tile k-1 is
    // contracted and tile k+1 is copied in.
    __shared__ __attribute__((aligned(16))) T Qs[3][kQT * D];
    __shared__ __attribute__((aligned(16))) T Ds[3][kQT * D];
    __shared__ __attribute__((aligned(16))) float lse_s[3][kQT], dlt_s[3][kQT];
    // P handed from wave A to wave B: fp16 for 16-bit inputs (10-bit mantissa,
    // so the dS that forms dK is close to the one the dQ kernel forms from
    // the same scores), fp32 otherwise.
    // Stored as 16-byte vectors [pair][q block][vector][lane] so a lane moves
    // its 16 values with 2 (fp16) or 4 (fp32) wide LDS accesses.
    using PexT = typename std::conditional<sizeof(T) == 2, _Float16, float>::type;
    constexpr int PPV = 16 / sizeof(PexT);     // values per 16-byte vector
    __shared__ __attribute__((aligned(16))) uint4 Pex[3][4][NQB][16 / PPV][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
    const int pair = wave & 3;
    const bool role_a = wave < 4;
    int item_ix, kvh;
    block_to_work(blockIdx.x, a.nitems, a.hkv, 1, item_ix, kvh);
    const int G = a.hq / a.hkv;
    const WorkItem it = load_const(a.items, item_ix);
    const int nkey = it.a1 - it.a0;
    const int kk = pair * 32 + (lane & 31);          // key offset in the item
    const bool key_ok = kk < nkey;
    const bool pair_on = pair * 32 < nkey;           // wave-uniform
    const int64_t krow = (int64_t)it.shard * a.n + it.a0 + kk;   // zigzag row of this lane's key
    const int64_t qrow0 = (int64_t)it.rank * a.n;
    const T *q = static_cast<const T *>(a.q);
    const T *dout = static_cast<const T *>(a.dout);

    // Key-side operand: K rows for wave A (S), V rows for wave B (dP).
    typename M::Op op[M::KS];
    if (key_ok) M::load_row_op(op, static_cast<const T *>(role_a ? a.k : a.v) + (krow * a.hkv + kvh) * D, hh);
    else M::zero_op(op);
    f32x16 acc[NB];   // dV^T (wave A) or dK^T (wave B)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;

    // Walk (query head of the group) x (listed query tile) as one sequence.
    const int ntile = it.tend - it.tbeg;
    const int nwork = G * ntile;
    // Row-major tiles of Q and dO are copied global -> LDS by the memory
    // unit, every wave issuing its share (Q^T and dO^T are read from them by
    // LDS transpose reads); the LSE and delta of a tile go through the
    // registers of the first kQT threads (rows past the tile get LSE = +inf,
    // so their P and dS are exactly 0).
    float lse_r = 0.0f, dlt_r = 0.0f;
    const DmaRows dma((uint32_t)(a.hq * D * sizeof(T)), wave, lane);
    TileWindow win(a.tiles, it.tbeg, ntile, lane);
    auto copy_tile = [&](int u, const TileRec &tn, T *qs, T *ds) __attribute__((always_inline)) {
        const int h = kvh * G + u / ntile;
        const int nq = tn.b1 - tn.b0;
        if (tid < kQT) {   // issued first: the counter waits below do not cover the copies
            const bool ok = tid < nq;
            lse_r = ok ? a.lse[(int64_t)h * a.T + qrow0 + tn.b0 + tid] : INFINITY;   // scaled when stored
            dlt_r = ok ? a.delta[(int64_t)h * a.T + qrow0 + tn.b0 + tid] : 0.0f;
        }
        dma.issue(tile_base<T, D>(q, qrow0 + tn.b0, a.hq, h), nq, qs);
        dma.issue(tile_base<T, D>(dout, qrow0 + tn.b0, a.hq, h), nq, ds);
    };
    auto store_stats = [&](float *lse_c, float *dlt_c) __attribute__((always_inline)) {
        if (tid < kQT) {
            lse_c[tid] = lse_r * kLog2e;
            dlt_c[tid] = dlt_r;
        }
    };
    TileRec cur = win.get(0);
    // Phase k (k = 0 .. nwork), one barrier each, software-pipelined across
    // the pair:
    //   wave A: dV^T += dO(k-1)^T P(k-1)  (P(k-1) still in its registers),
    //           then S(k), P(k) = exp(S - LSE), P(k) -> LDS;
    //   wave B: dS(k-1) = P(k-1) (dP(k-1) - delta)  (P from LDS, dP from its
    //           registers), dK^T += Q(k-1)^T dS(k-1), then dP(k).
    // Each role finishes the product of tile k-1 before it forms tile k's
    // block, so it still holds one block of registers, and A's exponentials
    // overlap B's products on their shared SIMD and vice versa.  Tile k+1 is
    // copied in at the start of the phase.  Buffers: tile k in c, k-1 in pv,
    // k+1 in nx (k mod 3, constant after unrolling by three).
    f32x16 x[NQB];   // wave A: P of the last formed tile; wave B: its dP
    // Every phase does both halves (a runtime "first/last phase" test here
    // costs dozens of registers): phase 0 contracts a zero block against
    // zeroed buffers, which adds exactly 0, and phase nwork forms a block from
    // a stale (finite) tile that is never used.
    auto phase = [&](int k, int c, int pv, int nx) __attribute__((always_inline)) {
        const TileRec tr = cur;
        if (k + 1 < nwork) {
            cur = win.get((k + 1) % ntile);
            copy_tile(k + 1, cur, Qs[nx], Ds[nx]);
        }
        if (pair_on) {
            if (role_a) {
                {
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) M::gemm_t_c(acc, Ds[pv], qb * 32, x[qb], lane);
                }
                __builtin_amdgcn_sched_barrier(0);   // keeps the two products' operands apart
                {
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) x[qb][i] = 0.0f;
                    if constexpr (NQB == 2)
                        M::gemm_rows_lds2(x[0], x[1], Qs[c], lane & 31, 32 + (lane & 31), op, hh);
                    else
                        M::gemm_rows_lds(x[0], Qs[c], lane & 31, op, hh);
                    const float *ls = lse_s[c];
                    // Only partial (diagonal) tiles need a mask: query rows past
                    // a ragged tile have P = 0 through their LSE, and the
                    // columns of keys past a ragged item are never written.
                    // Query row qq sees key kk iff qq >= kk - delta.
                    if (tr.kind != ZZ_TILE_FULL) {
#pragma unroll
                        for (int qb = 0; qb < NQB; ++qb) mask_rows_below(x[qb], kk - tr.delta - qb * 32 - 4 * hh);
                    }
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) {
                        float4 l4[4];   // LSE of this lane's 16 query rows (4 runs of 4)
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4)
                            l4[i4] = *reinterpret_cast<const float4 *>(ls + qb * 32 + c_row(4 * i4, hh));
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const float lv = i % 4 == 0 ? l4[i / 4].x : i % 4 == 1 ? l4[i / 4].y
                                           : i % 4 == 2 ? l4[i / 4].z : l4[i / 4].w;
                            x[qb][i] = __builtin_amdgcn_exp2f(fmaf(x[qb][i], a.scale_log2, -lv));
                        }
#pragma unroll
                        for (int vi = 0; vi < 16 / PPV; ++vi) {
                            PexT pv[PPV];
#pragma unroll
                            for (int e = 0; e < PPV; ++e) pv[e] = static_cast<PexT>(x[qb][vi * PPV + e]);
                            Pex[c][pair][qb][vi][lane] = *reinterpret_cast<const uint4 *>(pv);
                        }
                    }
                }
            } else {
                {
                    const float *dl = dlt_s[pv];
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) {
                        float4 d4[4];
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4)
                            d4[i4] = *reinterpret_cast<const float4 *>(dl + qb * 32 + c_row(4 * i4, hh));
#pragma unroll
                        for (int vi = 0; vi < 16 / PPV; ++vi) {
                            const uint4 raw = Pex[pv][pair][qb][vi][lane];
                            const PexT *pe = reinterpret_cast<const PexT *>(&raw);
#pragma unroll
                            for (int e = 0; e < PPV; ++e) {
                                const int i = vi * PPV + e;
                                const float dv = i % 4 == 0 ? d4[i / 4].x : i % 4 == 1 ? d4[i / 4].y
                                               : i % 4 == 2 ? d4[i / 4].z : d4[i / 4].w;
                                x[qb][i] = static_cast<float>(pe[e]) * (x[qb][i] - dv);
                            }
                        }
                        M::gemm_t_c(acc, Qs[pv], qb * 32, x[qb], lane);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                {
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) x[qb][i] = 0.0f;
                    if constexpr (NQB == 2)
                        M::gemm_rows_lds2(x[0], x[1], Ds[c], lane & 31, 32 + (lane & 31), op, hh);
                    else
                        M::gemm_rows_lds(x[0], Ds[c], lane & 31, op, hh);
                }
            }
        }
        if (k + 1 < nwork) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's copies of tile k+1 have landed
            store_stats(lse_s[nx], dlt_s[nx]);
        }
        __syncthreads();
    };
    copy_tile(0, cur, Qs[0], Ds[0]);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[qb][i] = 0.0f;
    {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int i = tid; i < kQT * D * (int)sizeof(T) / 16; i += kDkvThreads) {
            reinterpret_cast<uint4 *>(Qs[2])[i] = z;
            reinterpret_cast<uint4 *>(Ds[2])[i] = z;
        }
        for (int i = tid; i < (int)(sizeof(Pex[2]) / 16); i += kDkvThreads) (&Pex[2][0][0][0][0])[i] = z;
        if (tid < kQT) dlt_s[2][tid] = 0.0f;
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the key-side operand and tile 0 have landed
    store_stats(lse_s[0], dlt_s[0]);
    __syncthreads();
    for (int k = 0; k <= nwork; k += 3) {
        phase(k, 0, 2, 1);
        if (k + 1 <= nwork) phase(k + 1, 1, 0, 2);
        if (k + 2 <= nwork) phase(k + 2, 2, 1, 0);
    }
    if (!key_ok) return;
    if (role_a) add_row<NB>(a.dv + (krow * a.hkv + kvh) * D, acc, 1.0f, hh, a.accumulate != 0);
    else add_row<NB>(a.dk + (krow * a.hkv + kvh) * D, acc, a.scale, hh, a.accumulate != 0);
}

template <typename T, int D>
hipError_t launch_t(const zz_plan *p, int base, int rank, int step, BwdArgs a, int which, hipStream_t st) {
    const int pkv = base + ZZ_PASS_BWD_DKV, pq = base + ZZ_PASS_BWD_DQ;
    const Launch Lkv = launch_items(p, pkv, rank, step);
    if ((which & 1) && Lkv.n > 0) {
        a.items = Lkv.items; a.tiles = dev_tiles(p, pkv); a.nitems = Lkv.n;
        hipLaunchKernelGGL((bwd_dkv_kernel<T, D>), dim3(Lkv.n * p->hkv), dim3(kDkvThreads), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (which & 2) return launch_dq(p, pq, rank, step, a, st);
    return hipSuccess;
}

hipError_t launch_bwd_pass(const zz_plan *p, int base, int rank, int step, const void *q, const void *k,
                           const void *v, const void *dout, const float *lse, const float *delta, float *dq,
                           float *dk, float *dv, int accumulate, int which, hipStream_t st) {
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.lse = lse; a.delta = delta;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.items = nullptr; a.tiles = nullptr;
    a.T = p->T; a.n = (int32_t)(p->T / p->cp); a.hq = p->hq; a.hkv = p->hkv;
    a.scale = (float)(1.0 / std::sqrt((double)p->d));
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->d));
    a.accumulate = accumulate;
    if (p->dtype == ZZ_BF16) {
        if (p->d == 32) return launch_t<bf16, 32>(p, base, rank, step, a, which, st);
        if (p->d == 64) return launch_t<bf16, 64>(p, base, rank, step, a, which, st);
        return launch_t<bf16, 128>(p, base, rank, step, a, which, st);
    }
    if (p->d == 32) return launch_t<float, 32>(p, base, rank, step, a, which, st);
    if (p->d == 64) return launch_t<float, 64>(p, base, rank, step, a, which, st);
    return launch_t<float, 128>(p, base, rank, step, a, which, st);
}

}  // namespace

hipError_t launch_bwd_step(const zz_plan *p, int rank, int step, const void *q, const void *k, const void *v,
                           const void *dout, const float *lse, const float *delta, float *dq, float *dk,
                           float *dv, int accumulate, int which, hipStream_t st) {
    return launch_bwd_pass(p, 0, rank, step, q, k, v, dout, lse, delta, dq, dk, dv, accumulate, which, st);
}

hipError_t launch_bwd_gathered(const zz_plan *p, int rank, const void *q, const void *k, const void *v,
                               const void *dout, const float *lse, const float *delta, float *dq, float *dk,
                               float *dv, hipStream_t st) {
    return launch_bwd_pass(p, kPassGathered, rank, 0, q, k, v, dout, lse, delta, dq, dk, dv, 0, 3, st);
}

}  // namespace zz
