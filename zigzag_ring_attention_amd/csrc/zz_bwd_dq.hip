// Backward ring step of zigzag varlen attention, dQ kernel (FlagScale PR #910: the
// per-step backward of a ring driver).  With the global LSE of the merged
// forward, a step's contribution is a plain sum:
//   P = exp(S - LSE), dP = dO V^T, dS = P (dP - delta), delta = rowsum(dO O)
//   dQ_r += scale dS K_j,  dK_j += scale dS^T Q_r,  dV_j += P^T dO_r
// summed over the query heads of each key/value group.
//
// Query-major: S^T and dP^T with the queries in the lane dimension, like the
// forward step, then dQ^T += K^T dS^T.  Fully masked tiles are never
// visited (tile lists from the planner).

#include "zz_bwd.h"

namespace zz {
namespace {

// ---------------------------------------------------------------- dQ

// Keys per streamed tile (must match the planner's dQ tile): halved for fp32
// with D >= 64 so the double-buffered LDS stage fits.
template <typename T, int D> constexpr int k_tile() { return (sizeof(T) == 4 && D >= 64) ? 32 : 64; }
constexpr int kDqThreads = 512;    // eight waves own 32 query rows each

// Query-major: a workgroup owns up to 256 query rows of one head (eight
// waves of 32) and walks the item's key tiles, with the K and V tiles copied
// global -> LDS by the memory unit into double buffers (K^T is read from the
// K tile by LDS transpose reads).
template <typename T, int D>
__global__ void __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dq_kernel(BwdArgs a) {
    using M = Mfma<T, D>;
    constexpr int kKT = k_tile<T, D>();
    constexpr int NW = kDqThreads / 64;
    using DmaRows = Dma<kKT, M::W, NW>;
    constexpr int NB = D / 32;
    // K (S^T = K Q^T, and read transposed for dQ^T += K^T dS^T) and V
    // (dP^T = V dO^T), row-major.
    __shared__ __attribute__((aligned(16))) T Ks[2][kKT * D];
    __shared__ __attribute__((aligned(16))) T Vs[2][kKT * D];

    const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    int item_ix, head;
    block_to_work(blockIdx.x, a.nitems, a.hq, a.hq / a.hkv, item_ix, head);
    const int kvh = head / (a.hq / a.hkv);
    const WorkItem it = load_const(a.items, item_ix);
    const int nq = it.a1 - it.a0;
    const int qq = wave * 32 + (lane & 31);
    const bool row_ok = qq < nq;
    const bool wave_on = wave * 32 < nq;
    const int64_t zrow = (int64_t)it.rank * a.n + it.a0 + qq;
    const T *k = static_cast<const T *>(a.k);
    const T *v = static_cast<const T *>(a.v);

    typename M::Op qop[M::KS], dop[M::KS];
    float lse2 = 0.0f, dlt = 0.0f;
    if (row_ok) {
        M::load_row_op(qop, static_cast<const T *>(a.q) + (zrow * a.hq + head) * D, hh);
        M::load_row_op(dop, static_cast<const T *>(a.dout) + (zrow * a.hq + head) * D, hh);
        lse2 = a.lse[(int64_t)head * a.T + zrow] * kLog2e;
        dlt = a.delta[(int64_t)head * a.T + zrow];
    } else {
        M::zero_op(qop);
        M::zero_op(dop);
    }
    f32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
    const int64_t kv_row0 = (int64_t)it.shard * a.n;

    const DmaRows dma((uint32_t)(a.hkv * D * sizeof(T)), wave, lane);
    TileWindow win(a.tiles, it.tbeg, it.tend - it.tbeg, lane);
    auto copy_tile = [&](const TileRec &tn, T *ks, T *vs) __attribute__((always_inline)) {
        const int nk = tn.b1 - tn.b0;
        dma.issue(tile_base<T, D>(k, kv_row0 + tn.b0, a.hkv, kvh), nk, ks);
        dma.issue(tile_base<T, D>(v, kv_row0 + tn.b0, a.hkv, kvh), nk, vs);
    };
    // One tile, as in the forward step: the copy of tile t+1 overlaps this
    // tile's work; constant buffers (loop unrolled by two).
    TileRec cur = win.get(0);
    auto tile_step = [&](int t, const T *ks, const T *vs, T *ks_next, T *vs_next) __attribute__((always_inline)) {
        const TileRec tr = cur;
        const int nk = tr.b1 - tr.b0;
        cur = win.get(min(t + 1, it.tend - 1) - it.tbeg);
        copy_tile(cur, ks_next, vs_next);
        if (wave_on) {
#pragma unroll
            for (int kb = 0; kb < kKT / 32; ++kb) {
                // dP^T accumulates onto -delta (one value per lane: the lane's
                // query), so the chain yields dP - delta directly
                f32x16 s, dp;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[i] = 0.0f;
                    dp[i] = -dlt;
                }
                M::gemm_rows_lds_pair(s, ks, qop, dp, vs, dop, kb * 32 + (lane & 31), hh);
                // mask (partial and ragged tiles only): key kk is kept iff kk < nk
                // and, in a partial tile, kk <= qq + delta; rows of queries past
                // the item are never written
                if (tr.kind != ZZ_TILE_FULL || nk < kKT)
                    mask_rows_above(s, (tr.kind == ZZ_TILE_FULL ? nk - 1 : min(nk - 1, qq + tr.delta)) - kb * 32 -
                                           4 * hh);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -lse2));
                    dp[i] = p * dp[i];
                }
                M::gemm_t_c(acc, ks, kb * 32, dp, lane);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's copies of tile t+1 have landed
        __syncthreads();
    };
    copy_tile(cur, Ks[0], Vs[0]);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the query-side operands and tile 0 have landed
    __syncthreads();
    for (int t = it.tbeg; t < it.tend; t += 2) {
        tile_step(t, Ks[0], Vs[0], Ks[1], Vs[1]);
        if (t + 1 < it.tend) tile_step(t + 1, Ks[1], Vs[1], Ks[0], Vs[0]);
    }
    if (!row_ok) return;
    add_row<NB>(a.dq + (zrow * a.hq + head) * D, acc, a.scale, hh, a.accumulate != 0);
}

template <typename T, int D>
hipError_t launch_t(const zz_plan *p, int pass, int rank, int step, BwdArgs a, hipStream_t st) {
    const Launch L = launch_items(p, pass, rank, step);
    if (L.n == 0) return hipSuccess;
    a.items = L.items; a.tiles = dev_tiles(p, pass); a.nitems = L.n;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3(L.n * p->hq), dim3(kDqThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dq(const zz_plan *p, int pass, int rank, int step, BwdArgs a, hipStream_t st) {
    if (p->dtype == ZZ_BF16) {
        if (p->d == 32) return launch_t<bf16, 32>(p, pass, rank, step, a, st);
        if (p->d == 64) return launch_t<bf16, 64>(p, pass, rank, step, a, st);
        return launch_t<bf16, 128>(p, pass, rank, step, a, st);
    }
    if (p->d == 32) return launch_t<float, 32>(p, pass, rank, step, a, st);
    if (p->d == 64) return launch_t<float, 64>(p, pass, rank, step, a, st);
    return launch_t<float, 128>(p, pass, rank, step, a, st);
}

}  // namespace zz
