// Forward ring step of zigzag varlen attention (FlagScale PR #910: the
// per-step forward of a ring driver; MiniMax-01 issue #6: varlen ring
// attention over packed data).
//
// One workgroup = one work item (a tile of up to 128 query rows of one rank,
// inside one zigzag chunk) x one query head.  Four waves own 32 query rows
// each.  The workgroup walks the item's listed key tiles of shard
// j = (rank - step) mod CP -- fully masked tiles were pruned by the planner --
// with K and V tiles of up to 64 keys copied straight from global memory
// into double-buffered row-major LDS tiles by the memory unit (V^T is read
// from the V tile by LDS transpose reads).  Per tile and wave:
//   S^T = K Q^T * scale * log2(e)          (MFMA, fp32 accumulate)
//   mask only on PARTIAL tiles (diagonal chunk pair: key offset <= query
//   offset); keys past the ragged tile end are masked on every tile
//   online softmax per query: running max m (exchanged between the two lane
//   halves that hold the query's keys), rescale, exp2
//   O^T += V^T P^T                          (MFMA, P rounded to the input dtype)
// Epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2 (natural log), written as
// the step's partial or merged into the accumulator by log-sum-exp.
//
// Scale 1/sqrt(head_dim): MaxText PR #1133, scale_factor of the CP attention call.

#include "zz_mfma.h"

namespace zz {
namespace {

constexpr int kWaves = 4;
// s_waitcnt immediate that waits for vmcnt = 0 only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the others at their maximum).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per LDS tile

struct FwdArgs {
    const void *q, *k, *v;
    float *o, *lse;
    const WorkItem *items;
    const TileRec *tiles;
    int64_t T;          // total tokens
    int32_t n;          // rows per rank = T / cp
    int32_t hq, hkv;
    float scale_log2;   // softmax scale * log2(e)
    int32_t merge;
    int32_t nitems;     // work items in this launch
};

template <typename T, int D>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
fwd_step_kernel(FwdArgs a) {
    using M = Mfma<T, D>;
    using DmaKV = Dma<kBN, M::W, kWaves>;
    constexpr int NB = D / 32;   // 32-wide head-dim blocks of O^T
    // Double-buffered row-major K (A operand of S^T = K Q^T) and V (read
    // transposed as the A operand of O^T = V^T P^T).  One barrier per tile.
    __shared__ __attribute__((aligned(16))) T Ks[2][kBN * D];
    __shared__ __attribute__((aligned(16))) T Vs[2][kBN * D];

    const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    int item_ix, head;
    block_to_work(blockIdx.x, a.nitems, a.hq, a.hq / a.hkv, item_ix, head);
    const int kvh = head / (a.hq / a.hkv);
    const WorkItem it = load_const(a.items, item_ix);
    const int nq = it.a1 - it.a0;
    const int qq = wave * 32 + (lane & 31);          // query offset in the item
    const bool row_ok = qq < nq;
    const bool wave_on = wave * 32 < nq;             // wave-uniform
    const int64_t zrow = (int64_t)it.rank * a.n + it.a0 + qq;   // zigzag row of this lane's query
    const T *q = static_cast<const T *>(a.q);
    const T *k = static_cast<const T *>(a.k);
    const T *v = static_cast<const T *>(a.v);

    if (it.tbeg == it.tend) {
        // No visible key in this step: the partial is (0, -inf); merging it is a no-op.
        if (a.merge || !row_ok) return;
        float4 z = {0.f, 0.f, 0.f, 0.f};
        float *orow = a.o + (zrow * a.hq + head) * D;
        for (int e = 4 * hh; e < D; e += 8) *reinterpret_cast<float4 *>(orow + e) = z;
        if (hh == 0) a.lse[(int64_t)head * a.T + zrow] = -INFINITY;
        return;
    }

    typename M::Op qop[M::KS];
    if (row_ok) M::load_row_op(qop, q + (zrow * a.hq + head) * D, hh);
    else M::zero_op(qop);

    f32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
    // m: reference maximum of the scaled scores (log2 units) that every weight
    // of this query is taken relative to.  It is only moved when a tile's
    // maximum exceeds it by more than kLazy, so weights stay below 2^kLazy and
    // the O rescale is skipped on most tiles.
    constexpr float kLazy = 8.0f;
    float m = -INFINITY, lsum = 0.0f;
    const int64_t kv_row0 = (int64_t)it.shard * a.n;

    const DmaKV dma((uint32_t)(a.hkv * D * sizeof(T)), wave, lane);
    TileWindow win(a.tiles, it.tbeg, it.tend - it.tbeg, lane);
    auto copy_tile = [&](const TileRec &tn, T *ks, T *vs) __attribute__((always_inline)) {
        const int nk = tn.b1 - tn.b0;
        dma.issue(tile_base<T, D>(k, kv_row0 + tn.b0, a.hkv, kvh), nk, ks);
        dma.issue(tile_base<T, D>(v, kv_row0 + tn.b0, a.hkv, kvh), nk, vs);
    };
    // One tile: the copy of tile t+1 into the other buffer (its last readers
    // finished before the barrier that ended the previous tile) is issued
    // first and overlaps this tile's work; past the end it re-reads the last
    // tile into the unused buffer.  Called with constant buffers (the loop
    // below is unrolled by two), so every LDS address is a lane offset plus
    // an immediate.
    TileRec cur = win.get(0);
    auto tile_step = [&](int t, const T *ks, const T *vs, T *ks_next, T *vs_next) __attribute__((always_inline)) {
        const TileRec tr = cur;
        const int nk = tr.b1 - tr.b0;
        cur = win.get(min(t + 1, it.tend - 1) - it.tbeg);
        copy_tile(cur, ks_next, vs_next);
        if (wave_on) {
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
            M::gemm_rows_lds2(s[0], s[1], ks, lane & 31, 32 + (lane & 31), qop, hh);
            // mask (partial and ragged tiles only): key kk is kept iff
            // kk < nk and, in a partial tile, kk <= qq + delta
            if (tr.kind != ZZ_TILE_FULL || nk < kBN) {
                const int last = tr.kind == ZZ_TILE_FULL ? nk - 1 : min(nk - 1, qq + tr.delta);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) mask_rows_above(s[kb], last - kb * 32 - 4 * hh);
            }
            float mraw = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, s[kb][i]);
            mraw = fmaxf(mraw, swap_halves(mraw, lane));
            const float mt = mraw * a.scale_log2;     // scale > 0 commutes with max
            const bool move = mt > m + kLazy;         // false for an all-masked tile
            const float mnew = move ? mt : m;
            const float msafe = mnew == -INFINITY ? 0.0f : mnew;
            if (__builtin_amdgcn_ballot_w64(move)) {
                const float alpha = __builtin_amdgcn_exp2f(m - msafe);
                lsum *= alpha;
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;
            }
            m = mnew;
            float ps = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -msafe));
                    s[kb][i] = p;
                    ps += p;
                }
            lsum += ps;
            M::gemm_t_c(acc, vs, 0, s[0], lane);
            M::gemm_t_c(acc, vs, 32, s[1], lane);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's copies of tile t+1 have landed
        __syncthreads();
    };
    copy_tile(cur, Ks[0], Vs[0]);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int t = it.tbeg; t < it.tend; t += 2) {
        tile_step(t, Ks[0], Vs[0], Ks[1], Vs[1]);
        if (t + 1 < it.tend) tile_step(t + 1, Ks[1], Vs[1], Ks[0], Vs[0]);
    }
    if (!row_ok) return;

    // Epilogue: the lane pair (l, l^32) holds one query's keys split in two.
    const float ltot = lsum + swap_halves(lsum, lane);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    const float lse_b = ltot > 0.0f ? (m + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
    float *orow = a.o + (zrow * a.hq + head) * D;
    float *lse_p = a.lse + (int64_t)head * a.T + zrow;
    if (!a.merge) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                float4 w;
                w.x = acc[b][4 * i4 + 0] * inv;
                w.y = acc[b][4 * i4 + 1] * inv;
                w.z = acc[b][4 * i4 + 2] * inv;
                w.w = acc[b][4 * i4 + 3] * inv;
                *reinterpret_cast<float4 *>(orow + 32 * b + c_row(4 * i4, hh)) = w;
            }
        if (hh == 0) *lse_p = lse_b;
    } else {
        const MergeWeights w = merge_weights(*lse_p, lse_b);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                float4 *dst = reinterpret_cast<float4 *>(orow + 32 * b + c_row(4 * i4, hh));
                float4 o = *dst;
                o.x = merge_value(w, o.x, acc[b][4 * i4 + 0] * inv);
                o.y = merge_value(w, o.y, acc[b][4 * i4 + 1] * inv);
                o.z = merge_value(w, o.z, acc[b][4 * i4 + 2] * inv);
                o.w = merge_value(w, o.w, acc[b][4 * i4 + 3] * inv);
                *dst = o;
            }
        if (hh == 0) *lse_p = w.lse;
    }
}

template <typename T, int D>
hipError_t launch_t(const zz_plan *p, const Launch &L, const TileRec *tiles, const void *q, const void *k,
                    const void *v, float *o, float *lse, int merge, hipStream_t st) {
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.items = L.items; a.tiles = tiles;
    a.T = p->T; a.n = (int32_t)(p->T / p->cp); a.hq = p->hq; a.hkv = p->hkv;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->d));
    a.merge = merge;
    a.nitems = L.n;
    hipLaunchKernelGGL((fwd_step_kernel<T, D>), dim3(L.n * p->hq), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_fwd_pass(const zz_plan *p, int pass, int rank, int step, const void *q, const void *k,
                           const void *v, float *o, float *lse, int merge, hipStream_t st) {
    const Launch L = launch_items(p, pass, rank, step);
    if (L.n == 0) return hipSuccess;
    const TileRec *tiles = dev_tiles(p, pass);
    if (p->dtype == ZZ_BF16) {
        if (p->d == 32) return launch_t<bf16, 32>(p, L, tiles, q, k, v, o, lse, merge, st);
        if (p->d == 64) return launch_t<bf16, 64>(p, L, tiles, q, k, v, o, lse, merge, st);
        return launch_t<bf16, 128>(p, L, tiles, q, k, v, o, lse, merge, st);
    }
    if (p->d == 32) return launch_t<float, 32>(p, L, tiles, q, k, v, o, lse, merge, st);
    if (p->d == 64) return launch_t<float, 64>(p, L, tiles, q, k, v, o, lse, merge, st);
    return launch_t<float, 128>(p, L, tiles, q, k, v, o, lse, merge, st);
}

}  // namespace

hipError_t launch_fwd_step(const zz_plan *p, int rank, int step, const void *q, const void *k, const void *v,
                           float *o, float *lse, int merge, hipStream_t st) {
    return launch_fwd_pass(p, ZZ_PASS_FWD, rank, step, q, k, v, o, lse, merge, st);
}

hipError_t launch_fwd_gathered(const zz_plan *p, int rank, const void *q, const void *k, const void *v, float *o,
                               float *lse, hipStream_t st) {
    return launch_fwd_pass(p, kPassGathered + ZZ_PASS_FWD, rank, 0, q, k, v, o, lse, 0, st);
}

}  // namespace zz
