// Memory-bound kernels of libzz: zigzag permute / unpermute, fp32 -> dtype
// cast (optionally unpermuting), the standalone log-sum-exp merge, the
// backward pre-pass delta = rowsum(dO * O), and the debug visibility dump.
// All are HBM-bound: 16-byte vector accesses, whole rows per thread group.

#include "zz_device.h"

namespace zz {
namespace {

constexpr int kThreads = 256;

int grid_for(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    return (int)std::max<int64_t>(1, std::min<int64_t>(g, 256 * 64));
}

// Row-parallel launches: one wave per row, rows dealt to the grid's waves in
// a grid-stride loop; the 64 lanes of a wave walk the row's 16-byte vectors
// with several loads in flight per lane.  No per-element index arithmetic
// beyond an add: the row comes from the loop, the vector from the lane.
constexpr int kWavesPerBlock = kThreads / 64;

int grid_rows(int64_t rows) {
    return (int)std::max<int64_t>(1, std::min<int64_t>((rows + kWavesPerBlock - 1) / kWavesPerBlock, 256 * 32));
}

// Row gather / scatter by the zigzag row map: src[z] = packed token at
// zigzag row z.  Forward: out[z] = in[src[z]]; inverse: out[src[z]] = in[z].
// Eight 16-byte loads in flight per lane, loads and stores marked
// non-temporal (each byte is touched once): 5.4 TB/s on a 4 GiB bf16 tensor,
// against 5.2 TB/s with four ordinary loads in flight.
__global__ void __launch_bounds__(kThreads)
permute_kernel(const int4 *__restrict__ in, int4 *__restrict__ out, const int32_t *__restrict__ src,
               int64_t rows, int64_t vpr, int inverse) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t z = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); z < rows; z += nwaves) {
        const int64_t p = src[z];
        const i32x4 *s = reinterpret_cast<const i32x4 *>(in + (inverse ? z : p) * vpr);
        i32x4 *d = reinterpret_cast<i32x4 *>(out + (inverse ? p : z) * vpr);
        int64_t c = lane;
        for (; c + 448 < vpr; c += 512) {
            i32x4 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(s + c + 64 * u);
#pragma unroll
            for (int u = 0; u < 8; ++u) __builtin_nontemporal_store(x[u], d + c + 64 * u);
        }
        for (; c < vpr; c += 64) __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
    }
}

template <typename T> __device__ __forceinline__ void store4(T *dst, float4 v);
template <> __device__ __forceinline__ void store4<float>(float *dst, float4 v) {
    *reinterpret_cast<float4 *>(dst) = v;
}
template <> __device__ __forceinline__ void store4<bf16>(bf16 *dst, float4 v) {
    bf16x4 b = {to_bf16(v.x), to_bf16(v.y), to_bf16(v.z), to_bf16(v.w)};
    *reinterpret_cast<bf16x4 *>(dst) = b;
}

// fp32 zigzag rows -> element type, to zigzag or packed order (one wave per
// row, as the permute).
template <typename T>
__global__ void __launch_bounds__(kThreads)
cast_rows_kernel(const float4 *__restrict__ in, T *__restrict__ out, const int32_t *__restrict__ src,
                 int64_t rows, int64_t vpr, int unpermute) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t z = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); z < rows; z += nwaves) {
        const int64_t orow = unpermute ? (int64_t)src[z] : z;
        const float4 *s = in + z * vpr;
        T *d = out + orow * vpr * 4;
        int64_t c = lane;
        for (; c + 192 < vpr; c += 256) {
            const float4 a = s[c], b = s[c + 64], e = s[c + 128], f = s[c + 192];
            store4<T>(d + c * 4, a);
            store4<T>(d + (c + 64) * 4, b);
            store4<T>(d + (c + 128) * 4, e);
            store4<T>(d + (c + 192) * 4, f);
        }
        for (; c < vpr; c += 64) store4<T>(d + c * 4, s[c]);
    }
}

// Standalone merge.  A block owns kPairs (row, head) pairs: it reads both
// LSEs, forms the weights in shared memory, updates O, then writes the LSE.
constexpr int kPairs = 64;
__global__ void __launch_bounds__(kThreads)
lse_merge_kernel(float *__restrict__ o, float *__restrict__ lse, const float *__restrict__ o2,
                 const float *__restrict__ lse2, int64_t rows, int32_t heads, int32_t d) {
    __shared__ MergeWeights w[kPairs];
    const int64_t npairs = rows * heads;
    const int vp = d / 4;
    for (int64_t base = (int64_t)blockIdx.x * kPairs; base < npairs; base += (int64_t)gridDim.x * kPairs) {
        const int np = (int)std::min<int64_t>(kPairs, npairs - base);
        if (threadIdx.x < np) {
            const int64_t pr = base + threadIdx.x;
            const int64_t row = pr / heads, h = pr - row * heads;
            w[threadIdx.x] = merge_weights(lse[h * rows + row], lse2[h * rows + row]);
        }
        __syncthreads();
        for (int e = threadIdx.x; e < np * vp; e += kThreads) {
            const int u = e / vp, c = e - u * vp;
            const int64_t off = (base + u) * d + c * 4;
            float4 a = *reinterpret_cast<const float4 *>(o + off);
            const float4 b = *reinterpret_cast<const float4 *>(o2 + off);
            const MergeWeights ww = w[u];
            a.x = merge_value(ww, a.x, b.x);
            a.y = merge_value(ww, a.y, b.y);
            a.z = merge_value(ww, a.z, b.z);
            a.w = merge_value(ww, a.w, b.w);
            *reinterpret_cast<float4 *>(o + off) = a;
        }
        if (threadIdx.x < np) {
            const int64_t pr = base + threadIdx.x;
            const int64_t row = pr / heads, h = pr - row * heads;
            lse[h * rows + row] = w[threadIdx.x].lse;
        }
        __syncthreads();
    }
}

// delta[h, z] = sum_e dO[z,h,e] O[z,h,e]; a group of LPP lanes per (z, h).
template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
bwd_pre_kernel(const T *__restrict__ o, const T *__restrict__ dout, float *__restrict__ delta,
               int64_t rows, int32_t heads) {
    constexpr int EPV = 16 / sizeof(T);    // elements per 16-byte vector
    constexpr int LPP = D / EPV;           // lanes per (row, head)
    static_assert(LPP >= 1 && LPP <= 64 && (64 % LPP) == 0, "lanes per pair");
    const int64_t npairs = rows * heads;
    const int sub = threadIdx.x % LPP;
    for (int64_t pr = (blockIdx.x * (int64_t)kThreads + threadIdx.x) / LPP; pr < npairs;
         pr += (int64_t)gridDim.x * kThreads / LPP) {
        const int64_t off = pr * D + sub * EPV;
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            s += Elem<T>::to_float(o[off + e]) * Elem<T>::to_float(dout[off + e]);
#pragma unroll
        for (int m = LPP / 2; m >= 1; m /= 2) s += __shfl_xor(s, m, LPP);
        if (sub == 0) {
            const int64_t row = pr / heads, h = pr - row * heads;
            delta[h * rows + row] = s;
        }
    }
}

__global__ void __launch_bounds__(kThreads)
fill_u8_kernel(uint8_t *__restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        p[i] = 0;
}

// One block per work item: mark every visible pair of its listed tiles.
__global__ void __launch_bounds__(kThreads)
debug_mask_kernel(const WorkItem *__restrict__ items, const TileRec *__restrict__ tiles,
                  uint8_t *__restrict__ mask, int64_t n, int key_major) {
    const WorkItem it = items[blockIdx.x];
    for (int t = it.tbeg; t < it.tend; ++t) {
        const TileRec tr = tiles[t];
        const int q0 = key_major ? tr.b0 : it.a0, q1 = key_major ? tr.b1 : it.a1;
        const int k0 = key_major ? it.a0 : tr.b0, k1 = key_major ? it.a1 : tr.b1;
        const int nk = k1 - k0, cells = (q1 - q0) * nk;
        for (int e = threadIdx.x; e < cells; e += kThreads) {
            const int qq = e / nk, kk = e - qq * nk;
            if (tile_visible(tr.kind, tr.delta, qq, kk)) mask[(int64_t)(q0 + qq) * n + (k0 + kk)] = 1;
        }
    }
}

}  // namespace

hipError_t launch_permute(const zz_plan *p, const void *in, void *out, int64_t row_bytes, bool inverse,
                          hipStream_t st) {
    const int64_t vpr = row_bytes / 16;
    hipLaunchKernelGGL(permute_kernel, dim3(grid_rows(p->T)), dim3(kThreads), 0, st,
                       (const int4 *)in, (int4 *)out, dev_src(p), p->T, vpr, inverse ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_cast_rows(const zz_plan *p, const float *in, void *out, int32_t heads, bool unpermute,
                            hipStream_t st) {
    const int64_t vpr = (int64_t)heads * p->d / 4;
    const dim3 grid(grid_rows(p->T));
    if (p->dtype == ZZ_BF16)
        hipLaunchKernelGGL(cast_rows_kernel<bf16>, grid, dim3(kThreads), 0, st, (const float4 *)in,
                           (bf16 *)out, dev_src(p), p->T, vpr, unpermute ? 1 : 0);
    else
        hipLaunchKernelGGL(cast_rows_kernel<float>, grid, dim3(kThreads), 0, st, (const float4 *)in,
                           (float *)out, dev_src(p), p->T, vpr, unpermute ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_lse_merge(float *o, float *lse, const float *o2, const float *lse2, int64_t rows,
                            int32_t heads, int32_t d, hipStream_t st) {
    hipLaunchKernelGGL(lse_merge_kernel, dim3(grid_for(rows * heads, kPairs)), dim3(kThreads), 0, st, o,
                       lse, o2, lse2, rows, heads, d);
    return hipGetLastError();
}

hipError_t launch_bwd_pre(const zz_plan *p, const void *o, const void *dout, float *delta, hipStream_t st) {
    const int64_t pairs = p->T * p->hq;
    const dim3 grid(grid_for(pairs, 32)), block(kThreads);
#define ZZ_PRE(ET, DD)                                                                                 \
    hipLaunchKernelGGL((bwd_pre_kernel<ET, DD>), grid, block, 0, st, (const ET *)o, (const ET *)dout, delta, \
                       p->T, p->hq)
    if (p->dtype == ZZ_BF16) {
        if (p->d == 32) ZZ_PRE(bf16, 32); else if (p->d == 64) ZZ_PRE(bf16, 64); else ZZ_PRE(bf16, 128);
    } else {
        if (p->d == 32) ZZ_PRE(float, 32); else if (p->d == 64) ZZ_PRE(float, 64); else ZZ_PRE(float, 128);
    }
#undef ZZ_PRE
    return hipGetLastError();
}

hipError_t launch_debug_mask(const zz_plan *p, int pass, int rank, int step, uint8_t *mask, hipStream_t st) {
    const int64_t n = p->T / p->cp;
    hipLaunchKernelGGL(fill_u8_kernel, dim3(grid_for(n * n, kThreads * 4)), dim3(kThreads), 0, st, mask, n * n);
    const Launch L = launch_items(p, pass, rank, step);
    if (L.n > 0)
        hipLaunchKernelGGL(debug_mask_kernel, dim3(L.n), dim3(kThreads), 0, st, L.items, dev_tiles(p, pass),
                           mask, n, p->pass[pass].key_major ? 1 : 0);
    return hipGetLastError();
}

}  // namespace zz
