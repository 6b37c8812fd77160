// Device-side helpers shared by the libzz kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "zz_internal.h"

namespace zz {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Visibility inside a listed tile, shared by every kernel that applies the
// mask and by the debug dump.  qq / kk are the query / key offsets inside the
// tile; a PARTIAL tile comes from a diagonal chunk pair, where a key is
// visible iff its chunk offset does not exceed the query's (causal).
__device__ __forceinline__ bool tile_visible(int kind, int delta, int qq, int kk) {
    return kind == ZZ_TILE_FULL || kk <= qq + delta;
}

// Log-sum-exp merge of two partial results over disjoint key sets:
// L = log(e^a + e^b), O = e^(a-L) O_a + e^(b-L) O_b; (0, -inf) is the
// identity.  Used both by the standalone merge and by the fused epilogue of
// the forward step, so the two give bit-identical results.
struct MergeWeights {
    float wa, wb, lse;
};
__device__ __forceinline__ MergeWeights merge_weights(float a, float b) {
    const float m = fmaxf(a, b);
    if (m == -INFINITY) return MergeWeights{0.0f, 0.0f, -INFINITY};
    const float L = m + logf(expf(a - m) + expf(b - m));
    return MergeWeights{expf(a - L), expf(b - L), L};
}
__device__ __forceinline__ float merge_value(const MergeWeights &w, float oa, float ob) {
    return fmaf(w.wa, oa, w.wb * ob);
}

// Map a 1-D workgroup index to (work item, head).  Workgroups are dealt to
// the 8 XCDs of the chip round-robin, and each XCD has its own L2; when the
// key/value heads split evenly over the XCDs, every XCD gets whole key/value
// groups, and consecutive workgroups on an XCD are the G query heads of one
// item, so the workgroups that read the same K/V tiles share an L2.
// `group` = query heads per key/value head (1 for the key-major pass).
__device__ __forceinline__ void block_to_work(int b, int nitems, int nheads, int group, int &item, int &head) {
    const int nkv = nheads / group;
    if (nkv % 8 == 0) {
        const int x = b % 8, t = b / 8;
        const int per = nitems * group;
        const int kvh = x + 8 * (t / per);
        const int rem = t - (t / per) * per;
        item = rem / group;
        head = kvh * group + rem % group;
    } else {
        item = b / nheads;
        head = b % nheads;
    }
}

// Read of a table that stays constant for the whole launch (work items, tile
// lists) through the constant address space: with a wave-uniform index the
// compiler can use a scalar load, whose short latency and separate counter
// keep it off the path of the vector loads in flight.
template <typename T>
__device__ __forceinline__ T load_const(const T *p, int64_t i) {
    static_assert(sizeof(T) % 4 == 0, "tables hold 32-bit fields");
    typedef const int32_t __attribute__((address_space(4))) *ConstPtr;
    const ConstPtr src = (ConstPtr)(p + i);
    T out;
    int32_t *dst = reinterpret_cast<int32_t *>(&out);
#pragma unroll
    for (unsigned k = 0; k < sizeof(T) / 4; ++k) dst[k] = src[k];
    return out;
}

// The tile records of one work item (first .. first+count-1), fetched 64 at
// a time with one vector load per lane (lane l holds record wbase + l) and
// broadcast with readlane: the tile loops issue no scalar loads, whose
// latency the shared LDS/scalar counter would otherwise expose.  get() is
// called with wave-uniform indices; it refetches (rarely) when an index
// leaves the window.
struct TileWindow {
    const TileRec *tiles;
    int first, count, wbase, lane;
    i32x4 rec;
    __device__ __forceinline__ TileWindow(const TileRec *t, int first_, int count_, int lane_)
        : tiles(t), first(first_), count(count_), wbase(0), lane(lane_) {
        fetch();
    }
    __device__ __forceinline__ void fetch() {
        rec = *reinterpret_cast<const i32x4 *>(tiles + first + min(wbase + lane, count - 1));
    }
    __device__ __forceinline__ TileRec get(int j) {
        if (j < wbase || j >= wbase + 64) {
            wbase = j & ~63;
            fetch();
        }
        const int l = j - wbase;
        return TileRec{__builtin_amdgcn_readlane(rec.x, l), __builtin_amdgcn_readlane(rec.y, l),
                       __builtin_amdgcn_readlane(rec.z, l), __builtin_amdgcn_readlane(rec.w, l)};
    }
};

// float -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float to_float(float x) { return x; }
    static __device__ __forceinline__ float from_float(float x) { return x; }
};
template <> struct Elem<bf16> {
    static __device__ __forceinline__ float to_float(bf16 x) { return static_cast<float>(x); }
    static __device__ __forceinline__ bf16 from_float(float x) { return to_bf16(x); }
};

}  // namespace zz
