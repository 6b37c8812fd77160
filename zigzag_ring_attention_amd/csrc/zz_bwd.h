// Shared by the two backward kernels (zz_bwd.hip: dK/dV; zz_bwd_dq.hip: dQ):
// the argument block and the accumulator write-back.

#pragma once

#include "zz_mfma.h"

namespace zz {

// s_waitcnt immediate that waits for vmcnt = 0 only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the others at their maximum).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *lse, *delta;
    float *dq, *dk, *dv;
    const WorkItem *items;
    const TileRec *tiles;
    int64_t T;
    int32_t n, hq, hkv;
    float scale, scale_log2;
    int32_t accumulate;
    int32_t nitems;   // work items in this launch
};

// Read-add-write of a lane's column of a transposed accumulator (C layout:
// register i of block b is element 32*b + c_row(i, l/32) of the row).
template <int NB>
__device__ __forceinline__ void add_row(float *row, const f32x16 (&acc)[NB], float mul, int hh, bool accumulate) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            float4 *dst = reinterpret_cast<float4 *>(row + 32 * b + c_row(4 * i4, hh));
            float4 o = accumulate ? *dst : float4{0.f, 0.f, 0.f, 0.f};
            o.x += acc[b][4 * i4 + 0] * mul;
            o.y += acc[b][4 * i4 + 1] * mul;
            o.z += acc[b][4 * i4 + 2] * mul;
            o.w += acc[b][4 * i4 + 3] * mul;
            *dst = o;
        }
}

// dQ launch for one pass (zz_bwd_dq.hip; compiled on its own so its
// instruction schedule can be chosen apart from the dK/dV kernel's).
hipError_t launch_dq(const zz_plan *p, int pass, int rank, int step, BwdArgs a, hipStream_t st);

}  // namespace zz
