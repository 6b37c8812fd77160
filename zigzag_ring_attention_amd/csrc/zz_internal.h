// Internal declarations shared by the host planner, the C ABI and the HIP
// kernels of libzz.  Not part of the public interface (see include/zz.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/zz.h"

namespace zz {

// One unit of work of a pass in one ring step: a tile of the stationary side
// (query rows for the query-major passes, key rows for the key-major pass)
// and the range of its visible tiles of the streamed side.
struct WorkItem {
    int32_t rank;   // simulated CP rank (owner of the query rows)
    int32_t shard;  // key/value shard j = (rank - step) mod cp
    int32_t a0, a1; // stationary rows, local to the rank (queries) or shard (keys)
    int32_t tbeg, tend;  // range in the pass's tile array
    int32_t pad0, pad1;
};
static_assert(sizeof(WorkItem) == 32, "WorkItem layout");

// A visible tile of the streamed side.  For PARTIAL tiles the visible pairs
// are those with (key offset in tile) <= (query offset in tile) + delta.
struct TileRec {
    int32_t b0, b1;  // streamed rows (keys for query-major, queries for key-major)
    int32_t kind;    // ZZ_TILE_FULL or ZZ_TILE_PARTIAL
    int32_t delta;
};
static_assert(sizeof(TileRec) == 16, "TileRec layout");

struct PassTables {
    int32_t bm = 0, bn = 0;      // query rows x key rows per tile
    bool key_major = false;      // stationary side is keys (BWD_DKV)
    bool keep_empty = false;     // list stationary tiles with no visible tile (FWD)
    std::vector<WorkItem> items; // grouped by (step, rank); LPT order inside a rank
    std::vector<TileRec> tiles;
    std::vector<WorkItem> ordered;   // per step: every rank's items in launch order
    std::vector<int64_t> rank_off;   // [(step*cp + rank)] -> first item; size cp*cp+1
    std::vector<int64_t> order_off;  // [step] -> first entry of `ordered`; size cp+1
    std::vector<int64_t> useful;     // [(step*cp + rank)] visible pairs (per head)
    std::vector<int64_t> issued;     // [(step*cp + rank)] pairs covered by visited tiles
    size_t off_items = 0, off_tiles = 0, off_ordered = 0;  // byte offsets in the workspace
};

}  // namespace zz

struct zz_plan {
    int64_t T = 0;
    int32_t nseq = 0, cp = 0, hq = 0, hkv = 0, d = 0;
    zz_dtype dtype = ZZ_BF16;
    std::vector<int32_t> cu;     // packed cu_seqlens
    std::vector<int32_t> src;    // zigzag row -> packed token
    // pass[ZZ_PASS_FWD..ZZ_PASS_BWD_DKV] are the ring passes; pass[kPassGathered
    // + ZZ_PASS_*] are the same walks against every shard at once (one
    // "step": their rank_off has cp+1 entries, their order_off 2).
    zz::PassTables pass[6];
    size_t off_src = 0;
    size_t ws_bytes = 0;
    std::vector<uint8_t> image;  // host image of the device workspace
    const uint8_t *d_ws = nullptr;  // bound device workspace (after upload)
    // Set by zz_plan_upload_static: the device whose static workspace holds
    // this plan's tables, and that workspace's upload count at the time (a
    // later upload into it makes the plan stale).  -1: a caller's workspace.
    int32_t static_dev = -1;
    uint64_t static_gen = 0;
};

namespace zz {

// Host planner (zz_plan.cpp).
zz_status build_plan(const int32_t *cu, int32_t nseq, int32_t cp, int32_t hq, int32_t hkv,
                     int32_t d, zz_dtype dt, int32_t bm, int32_t bn, zz_plan **out,
                     std::string *err);

// Internal pass index of the gathered walks: kPassGathered + ZZ_PASS_FWD /
// _BWD_DQ / _BWD_DKV (not public zz_pass values).
constexpr int kPassGathered = 3;

// Device-side pointers into a bound plan's workspace.
inline const int32_t *dev_src(const zz_plan *p) {
    return reinterpret_cast<const int32_t *>(p->d_ws + p->off_src);
}
inline const WorkItem *dev_items(const zz_plan *p, int pass) {
    return reinterpret_cast<const WorkItem *>(p->d_ws + p->pass[pass].off_items);
}
inline const TileRec *dev_tiles(const zz_plan *p, int pass) {
    return reinterpret_cast<const TileRec *>(p->d_ws + p->pass[pass].off_tiles);
}
inline const WorkItem *dev_ordered(const zz_plan *p, int pass) {
    return reinterpret_cast<const WorkItem *>(p->d_ws + p->pass[pass].off_ordered);
}

// Item selection of one launch: a contiguous range of work items, one
// rank's (in its longest-first order) or, for all ranks, the step's items in
// launch order.
struct Launch {
    const WorkItem *items;
    int32_t n;
};
Launch launch_items(const zz_plan *p, int pass, int rank, int step);

// Kernel launchers (HIP translation units).  They assume validated arguments.
hipError_t launch_permute(const zz_plan *p, const void *in, void *out, int64_t row_bytes,
                          bool inverse, hipStream_t st);
hipError_t launch_cast_rows(const zz_plan *p, const float *in, void *out, int32_t heads,
                            bool unpermute, hipStream_t st);
hipError_t launch_lse_merge(float *o, float *lse, const float *o2, const float *lse2, int64_t rows,
                            int32_t heads, int32_t d, hipStream_t st);
hipError_t launch_bwd_pre(const zz_plan *p, const void *o, const void *dout, float *delta,
                          hipStream_t st);
hipError_t launch_debug_mask(const zz_plan *p, int pass, int rank, int step, uint8_t *mask,
                             hipStream_t st);
// Forward of rank (or all ranks) against every shard in one launch: writes
// the normalised O and the LSE, no merge.
hipError_t launch_fwd_gathered(const zz_plan *p, int rank, const void *q, const void *k, const void *v,
                               float *o, float *lse, hipStream_t st);
// Backward of rank r against every shard (dq of its rows, dk/dv of its shard)
// in one launch per kernel; writes (no accumulation across calls).
hipError_t launch_bwd_gathered(const zz_plan *p, int rank, const void *q, const void *k, const void *v,
                               const void *dout, const float *lse, const float *delta, float *dq, float *dk,
                               float *dv, hipStream_t st);
hipError_t launch_fwd_step(const zz_plan *p, int rank, int step, const void *q, const void *k,
                           const void *v, float *o, float *lse, int merge, hipStream_t st);
// which: 1 = dK/dV kernel, 2 = dQ kernel, 3 = both.
hipError_t launch_bwd_step(const zz_plan *p, int rank, int step, const void *q, const void *k,
                           const void *v, const void *dout, const float *lse, const float *delta,
                           float *dq, float *dk, float *dv, int accumulate, int which, hipStream_t st);

}  // namespace zz
