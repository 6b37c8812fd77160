// C ABI of libzz (declared in include/zz.h): argument checks, then launches.
// Nothing here throws across the ABI; every failure becomes a zz_status with a
// per-thread message.

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "zz_internal.h"

namespace {

thread_local std::string g_err;

zz_status fail(zz_status s, const std::string &msg) {
    g_err = msg;
    return s;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------- static plan workspace
// The workspace of zz_plan_upload_static, for callers that cannot allocate
// device memory.  Every GPU the library runs on holds its own copy of this
// array until the process ends.  In host code the array's name is not a
// device address: each device's address is looked up once, with that device
// current, by hipGetSymbolAddress, kept in g_static, and used everywhere
// host code needs the array (the upload copy, the kernels' table pointers).
static __device__ __align__(256) uint8_t scratch[ZZ_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
struct StaticSlot {
    uint8_t *ptr = nullptr;    // device address of `scratch` on this device
    uint64_t generation = 0;   // uploads into it so far
};
std::mutex g_static_mu;
StaticSlot g_static[kMaxDevices];

zz_status check_plan(const zz_plan *p, bool need_upload = true) {
    if (!p) return fail(ZZ_ERR_ARG, "null plan");
    if (need_upload && !p->d_ws) return fail(ZZ_ERR_STATE, "plan not uploaded (call zz_plan_upload)");
    if (need_upload && p->static_dev >= 0) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != p->static_dev)
            return fail(ZZ_ERR_STATE, "plan is bound to the static workspace of another device");
        std::lock_guard<std::mutex> lk(g_static_mu);
        if (g_static[p->static_dev].generation != p->static_gen)
            return fail(ZZ_ERR_STATE, "the static workspace now holds another plan's tables; upload this plan again");
    }
    return ZZ_OK;
}

zz_status check_rank_step(const zz_plan *p, int32_t rank, int32_t step, bool allow_all_rank) {
    if (step < 0 || step >= p->cp) return fail(ZZ_ERR_ARG, "step out of range");
    if (rank == ZZ_ALL_RANKS && allow_all_rank) return ZZ_OK;
    if (rank < 0 || rank >= p->cp) return fail(ZZ_ERR_ARG, "rank out of range");
    return ZZ_OK;
}

zz_status check_ptrs(std::initializer_list<const void *> ps) {
    for (const void *x : ps) {
        if (!x) return fail(ZZ_ERR_ARG, "null device pointer");
        if (!aligned16(x)) return fail(ZZ_ERR_ALIGN, "device pointer not 16-byte aligned");
    }
    return ZZ_OK;
}

// One buffer of a call: its extent in bytes and whether the call writes it.
struct Span {
    const char *name;
    const void *p;
    uint64_t bytes;
    bool written;
};

// A buffer the call writes must not overlap any other buffer of the call
// (the kernels read and write whole rows in parallel, so an overlap is a
// race); buffers that are only read may share memory.
zz_status check_disjoint(std::initializer_list<Span> spans) {
    for (const Span &a : spans) {
        if (!a.written || a.bytes == 0) continue;
        const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
        for (const Span &b : spans) {
            if (&a == &b || b.bytes == 0) continue;
            const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
            if (a0 < b1 && b0 < a1)
                return fail(ZZ_ERR_ARG, std::string("buffers overlap: ") + a.name + " and " + b.name);
        }
    }
    return ZZ_OK;
}

// Whole-buffer extents of the plan's tensors.
uint64_t rows_bytes(const zz_plan *p, int32_t heads, bool fp32) {
    return (uint64_t)p->T * heads * p->d * (fp32 || p->dtype == ZZ_F32 ? 4u : 2u);
}
uint64_t stat_bytes(const zz_plan *p) { return (uint64_t)p->T * p->hq * 4u; }

zz_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ZZ_OK;
    return fail(ZZ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define ZZ_TRY(x)                      \
    do {                               \
        zz_status _s = (x);            \
        if (_s != ZZ_OK) return _s;    \
    } while (0)

}  // namespace

extern "C" {


const char *zz_status_str(zz_status s) {
    switch (s) {
        case ZZ_OK: return "ok";
        case ZZ_ERR_ARG: return "invalid argument";
        case ZZ_ERR_SHAPE: return "inconsistent shape";
        case ZZ_ERR_DTYPE: return "unsupported dtype";
        case ZZ_ERR_ALIGN: return "misaligned pointer or row size";
        case ZZ_ERR_WORKSPACE: return "workspace or output buffer too small";
        case ZZ_ERR_HIP: return "HIP error";
        case ZZ_ERR_STATE: return "plan not uploaded";
    }
    return "unknown status";
}

const char *zz_last_error(void) { return g_err.c_str(); }

zz_status zz_plan_create(const int32_t *cu_seqlens, int32_t nseq, int32_t cp, int32_t hq,
                         int32_t hkv, int32_t head_dim, zz_dtype dtype, int32_t bm, int32_t bn,
                         zz_plan **out) {
    g_err.clear();
    std::string err;
    zz_status s = zz::build_plan(cu_seqlens, nseq, cp, hq, hkv, head_dim, dtype, bm, bn, out, &err);
    if (s != ZZ_OK) return fail(s, err);
    return ZZ_OK;
}

void zz_plan_destroy(zz_plan *plan) { delete plan; }

size_t zz_plan_workspace_bytes(const zz_plan *plan) { return plan ? plan->ws_bytes : 0; }

zz_status zz_plan_upload(zz_plan *plan, void *d_ws, size_t ws_bytes, void *stream) {
    ZZ_TRY(check_plan(plan, false));
    ZZ_TRY(check_ptrs({d_ws}));
    if (ws_bytes < plan->ws_bytes) return fail(ZZ_ERR_WORKSPACE, "workspace smaller than zz_plan_workspace_bytes");
    hipStream_t st = (hipStream_t)stream;
    ZZ_TRY(hip_status(hipMemcpyAsync(d_ws, plan->image.data(), plan->ws_bytes, hipMemcpyHostToDevice, st),
                      "plan upload"));
    // The host image must outlive the copy: wait for it here, once per plan.
    ZZ_TRY(hip_status(hipStreamSynchronize(st), "plan upload sync"));
    plan->d_ws = (const uint8_t *)d_ws;
    plan->static_dev = -1;
    return ZZ_OK;
}

zz_status zz_plan_upload_static(zz_plan *plan, void *stream) {
    ZZ_TRY(check_plan(plan, false));
    if (plan->ws_bytes > (size_t)ZZ_STATIC_WORKSPACE_BYTES)
        return fail(ZZ_ERR_WORKSPACE, "plan workspace of " + std::to_string(plan->ws_bytes) +
                                          " bytes exceeds the static workspace (" +
                                          std::to_string((size_t)ZZ_STATIC_WORKSPACE_BYTES) +
                                          " bytes); use zz_plan_upload");
    int dev = -1;
    ZZ_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
    if (dev < 0 || dev >= kMaxDevices) return fail(ZZ_ERR_ARG, "device index beyond the static workspace table");
    std::lock_guard<std::mutex> lk(g_static_mu);
    StaticSlot &slot = g_static[dev];
    if (!slot.ptr) {
        void *addr = nullptr;
        ZZ_TRY(hip_status(hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)), "static workspace address"));
        slot.ptr = static_cast<uint8_t *>(addr);
    }
    // Any plan bound here before is stale from now on, even if the copy fails.
    ++slot.generation;
    plan->d_ws = nullptr;
    hipStream_t st = (hipStream_t)stream;
    ZZ_TRY(hip_status(hipMemcpyAsync(slot.ptr, plan->image.data(), plan->ws_bytes, hipMemcpyHostToDevice, st),
                      "static plan upload"));
    ZZ_TRY(hip_status(hipStreamSynchronize(st), "static plan upload sync"));
    plan->d_ws = slot.ptr;
    plan->static_dev = dev;
    plan->static_gen = slot.generation;
    return ZZ_OK;
}

zz_status zz_plan_shape(const zz_plan *p, int64_t *total_tokens, int32_t *nseq, int32_t *cp,
                        int32_t *hq, int32_t *hkv, int32_t *head_dim, int32_t *dtype) {
    ZZ_TRY(check_plan(p, false));
    if (total_tokens) *total_tokens = p->T;
    if (nseq) *nseq = p->nseq;
    if (cp) *cp = p->cp;
    if (hq) *hq = p->hq;
    if (hkv) *hkv = p->hkv;
    if (head_dim) *head_dim = p->d;
    if (dtype) *dtype = (int32_t)p->dtype;
    return ZZ_OK;
}

zz_status zz_plan_local_cu_seqlens(const zz_plan *p, int32_t *out) {
    ZZ_TRY(check_plan(p, false));
    if (!out) return fail(ZZ_ERR_ARG, "null output");
    for (int32_t i = 0; i <= p->nseq; ++i) out[i] = p->cu[i] / p->cp;
    return ZZ_OK;
}

zz_status zz_plan_zigzag_dst(const zz_plan *p, int64_t *out) {
    ZZ_TRY(check_plan(p, false));
    if (!out) return fail(ZZ_ERR_ARG, "null output");
    for (int64_t z = 0; z < p->T; ++z) out[p->src[(size_t)z]] = z;
    return ZZ_OK;
}

zz_status zz_plan_tile_shape(const zz_plan *p, zz_pass pass, int32_t *bm, int32_t *bn) {
    ZZ_TRY(check_plan(p, false));
    if (pass < ZZ_PASS_FWD || pass > ZZ_PASS_BWD_DKV) return fail(ZZ_ERR_ARG, "bad pass");
    if (bm) *bm = p->pass[pass].bm;
    if (bn) *bn = p->pass[pass].bn;
    return ZZ_OK;
}

// Tiles of items [b, e) of a pass as (q0, q1, k0, k1, kind), the stationary
// rows shifted by `stat_base` and the streamed rows by `stream_base`, sorted
// by (q0, k0) and copied out under the capacity rule of zz_plan_tiles.
static zz_status emit_tiles(const zz::PassTables &t, int64_t b, int64_t e, int64_t stat_base, int64_t stream_base,
                     int32_t *out, int64_t cap, int64_t *n) {
    struct Q { int32_t q0, q1, k0, k1, kind; };
    std::vector<Q> v;
    for (int64_t u = b; u < e; ++u) {
        const zz::WorkItem &it = t.items[(size_t)u];
        const int32_t s0 = (int32_t)(stat_base + it.a0), s1 = (int32_t)(stat_base + it.a1);
        for (int32_t x = it.tbeg; x < it.tend; ++x) {
            const zz::TileRec &tr = t.tiles[(size_t)x];
            const int32_t m0 = (int32_t)(stream_base + tr.b0), m1 = (int32_t)(stream_base + tr.b1);
            if (t.key_major) v.push_back(Q{m0, m1, s0, s1, tr.kind});
            else v.push_back(Q{s0, s1, m0, m1, tr.kind});
        }
    }
    std::sort(v.begin(), v.end(), [](const Q &a, const Q &c) {
        return a.q0 != c.q0 ? a.q0 < c.q0 : a.k0 < c.k0;
    });
    *n = (int64_t)v.size();
    for (int64_t u = 0; u < std::min<int64_t>(cap, (int64_t)v.size()); ++u) {
        const Q &x = v[(size_t)u];
        int32_t *o = out + 5 * u;
        o[0] = x.q0; o[1] = x.q1; o[2] = x.k0; o[3] = x.k1; o[4] = x.kind;
    }
    if ((int64_t)v.size() > cap) return fail(ZZ_ERR_WORKSPACE, "tile output capacity too small");
    return ZZ_OK;
}

zz_status zz_plan_tiles(const zz_plan *p, zz_pass pass, int32_t rank, int32_t step, int32_t *out,
                        int64_t cap, int64_t *n) {
    ZZ_TRY(check_plan(p, false));
    if (pass < ZZ_PASS_FWD || pass > ZZ_PASS_BWD_DKV) return fail(ZZ_ERR_ARG, "bad pass");
    ZZ_TRY(check_rank_step(p, rank, step, false));
    if (!n || (cap > 0 && !out)) return fail(ZZ_ERR_ARG, "null output");
    const zz::PassTables &t = p->pass[pass];
    const int64_t b = t.rank_off[(size_t)step * p->cp + rank], e = t.rank_off[(size_t)step * p->cp + rank + 1];
    return emit_tiles(t, b, e, 0, 0, out, cap, n);
}

zz_status zz_plan_gathered_tiles(const zz_plan *p, zz_pass pass, int32_t owner, int32_t *out, int64_t cap,
                                 int64_t *n) {
    ZZ_TRY(check_plan(p, false));
    if (pass < ZZ_PASS_FWD || pass > ZZ_PASS_BWD_DKV) return fail(ZZ_ERR_ARG, "bad pass");
    if (owner < 0 || owner >= p->cp) return fail(ZZ_ERR_ARG, "owner out of range");
    if (!n || (cap > 0 && !out)) return fail(ZZ_ERR_ARG, "null output");
    const zz::PassTables &t = p->pass[zz::kPassGathered + pass];
    // stationary rows are local to the owner; streamed rows are already global
    return emit_tiles(t, t.rank_off[(size_t)owner], t.rank_off[(size_t)owner + 1], (int64_t)owner * (p->T / p->cp),
                      0, out, cap, n);
}

zz_status zz_plan_pair_counts(const zz_plan *p, zz_pass pass, int32_t rank, int32_t step,
                              int64_t *useful, int64_t *issued) {
    ZZ_TRY(check_plan(p, false));
    if (pass < ZZ_PASS_FWD || pass > ZZ_PASS_BWD_DKV) return fail(ZZ_ERR_ARG, "bad pass");
    if (rank != ZZ_ALL_RANKS && (rank < 0 || rank >= p->cp)) return fail(ZZ_ERR_ARG, "rank out of range");
    if (step != ZZ_ALL_STEPS && (step < 0 || step >= p->cp)) return fail(ZZ_ERR_ARG, "step out of range");
    const zz::PassTables &t = p->pass[pass];
    int64_t u = 0, is = 0;
    for (int32_t s = 0; s < p->cp; ++s)
        for (int32_t r = 0; r < p->cp; ++r) {
            if ((step != ZZ_ALL_STEPS && s != step) || (rank != ZZ_ALL_RANKS && r != rank)) continue;
            u += t.useful[(size_t)s * p->cp + r];
            is += t.issued[(size_t)s * p->cp + r];
        }
    if (useful) *useful = u;
    if (issued) *issued = is;
    return ZZ_OK;
}

zz_status zz_plan_rank_useful_pairs(const zz_plan *p, int64_t *out) {
    ZZ_TRY(check_plan(p, false));
    if (!out) return fail(ZZ_ERR_ARG, "null output");
    const zz::PassTables &t = p->pass[ZZ_PASS_FWD];
    for (int32_t r = 0; r < p->cp; ++r) {
        int64_t u = 0;
        for (int32_t s = 0; s < p->cp; ++s) u += t.useful[(size_t)s * p->cp + r];
        out[r] = u;
    }
    return ZZ_OK;
}

zz_status zz_zigzag_permute(const zz_plan *p, const void *x_packed, void *x_zz, int64_t row_bytes,
                            void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_ptrs({x_packed, x_zz}));
    if (row_bytes <= 0 || row_bytes % 16) return fail(ZZ_ERR_ALIGN, "row_bytes must be a positive multiple of 16");
    ZZ_TRY(check_disjoint({{"x_packed", x_packed, (uint64_t)p->T * row_bytes, false},
                           {"x_zz", x_zz, (uint64_t)p->T * row_bytes, true}}));
    return hip_status(zz::launch_permute(p, x_packed, x_zz, row_bytes, false, (hipStream_t)stream), "permute");
}

zz_status zz_zigzag_unpermute(const zz_plan *p, const void *x_zz, void *x_packed, int64_t row_bytes,
                              void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_ptrs({x_packed, x_zz}));
    if (row_bytes <= 0 || row_bytes % 16) return fail(ZZ_ERR_ALIGN, "row_bytes must be a positive multiple of 16");
    ZZ_TRY(check_disjoint({{"x_zz", x_zz, (uint64_t)p->T * row_bytes, false},
                           {"x_packed", x_packed, (uint64_t)p->T * row_bytes, true}}));
    return hip_status(zz::launch_permute(p, x_zz, x_packed, row_bytes, true, (hipStream_t)stream), "unpermute");
}

zz_status zz_varlen_ring_step_fwd(const zz_plan *p, int32_t rank, int32_t step, const void *q_zz,
                                  const void *k_zz, const void *v_zz, float *o_acc, float *lse_acc,
                                  int32_t merge, void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_rank_step(p, rank, step, true));
    ZZ_TRY(check_ptrs({q_zz, k_zz, v_zz, o_acc, lse_acc}));
    ZZ_TRY(check_disjoint({{"q_zz", q_zz, rows_bytes(p, p->hq, false), false},
                           {"k_zz", k_zz, rows_bytes(p, p->hkv, false), false},
                           {"v_zz", v_zz, rows_bytes(p, p->hkv, false), false},
                           {"o_acc", o_acc, rows_bytes(p, p->hq, true), true},
                           {"lse_acc", lse_acc, stat_bytes(p), true}}));
    if (merge != 0 && merge != 1) return fail(ZZ_ERR_ARG, "merge must be 0 or 1");
    return hip_status(zz::launch_fwd_step(p, rank, step, q_zz, k_zz, v_zz, o_acc, lse_acc, merge,
                                          (hipStream_t)stream), "varlen_ring_step_fwd");
}

zz_status zz_varlen_gathered_fwd(const zz_plan *p, int32_t rank, const void *q_zz, const void *k_zz,
                                 const void *v_zz, float *o, float *lse, void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_rank_step(p, rank, 0, true));
    ZZ_TRY(check_ptrs({q_zz, k_zz, v_zz, o, lse}));
    ZZ_TRY(check_disjoint({{"q_zz", q_zz, rows_bytes(p, p->hq, false), false},
                           {"k_zz", k_zz, rows_bytes(p, p->hkv, false), false},
                           {"v_zz", v_zz, rows_bytes(p, p->hkv, false), false},
                           {"o", o, rows_bytes(p, p->hq, true), true},
                           {"lse", lse, stat_bytes(p), true}}));
    return hip_status(zz::launch_fwd_gathered(p, rank, q_zz, k_zz, v_zz, o, lse, (hipStream_t)stream),
                      "varlen_gathered_fwd");
}

zz_status zz_varlen_gathered_bwd(const zz_plan *p, int32_t rank, const void *q_zz, const void *k_zz,
                                 const void *v_zz, const void *do_zz, const float *lse, const float *delta,
                                 float *dq, float *dk, float *dv, void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_rank_step(p, rank, 0, true));
    ZZ_TRY(check_ptrs({q_zz, k_zz, v_zz, do_zz, lse, delta, dq, dk, dv}));
    ZZ_TRY(check_disjoint({{"q_zz", q_zz, rows_bytes(p, p->hq, false), false},
                           {"k_zz", k_zz, rows_bytes(p, p->hkv, false), false},
                           {"v_zz", v_zz, rows_bytes(p, p->hkv, false), false},
                           {"do_zz", do_zz, rows_bytes(p, p->hq, false), false},
                           {"lse", lse, stat_bytes(p), false},
                           {"delta", delta, stat_bytes(p), false},
                           {"dq", dq, rows_bytes(p, p->hq, true), true},
                           {"dk", dk, rows_bytes(p, p->hkv, true), true},
                           {"dv", dv, rows_bytes(p, p->hkv, true), true}}));
    return hip_status(zz::launch_bwd_gathered(p, rank, q_zz, k_zz, v_zz, do_zz, lse, delta, dq, dk, dv,
                                              (hipStream_t)stream), "varlen_gathered_bwd");
}

zz_status zz_lse_merge(float *o_acc, float *lse_acc, const float *o_part, const float *lse_part,
                       int64_t rows, int32_t heads, int32_t head_dim, void *stream) {
    ZZ_TRY(check_ptrs({o_acc, lse_acc, o_part, lse_part}));
    if (rows < 0 || heads < 1 || head_dim < 1 || head_dim % 4) return fail(ZZ_ERR_ARG, "bad merge shape (head_dim % 4 == 0)");
    if (rows == 0) return ZZ_OK;
    const uint64_t ob = (uint64_t)rows * heads * head_dim * 4u, lb = (uint64_t)rows * heads * 4u;
    ZZ_TRY(check_disjoint({{"o_acc", o_acc, ob, true}, {"lse_acc", lse_acc, lb, true},
                           {"o_part", o_part, ob, false}, {"lse_part", lse_part, lb, false}}));
    return hip_status(zz::launch_lse_merge(o_acc, lse_acc, o_part, lse_part, rows, heads, head_dim,
                                           (hipStream_t)stream), "lse_merge");
}

zz_status zz_finalize_fwd(const zz_plan *p, const float *o_acc, void *o_out, int32_t unpermute,
                          void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_ptrs({o_acc, o_out}));
    ZZ_TRY(check_disjoint({{"o_acc", o_acc, rows_bytes(p, p->hq, true), false},
                           {"o_out", o_out, rows_bytes(p, p->hq, false), true}}));
    return hip_status(zz::launch_cast_rows(p, o_acc, o_out, p->hq, unpermute != 0, (hipStream_t)stream),
                      "finalize_fwd");
}

zz_status zz_bwd_preprocess(const zz_plan *p, const void *o_zz, const void *do_zz, float *delta,
                            void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_ptrs({o_zz, do_zz, delta}));
    ZZ_TRY(check_disjoint({{"o_zz", o_zz, rows_bytes(p, p->hq, false), false},
                           {"do_zz", do_zz, rows_bytes(p, p->hq, false), false},
                           {"delta", delta, stat_bytes(p), true}}));
    return hip_status(zz::launch_bwd_pre(p, o_zz, do_zz, delta, (hipStream_t)stream), "bwd_preprocess");
}

zz_status zz_varlen_ring_step_bwd(const zz_plan *p, int32_t rank, int32_t step, const void *q_zz,
                                  const void *k_zz, const void *v_zz, const void *do_zz,
                                  const float *lse, const float *delta, float *dq_acc,
                                  float *dk_acc, float *dv_acc, int32_t accumulate, void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_rank_step(p, rank, step, true));
    ZZ_TRY(check_ptrs({q_zz, k_zz, v_zz, do_zz, lse, delta, dq_acc, dk_acc, dv_acc}));
    ZZ_TRY(check_disjoint({{"q_zz", q_zz, rows_bytes(p, p->hq, false), false},
                           {"k_zz", k_zz, rows_bytes(p, p->hkv, false), false},
                           {"v_zz", v_zz, rows_bytes(p, p->hkv, false), false},
                           {"do_zz", do_zz, rows_bytes(p, p->hq, false), false},
                           {"lse", lse, stat_bytes(p), false},
                           {"delta", delta, stat_bytes(p), false},
                           {"dq_acc", dq_acc, rows_bytes(p, p->hq, true), true},
                           {"dk_acc", dk_acc, rows_bytes(p, p->hkv, true), true},
                           {"dv_acc", dv_acc, rows_bytes(p, p->hkv, true), true}}));
    if (accumulate != 0 && accumulate != 1) return fail(ZZ_ERR_ARG, "accumulate must be 0 or 1");
    return hip_status(zz::launch_bwd_step(p, rank, step, q_zz, k_zz, v_zz, do_zz, lse, delta, dq_acc,
                                          dk_acc, dv_acc, accumulate, 3, (hipStream_t)stream),
                      "varlen_ring_step_bwd");
}

zz_status zz_varlen_ring_step_bwd_dkv(const zz_plan *p, int32_t rank, int32_t step, const void *q_zz,
                                      const void *k_zz, const void *v_zz, const void *do_zz,
                                      const float *lse, const float *delta, float *dk_acc,
                                      float *dv_acc, int32_t accumulate, void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_rank_step(p, rank, step, true));
    ZZ_TRY(check_ptrs({q_zz, k_zz, v_zz, do_zz, lse, delta, dk_acc, dv_acc}));
    ZZ_TRY(check_disjoint({{"q_zz", q_zz, rows_bytes(p, p->hq, false), false},
                           {"k_zz", k_zz, rows_bytes(p, p->hkv, false), false},
                           {"v_zz", v_zz, rows_bytes(p, p->hkv, false), false},
                           {"do_zz", do_zz, rows_bytes(p, p->hq, false), false},
                           {"lse", lse, stat_bytes(p), false},
                           {"delta", delta, stat_bytes(p), false},
                           {"dk_acc", dk_acc, rows_bytes(p, p->hkv, true), true},
                           {"dv_acc", dv_acc, rows_bytes(p, p->hkv, true), true}}));
    if (accumulate != 0 && accumulate != 1) return fail(ZZ_ERR_ARG, "accumulate must be 0 or 1");
    return hip_status(zz::launch_bwd_step(p, rank, step, q_zz, k_zz, v_zz, do_zz, lse, delta, nullptr,
                                          dk_acc, dv_acc, accumulate, 1, (hipStream_t)stream),
                      "varlen_ring_step_bwd_dkv");
}

zz_status zz_varlen_ring_step_bwd_dq(const zz_plan *p, int32_t rank, int32_t step, const void *q_zz,
                                     const void *k_zz, const void *v_zz, const void *do_zz,
                                     const float *lse, const float *delta, float *dq_acc,
                                     int32_t accumulate, void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_rank_step(p, rank, step, true));
    ZZ_TRY(check_ptrs({q_zz, k_zz, v_zz, do_zz, lse, delta, dq_acc}));
    ZZ_TRY(check_disjoint({{"q_zz", q_zz, rows_bytes(p, p->hq, false), false},
                           {"k_zz", k_zz, rows_bytes(p, p->hkv, false), false},
                           {"v_zz", v_zz, rows_bytes(p, p->hkv, false), false},
                           {"do_zz", do_zz, rows_bytes(p, p->hq, false), false},
                           {"lse", lse, stat_bytes(p), false},
                           {"delta", delta, stat_bytes(p), false},
                           {"dq_acc", dq_acc, rows_bytes(p, p->hq, true), true}}));
    if (accumulate != 0 && accumulate != 1) return fail(ZZ_ERR_ARG, "accumulate must be 0 or 1");
    return hip_status(zz::launch_bwd_step(p, rank, step, q_zz, k_zz, v_zz, do_zz, lse, delta, dq_acc,
                                          nullptr, nullptr, accumulate, 2, (hipStream_t)stream),
                      "varlen_ring_step_bwd_dq");
}

zz_status zz_finalize_bwd(const zz_plan *p, const float *dq_acc, const float *dk_acc,
                          const float *dv_acc, void *dq_out, void *dk_out, void *dv_out,
                          int32_t unpermute, void *stream) {
    ZZ_TRY(check_plan(p));
    ZZ_TRY(check_ptrs({dq_acc, dk_acc, dv_acc, dq_out, dk_out, dv_out}));
    ZZ_TRY(check_disjoint({{"dq_acc", dq_acc, rows_bytes(p, p->hq, true), false},
                           {"dk_acc", dk_acc, rows_bytes(p, p->hkv, true), false},
                           {"dv_acc", dv_acc, rows_bytes(p, p->hkv, true), false},
                           {"dq_out", dq_out, rows_bytes(p, p->hq, false), true},
                           {"dk_out", dk_out, rows_bytes(p, p->hkv, false), true},
                           {"dv_out", dv_out, rows_bytes(p, p->hkv, false), true}}));
    hipStream_t st = (hipStream_t)stream;
    ZZ_TRY(hip_status(zz::launch_cast_rows(p, dq_acc, dq_out, p->hq, unpermute != 0, st), "finalize_bwd dq"));
    ZZ_TRY(hip_status(zz::launch_cast_rows(p, dk_acc, dk_out, p->hkv, unpermute != 0, st), "finalize_bwd dk"));
    return hip_status(zz::launch_cast_rows(p, dv_acc, dv_out, p->hkv, unpermute != 0, st), "finalize_bwd dv");
}

zz_status zz_debug_mask(const zz_plan *p, zz_pass pass, int32_t rank, int32_t step, uint8_t *d_mask,
                        void *stream) {
    ZZ_TRY(check_plan(p));
    if (pass < ZZ_PASS_FWD || pass > ZZ_PASS_BWD_DKV) return fail(ZZ_ERR_ARG, "bad pass");
    ZZ_TRY(check_rank_step(p, rank, step, false));
    ZZ_TRY(check_ptrs({d_mask}));
    return hip_status(zz::launch_debug_mask(p, pass, rank, step, d_mask, (hipStream_t)stream), "debug_mask");
}

}  // extern "C"
