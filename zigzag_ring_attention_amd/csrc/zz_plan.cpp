// Host planner of libzz: validates a packed batch and builds the device tables
// of the three tile walks (forward, backward dQ, backward dK/dV).
//
// Zigzag split (ring-attention-pytorch issue #20, "Zigzag attention
// support?", extract_local snippet): every sequence is cut into 2*CP chunks
// of c = L/(2CP) tokens and rank r holds chunk r followed by chunk 2CP-1-r.
// For packed input the split is applied per sequence; a rank's rows list the
// sequences in order, and ranks are stacked rank-major, so rank r's rows start
// at r*T/CP and sequence i starts at cu[i]/CP inside every rank.
//
// Ring step s pairs rank r with key shard j = (r - s) mod CP.  Inside one
// sequence, query chunk a sees key chunk b fully when a > b, not at all when
// a < b, and lower-triangularly when a == b (causal, MaxText PR #1133: the
// load-balanced CP attention is causal).  Different sequences never see each
// other (EasyDeL issue #129, packed examples).  Tiles are laid on a grid that
// restarts at every chunk boundary, so a tile never straddles two chunks and
// its kind follows from the chunk pair: fully visible, partially visible
// (diagonal chunk pair, only (key offset) <= (query offset)), or invisible.
// Invisible tiles are never listed (FlagScale PR #910: pruning of redundant
// computation).

#include <algorithm>
#include <cstring>
#include <new>

#include "zz_internal.h"

namespace zz {
namespace {

struct Chunk {
    int32_t index;  // chunk number inside its sequence, 0..2cp-1
    int32_t start;  // local row of its first token (rank-local or shard-local)
    int32_t len;
};

// The two chunks of every sequence that rank (or shard) `who` holds, in
// local order.
std::vector<std::vector<Chunk>> local_chunks(const std::vector<int32_t> &cu, int32_t cp, int32_t who) {
    std::vector<std::vector<Chunk>> out;
    int32_t nseq = (int32_t)cu.size() - 1;
    for (int32_t i = 0; i < nseq; ++i) {
        int32_t c = (cu[i + 1] - cu[i]) / (2 * cp);
        int32_t base = cu[i] / cp;
        out.push_back({Chunk{who, base, c}, Chunk{2 * cp - 1 - who, base + c, c}});
    }
    return out;
}

// Kind and delta of the tile (query offsets [qa0,qa1) of chunk qa) x
// (key offsets [kb0,kb1) of chunk kb); 0 = invisible.
int classify(int32_t qa, int32_t qa0, int32_t qa1, int32_t kb, int32_t kb0, int32_t kb1,
             int32_t *delta) {
    *delta = qa0 - kb0;
    if (qa > kb) return ZZ_TILE_FULL;
    if (qa < kb) return 0;
    if (kb1 - 1 <= qa0) return ZZ_TILE_FULL;
    if (kb0 > qa1 - 1) return 0;
    return ZZ_TILE_PARTIAL;
}

// Visible pairs of a tile.
int64_t tile_pairs(int kind, int32_t q0, int32_t q1, int32_t k0, int32_t k1, int32_t delta) {
    int64_t nk = k1 - k0;
    if (kind == ZZ_TILE_FULL) return (int64_t)(q1 - q0) * nk;
    int64_t s = 0;
    for (int32_t qq = 0; qq < q1 - q0; ++qq) s += std::max<int64_t>(0, std::min<int64_t>(nk, qq + delta + 1));
    return s;
}

// Launch order of a pass's items, longest first.  When a query-major walk
// (forward, dQ) of many workgroups mixes long and short items -- median work
// under a quarter of the largest, as with packed short documents -- the
// order alternates longest and shortest, so the latency-bound short items
// run next to long ones instead of all together at the end of the launch
// (15 documents of 64-16384 tokens: dQ 4-8% and forward 1-1.6% faster).
// Items of one long sequence are close in size and keep longest-first
// (alternating cost them 0.2-0.4%), as do launches of only a few rounds of
// workgroups (alternating cost 8192 tokens of 5 documents 5%), and the
// key-major dK/dV walk always does (alternating made it 13-19% slower).
void launch_order(const zz_plan *p, const PassTables &t, const std::vector<int64_t> &item_work,
                  std::vector<int32_t> &ord) {
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) { return item_work[x] > item_work[y]; });
    if (t.key_major) return;
    // a launch of a few rounds of workgroups (8192 = 16 rounds of two per CU
    // on 256 CUs) finishes soonest with the longest items started first
    if ((int64_t)ord.size() * p->hq < 8192) return;
    // items with no visible tile (kept by the forward only to clear their
    // rows) cost nothing and do not count
    size_t busy = 0;
    while (busy < ord.size() && item_work[(size_t)ord[busy]] > 0) ++busy;
    if (busy < 2) return;
    const int64_t largest = item_work[(size_t)ord.front()], median = item_work[(size_t)ord[busy / 2]];
    if (4 * median >= largest) return;
    std::vector<int32_t> z;
    z.reserve(ord.size());
    size_t lo = 0, hi = ord.size();
    while (lo < hi) {
        z.push_back(ord[lo++]);
        if (lo < hi) z.push_back(ord[--hi]);
    }
    ord.swap(z);
}

void build_pass(zz_plan *p, PassTables &t) {
    const int32_t cp = p->cp;
    t.items.clear();
    t.tiles.clear();
    t.ordered.clear();
    t.rank_off.assign((size_t)cp * cp + 1, 0);
    t.order_off.assign((size_t)cp + 1, 0);
    t.useful.assign((size_t)cp * cp, 0);
    t.issued.assign((size_t)cp * cp, 0);
    std::vector<int64_t> item_work;  // issued pairs per item, for LPT

    for (int32_t s = 0; s < cp; ++s) {
        for (int32_t r = 0; r < cp; ++r) {
            const int32_t j = ((r - s) % cp + cp) % cp;
            t.rank_off[(size_t)s * cp + r] = (int64_t)t.items.size();
            auto qch = local_chunks(p->cu, cp, r);
            auto kch = local_chunks(p->cu, cp, j);
            const size_t first_item = t.items.size();
            for (int32_t i = 0; i < p->nseq; ++i) {
                // Stationary side: queries (query-major) or keys (key-major).
                const auto &st = t.key_major ? kch[i] : qch[i];
                const auto &sm = t.key_major ? qch[i] : kch[i];
                const int32_t sstep = t.key_major ? t.bn : t.bm;
                const int32_t mstep = t.key_major ? t.bm : t.bn;
                for (const Chunk &a : st) {
                    for (int32_t a0 = 0; a0 < a.len; a0 += sstep) {
                        const int32_t a1 = std::min(a0 + sstep, a.len);
                        WorkItem it{r, j, a.start + a0, a.start + a1, (int32_t)t.tiles.size(), 0, 0, 0};
                        int64_t work = 0;
                        for (const Chunk &b : sm) {
                            for (int32_t b0 = 0; b0 < b.len; b0 += mstep) {
                                const int32_t b1 = std::min(b0 + mstep, b.len);
                                int32_t delta, kind;
                                int32_t q0, q1, k0, k1;
                                if (t.key_major) {
                                    kind = classify(b.index, b0, b1, a.index, a0, a1, &delta);
                                    q0 = b0; q1 = b1; k0 = a0; k1 = a1;
                                } else {
                                    kind = classify(a.index, a0, a1, b.index, b0, b1, &delta);
                                    q0 = a0; q1 = a1; k0 = b0; k1 = b1;
                                }
                                if (!kind) continue;
                                t.tiles.push_back(TileRec{b.start + b0, b.start + b1, kind, delta});
                                const int64_t area = (int64_t)(q1 - q0) * (k1 - k0);
                                work += area;
                                t.issued[(size_t)s * cp + r] += area;
                                t.useful[(size_t)s * cp + r] += tile_pairs(kind, q0, q1, k0, k1, delta);
                            }
                        }
                        it.tend = (int32_t)t.tiles.size();
                        if (it.tend > it.tbeg || t.keep_empty) {
                            t.items.push_back(it);
                            item_work.push_back(work);
                        }
                    }
                }
            }
            // Longest first inside the rank (stable, so ties keep row order).
            std::vector<size_t> idx(t.items.size() - first_item);
            for (size_t u = 0; u < idx.size(); ++u) idx[u] = first_item + u;
            std::stable_sort(idx.begin(), idx.end(),
                             [&](size_t x, size_t y) { return item_work[x] > item_work[y]; });
            std::vector<WorkItem> tmp;
            std::vector<int64_t> tw;
            for (size_t u : idx) { tmp.push_back(t.items[u]); tw.push_back(item_work[u]); }
            std::copy(tmp.begin(), tmp.end(), t.items.begin() + first_item);
            std::copy(tw.begin(), tw.end(), item_work.begin() + first_item);
        }
        // Whole-step launch order over every rank.
        t.order_off[s] = (int64_t)t.ordered.size();
        const int64_t b = t.rank_off[(size_t)s * cp], e = (int64_t)t.items.size();
        std::vector<int32_t> ord;
        for (int64_t u = b; u < e; ++u) ord.push_back((int32_t)u);
        launch_order(p, t, item_work, ord);
        for (int32_t u : ord) t.ordered.push_back(t.items[(size_t)u]);
    }
    t.rank_off[(size_t)cp * cp] = (int64_t)t.items.size();
    t.order_off[cp] = (int64_t)t.ordered.size();
}

// Gathered walks: every stationary item of rank r (its query rows for the
// query-major walks, its key/value shard for the key-major one) lists the
// visible tiles of every other rank's streamed rows, given in the global
// zigzag order (rank j's rows start at j*T/cp), so the items carry a zero
// base on the streamed side and one launch covers what the cp ring steps
// cover -- the all-gather alternative to the ring (ring-attention-pytorch
// issue #20, "Zigzag attention support?": the maintainer reads the scheme as
// gathering keys and values across ranks, which GQA makes affordable, and
// plans to offer that gather as an option).
void build_gathered_pass(zz_plan *p, PassTables &t) {
    const int32_t cp = p->cp;
    const int64_t n = p->T / cp;
    t.items.clear();
    t.tiles.clear();
    t.ordered.clear();
    t.rank_off.assign((size_t)cp + 1, 0);
    t.order_off.assign(2, 0);
    t.useful.assign((size_t)cp, 0);
    t.issued.assign((size_t)cp, 0);
    std::vector<int64_t> item_work;
    std::vector<std::vector<std::vector<Chunk>>> ch((size_t)cp);
    for (int32_t j = 0; j < cp; ++j) ch[(size_t)j] = local_chunks(p->cu, cp, j);
    const int32_t sstep = t.key_major ? t.bn : t.bm;
    const int32_t mstep = t.key_major ? t.bm : t.bn;
    for (int32_t r = 0; r < cp; ++r) {
        t.rank_off[(size_t)r] = (int64_t)t.items.size();
        const size_t first_item = t.items.size();
        for (int32_t i = 0; i < p->nseq; ++i) {
            for (const Chunk &a : ch[(size_t)r][(size_t)i]) {
                for (int32_t a0 = 0; a0 < a.len; a0 += sstep) {
                    const int32_t a1 = std::min(a0 + sstep, a.len);
                    // query-major: rank r's queries, keys at global rows (shard 0);
                    // key-major: shard r's keys, queries at global rows (rank 0)
                    WorkItem it{t.key_major ? 0 : r, t.key_major ? r : 0, a.start + a0, a.start + a1,
                                (int32_t)t.tiles.size(), 0, 0, 0};
                    int64_t work = 0;
                    for (int32_t j = 0; j < cp; ++j) {
                        for (const Chunk &b : ch[(size_t)j][(size_t)i]) {
                            for (int32_t b0 = 0; b0 < b.len; b0 += mstep) {
                                const int32_t b1 = std::min(b0 + mstep, b.len);
                                int32_t delta, kind, q0, q1, k0, k1;
                                if (t.key_major) {
                                    kind = classify(b.index, b0, b1, a.index, a0, a1, &delta);
                                    q0 = b0; q1 = b1; k0 = a0; k1 = a1;
                                } else {
                                    kind = classify(a.index, a0, a1, b.index, b0, b1, &delta);
                                    q0 = a0; q1 = a1; k0 = b0; k1 = b1;
                                }
                                if (!kind) continue;
                                const int32_t g0 = (int32_t)(j * n + b.start + b0), g1 = (int32_t)(j * n + b.start + b1);
                                t.tiles.push_back(TileRec{g0, g1, kind, delta});
                                const int64_t area = (int64_t)(q1 - q0) * (k1 - k0);
                                work += area;
                                t.issued[(size_t)r] += area;
                                t.useful[(size_t)r] += tile_pairs(kind, q0, q1, k0, k1, delta);
                            }
                        }
                    }
                    it.tend = (int32_t)t.tiles.size();
                    if (it.tend > it.tbeg || t.keep_empty) {
                        t.items.push_back(it);
                        item_work.push_back(work);
                    }
                }
            }
        }
        std::vector<size_t> idx(t.items.size() - first_item);
        for (size_t u = 0; u < idx.size(); ++u) idx[u] = first_item + u;
        std::stable_sort(idx.begin(), idx.end(), [&](size_t x, size_t y) { return item_work[x] > item_work[y]; });
        std::vector<WorkItem> tmp;
        std::vector<int64_t> tw;
        for (size_t u : idx) { tmp.push_back(t.items[u]); tw.push_back(item_work[u]); }
        std::copy(tmp.begin(), tmp.end(), t.items.begin() + first_item);
        std::copy(tw.begin(), tw.end(), item_work.begin() + first_item);
    }
    t.rank_off[(size_t)cp] = (int64_t)t.items.size();
    std::vector<int32_t> ord;
    for (size_t u = 0; u < t.items.size(); ++u) ord.push_back((int32_t)u);
    launch_order(p, t, item_work, ord);
    for (int32_t u : ord) t.ordered.push_back(t.items[(size_t)u]);
    t.order_off[1] = (int64_t)t.ordered.size();
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

zz_status build_plan(const int32_t *cu, int32_t nseq, int32_t cp, int32_t hq, int32_t hkv,
                     int32_t d, zz_dtype dt, int32_t bm, int32_t bn, zz_plan **out,
                     std::string *err) {
    if (!cu || !out) { *err = "null argument"; return ZZ_ERR_ARG; }
    if (nseq < 1) { *err = "nseq must be >= 1"; return ZZ_ERR_ARG; }
    if (cp < 1 || cp > 64) { *err = "cp must be in [1, 64]"; return ZZ_ERR_ARG; }
    if (hq < 1 || hkv < 1 || hq % hkv != 0) { *err = "hq must be a positive multiple of hkv"; return ZZ_ERR_SHAPE; }
    if (d != 32 && d != 64 && d != 128) { *err = "head_dim must be 32, 64 or 128"; return ZZ_ERR_SHAPE; }
    if (dt != ZZ_F32 && dt != ZZ_BF16) { *err = "dtype must be ZZ_F32 or ZZ_BF16"; return ZZ_ERR_DTYPE; }
    if (bm < 1 || bm > 128 || bn < 1 || bn > 64) { *err = "tile must satisfy 1<=bm<=128, 1<=bn<=64"; return ZZ_ERR_ARG; }
    if (cu[0] != 0) { *err = "cu_seqlens[0] must be 0"; return ZZ_ERR_SHAPE; }
    for (int32_t i = 0; i < nseq; ++i) {
        const int64_t L = (int64_t)cu[i + 1] - cu[i];
        if (L <= 0) { *err = "cu_seqlens must be strictly increasing"; return ZZ_ERR_SHAPE; }
        if (L % (2 * cp) != 0) {
            *err = "sequence " + std::to_string(i) + " has length " + std::to_string(L) +
                   ", not a multiple of 2*cp=" + std::to_string(2 * cp);
            return ZZ_ERR_SHAPE;
        }
    }
    zz_plan *p = new (std::nothrow) zz_plan();
    if (!p) { *err = "out of host memory"; return ZZ_ERR_ARG; }
    p->T = cu[nseq];
    p->nseq = nseq; p->cp = cp; p->hq = hq; p->hkv = hkv; p->d = d; p->dtype = dt;
    p->cu.assign(cu, cu + nseq + 1);

    // Zigzag row map: token at offset o of chunk x of sequence i sits on rank
    // rho = (x < cp ? x : 2cp-1-x), in that rank's half eta = (x >= cp).
    p->src.assign((size_t)p->T, 0);
    const int64_t n = p->T / cp;
    for (int32_t i = 0; i < nseq; ++i) {
        const int32_t c = (cu[i + 1] - cu[i]) / (2 * cp);
        for (int32_t x = 0; x < 2 * cp; ++x) {
            const int32_t rho = x < cp ? x : 2 * cp - 1 - x;
            const int32_t eta = x >= cp ? 1 : 0;
            for (int32_t o = 0; o < c; ++o) {
                const int64_t z = rho * n + cu[i] / cp + (int64_t)eta * c + o;
                p->src[(size_t)z] = cu[i] + x * c + o;
            }
        }
    }

    PassTables &fw = p->pass[ZZ_PASS_FWD];
    fw.bm = bm; fw.bn = bn; fw.key_major = false; fw.keep_empty = true;
    PassTables &dq = p->pass[ZZ_PASS_BWD_DQ];
    // dQ: 256 query rows per item; fp32 key tiles halved for D >= 64 (LDS).
    dq.bm = 256; dq.bn = (dt == ZZ_F32 && d >= 64) ? 32 : 64; dq.key_major = false; dq.keep_empty = false;
    PassTables &dkv = p->pass[ZZ_PASS_BWD_DKV];
    // fp32 query tiles of 64 or 128 columns are halved so the double-buffered
    // LDS stage of the dK/dV kernel fits.
    dkv.bm = (dt == ZZ_F32 && d >= 64) ? 32 : 64;
    dkv.bn = 128; dkv.key_major = true; dkv.keep_empty = false;
    for (int k = ZZ_PASS_FWD; k <= ZZ_PASS_BWD_DKV; ++k) {
        PassTables &g = p->pass[kPassGathered + k];
        const PassTables &r = p->pass[k];
        g.bm = r.bm; g.bn = r.bn; g.key_major = r.key_major; g.keep_empty = r.keep_empty;
        build_pass(p, p->pass[k]);
        build_gathered_pass(p, g);
    }

    // Workspace image: zigzag map, then items / tiles / order of each pass.
    size_t off = 0;
    p->off_src = off; off = align_up(off + sizeof(int32_t) * p->src.size());
    for (auto &t : p->pass) {
        t.off_items = off; off = align_up(off + sizeof(WorkItem) * t.items.size());
        t.off_tiles = off; off = align_up(off + sizeof(TileRec) * t.tiles.size());
        t.off_ordered = off; off = align_up(off + sizeof(WorkItem) * t.ordered.size());
    }
    p->ws_bytes = std::max<size_t>(off, 256);
    p->image.assign(p->ws_bytes, 0);
    std::memcpy(p->image.data() + p->off_src, p->src.data(), sizeof(int32_t) * p->src.size());
    for (auto &t : p->pass) {
        if (!t.items.empty()) std::memcpy(p->image.data() + t.off_items, t.items.data(), sizeof(WorkItem) * t.items.size());
        if (!t.tiles.empty()) std::memcpy(p->image.data() + t.off_tiles, t.tiles.data(), sizeof(TileRec) * t.tiles.size());
        if (!t.ordered.empty())
            std::memcpy(p->image.data() + t.off_ordered, t.ordered.data(), sizeof(WorkItem) * t.ordered.size());
    }
    *out = p;
    return ZZ_OK;
}

Launch launch_items(const zz_plan *p, int pass, int rank, int step) {
    const PassTables &t = p->pass[pass];
    const int cp = p->cp;
    if (rank < 0) {
        const int64_t b = t.order_off[step], e = t.order_off[step + 1];
        return Launch{dev_ordered(p, pass) + b, (int32_t)(e - b)};
    }
    const int64_t b = t.rank_off[(size_t)step * cp + rank], e = t.rank_off[(size_t)step * cp + rank + 1];
    return Launch{dev_items(p, pass) + b, (int32_t)(e - b)};
}

}  // namespace zz
