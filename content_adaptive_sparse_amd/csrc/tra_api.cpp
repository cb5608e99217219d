// C ABI of the entropy-radius block-sparse attention library: argument
// validation, tile-grid arithmetic, stream-ordered scratch memory and the
// launch sequences (probe -> walk plan -> attention, and the staged calls).
// Declarations and the contract of every entry point are in
// include/tra_attention.h.
#include "tra_attention.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "tra_internal.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool is_dense(int r_min, int r_max) { return r_min == TRA_RADIUS_INF && r_max == TRA_RADIUS_INF; }

int make_grid(int T, int H, int W, int block, tra::Grid *g) {
    if (T < 1 || H < 1 || W < 1) return TRA_ERR_INVALID_ARG;
    if (block != tra::kBlockTokens) return TRA_ERR_UNSUPPORTED;
    const int64_t nby = (H + tra::kTileSide - 1) / tra::kTileSide;
    const int64_t nbx = (W + tra::kTileSide - 1) / tra::kTileSide;
    const int64_t nb = (int64_t)T * nby * nbx;
    // block ids stay below 2^24 and tile counts per axis below 2^15 (the
    // attention kernel's multiply-shift division is exact in that range)
    if (nb >= (int64_t(1) << 24) || nby >= (1 << 15) || nbx >= (1 << 15)) return TRA_ERR_UNSUPPORTED;
    if ((int64_t)T * H * W > INT32_MAX) return TRA_ERR_UNSUPPORTED;
    g->T = T; g->H = H; g->W = W;
    g->nby = (int)nby; g->nbx = (int)nbx; g->nb = (int)nb;
    return TRA_OK;
}

int check_radii(int r_min, int r_max) {
    if (is_dense(r_min, r_max)) return TRA_OK;
    if (r_min < 0 || r_max < r_min) return TRA_ERR_INVALID_ARG;
    return TRA_OK;
}

int check_dims(int heads, int head_dim, const tra::Grid &g) {
    if (heads < 1 || head_dim < 1) return TRA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return TRA_ERR_UNSUPPORTED;
    if (heads > 65535) return TRA_ERR_UNSUPPORTED;
    // packed tiles and tokens, per tensor
    if ((int64_t)heads * g.nb * tra::kBlockTokens * head_dim > kMaxElems) return TRA_ERR_UNSUPPORTED;
    if ((int64_t)heads * g.nb > INT32_MAX) return TRA_ERR_UNSUPPORTED;
    return TRA_OK;
}

int64_t maxcnt_of(const tra::Grid &g, int r_max) {
    if (r_max == TRA_RADIUS_INF) return g.nb;
    const int64_t w = 2 * (int64_t)r_max + 1;
    const int64_t a = w < g.T ? w : g.T;
    const int64_t b = w < g.nby ? w : g.nby;
    const int64_t c = w < g.nbx ? w : g.nbx;
    return a * b * c;
}

// Library-owned stream-ordered memory pool per device.  Freed scratch stays in
// the pool (release threshold = max) so repeated calls do not reach the driver.
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices] = {};

hipError_t pool_for_current_device(hipMemPool_t *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (!g_pool[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        e = hipMemPoolCreate(&p, &props);
        if (e != hipSuccess) return e;
        uint64_t threshold = UINT64_MAX;
        e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &threshold);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(p);
            return e;
        }
        g_pool[dev] = p;
    }
    *out = g_pool[dev];
    return hipSuccess;
}

// Scratch carved from one stream-ordered allocation; freed on the stream when
// the scope ends (after every kernel that uses it has been enqueued).
class Scratch {
  public:
    explicit Scratch(hipStream_t s) : s_(s) {}
    ~Scratch() {
        if (base_) (void)hipFreeAsync(base_, s_);
    }
    // Reserve `bytes` (256-byte aligned); returns the offset.
    size_t reserve(size_t bytes) {
        const size_t off = size_;
        size_ += (bytes + 255) & ~size_t(255);
        return off;
    }
    int allocate() {
        if (size_ == 0) return TRA_OK;
        hipMemPool_t pool = nullptr;
        if (pool_for_current_device(&pool) != hipSuccess) return TRA_ERR_HIP;
        const hipError_t e = hipMallocFromPoolAsync(&base_, size_, pool, s_);
        if (e == hipErrorOutOfMemory) return TRA_ERR_NOMEM;
        if (e != hipSuccess) {
            base_ = nullptr;
            return TRA_ERR_HIP;
        }
        return TRA_OK;
    }
    template <typename T>
    T *at(size_t off) const {
        return reinterpret_cast<T *>(static_cast<char *>(base_) + off);
    }

  private:
    hipStream_t s_;
    void *base_ = nullptr;
    size_t size_ = 0;
};

int hip_status(hipError_t e) { return e == hipSuccess ? TRA_OK : TRA_ERR_HIP; }

// Work items of the attention kernel: pairs of neighbouring query blocks.
size_t walk_rows(const tra::Grid &g, int heads) { return (size_t)tra::walk_items(g, heads); }
size_t order_len(const tra::Grid &g, int heads) { return (size_t)tra::order_ints(g, heads); }

// ---- optional per-kernel event timing ----
struct ProfRecord {
    int kind;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;

// Brackets one kernel launch with events on its stream when profiling is on.
class ProfScope {
  public:
    ProfScope(int kind, hipStream_t s) : s_(s) {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        if (!g_prof_on) return;
        rec_.kind = kind;
        if (hipEventCreate(&rec_.start) != hipSuccess) return;
        if (hipEventCreate(&rec_.stop) != hipSuccess) {
            (void)hipEventDestroy(rec_.start);
            return;
        }
        active_ = hipEventRecord(rec_.start, s_) == hipSuccess;
        if (!active_) {
            (void)hipEventDestroy(rec_.start);
            (void)hipEventDestroy(rec_.stop);
        }
    }
    ~ProfScope() {
        if (!active_) return;
        (void)hipEventRecord(rec_.stop, s_);
        std::lock_guard<std::mutex> lock(g_prof_mu);
        g_prof.push_back(rec_);
    }

  private:
    hipStream_t s_;
    ProfRecord rec_{};
    bool active_ = false;
};

// Packed K/V of one call: K and V^T tiles, the partial maxima of |v| and the
// per-head V exponents (see launch_vmax).
struct PackedOffsets {
    size_t kt, vt, vpart, vexp, sched;
};
struct Packed {
    uint16_t *kt, *vt;
    uint32_t *vpart;
    int32_t *vexp;
    int32_t *sched;  // the attention launch's work-claiming counters
};

PackedOffsets reserve_packed(Scratch &ws, const tra::Grid &g, int heads, int head_dim) {
    const size_t tiles = (size_t)heads * g.nb * tra::packed_tile_elems(head_dim) * 2;
    PackedOffsets o;
    o.kt = ws.reserve(tiles);
    o.vt = ws.reserve(tiles);
    o.vpart = ws.reserve((size_t)heads * tra::kVmaxParts * sizeof(uint32_t));
    o.vexp = ws.reserve((size_t)heads * sizeof(int32_t));
    o.sched = ws.reserve(tra::kSchedBytes);
    return o;
}

Packed packed_at(const Scratch &ws, const PackedOffsets &o) {
    return Packed{ws.at<uint16_t>(o.kt), ws.at<uint16_t>(o.vt), ws.at<uint32_t>(o.vpart),
                  ws.at<int32_t>(o.vexp), ws.at<int32_t>(o.sched)};
}

// The head's largest |v|, then the tile packing of k and v (and, with q given,
// the pooled means of q and k).
hipError_t pack_kv(int head_dim, const void *q, const void *k, const void *v, const tra::Grid &g,
                   int heads, float *qp, float *kp, const Packed &p, hipStream_t stream) {
    hipError_t e;
    {
        ProfScope ps(TRA_KERNEL_VMAX, stream);
        e = tra::launch_vmax(head_dim, (const uint16_t *)v, g, heads, p.vpart, p.sched, stream);
    }
    if (e != hipSuccess) return e;
    ProfScope ps(TRA_KERNEL_PACK_POOL, stream);
    return tra::launch_pack_pool(head_dim, q != nullptr, true, (const uint16_t *)q,
                                 (const uint16_t *)k, (const uint16_t *)v, g, heads, qp, kp, p.kt,
                                 p.vt, p.vpart, p.vexp, stream);
}

// Bytes of tra_probe's workspace: the pooled means of q and k.
size_t probe_ws_bytes(const tra::Grid &g, int heads, int head_dim) {
    const size_t pooled = (size_t)heads * g.nb * head_dim * sizeof(float);
    return 2 * ((pooled + 255) & ~size_t(255));
}

}  // namespace

extern "C" {

const char *tra_status_string(int status) {
    switch (status) {
        case TRA_OK: return "TRA_OK";
        case TRA_ERR_INVALID_ARG: return "TRA_ERR_INVALID_ARG";
        case TRA_ERR_UNSUPPORTED: return "TRA_ERR_UNSUPPORTED";
        case TRA_ERR_HIP: return "TRA_ERR_HIP";
        case TRA_ERR_NOMEM: return "TRA_ERR_NOMEM";
        case TRA_ERR_TOO_LARGE: return "TRA_ERR_TOO_LARGE";
        default: return "TRA_ERR_UNKNOWN";
    }
}

int tra_version(void) { return 200; }

int tra_grid(int T, int H, int W, int block, int *nby, int *nbx, int *nb) {
    tra::Grid g;
    const int rc = make_grid(T, H, W, block, &g);
    if (rc != TRA_OK) return rc;
    if (nby) *nby = g.nby;
    if (nbx) *nbx = g.nbx;
    if (nb) *nb = g.nb;
    return TRA_OK;
}

int64_t tra_maxcnt(int T, int H, int W, int block, int r_max) {
    tra::Grid g;
    const int rc = make_grid(T, H, W, block, &g);
    if (rc != TRA_OK) return rc;
    if (r_max < 0) return TRA_ERR_INVALID_ARG;
    return maxcnt_of(g, r_max);
}

int64_t tra_workspace_bytes(int T, int H, int W, int heads, int head_dim, int block, int r_max) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc != TRA_OK) return rc;
    if (r_max < 0) return TRA_ERR_INVALID_ARG;
    return (int64_t)probe_ws_bytes(g, heads, head_dim);
}

int tra_probe(const void *q, const void *k, int T, int H, int W, int heads, int head_dim,
              int block, int r_min, int r_max, int32_t *radius, float *h_norm, void *ws,
              hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc == TRA_OK) rc = check_radii(r_min, r_max);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !radius) return TRA_ERR_INVALID_ARG;
    hipError_t e;
    if (is_dense(r_min, r_max)) {
        ProfScope p(TRA_KERNEL_FILL, stream);
        e = tra::launch_fill_dense(g, heads, radius, h_norm, stream);
        return hip_status(e);
    }

    // the pooled means live in the caller's workspace, else in library scratch
    Scratch pool(stream);
    const size_t half = probe_ws_bytes(g, heads, head_dim) / 2;
    char *base = static_cast<char *>(ws);
    if (!base) {
        const size_t o = pool.reserve(2 * half);
        if ((rc = pool.allocate()) != TRA_OK) return rc;
        base = pool.at<char>(o);
    }
    float *qp = reinterpret_cast<float *>(base), *kp = reinterpret_cast<float *>(base + half);
    {
        ProfScope p(TRA_KERNEL_PACK_POOL, stream);
        e = tra::launch_pack_pool(head_dim, true, false, (const uint16_t *)q, (const uint16_t *)k,
                                  nullptr, g, heads, qp, kp, nullptr, nullptr, nullptr, nullptr,
                                  stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_ENTROPY, stream);
        e = tra::launch_entropy(head_dim, qp, kp, g, heads, r_min, r_max, radius, h_norm, stream);
    }
    return hip_status(e);
}

int tra_probe_static(const void *q, const void *k, int T, int H, int W, int heads, int head_dim,
                     int block, int r_min, int r_max, int32_t *radius, float *h_norm,
                     hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc == TRA_OK) rc = check_radii(r_min, r_max);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !radius) return TRA_ERR_INVALID_ARG;
    if (probe_ws_bytes(g, heads, head_dim) > tra::kStaticScratchBytes) return TRA_ERR_TOO_LARGE;
    void *ws = nullptr;
    if (tra::static_scratch(&ws) != hipSuccess) return TRA_ERR_HIP;
    return tra_probe(q, k, T, H, W, heads, head_dim, block, r_min, r_max, radius, h_norm, ws,
                     stream);
}

int64_t tra_static_scratch_bytes(void) { return (int64_t)tra::kStaticScratchBytes; }

int tra_mask(const int32_t *radius, int T, int H, int W, int heads, int block, int r_max,
             int32_t *idx, int32_t *cnt, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc != TRA_OK) return rc;
    if (heads < 1 || r_max < 0) return TRA_ERR_INVALID_ARG;
    if ((int64_t)heads * g.nb > INT32_MAX) return TRA_ERR_UNSUPPORTED;
    if (!radius || !idx || !cnt) return TRA_ERR_INVALID_ARG;
    ProfScope p(TRA_KERNEL_MASK, stream);
    return hip_status(tra::launch_mask(radius, g, heads, r_max, maxcnt_of(g, r_max), idx, cnt, stream));
}

// The attention walk of the lists: the pair table, the union of each pair's
// two lists, then the work order of the pairs (XCD ranges, longest length
// class first).
static hipError_t plan_walk(const int32_t *idx, const int32_t *cnt, const float *lw,
                            int64_t maxcnt, const tra::Grid &g, int heads, int2 *pairs,
                            int32_t *ulist, int32_t *ulen, float2 *ubias, int32_t *order,
                            hipStream_t stream) {
    hipError_t e;
    {
        ProfScope p(TRA_KERNEL_PAIR, stream);
        // the work order's memory holds the candidate walk lengths meanwhile
        e = tra::launch_pair(idx, cnt, maxcnt, g, heads, pairs, order, stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_UNION, stream);
        e = tra::launch_union(idx, cnt, lw, maxcnt, g, heads, pairs, ulist, ulen, ubias, stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_ORDER, stream);
        e = tra::launch_order(ulen, g, heads, maxcnt, order, stream);
    }
    return e;
}

// The walk plan of the radius mask's lists, taken straight from the radii:
// the radius pair table, the union of each pair's two key boxes, the order.
// Each block meets the same entries in the same order as along plan_walk of
// the lists (the pairing differs; results do not).
static hipError_t plan_walk_radius(const int32_t *radius, int r_max, int64_t maxcnt,
                                   const tra::Grid &g, int heads, int2 *pairs, int32_t *ulist,
                                   int32_t *ulen, int32_t *order, hipStream_t stream) {
    hipError_t e;
    {
        ProfScope p(TRA_KERNEL_PAIR, stream);
        e = tra::launch_pair_radius(radius, r_max, maxcnt, g, heads, pairs, stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_UNION, stream);
        e = tra::launch_radius_walk(radius, r_max, maxcnt, g, heads, pairs, ulist, ulen, stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_ORDER, stream);
        e = tra::launch_order(ulen, g, heads, maxcnt, order, stream);
    }
    return e;
}

// Layout of a walk plan in one buffer: work order, walk lengths, walks, the
// pair table and (for weighted lists) the walks' per-side log2 weights; each
// part 256-byte aligned.
struct PlanLayout {
    size_t o_order, o_ulen, o_ulist, o_pairs, o_ubias, bytes;
    int64_t ustride;
    bool weighted;
};

static PlanLayout plan_layout(const tra::Grid &g, int heads, int64_t maxcnt,
                              bool weighted = false) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    PlanLayout L;
    const size_t rows = walk_rows(g, heads);
    L.ustride = tra::union_stride(maxcnt);
    L.weighted = weighted;
    L.o_order = 0;
    L.o_ulen = up(order_len(g, heads) * sizeof(int32_t));
    L.o_ulist = L.o_ulen + up(rows * sizeof(int32_t));
    L.o_pairs = L.o_ulist + up(rows * (size_t)L.ustride * sizeof(int32_t));
    L.o_ubias = L.o_pairs + up(rows * sizeof(int2));
    L.bytes = L.o_ubias + (weighted ? up(rows * (size_t)L.ustride * sizeof(float2)) : 0);
    return L;
}

static hipError_t plan_walk_into(const int32_t *idx, const int32_t *cnt, const float *lw,
                                 int64_t maxcnt, const tra::Grid &g, int heads, char *plan,
                                 const PlanLayout &L, hipStream_t stream) {
    return plan_walk(idx, cnt, lw, maxcnt, g, heads, (int2 *)(plan + L.o_pairs),
                     (int32_t *)(plan + L.o_ulist), (int32_t *)(plan + L.o_ulen),
                     L.weighted ? (float2 *)(plan + L.o_ubias) : nullptr,
                     (int32_t *)(plan + L.o_order), stream);
}

// The attention kernel along a walk plan (nullptr: dense mode) over packed K/V.
static hipError_t attn_launch(const void *q, const Packed &pk, const tra::Grid &g, int heads,
                              int head_dim, const char *plan, const PlanLayout &L, void *out,
                              hipStream_t stream, const tra::EntropyOut *eo = nullptr) {
    ProfScope p(TRA_KERNEL_ATTN, stream);
    const int32_t *order = plan ? (const int32_t *)(plan + L.o_order) : nullptr;
    const int32_t *ulen = plan ? (const int32_t *)(plan + L.o_ulen) : nullptr;
    const int32_t *ulist = plan ? (const int32_t *)(plan + L.o_ulist) : nullptr;
    const float2 *ubias = plan && L.weighted ? (const float2 *)(plan + L.o_ubias) : nullptr;
    const int2 *pairs = plan ? (const int2 *)(plan + L.o_pairs) : nullptr;
    return tra::launch_attn(head_dim, (const uint16_t *)q, pk.kt, pk.vt, pk.vexp, pairs, ulist,
                            ulen, ubias, plan ? L.ustride : 0, order, pk.sched, g, heads,
                            (float *)out, stream, eo);
}

// Pack k and v, then attention along a walk plan (nullptr: dense mode).
static int attn_with_plan(const void *q, const void *k, const void *v, const tra::Grid &g,
                          int heads, int head_dim, const char *plan, const PlanLayout &L,
                          void *out, hipStream_t stream) {
    Scratch ws(stream);
    const PackedOffsets po = reserve_packed(ws, g, heads, head_dim);
    int rc = ws.allocate();
    if (rc != TRA_OK) return rc;
    const Packed pk = packed_at(ws, po);
    hipError_t e = pack_kv(head_dim, nullptr, k, v, g, heads, nullptr, nullptr, pk, stream);
    if (e == hipSuccess) e = attn_launch(q, pk, g, heads, head_dim, plan, L, out, stream);
    return hip_status(e);
}

// Walk plans above 2^44 bytes are refused (they could not be allocated anyway).
static int check_plan(const tra::Grid &g, int heads, int64_t maxcnt) {
    if (maxcnt < 1 || maxcnt > (int64_t)1 << 30) return TRA_ERR_INVALID_ARG;
    const double bytes = (double)walk_rows(g, heads) * (double)tra::union_stride(maxcnt) * 4.0;
    return bytes > (double)((int64_t)1 << 44) ? TRA_ERR_UNSUPPORTED : TRA_OK;
}

int64_t tra_plan_bytes(int T, int H, int W, int heads, int block, int64_t maxcnt) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, 64, g);
    if (rc == TRA_OK) rc = check_plan(g, heads, maxcnt);
    if (rc != TRA_OK) return rc;
    return (int64_t)plan_layout(g, heads, maxcnt).bytes;
}

int tra_plan(const int32_t *idx, const int32_t *cnt, int64_t maxcnt, int T, int H, int W,
             int heads, int block, void *plan, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, 64, g);
    if (rc == TRA_OK) rc = check_plan(g, heads, maxcnt);
    if (rc != TRA_OK) return rc;
    if (!idx || !cnt || !plan) return TRA_ERR_INVALID_ARG;
    return hip_status(plan_walk_into(idx, cnt, nullptr, maxcnt, g, heads, static_cast<char *>(plan),
                                     plan_layout(g, heads, maxcnt), stream));
}

int tra_plan_radius(const int32_t *radius, int T, int H, int W, int heads, int block, int r_max,
                    void *plan, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, 64, g);
    if (rc != TRA_OK) return rc;
    if (r_max < 0) return TRA_ERR_INVALID_ARG;
    const int64_t maxcnt = maxcnt_of(g, r_max);
    if ((rc = check_plan(g, heads, maxcnt)) != TRA_OK) return rc;
    if (!radius || !plan) return TRA_ERR_INVALID_ARG;
    const PlanLayout L = plan_layout(g, heads, maxcnt);
    char *pl = static_cast<char *>(plan);
    return hip_status(plan_walk_radius(radius, r_max, maxcnt, g, heads, (int2 *)(pl + L.o_pairs),
                                       (int32_t *)(pl + L.o_ulist), (int32_t *)(pl + L.o_ulen),
                                       (int32_t *)(pl + L.o_order), stream));
}

int tra_attn_plan(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                  int head_dim, int block, const void *plan, int64_t maxcnt, void *out,
                  hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc == TRA_OK) rc = check_plan(g, heads, maxcnt);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out || !plan) return TRA_ERR_INVALID_ARG;
    return attn_with_plan(q, k, v, g, heads, head_dim, static_cast<const char *>(plan),
                          plan_layout(g, heads, maxcnt), out, stream);
}

// Lists (with optional log-weights) -> walk plan in library scratch -> attention,
// all on the caller's stream.  (Packing k and v on a second stream beside the
// latency-bound plan kernels measured slightly slower: the HBM-bound packing
// slows the kernels beside it more than it overlaps them.)
static int attn_lists(const void *q, const void *k, const void *v, const tra::Grid &g, int heads,
                      int head_dim, const int32_t *idx, const int32_t *cnt, const float *lw,
                      int64_t maxcnt, void *out, hipStream_t stream) {
    const PlanLayout L = plan_layout(g, heads, maxcnt, lw != nullptr);
    Scratch ws(stream);
    const PackedOffsets po = reserve_packed(ws, g, heads, head_dim);
    const size_t o_plan = ws.reserve(L.bytes);
    int rc = ws.allocate();
    if (rc != TRA_OK) return rc;
    const Packed pk = packed_at(ws, po);
    char *plan = ws.at<char>(o_plan);
    hipError_t e = pack_kv(head_dim, nullptr, k, v, g, heads, nullptr, nullptr, pk, stream);
    if (e == hipSuccess) e = plan_walk_into(idx, cnt, lw, maxcnt, g, heads, plan, L, stream);
    if (e == hipSuccess) e = attn_launch(q, pk, g, heads, head_dim, plan, L, out, stream);
    return hip_status(e);
}

int tra_attn(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
             int head_dim, int block, const int32_t *idx, const int32_t *cnt, int64_t maxcnt,
             void *out, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out) return TRA_ERR_INVALID_ARG;
    if ((idx == nullptr) != (cnt == nullptr)) return TRA_ERR_INVALID_ARG;
    if (idx && (rc = check_plan(g, heads, maxcnt)) != TRA_OK) return rc;
    if (!idx) return attn_with_plan(q, k, v, g, heads, head_dim, nullptr, PlanLayout{}, out, stream);
    return attn_lists(q, k, v, g, heads, head_dim, idx, cnt, nullptr, maxcnt, out, stream);
}

int tra_attn_weighted(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                      int head_dim, int block, const int32_t *idx, const int32_t *cnt,
                      const float *lw, int64_t maxcnt, void *out, hipStream_t stream) {
    if (!lw) return tra_attn(q, k, v, T, H, W, heads, head_dim, block, idx, cnt, maxcnt, out, stream);
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out || !idx || !cnt) return TRA_ERR_INVALID_ARG;
    if ((rc = check_plan(g, heads, maxcnt)) != TRA_OK) return rc;
    return attn_lists(q, k, v, g, heads, head_dim, idx, cnt, lw, maxcnt, out, stream);
}

// Launches timed back to back get a zeroed set of work-claiming counters each.
constexpr int kMaxTimedReps = 4096;

// Packs k and v into pk, then times `reps` back-to-back attention launches
// along the plan (nullptr: dense mode) between one pair of events on `stream`;
// sched_sets: reps sets of work-claiming counters (kSchedBytes each), zeroed
// before the timed launches.
static int time_attn_launches(const void *q, const void *k, const void *v, const tra::Grid &g,
                              int heads, int head_dim, const char *plan, const PlanLayout &L,
                              const Packed &pk, int32_t *sched_sets, int reps, void *out,
                              float *ms, hipStream_t stream) {
    const int64_t set_ints = (int64_t)(tra::kSchedBytes / sizeof(int32_t));
    hipError_t e = pack_kv(head_dim, nullptr, k, v, g, heads, nullptr, nullptr, pk, stream);
    if (e == hipSuccess) e = tra::launch_zero(sched_sets, set_ints * reps, stream);
    if (e != hipSuccess) return hip_status(e);
    hipEvent_t ev[2];
    if (hipEventCreate(&ev[0]) != hipSuccess) return TRA_ERR_HIP;
    if (hipEventCreate(&ev[1]) != hipSuccess) {
        (void)hipEventDestroy(ev[0]);
        return TRA_ERR_HIP;
    }
    e = hipEventRecord(ev[0], stream);
    for (int i = 0; i < reps && e == hipSuccess; ++i) {
        Packed pi = pk;
        pi.sched = sched_sets + set_ints * i;
        e = attn_launch(q, pi, g, heads, head_dim, plan, L, out, stream);
    }
    if (e == hipSuccess) e = hipEventRecord(ev[1], stream);
    if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[0], ev[1]);
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (e != hipSuccess) return TRA_ERR_HIP;
    *ms = t / (float)reps;
    return TRA_OK;
}

int tra_time_attn(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                  int head_dim, int block, const int32_t *idx, const int32_t *cnt,
                  const float *lw, int64_t maxcnt, int reps, void *out, float *ms,
                  hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out || !ms || reps < 1 || reps > kMaxTimedReps)
        return TRA_ERR_INVALID_ARG;
    if ((idx == nullptr) != (cnt == nullptr) || (lw && !idx)) return TRA_ERR_INVALID_ARG;
    if (idx && (rc = check_plan(g, heads, maxcnt)) != TRA_OK) return rc;
    const PlanLayout L = idx ? plan_layout(g, heads, maxcnt, lw != nullptr) : PlanLayout{};
    Scratch ws(stream);
    const PackedOffsets po = reserve_packed(ws, g, heads, head_dim);
    const size_t o_plan = idx ? ws.reserve(L.bytes) : 0;
    const size_t o_sets = ws.reserve(tra::kSchedBytes * (size_t)reps);
    if ((rc = ws.allocate()) != TRA_OK) return rc;
    const Packed pk = packed_at(ws, po);
    char *plan = idx ? ws.at<char>(o_plan) : nullptr;
    hipError_t e = hipSuccess;
    if (idx) e = plan_walk_into(idx, cnt, lw, maxcnt, g, heads, plan, L, stream);
    if (e != hipSuccess) return hip_status(e);
    return time_attn_launches(q, k, v, g, heads, head_dim, plan, L, pk, ws.at<int32_t>(o_sets),
                              reps, out, ms, stream);
}

int tra_time_attn_plan(const void *q, const void *k, const void *v, int T, int H, int W,
                       int heads, int head_dim, int block, const void *plan, int64_t maxcnt,
                       int reps, void *out, float *ms, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out || !ms || reps < 1 || reps > kMaxTimedReps)
        return TRA_ERR_INVALID_ARG;
    if (plan && (rc = check_plan(g, heads, maxcnt)) != TRA_OK) return rc;
    const PlanLayout L = plan ? plan_layout(g, heads, maxcnt) : PlanLayout{};
    Scratch ws(stream);
    const PackedOffsets po = reserve_packed(ws, g, heads, head_dim);
    const size_t o_sets = ws.reserve(tra::kSchedBytes * (size_t)reps);
    if ((rc = ws.allocate()) != TRA_OK) return rc;
    return time_attn_launches(q, k, v, g, heads, head_dim, static_cast<const char *>(plan), L,
                              packed_at(ws, po), ws.at<int32_t>(o_sets), reps, out, ms, stream);
}

int tra_sip_mask(const void *q, const void *k, const float *u, int T, int H, int W, int heads,
                 int head_dim, int block, float m, int32_t *idx, int32_t *cnt, float *lw,
                 hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !u || !idx || !cnt || !lw || !(m >= 0.f) || !isfinite(m))
        return TRA_ERR_INVALID_ARG;
    if ((double)heads * g.nb * g.nb > (double)((int64_t)1 << 40)) return TRA_ERR_UNSUPPORTED;
    const size_t rows = (size_t)heads * g.nb;
    Scratch ws(stream);
    const size_t pooled = rows * head_dim * sizeof(float);
    const size_t o_qp = ws.reserve(pooled), o_kp = ws.reserve(pooled);
    const size_t o_r = ws.reserve(rows * sizeof(int32_t));
    const size_t o_lg = ws.reserve(rows * (size_t)g.nb * sizeof(float));
    if ((rc = ws.allocate()) != TRA_OK) return rc;
    float *qp = ws.at<float>(o_qp), *kp = ws.at<float>(o_kp), *lg = ws.at<float>(o_lg);
    int32_t *radius = ws.at<int32_t>(o_r);
    hipError_t e;
    {
        ProfScope p(TRA_KERNEL_PACK_POOL, stream);
        e = tra::launch_pack_pool(head_dim, true, false, (const uint16_t *)q, (const uint16_t *)k,
                                  nullptr, g, heads, qp, kp, nullptr, nullptr, nullptr, nullptr,
                                  stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_ENTROPY, stream);
        e = tra::launch_entropy(head_dim, qp, kp, g, heads, 0, 0, radius, nullptr, stream, lg);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_SIP, stream);
        e = tra::launch_sip(lg, u, g, heads, m, idx, cnt, lw, stream);
    }
    return hip_status(e);
}

static int check_token_params(float tau, float gamma) {
    if (!(tau > 0.f) || !isfinite(tau) || !(gamma >= 0.f) || !isfinite(gamma))
        return TRA_ERR_INVALID_ARG;
    return TRA_OK;
}

static float two_gamma_log2e(float gamma) { return (float)(2.0 * gamma * 1.4426950408889634); }

int tra_token_probe(const void *q, const void *k, int T, int H, int W, int heads, int head_dim,
                    int block, float tau, float gamma, float *entropy, float *r0,
                    hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc == TRA_OK) rc = check_token_params(tau, gamma);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !r0) return TRA_ERR_INVALID_ARG;
    Scratch ws(stream);
    const size_t tiles = (size_t)heads * g.nb * tra::packed_tile_elems(head_dim) * 2;
    const size_t o_kt = ws.reserve(tiles);
    const size_t o_ent = entropy ? 0 : ws.reserve((size_t)heads * T * H * W * sizeof(float));
    if ((rc = ws.allocate()) != TRA_OK) return rc;
    uint16_t *kt = ws.at<uint16_t>(o_kt);
    float *ent = entropy ? entropy : ws.at<float>(o_ent);
    hipError_t e;
    {
        ProfScope p(TRA_KERNEL_PACK_POOL, stream);
        e = tra::launch_pack_k(head_dim, (const uint16_t *)k, g, heads, kt, stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_TOKEN_ENTROPY, stream);
        e = tra::launch_token_entropy(head_dim, (const uint16_t *)q, kt, g, heads, tau, gamma, ent,
                                      r0, stream);
    }
    return hip_status(e);
}

int tra_token_warmup(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                     int head_dim, int block, float tau, float gamma, void *out, float *entropy,
                     float *r0, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc == TRA_OK) rc = check_token_params(tau, gamma);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out || !r0) return TRA_ERR_INVALID_ARG;
    Scratch ws(stream);
    const PackedOffsets po = reserve_packed(ws, g, heads, head_dim);
    const size_t o_ent = entropy ? 0 : ws.reserve((size_t)heads * T * H * W * sizeof(float));
    if ((rc = ws.allocate()) != TRA_OK) return rc;
    const Packed pk = packed_at(ws, po);
    const tra::EntropyOut eo{entropy ? entropy : ws.at<float>(o_ent), r0, tau,
                             two_gamma_log2e(gamma)};
    hipError_t e = pack_kv(head_dim, nullptr, k, v, g, heads, nullptr, nullptr, pk, stream);
    if (e == hipSuccess) e = attn_launch(q, pk, g, heads, head_dim, nullptr, PlanLayout{}, out, stream, &eo);
    return hip_status(e);
}

int tra_token_mask(const float *r0, int T, int H, int W, int heads, int block, float gamma,
                   int min_votes, int32_t *idx, int32_t *cnt, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, 64, g);
    if (rc == TRA_OK) rc = check_token_params(1.f, gamma);
    if (rc != TRA_OK) return rc;
    if (!r0 || !idx || !cnt || min_votes < 1 || min_votes > tra::kBlockTokens)
        return TRA_ERR_INVALID_ARG;
    ProfScope p(TRA_KERNEL_TOKEN_MASK, stream);
    return hip_status(tra::launch_token_mask(r0, g, heads, gamma, min_votes, g.nb, idx, cnt, stream));
}

int tra_token_attention(const void *q, const void *k, const void *v, int T, int H, int W,
                        int heads, int head_dim, int block, float tau, float gamma,
                        int min_votes, void *out, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc == TRA_OK) rc = check_token_params(tau, gamma);
    if (rc == TRA_OK) rc = check_plan(g, heads, g.nb);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out || min_votes < 1 || min_votes > tra::kBlockTokens)
        return TRA_ERR_INVALID_ARG;
    const size_t rows = (size_t)heads * g.nb;
    const size_t toks = (size_t)heads * T * H * W;
    const PlanLayout L = plan_layout(g, heads, g.nb);
    Scratch ws(stream);
    const PackedOffsets po = reserve_packed(ws, g, heads, head_dim);
    const size_t o_ent = ws.reserve(toks * sizeof(float)), o_r0 = ws.reserve(toks * sizeof(float));
    const size_t o_idx = ws.reserve(rows * (size_t)g.nb * sizeof(int32_t));
    const size_t o_cnt = ws.reserve(rows * sizeof(int32_t));
    const size_t o_plan = ws.reserve(L.bytes);
    if ((rc = ws.allocate()) != TRA_OK) return rc;
    const Packed pk = packed_at(ws, po);
    float *ent = ws.at<float>(o_ent), *r0 = ws.at<float>(o_r0);
    int32_t *idx = ws.at<int32_t>(o_idx), *cnt = ws.at<int32_t>(o_cnt);
    char *plan = ws.at<char>(o_plan);
    hipError_t e = pack_kv(head_dim, nullptr, k, v, g, heads, nullptr, nullptr, pk, stream);
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_TOKEN_ENTROPY, stream);
        e = tra::launch_token_entropy(head_dim, (const uint16_t *)q, pk.kt, g, heads, tau, gamma,
                                      ent, r0, stream);
    }
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_TOKEN_MASK, stream);
        e = tra::launch_token_mask(r0, g, heads, gamma, min_votes, g.nb, idx, cnt, stream);
    }
    if (e == hipSuccess) e = plan_walk_into(idx, cnt, nullptr, g.nb, g, heads, plan, L, stream);
    if (e == hipSuccess) e = attn_launch(q, pk, g, heads, head_dim, plan, L, out, stream);
    return hip_status(e);
}

int tra_attention(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                  int head_dim, int block, int r_min, int r_max, void *out, hipStream_t stream) {
    tra::Grid g;
    int rc = make_grid(T, H, W, block, &g);
    if (rc == TRA_OK) rc = check_dims(heads, head_dim, g);
    if (rc == TRA_OK) rc = check_radii(r_min, r_max);
    if (rc != TRA_OK) return rc;
    if (!q || !k || !v || !out) return TRA_ERR_INVALID_ARG;

    const bool dense = is_dense(r_min, r_max);
    if (dense) return attn_with_plan(q, k, v, g, heads, head_dim, nullptr, PlanLayout{}, out, stream);

    const int64_t maxcnt = maxcnt_of(g, r_max);
    const size_t rows = (size_t)heads * g.nb;
    const PlanLayout L = plan_layout(g, heads, maxcnt);
    Scratch ws(stream);
    const PackedOffsets po = reserve_packed(ws, g, heads, head_dim);
    const size_t o_qp = ws.reserve(rows * head_dim * sizeof(float));
    const size_t o_kp = ws.reserve(rows * head_dim * sizeof(float));
    const size_t o_r = ws.reserve(rows * sizeof(int32_t));
    const size_t o_plan = ws.reserve(L.bytes);
    if ((rc = ws.allocate()) != TRA_OK) return rc;
    const Packed pk = packed_at(ws, po);
    float *qp = ws.at<float>(o_qp), *kp = ws.at<float>(o_kp);
    int32_t *radius = ws.at<int32_t>(o_r);
    char *plan = ws.at<char>(o_plan);

    // One stream: V's scale, then one pass over q, k, v that pools q and k and
    // packs k and v, the entropy, and the walk plan straight from the radii
    // (the radius mask's lists are never written out).  Packing on a second
    // stream beside the latency-bound entropy and plan kernels measured no
    // faster: the HBM-bound packing slows the kernels beside it as much as it
    // overlaps them.
    hipError_t e = pack_kv(head_dim, q, k, v, g, heads, qp, kp, pk, stream);
    if (e == hipSuccess) {
        ProfScope p(TRA_KERNEL_ENTROPY, stream);
        e = tra::launch_entropy(head_dim, qp, kp, g, heads, r_min, r_max, radius, nullptr, stream);
    }
    if (e == hipSuccess)
        e = plan_walk_radius(radius, r_max, maxcnt, g, heads, (int2 *)(plan + L.o_pairs),
                             (int32_t *)(plan + L.o_ulist), (int32_t *)(plan + L.o_ulen),
                             (int32_t *)(plan + L.o_order), stream);
    if (e == hipSuccess) e = attn_launch(q, pk, g, heads, head_dim, plan, L, out, stream);
    return hip_status(e);
}

int tra_release_scratch(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TRA_ERR_HIP;
    hipMemPool_t p = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_pool_mu);
        p = g_pool[dev];
    }
    if (!p) return TRA_OK;
    return hip_status(hipMemPoolTrimTo(p, 0));
}

int tra_profile_begin(void) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_on = true;
    return TRA_OK;
}

int tra_profile_end(double *ms, int *launches, int n) {
    std::vector<ProfRecord> recs;
    {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        g_prof_on = false;
        recs.swap(g_prof);
    }
    for (int i = 0; i < n; ++i) {
        if (ms) ms[i] = 0.0;
        if (launches) launches[i] = 0;
    }
    int rc = TRA_OK;
    for (const ProfRecord &r : recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
            rc = TRA_ERR_HIP;
        else if (r.kind < n) {
            if (ms) ms[r.kind] += t;
            if (launches) launches[r.kind] += 1;
        }
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    return rc;
}

}  // extern "C"
