// Host side of the crkv C ABI: argument validation, the per-call plan
// (segment table, key tiles, work items, impact-partial slots), the upload of
// that plan through a per-device ring on a copy stream, and the kernel
// launches.
//
// Nothing here synchronises the caller's stream. The only host waits are on
// ring-slot events, which complete once the work of the call four uploads
// earlier has run, and, when the library's scratch buffer or a ring slot has
// to grow, on the work of the call that used it last.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "crkv.h"
#include "crkv_internal.h"

namespace crkv {
hipError_t launch_attn_bf16_wave(int d, int rt, const AttnArgs &args, int n_items, hipStream_t stream);
hipError_t launch_attn_bf16_pair(int d, int rt, const AttnArgs &args, int n_items, hipStream_t stream);
hipError_t launch_attn_q8(int d, int rt, const AttnArgs &args, int n_items, hipStream_t stream);
hipError_t launch_attn_lse(int d, bool kv8, const AttnArgs &args, int n_items, hipStream_t stream);
hipError_t launch_attn_out_combine(int d, const CombineArgs &args, int n_items, hipStream_t stream);
hipError_t launch_decode_bf16(int d, const DecodeArgs &args, int n_items, int n_pairs, hipStream_t stream);
hipError_t launch_attn_f32(int d, const AttnArgs &args, int n_items, hipStream_t stream);
hipError_t launch_combine(const ProbDesc *probs, int n_probs, int max_keys, hipStream_t stream);
hipError_t launch_topk_one(const TopkDesc &td, hipStream_t stream);
hipError_t launch_topk_batched(const TopkDesc *descs, int n, hipStream_t stream);
hipError_t launch_topk_inline(const TopkDesc *descs, int n, hipStream_t stream);
hipError_t launch_kvsel(bool scatter, const SelArgs &args, int n_items, hipStream_t stream);
hipError_t launch_rope_shift(int d, bool bf16, const RopeArgs &args, int n_items, hipStream_t stream);
hipError_t launch_quantize_q8(int d, const Q8Args &v_args, int n_v, const Q8Args &k_args, int n_k,
                              hipStream_t stream);
hipError_t launch_decode_q8(int d, const DecodeArgs &args, int n_items, int n_pairs, hipStream_t stream);
}  // namespace crkv

using namespace crkv;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(e == hipErrorOutOfMemory ? CRKV_E_NOMEM : CRKV_E_HIP, "%s: %s", what,
                hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------ plan upload ring
// A call's plan tables are written into the pinned host half of a ring slot
// and copied to the slot's device half on a copy stream the library owns per
// device; the caller's stream waits for that copy on an event. The copy
// therefore runs while earlier work on the caller's stream still executes
// (an upload on the caller's stream itself was measured to leave a gap of
// tens of microseconds between kernels: the hand-off to the copy engine and
// back). A slot is reused only after the event recorded behind the work that
// read it has completed, so a slot in use is never overwritten. A slot also
// keeps a host copy of the bytes it last uploaded: a call whose tables are
// byte-for-byte the same (a repeated call on the same tensors) skips the
// copy and the wait, the slot's device half already holding them. The
// ring's mutex is held from plan_acquire to plan_release.
struct PlanRing {
    static constexpr int kSlots = 4;
    struct Slot {
        unsigned char *host = nullptr;
        unsigned char *dev = nullptr;
        size_t cap = 0;
        hipEvent_t copied = nullptr;
        hipEvent_t consumed = nullptr;
        bool pending = false;
        std::vector<unsigned char> shadow;   // the bytes of the last upload into `dev`
    };
    std::mutex mu;
    hipStream_t copy = nullptr;
    Slot slots[kSlots];
    int next = 0;
};

std::mutex g_rings_mu;
std::map<int, std::unique_ptr<PlanRing>> g_rings;

struct PlanLease {
    PlanRing *ring = nullptr;
    PlanRing::Slot *slot = nullptr;
    unsigned char *host = nullptr;   // write the tables here
    unsigned char *dev = nullptr;    // their device address
    bool committed = false;
};

// Takes the next ring slot with room for `bytes` of tables.
int plan_acquire(PlanLease &l, size_t bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    PlanRing *ring;
    {
        std::lock_guard<std::mutex> lk(g_rings_mu);
        auto &r = g_rings[dev];
        if (!r)
            r.reset(new PlanRing());
        ring = r.get();
    }
    ring->mu.lock();
    auto bail = [&](hipError_t err, const char *what) {
        ring->mu.unlock();
        return hip_fail(err, what);
    };
    if (!ring->copy) {
        e = hipStreamCreateWithFlags(&ring->copy, hipStreamNonBlocking);
        if (e != hipSuccess) {
            ring->copy = nullptr;
            return bail(e, "hipStreamCreate(plan copy)");
        }
    }
    PlanRing::Slot &s = ring->slots[ring->next];
    if (!s.copied) {
        e = hipEventCreateWithFlags(&s.copied, hipEventDisableTiming);
        if (e != hipSuccess) {
            s.copied = nullptr;
            return bail(e, "hipEventCreate(plan)");
        }
    }
    if (!s.consumed) {
        e = hipEventCreateWithFlags(&s.consumed, hipEventDisableTiming);
        if (e != hipSuccess) {
            s.consumed = nullptr;
            return bail(e, "hipEventCreate(plan)");
        }
    }
    if (s.pending) {
        e = hipEventSynchronize(s.consumed);
        if (e != hipSuccess)
            return bail(e, "hipEventSynchronize(plan slot)");
        s.pending = false;
    }
    if (s.cap < bytes) {
        if (s.host)
            (void)hipHostFree(s.host);
        if (s.dev)
            (void)hipFree(s.dev);
        s.host = nullptr;
        s.dev = nullptr;
        s.cap = 0;
        s.shadow.clear();
        const size_t cap = align_up(std::max<size_t>(bytes, 65536), 65536);
        e = hipHostMalloc(reinterpret_cast<void **>(&s.host), cap, hipHostMallocDefault);
        if (e != hipSuccess) {
            s.host = nullptr;
            return bail(e, "hipHostMalloc(plan)");
        }
        e = hipMalloc(reinterpret_cast<void **>(&s.dev), cap);
        if (e != hipSuccess) {
            s.dev = nullptr;
            return bail(e, "hipMalloc(plan)");
        }
        s.cap = cap;
    }
    ring->next = (ring->next + 1) % PlanRing::kSlots;
    l.ring = ring;
    l.slot = &s;
    l.host = s.host;
    l.dev = s.dev;
    l.committed = false;
    return CRKV_OK;
}

// Enqueues the copy of the slot's first `bytes` and makes `stream` wait for it.
int plan_commit(PlanLease &l, size_t bytes, hipStream_t stream)
{
    PlanRing::Slot &s = *l.slot;
    // The slot's last upload completed before the work that read it, which
    // plan_acquire waited for; identical bytes need no copy.
    if (s.shadow.size() == bytes && std::memcmp(s.shadow.data(), s.host, bytes) == 0) {
        l.committed = true;
        return CRKV_OK;
    }
    s.shadow.clear();
    hipError_t e = hipMemcpyAsync(s.dev, s.host, bytes, hipMemcpyHostToDevice, l.ring->copy);
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpyAsync(plan)");
    e = hipEventRecord(s.copied, l.ring->copy);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(stream, s.copied, 0);
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(l.ring->copy);
        return hip_fail(e, "plan copy ordering");
    }
    s.shadow.assign(s.host, s.host + bytes);
    l.committed = true;
    return CRKV_OK;
}

// Marks the slot busy until the work enqueued on `stream` so far has run.
void plan_release(PlanLease &l, hipStream_t stream)
{
    if (!l.ring)
        return;
    PlanRing::Slot &s = *l.slot;
    if (l.committed) {
        if (hipEventRecord(s.consumed, stream) == hipSuccess)
            s.pending = true;
        else
            (void)hipStreamSynchronize(stream);
    }
    l.ring->mu.unlock();
    l.ring = nullptr;
    l.slot = nullptr;
}

// ------------------------------------------------------------ scratch
// Without a caller workspace, a call uses one scratch buffer the library keeps
// per device (a per-call stream-ordered free was measured to block the host
// until the launched kernels finished, which serialises host preparation with
// the GPU). The buffer grows when a call needs more and lives until the
// process ends. Calls that share it are ordered on the device: a call on a
// different stream from the previous user waits on the event recorded behind
// that user's work. The mutex is held from scratch_get to scratch_release.
struct ScratchCache {
    std::mutex mu;
    void *ptr = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    hipStream_t last = nullptr;
    bool used = false;
};

std::mutex g_scratch_mu;
std::map<int, std::unique_ptr<ScratchCache>> g_scratch;

struct Scratch {
    void *ptr = nullptr;
    ScratchCache *cache = nullptr;   // non-null while the library buffer is held
};

int scratch_get(Scratch &sc, size_t bytes, const crkv_opts &o, hipStream_t stream)
{
    if (o.workspace) {
        if (o.workspace_bytes < bytes)
            return fail(CRKV_E_INVAL, "workspace too small: %zu bytes given, %zu needed",
                        o.workspace_bytes, bytes);
        if (reinterpret_cast<uintptr_t>(o.workspace) & 255u)
            return fail(CRKV_E_INVAL, "workspace must be 256-byte aligned");
        sc.ptr = o.workspace;
        sc.cache = nullptr;
        return CRKV_OK;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    ScratchCache *c;
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        auto &p = g_scratch[dev];
        if (!p)
            p.reset(new ScratchCache());
        c = p.get();
    }
    c->mu.lock();
    if (!c->ev) {
        e = hipEventCreateWithFlags(&c->ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            c->ev = nullptr;
            c->mu.unlock();
            return hip_fail(e, "hipEventCreate(scratch)");
        }
    }
    if (c->used && c->last != stream) {
        e = hipStreamWaitEvent(stream, c->ev, 0);
        if (e != hipSuccess) {
            c->mu.unlock();
            return hip_fail(e, "hipStreamWaitEvent(scratch)");
        }
    }
    if (c->cap < bytes) {
        if (c->ptr) {
            // the previous user's work must be done before the memory goes
            e = hipEventSynchronize(c->ev);
            if (e == hipSuccess)
                e = hipFree(c->ptr);
            c->ptr = nullptr;
            c->cap = 0;
            if (e != hipSuccess) {
                c->mu.unlock();
                return hip_fail(e, "hipFree(scratch)");
            }
        }
        const size_t cap = align_up(std::max<size_t>(bytes, 1), size_t(1) << 20);
        e = hipMalloc(&c->ptr, cap);
        if (e != hipSuccess) {
            c->ptr = nullptr;
            c->mu.unlock();
            return hip_fail(e, "hipMalloc(scratch)");
        }
        c->cap = cap;
    }
    sc.ptr = c->ptr;
    sc.cache = c;
    return CRKV_OK;
}

// Ends the call's use of the scratch: records the library buffer's event
// behind the work just enqueued on `stream` and lets the next call have it.
void scratch_release(Scratch &sc, hipStream_t stream)
{
    if (ScratchCache *c = sc.cache) {
        if (hipEventRecord(c->ev, stream) == hipSuccess) {
            c->last = stream;
            c->used = true;
        } else {
            // nothing to order against: make the next user wait for the device
            (void)hipDeviceSynchronize();
            c->used = false;
        }
        c->mu.unlock();
    }
    sc.ptr = nullptr;
    sc.cache = nullptr;
}

// ------------------------------------------------------------ validation
int check_opts(const crkv_opts &o)
{
    if (o.dtype != CRKV_F32 && o.dtype != CRKV_BF16)
        return fail(CRKV_E_INVAL, "opts.dtype %d is not CRKV_F32 or CRKV_BF16", o.dtype);
    if (o.mode < CRKV_IMPACT_QUERY_ROWS || o.mode > CRKV_IMPACT_ALL_ROWS)
        return fail(CRKV_E_INVAL, "opts.mode %d is not a crkv_mode", o.mode);
    if (o.deterministic != 0 && o.deterministic != 1)
        return fail(CRKV_E_INVAL, "opts.deterministic %d is not 0 or 1", o.deterministic);
    if (o.workspace && (reinterpret_cast<uintptr_t>(o.workspace) & 255u))
        return fail(CRKV_E_INVAL, "workspace must be 256-byte aligned");
    return CRKV_OK;
}

int check_problem(const crkv_problem &p, int idx, int H, int H_kv, int d, int mode, bool need_impact = true)
{
    if (!p.Q || !p.out || (need_impact && !p.impact))
        return fail(CRKV_E_INVAL, "problem %d: Q, out and impact must be non-null", idx);
    if (!p.chunk_K || !p.chunk_V || !p.chunk_len)
        return fail(CRKV_E_INVAL, "problem %d: chunk_K, chunk_V and chunk_len must be non-null", idx);
    if (p.m < 0)
        return fail(CRKV_E_INVAL, "problem %d: m = %d < 0", idx, p.m);
    if (p.q_len < 1)
        return fail(CRKV_E_INVAL, "problem %d: q_len = %d < 1", idx, p.q_len);
    if (p.chunk_len[p.m] < p.q_len)
        return fail(CRKV_E_INVAL, "problem %d: chunk_len[m] = %d is less than q_len = %d", idx,
                    p.chunk_len[p.m], p.q_len);
    int64_t n = 0;
    for (int c = 0; c <= p.m; ++c) {
        const int32_t len = p.chunk_len[c];
        if (len < 0)
            return fail(CRKV_E_INVAL, "problem %d: chunk_len[%d] = %d < 0", idx, c, len);
        if (len > 0 && (!p.chunk_K[c] || !p.chunk_V[c]))
            return fail(CRKV_E_INVAL, "problem %d: chunk %d has %d keys but a null K or V", idx, c, len);
        if (len > 0 && (!aligned16(p.chunk_K[c]) || !aligned16(p.chunk_V[c])))
            return fail(CRKV_E_INVAL, "problem %d: chunk %d K/V must be 16-byte aligned", idx, c);
        n += len;
    }
    if (n >= (int64_t)1 << 30)
        return fail(CRKV_E_UNSUPPORTED, "problem %d: %lld keys exceed 2^30", idx, (long long)n);
    const int64_t rows = mode == CRKV_IMPACT_QUERY_ROWS ? p.q_len : n;
    if (rows * (int64_t)H * d >= (int64_t)1 << 40 || rows * (int64_t)(H / H_kv) >= (int64_t)1 << 30)
        return fail(CRKV_E_UNSUPPORTED, "problem %d: too many rows", idx);
    if (!aligned16(p.Q) || !aligned16(p.out))
        return fail(CRKV_E_INVAL, "problem %d: Q and out must be 16-byte aligned", idx);
    if (need_impact && (reinterpret_cast<uintptr_t>(p.impact) & 3u))
        return fail(CRKV_E_INVAL, "problem %d: impact must be 4-byte aligned", idx);
    return CRKV_OK;
}

int check_shape(int n_problems, int H, int H_kv, int d)
{
    if (n_problems < 1)
        return fail(CRKV_E_INVAL, "n_problems = %d < 1", n_problems);
    if (H < 1 || H_kv < 1)
        return fail(CRKV_E_INVAL, "H = %d and H_kv = %d must be >= 1", H, H_kv);
    if (H % H_kv != 0)
        return fail(CRKV_E_INVAL, "H = %d is not a multiple of H_kv = %d", H, H_kv);
    if (d != 64 && d != 128)
        return fail(CRKV_E_UNSUPPORTED, "d = %d: only 64 and 128 are supported", d);
    return CRKV_OK;
}

// ------------------------------------------------------------ plan
struct Plan {
    std::vector<ProbDesc> probs;
    std::vector<SegDesc> segs;
    std::vector<KTile> tiles;
    std::vector<int32_t> slot_end;
    std::vector<ItemDesc> items;
    std::vector<OutCombItem> comb;   // row tiles of blocks split into key ranges
    std::vector<size_t> seg_base, tile_base, slot_base, partial_base;   // per problem
    size_t off_probs = 0, off_items = 0, off_segs = 0, off_tiles = 0, off_slots = 0, off_comb = 0;
    size_t table_bytes = 0;     // plan tables (uploaded through the ring)
    size_t scratch_bytes = 0;   // impact partials, pass-1 states, output partials (workspace or library scratch)
    size_t state_off = 0;       // byte offset of the pass-1 states in the scratch
    size_t opart_off = 0;       // byte offset of the output partials in the scratch
    bool lse_kernel = false;    // pass 1 runs as attn_lse_kernel (else inside pass 2's kernel)
    int cap_rows = 0;           // packed rows per block
    int max_keys = 0;
    int rt = 1;                 // row tiles per wave (wave kernel) or wave pair (pair kernel)
    int kernel = kBf16Wave;     // bf16 kernel of the launch
    int64_t model_cycles = 0;   // modelled duration of pass 2's kernel (the planner's cost model)
    int64_t work_cycles = 0;    // modelled work of its items, summed
    int split_blocks = 0, max_ranges = 1;
};

int64_t packed_rows(const crkv_problem &p, int G, int mode)
{
    int64_t n = 0;
    for (int c = 0; c <= p.m; ++c)
        n += p.chunk_len[c];
    return (int64_t)G * (mode == CRKV_IMPACT_QUERY_ROWS ? p.q_len : n);
}

int64_t step_cycles(int kernel, int rt)
{
    return kernel == kBf16Wave ? kWaveStepFixed + (int64_t)kWaveStepPerTile * rt
                               : kPairStepFixed + (int64_t)kPairStepPerTile * rt;
}

// The bf16 kernel and its row tiles per wave (or wave pair) for a launch.
// Every workgroup runs kWaves * rt row tiles per key tile whether or not they
// are all real rows; its cost per key step is modelled as fixed + per_tile * rt
// SIMD cycles (measured per kernel), and its key steps as the key tiles up to
// its last row. The choice minimises the modelled sum over all workgroups.
// CRKV_BF16_KERNEL (wave | pair) and CRKV_ROW_TILES force a built choice
// (tuning experiments and tests).
void choose_bf16(const crkv_problem *problems, int n_problems, int G, int mode, bool q8, int &kernel, int &rt)
{
    const char *ek = q8 ? "wave" : getenv("CRKV_BF16_KERNEL");   // 8-bit segments: the wave kernel's builds
    const char *er = getenv("CRKV_ROW_TILES");
    const int forced_rt = er ? atoi(er) : 0;
    int64_t best_cost = INT64_MAX;
    kernel = q8 ? kBf16Wave : kBf16Pair;
    rt = q8 ? kQ8RowTiles[0] : kPairRowTiles[0];
    for (int k = kBf16Wave; k <= kBf16Pair; ++k) {
        if (ek && strcmp(ek, k == kBf16Wave ? "wave" : "pair") != 0)
            continue;
        const int *choices = k == kBf16Wave ? kWaveRowTiles : kPairRowTiles;
        const int n_choices = k == kBf16Wave ? kNumWaveRowTiles : 3;
        for (int c = 0; c < n_choices; ++c) {
            const int r = choices[c];
            if (forced_rt && r != forced_rt)
                continue;
            if (q8 && r != kQ8RowTiles[0] && r != kQ8RowTiles[1])
                continue;
            if (k == kBf16Wave && mode == CRKV_IMPACT_CROSS_DOC && r > kWaveMaxRowTilesCross)
                continue;
            const int64_t cap = (int64_t)kWaves * r;
            int64_t steps = 0;
            for (int i = 0; i < n_problems; ++i) {
                const crkv_problem &p = problems[i];
                int64_t n_keys = 0;
                for (int j = 0; j <= p.m; ++j)
                    n_keys += p.chunk_len[j];
                const int64_t packed = packed_rows(p, G, mode);
                const int64_t nrt = (packed + kRowTile - 1) / kRowTile;
                const int64_t pos0 = mode == CRKV_IMPACT_QUERY_ROWS ? n_keys - p.q_len : 0;
                for (int64_t tb = 0; tb < nrt; tb += cap) {
                    const int64_t last_row = std::min(packed, (tb + cap) * kRowTile) - 1;
                    steps += (pos0 + last_row / G + kKeyTile) / kKeyTile;
                }
            }
            const int64_t cost = steps * step_cycles(k, r);
            if (cost <= best_cost) {   // ties go to the later (larger) build
                best_cost = cost;
                kernel = k;
                rt = r;
            }
        }
    }
}

// A row block before it is cut into key ranges: its item fields except the
// range ones, and every key tile its last row sees.
struct Block {
    ItemDesc it;
    int n_kt;
    int n_ranges = 1;
};
using Groups = std::vector<std::vector<Block>>;   // per (problem, KV head)

constexpr int kXcd = 8;                 // workgroup i runs on XCD i % 8
constexpr int kCUsPerXcd = kCUs / kXcd;
constexpr int64_t kItemOverheadSteps = 2;   // Q load, lse, epilogue of a workgroup, in key steps
constexpr int64_t kLaunchCycles = 8000;     // one more kernel in the stream (about 3.5 us)
constexpr int64_t kBytesPerCycle = 1800;    // HBM bytes per shader cycle, streaming (about 4 TB/s)

bool item_order_lpt()
{
    const char *e = getenv("CRKV_ITEM_ORDER");
    return !(e && strcmp(e, "group") == 0);
}

// Key tiles of range r of a block cut into n ranges of nearly equal length.
inline int range_begin(int n_kt, int n, int r) { return (int)((int64_t)r * n_kt / n); }

// Dispatch order: groups longest first, each to the XCD with the least
// modelled work so far, so that the row blocks (and key ranges) of one
// (problem, KV head) run on the same XCD and share their K/V reads through
// its L2; on each XCD the longest items first, so that its last items, which
// set when it finishes, are short (a group's items have nearly equal key
// counts and stay next to each other). The model: on each XCD the items start
// in that order on whichever of its CUs frees first (one workgroup per CU),
// each taking (key tiles + fixed part) steps of `step` cycles.
struct Dealer {
    bool lpt = true;   // false: each group's items together, its longest first (CRKV_ITEM_ORDER=group)
    std::vector<std::pair<int64_t, int>> order;   // (cost, group)
    std::vector<int> xcd;                         // per group
    std::vector<int32_t> n_kt[kXcd];              // per XCD: key tiles of its items
    std::vector<int64_t> cu;

    void assign(const Groups &groups, int64_t step)
    {
        order.clear();
        for (size_t g = 0; g < groups.size(); ++g) {
            int64_t c = 0;
            for (const Block &b : groups[g])
                c += (b.n_kt + kItemOverheadSteps * b.n_ranges) * step;
            order.emplace_back(c, (int)g);
        }
        std::stable_sort(order.begin(), order.end(),
                         [](const std::pair<int64_t, int> &x, const std::pair<int64_t, int> &y) {
                             return x.first > y.first;
                         });
        xcd.assign(groups.size(), 0);
        int64_t load[kXcd] = {};
        for (const auto &o : order) {
            const int x = (int)(std::min_element(load, load + kXcd) - load);
            xcd[o.second] = x;
            load[x] += o.first;
        }
    }

    // Modelled duration of the items.
    int64_t model(const Groups &groups, int64_t step)
    {
        assign(groups, step);
        for (auto &v : n_kt)
            v.clear();
        for (const auto &o : order) {
            auto &v = n_kt[xcd[o.second]];
            const size_t first = v.size();
            for (const Block &b : groups[o.second])
                for (int r = 0; r < b.n_ranges; ++r)
                    v.push_back(range_begin(b.n_kt, b.n_ranges, r + 1) - range_begin(b.n_kt, b.n_ranges, r));
            if (!lpt)
                std::sort(v.begin() + first, v.end(), std::greater<int32_t>());
        }
        int64_t makespan = 0;
        for (auto &v : n_kt) {
            if (lpt)
                std::sort(v.begin(), v.end(), std::greater<int32_t>());
            cu.assign(kCUsPerXcd, 0);   // min-heap of the CUs' free times
            for (int32_t n : v) {
                std::pop_heap(cu.begin(), cu.end(), std::greater<int64_t>());
                cu.back() += (n + kItemOverheadSteps) * step;
                makespan = std::max(makespan, cu.back());
                std::push_heap(cu.begin(), cu.end(), std::greater<int64_t>());
            }
        }
        return makespan;
    }

    // The work items in dispatch order (workgroup i runs on XCD i % 8).
    void emit(const Groups &groups, int64_t step, std::vector<ItemDesc> &out)
    {
        assign(groups, step);
        std::vector<std::vector<ItemDesc>> q(kXcd);
        auto longer = [](const ItemDesc &x, const ItemDesc &y) { return x.n_ktiles > y.n_ktiles; };
        for (const auto &o : order) {
            auto &v = q[xcd[o.second]];
            const size_t first = v.size();
            for (const Block &b : groups[o.second])
                for (int r = 0; r < b.n_ranges; ++r) {
                    ItemDesc it = b.it;
                    it.kt_begin = range_begin(b.n_kt, b.n_ranges, r);
                    it.n_ktiles = range_begin(b.n_kt, b.n_ranges, r + 1) - it.kt_begin;
                    it.range = r;
                    it.n_ranges = b.n_ranges;
                    v.push_back(it);
                }
            if (!lpt)
                std::stable_sort(v.begin() + first, v.end(), longer);
        }
        size_t depth = 0;
        for (auto &v : q) {
            if (lpt)
                std::stable_sort(v.begin(), v.end(), longer);
            depth = std::max(depth, v.size());
        }
        ItemDesc empty{};   // n_rowtiles = 0: the workgroup exits at once
        for (size_t d = 0; d < depth; ++d)
            for (int x = 0; x < kXcd; ++x)
                out.push_back(d < q[x].size() ? q[x][d] : empty);
        while (!out.empty() && out.back().n_rowtiles == 0)
            out.pop_back();
    }
};

// Cuts row blocks into key ranges where the modelled duration drops. A block
// of one (problem, KV head) otherwise streams all of its keys in one
// workgroup: a batch with few row blocks (one problem, short query) leaves
// most of the chip idle, and one with blocks of very different lengths
// (ragged requests) finishes on its longest ones. Candidates aim every item
// at 1/4 .. 4 times the per-CU share of the work; a block gets ceil(cost /
// aim) ranges of at least kMinRangeTiles key tiles, and the candidate with
// the least modelled duration wins (no split on ties). A split costs
// the fp32 output partials (written, then read by the combine), and one more
// kernel (the combine, plus pass 1 on its own for plans that would fuse it).
// CRKV_KEY_SPLIT = off, or a number of ranges for every block (tests).
void choose_ranges(Groups &groups, int64_t step, int cap_rows, int d, bool lse_kernel_anyway)
{
    const char *e = getenv("CRKV_KEY_SPLIT");
    if (e && strcmp(e, "off") == 0)
        return;
    if (e && atoi(e) > 0) {
        const int n = atoi(e);
        for (auto &g : groups)
            for (Block &b : g)
                b.n_ranges = std::max(1, std::min(n, b.n_kt));
        return;
    }
    // The choice depends only on the blocks' key tiles and row tiles, the
    // step cost, d and the pass-1 form: batches of one shape (every call of
    // a serving loop) reuse it.
    std::vector<int64_t> sig;
    sig.reserve(4 + 2 * groups.size() * (groups.empty() ? 0 : groups[0].size()));
    sig.push_back(step);
    sig.push_back(d);
    sig.push_back(lse_kernel_anyway + 2 * item_order_lpt());
    sig.push_back((int64_t)groups.size());
    for (auto &g : groups) {
        sig.push_back(-(int64_t)g.size());
        for (const Block &b : g)
            sig.push_back(((int64_t)b.n_kt << 20) | b.it.n_rowtiles);
    }
    static std::mutex memo_mu;
    static std::map<std::vector<int64_t>, std::vector<int>> memo;
    {
        std::lock_guard<std::mutex> lk(memo_mu);
        auto it = memo.find(sig);
        if (it != memo.end()) {
            size_t i = 0;
            for (auto &g : groups)
                for (Block &b : g)
                    b.n_ranges = it->second.empty() ? 1 : it->second[i++];
            return;
        }
    }
    auto remember = [&](const std::vector<int> &r) {
        std::lock_guard<std::mutex> lk(memo_mu);
        if (memo.size() >= 64)
            memo.clear();
        memo.emplace(std::move(sig), r);
    };
    static thread_local Dealer dealer;
    dealer.lpt = item_order_lpt();
    int64_t work = 0;
    for (auto &g : groups)
        for (const Block &b : g)
            work += (b.n_kt + kItemOverheadSteps) * step;
    int64_t best = dealer.model(groups, step);
    if (best * kCUs <= work + work / 32) {
        remember({});
        return;   // within 3 % of an even spread already: nothing for ranges to gain
    }
    std::vector<int> best_r;   // empty: no split
    int64_t last_aim = -1;
    for (int g8 : {2, 3, 4, 5, 6, 8, 10, 12, 16, 24, 32}) {   // aim = g8 / 8 of the per-CU share
        const int64_t aim = std::max<int64_t>(work * g8 / ((int64_t)kCUs * 8), (kMinRangeTiles + kItemOverheadSteps) * step);
        if (aim == last_aim)
            continue;
        last_aim = aim;
        int64_t opart_bytes = 0, cand_work = 0, cand_max = 0;
        std::vector<int> r;
        for (auto &g : groups)
            for (Block &b : g) {
                const int64_t cost = (b.n_kt + kItemOverheadSteps) * step;
                const int64_t want = (cost + aim - 1) / aim;
                b.n_ranges = (int)std::max<int64_t>(1, std::min<int64_t>(want, b.n_kt / kMinRangeTiles));
                if (b.n_ranges > 1)
                    opart_bytes += (int64_t)b.n_ranges * b.it.n_rowtiles * kRowTile * d * 4;
                cand_work += (b.n_kt + kItemOverheadSteps * b.n_ranges) * step;
                cand_max = std::max(cand_max, ((b.n_kt + b.n_ranges - 1) / b.n_ranges + kItemOverheadSteps) * step);
                r.push_back(b.n_ranges);
            }
        if (opart_bytes == 0 || opart_bytes > ((int64_t)1 << 32))   // offsets are int32 floats
            continue;
        const int64_t extra = 2 * opart_bytes / kBytesPerCycle + kLaunchCycles + (lse_kernel_anyway ? 0 : kLaunchCycles);
        if (std::max(cand_work / kCUs, cand_max) + extra >= best)
            continue;   // cannot win
        const int64_t t = dealer.model(groups, step) + extra;
        if (t < best) {
            best = t;
            best_r = std::move(r);
        }
    }
    size_t i = 0;
    for (auto &g : groups)
        for (Block &b : g)
            b.n_ranges = best_r.empty() ? 1 : best_r[i++];
    remember(best_r);
}

// Builds the plan for a validated batch (key_ranges = false: no block is cut
// into key ranges, whatever the model says).
void build_plan(Plan &pl, const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                const crkv_opts &o, bool key_ranges = true)
{
    const int G = H / H_kv;
    const bool q8 = o.dtype == CRKV_KV_Q8;
    const bool bf16 = o.dtype == CRKV_BF16 || q8;   // Q and out bf16
    if (bf16)
        choose_bf16(problems, n_problems, G, o.mode, q8, pl.kernel, pl.rt);
    else
        pl.rt = 1;
    const int cap = bf16 ? kWaves * pl.rt : 1;   // row tiles per workgroup
    pl.cap_rows = cap * kRowTile;
    Groups groups;
    size_t partial_floats = 0;
    pl.probs.resize(n_problems);
    {
        size_t n_tiles = 0, n_segs = 0;
        for (int pi = 0; pi < n_problems; ++pi) {
            n_segs += problems[pi].m + 1;
            for (int c = 0; c <= problems[pi].m; ++c)
                n_tiles += (problems[pi].chunk_len[c] + kKeyTile - 1) / kKeyTile;
        }
        pl.tiles.reserve(n_tiles);
        pl.segs.reserve(n_segs);
        groups.reserve((size_t)n_problems * H_kv);
    }
    for (int pi = 0; pi < n_problems; ++pi) {
        const crkv_problem &p = problems[pi];
        int32_t n_doc = 0;
        for (int c = 0; c < p.m; ++c)
            n_doc += p.chunk_len[c];
        const int32_t N = n_doc + p.chunk_len[p.m];
        const bool query = o.mode == CRKV_IMPACT_QUERY_ROWS;
        const int32_t rows = query ? p.q_len : N;
        const int32_t pos0 = query ? N - p.q_len : 0;   // query rows are the last q_len positions
        pl.seg_base.push_back(pl.segs.size());
        pl.tile_base.push_back(pl.tiles.size());
        int32_t start = 0;
        for (int c = 0; c <= p.m; ++c) {
            const int32_t len = p.chunk_len[c];
            pl.segs.push_back(SegDesc{p.chunk_K[c], p.chunk_V[c], len, start});
            const size_t esz = q8 ? 1 : o.dtype == CRKV_BF16 ? 2 : 4;   // 8-bit: code bytes
            for (int32_t t = 0; t < len; t += kKeyTile) {
                KTile kt;
                kt.K = static_cast<const unsigned char *>(p.chunk_K[c]) + (size_t)t * d * esz;
                kt.V = static_cast<const unsigned char *>(p.chunk_V[c]) + (size_t)t * d * esz;
                kt.n_valid = std::min(kKeyTile, len - t);
                kt.key0 = start + t;
                kt.seg_len = len;
                kt.seg_lo = start;
                pl.tiles.push_back(kt);
            }
            start += len;
        }
        const KTile *ptiles = pl.tiles.data() + pl.tile_base.back();
        const int n_tiles = (int)(pl.tiles.size() - pl.tile_base.back());
        const int64_t packed = (int64_t)G * rows;
        const int nrt = (int)((packed + kRowTile - 1) / kRowTile);
        const int nblk = (nrt + cap - 1) / cap;
        const int n_slots = H_kv * nblk;
        pl.slot_base.push_back(pl.slot_end.size());
        pl.slot_end.resize(pl.slot_end.size() + n_slots, 0);
        pl.partial_base.push_back(partial_floats);
        partial_floats += align_up((size_t)n_slots * N, 64);
        ProbDesc &pd = pl.probs[pi];
        memset(&pd, 0, sizeof pd);
        pd.n_tiles = n_tiles;
        pd.n_seg = p.m + 1;
        pd.n_doc = n_doc;
        pd.n_keys = N;
        pd.rows = rows;
        pd.pos0 = pos0;
        pd.n_slots = n_slots;
        pl.max_keys = std::max(pl.max_keys, (int)N);
        for (int kv = 0; kv < H_kv; ++kv) {
            std::vector<Block> g;
            for (int b = 0; b < nblk; ++b) {
                const int tb = b * cap;
                const int te = std::min(nrt, tb + cap);
                const int64_t last_row = std::min<int64_t>(packed, (int64_t)te * kRowTile) - 1;
                const int64_t key_end = pos0 + last_row / G + 1;
                const int n_kt = (int)(std::partition_point(ptiles, ptiles + n_tiles,
                                                            [&](const KTile &t) { return t.key0 < key_end; }) -
                                       ptiles);
                const int slot = kv * nblk + b;
                pl.slot_end[pl.slot_base.back() + slot] =
                    n_kt ? ptiles[n_kt - 1].key0 + ptiles[n_kt - 1].n_valid : 0;
                Block blk;
                memset(&blk.it, 0, sizeof blk.it);
                blk.it.prob = pi;
                blk.it.kv_head = kv;
                blk.it.tile_begin = tb;
                blk.it.n_rowtiles = te - tb;
                blk.it.slot = slot;
                blk.it.opart = -1;
                blk.n_kt = n_kt;
                g.push_back(blk);
            }
            groups.push_back(std::move(g));
        }
    }

    // Pass 1 on its own (attn_lse_kernel, two waves per SIMD) for the
    // one-wave kernel and for any plan with key ranges; the pair kernel
    // otherwise keeps it fused. CRKV_SWEEP1 = fused (no key ranges either) or
    // split forces a form.
    const char *es = getenv("CRKV_SWEEP1");
    const bool fused_only = es && strcmp(es, "fused") == 0;
    const bool split_anyway = es && strcmp(es, "split") == 0;
    const int64_t step = bf16 ? step_cycles(pl.kernel, pl.rt) : 1;
    const bool lse_anyway = bf16 && !fused_only && (pl.kernel == kBf16Wave || split_anyway);
    if (bf16 && !fused_only && key_ranges)
        choose_ranges(groups, step, pl.cap_rows, d, lse_anyway);
    bool any_split = false;
    for (auto &g : groups)
        for (Block &b : g)
            any_split |= b.n_ranges > 1;
    pl.lse_kernel = lse_anyway || any_split;

    // Per block: n_ranges pass-1 states of cap_rows rows; split blocks also
    // n_ranges fp32 output partials of cap_rows x d.
    int64_t state_f2 = 0, opart_f = 0;
    for (auto &g : groups)
        for (Block &b : g) {
            b.it.state = (int32_t)state_f2;
            if (pl.lse_kernel)
                state_f2 += (int64_t)b.n_ranges * pl.cap_rows;
            if (b.n_ranges > 1) {
                b.it.opart = (int32_t)opart_f;
                for (int t = 0; t < b.it.n_rowtiles; ++t) {
                    OutCombItem ci{};
                    ci.prob = b.it.prob;
                    ci.kv_head = b.it.kv_head;
                    ci.tile = b.it.tile_begin + t;
                    ci.n_ranges = b.n_ranges;
                    ci.opart = (int32_t)(opart_f + (int64_t)t * kRowTile * d);
                    pl.comb.push_back(ci);
                }
                opart_f += (int64_t)b.n_ranges * pl.cap_rows * d;
            }
        }
    {
        Dealer dealer;
        dealer.lpt = item_order_lpt();
        pl.model_cycles = dealer.model(groups, step);
        dealer.emit(groups, step, pl.items);
    }
    for (const ItemDesc &it : pl.items)
        if (it.n_rowtiles)
            pl.work_cycles += (it.n_ktiles + kItemOverheadSteps) * step;
    for (auto &g : groups)
        for (Block &b : g) {
            pl.split_blocks += b.n_ranges > 1;
            pl.max_ranges = std::max(pl.max_ranges, b.n_ranges);
        }

    pl.off_probs = 0;
    pl.off_items = align_up(pl.off_probs + pl.probs.size() * sizeof(ProbDesc), 256);
    pl.off_segs = align_up(pl.off_items + pl.items.size() * sizeof(ItemDesc), 256);
    pl.off_tiles = align_up(pl.off_segs + pl.segs.size() * sizeof(SegDesc), 256);
    pl.off_slots = align_up(pl.off_tiles + pl.tiles.size() * sizeof(KTile), 256);
    pl.off_comb = align_up(pl.off_slots + pl.slot_end.size() * sizeof(int32_t), 256);
    pl.table_bytes = align_up(pl.off_comb + pl.comb.size() * sizeof(OutCombItem), 256);
    size_t bytes = std::max<size_t>(partial_floats * sizeof(float), 256);
    pl.state_off = align_up(bytes, 256);
    bytes = pl.state_off + (size_t)state_f2 * 2 * sizeof(float);
    pl.opart_off = align_up(bytes, 256);
    pl.scratch_bytes = pl.opart_off + (size_t)opart_f * sizeof(float);
}

// Kernel arguments of a planned launch, tables at `dev`, scratch at `scratch`.
struct LaunchArgs {
    AttnArgs attn;
    CombineArgs comb;
    int n_items = 0, n_comb = 0;
    int dtype = CRKV_F32, kernel = kBf16Wave, rt = 1, d = 0;
};

LaunchArgs make_args(const Plan &pl, int H, int H_kv, int d, const crkv_opts &o, const unsigned char *dev,
                     void *scratch)
{
    LaunchArgs la{};
    AttnArgs &args = la.attn;
    args.probs = reinterpret_cast<const ProbDesc *>(dev + pl.off_probs);
    args.items = reinterpret_cast<const ItemDesc *>(dev + pl.off_items);
    args.H = H;
    args.H_kv = H_kv;
    args.G = H / H_kv;
    args.cross = o.mode == CRKV_IMPACT_CROSS_DOC ? 1 : 0;
    args.c_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    args.cap_rows = pl.cap_rows;
    unsigned char *sc = static_cast<unsigned char *>(scratch);
    if (pl.lse_kernel)
        args.state = reinterpret_cast<float *>(sc + pl.state_off);
    if (!pl.comb.empty())
        args.opart = reinterpret_cast<float *>(sc + pl.opart_off);
    la.comb.probs = args.probs;
    la.comb.items = reinterpret_cast<const OutCombItem *>(dev + pl.off_comb);
    la.comb.opart = args.opart;
    la.comb.G = args.G;
    la.comb.range_stride = pl.cap_rows * d;
    la.n_items = (int)pl.items.size();
    la.n_comb = (int)pl.comb.size();
    la.dtype = o.dtype;
    la.kernel = pl.kernel;
    la.rt = pl.rt;
    la.d = d;
    return la;
}

// The attention kernels of a launch: pass 1 on its own first when the plan
// runs it so, then the kernel the plan chose, then the sum of the output
// partials of blocks split into key ranges.
hipError_t launch_attn_kernels(const LaunchArgs &la, hipStream_t stream)
{
    const AttnArgs &args = la.attn;
    hipError_t e = hipSuccess;
    if (args.state)
        e = launch_attn_lse(la.d, la.dtype == CRKV_KV_Q8, args, la.n_items, stream);
    if (e == hipSuccess)
        e = la.dtype == CRKV_KV_Q8       ? launch_attn_q8(la.d, la.rt, args, la.n_items, stream)
            : la.dtype != CRKV_BF16      ? launch_attn_f32(la.d, args, la.n_items, stream)
            : la.kernel == kBf16Wave     ? launch_attn_bf16_wave(la.d, la.rt, args, la.n_items, stream)
                                         : launch_attn_bf16_pair(la.d, la.rt, args, la.n_items, stream);
    if (e == hipSuccess && la.n_comb)
        e = launch_attn_out_combine(la.d, la.comb, la.n_comb, stream);
    return e;
}

// Writes the plan tables (with device addresses inside `dev`, the tables'
// device copy, and `scratch`, the partials) into `host`.
void fill_tables(Plan &pl, const crkv_problem *problems, unsigned char *host, unsigned char *dev,
                 float *scratch)
{
    for (size_t pi = 0; pi < pl.probs.size(); ++pi) {
        ProbDesc &pd = pl.probs[pi];
        pd.Q = problems[pi].Q;
        pd.out = problems[pi].out;
        pd.impact = problems[pi].impact;
        pd.partial = scratch + pl.partial_base[pi];
        pd.tiles = reinterpret_cast<const KTile *>(dev + pl.off_tiles) + pl.tile_base[pi];
        pd.segs = reinterpret_cast<const SegDesc *>(dev + pl.off_segs) + pl.seg_base[pi];
        pd.slot_end = reinterpret_cast<const int32_t *>(dev + pl.off_slots) + pl.slot_base[pi];
    }
    memset(host, 0, pl.table_bytes);
    memcpy(host + pl.off_probs, pl.probs.data(), pl.probs.size() * sizeof(ProbDesc));
    memcpy(host + pl.off_items, pl.items.data(), pl.items.size() * sizeof(ItemDesc));
    memcpy(host + pl.off_segs, pl.segs.data(), pl.segs.size() * sizeof(SegDesc));
    memcpy(host + pl.off_tiles, pl.tiles.data(), pl.tiles.size() * sizeof(KTile));
    memcpy(host + pl.off_slots, pl.slot_end.data(), pl.slot_end.size() * sizeof(int32_t));
    memcpy(host + pl.off_comb, pl.comb.data(), pl.comb.size() * sizeof(OutCombItem));
}

crkv_opts resolve(const crkv_opts *opts)
{
    crkv_opts o;
    crkv_opts_init(&o);
    if (opts)
        o = *opts;
    return o;
}

int validate_batch(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                   const crkv_opts &o)
{
    // 8-bit segments (CRKV_KV_Q8) come with bf16 Q and out
    crkv_opts oc = o;
    if (oc.dtype == CRKV_KV_Q8)
        oc.dtype = CRKV_BF16;
    int rc = check_opts(oc);
    if (rc)
        return rc;
    rc = check_shape(n_problems, H, H_kv, d);
    if (rc)
        return rc;
    if (!problems)
        return fail(CRKV_E_INVAL, "problems must be non-null");
    for (int i = 0; i < n_problems; ++i) {
        rc = check_problem(problems[i], i, H, H_kv, d, o.mode);
        if (rc)
            return rc;
    }
    return CRKV_OK;
}

int check_topk_args(const float *impact, int n, int k, const int32_t *idx, int which)
{
    if (!impact || !idx)
        return fail(CRKV_E_INVAL, "top-k %d: impact and idx must be non-null", which);
    if (n < 1)
        return fail(CRKV_E_INVAL, "top-k %d: n = %d < 1", which, n);
    if (k < 1 || k > n)
        return fail(CRKV_E_INVAL, "top-k %d: k = %d outside [1, n = %d]", which, k, n);
    if (k > kTopkMaxK)
        return fail(CRKV_E_UNSUPPORTED, "top-k %d: k = %d exceeds %d", which, k, kTopkMaxK);
    if ((reinterpret_cast<uintptr_t>(impact) & 3u) || (reinterpret_cast<uintptr_t>(idx) & 3u))
        return fail(CRKV_E_INVAL, "top-k %d: impact and idx must be 4-byte aligned", which);
    return CRKV_OK;
}

// Enqueues the attention kernels the plan chose and the impact combine, with
// the plan's tables at `dev` (device copy already enqueued on `stream`) and
// its scratch at `scratch`.
hipError_t launch_planned(const Plan &pl, int n_problems, int H, int H_kv, int d, const crkv_opts &o,
                          const unsigned char *dev, void *scratch, hipStream_t stream)
{
    const LaunchArgs la = make_args(pl, H, H_kv, d, o, dev, scratch);
    hipError_t e = hipSuccess;
    if (o.timing_events[0])
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[0]), stream);
    if (e == hipSuccess)
        e = launch_attn_kernels(la, stream);
    if (e == hipSuccess && o.timing_events[1])
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[1]), stream);
    if (e == hipSuccess)
        e = launch_combine(la.attn.probs, n_problems, pl.max_keys, stream);
    return e;
}

// ------------------------------------------------------------ static scratch
// Device memory for crkv_attn_chunks_batched_static, the entry point for
// callers that cannot allocate: a file-scope array each device holds once the
// library's code is loaded on it, until the process ends. In host code the
// array's name is only a stand-in, so its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and kept; host
// code passes that address, never the name, to kernels and copies. Every call
// on a device shares the one array and leaves its contents behind; calls that
// overlap on one device (different streams, or threads) race.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

std::mutex g_static_mu;
std::map<int, unsigned char *> g_static_ptr;

int static_scratch(unsigned char **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_static_mu);
    auto it = g_static_ptr.find(dev);
    if (it == g_static_ptr.end()) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        it = g_static_ptr.emplace(dev, static_cast<unsigned char *>(ptr)).first;
    }
    *out = it->second;
    return CRKV_OK;
}

}  // namespace

// ================================================================== C ABI

// ------------------------------------------------------------ decode plan
// Workgroups the split of a decode launch aims for: two per CU of MI355X
// (the split kernel's occupancy), i.e. one round; measured best among
// 256 .. 8192 on the 32-layer decode workload (more rounds add merge work and
// a partial last round).
constexpr int64_t kDecodeTargetItems = 2 * 256;

struct DecodePlan {
    std::vector<ProbDesc> probs;
    std::vector<KTile> tiles;
    std::vector<DecodeItem> items;
    std::vector<DecodePair> pairs;
    std::vector<size_t> tile_base;   // per problem
    size_t off_probs = 0, off_items = 0, off_pairs = 0, off_tiles = 0;
    size_t table_bytes = 0;     // plan tables (uploaded through the ring)
    size_t scratch_bytes = 0;   // per-range partials (workspace or library scratch)
    int split = 0;   // key tiles per range
};

int validate_decode(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                    const crkv_opts &o)
{
    if (o.dtype != CRKV_BF16 && o.dtype != CRKV_KV_Q8)
        return fail(CRKV_E_UNSUPPORTED, "decode: opts.dtype %d (only CRKV_BF16 and CRKV_KV_Q8)", o.dtype);
    crkv_opts ob = o;   // the remaining options are checked as for bf16
    ob.dtype = CRKV_BF16;
    int rc = check_opts(ob);
    if (rc)
        return rc;
    rc = check_shape(n_problems, H, H_kv, d);
    if (rc)
        return rc;
    if (H / H_kv > kDecodeMaxGroup)
        return fail(CRKV_E_UNSUPPORTED, "decode: H / H_kv = %d query heads per KV head exceed %d",
                    H / H_kv, kDecodeMaxGroup);
    if (!problems)
        return fail(CRKV_E_INVAL, "problems must be non-null");
    for (int i = 0; i < n_problems; ++i) {
        if (problems[i].q_len != 1)
            return fail(CRKV_E_INVAL, "decode problem %d: q_len = %d, must be 1", i, problems[i].q_len);
        rc = check_problem(problems[i], i, H, H_kv, d, CRKV_IMPACT_QUERY_ROWS, false);
        if (rc)
            return rc;
    }
    return CRKV_OK;
}

// Key tiles of a problem (never straddling a segment) appended to `tiles`.
void append_tiles(std::vector<KTile> &tiles, const crkv_problem &p, int d, size_t esz)
{
    int32_t start = 0;
    for (int c = 0; c <= p.m; ++c) {
        const int32_t len = p.chunk_len[c];
        for (int32_t t = 0; t < len; t += kKeyTile) {
            KTile kt;
            kt.K = static_cast<const unsigned char *>(p.chunk_K[c]) + (size_t)t * d * esz;
            kt.V = static_cast<const unsigned char *>(p.chunk_V[c]) + (size_t)t * d * esz;
            kt.n_valid = std::min(kKeyTile, len - t);
            kt.key0 = start + t;
            kt.seg_len = len;
            kt.seg_lo = start;
            tiles.push_back(kt);
        }
        start += len;
    }
}

// Splits every (problem, KV head) into ranges of `split` key tiles, with
// `split` chosen so that the launch has about kDecodeTargetItems workgroups
// (a multiple of the split kernel's 4 waves, at least 4 tiles, at most 256).
void build_decode_plan(DecodePlan &pl, const crkv_problem *problems, int n_problems, int H, int H_kv,
                       int d, size_t esz)
{
    const int G = H / H_kv;
    int64_t all_tiles = 0;
    pl.probs.resize(n_problems);
    for (int pi = 0; pi < n_problems; ++pi) {
        pl.tile_base.push_back(pl.tiles.size());
        append_tiles(pl.tiles, problems[pi], d, esz);
        all_tiles += (int64_t)(pl.tiles.size() - pl.tile_base.back()) * H_kv;
    }
    int64_t split = (all_tiles + kDecodeTargetItems - 1) / kDecodeTargetItems;
    split = std::min<int64_t>(256, std::max<int64_t>(kDecodeWaves, split));
    split = (split + kDecodeWaves - 1) / kDecodeWaves * kDecodeWaves;
    pl.split = (int)split;
    for (int pi = 0; pi < n_problems; ++pi) {
        const crkv_problem &p = problems[pi];
        const int n_tiles = (int)((pi + 1 < n_problems ? pl.tile_base[pi + 1] : pl.tiles.size()) - pl.tile_base[pi]);
        int32_t n_keys = 0;
        for (int c = 0; c <= p.m; ++c)
            n_keys += p.chunk_len[c];
        ProbDesc &pd = pl.probs[pi];
        memset(&pd, 0, sizeof pd);
        pd.n_tiles = n_tiles;
        pd.n_seg = p.m + 1;
        pd.n_keys = n_keys;
        pd.rows = 1;
        pd.pos0 = n_keys - 1;
        for (int kv = 0; kv < H_kv; ++kv) {
            DecodePair pp{pi, kv, (int32_t)pl.items.size(), 0};
            for (int tb = 0; tb < n_tiles; tb += pl.split) {
                DecodeItem it{};
                it.prob = pi;
                it.kv_head = kv;
                it.tile_begin = tb;
                it.n_tiles = std::min(pl.split, n_tiles - tb);
                it.part = (int32_t)pl.items.size();
                pl.items.push_back(it);
                ++pp.n_parts;
            }
            pl.pairs.push_back(pp);
        }
    }
    pl.off_probs = 0;
    pl.off_items = align_up(pl.off_probs + pl.probs.size() * sizeof(ProbDesc), 256);
    pl.off_pairs = align_up(pl.off_items + pl.items.size() * sizeof(DecodeItem), 256);
    pl.off_tiles = align_up(pl.off_pairs + pl.pairs.size() * sizeof(DecodePair), 256);
    pl.table_bytes = align_up(pl.off_tiles + pl.tiles.size() * sizeof(KTile), 256);
    pl.scratch_bytes = std::max<size_t>(pl.items.size() * (size_t)G * (2 + d) * sizeof(float), 256);
    (void)H;
}

// ------------------------------------------------------------ selected-key K/V gather / scatter
int validate_sel(const crkv_kv_select *sel, int n, int H_kv, int d, const crkv_opts &o)
{
    int rc = check_opts(o);
    if (rc)
        return rc;
    if (n < 1 || !sel)
        return fail(CRKV_E_INVAL, "n = %d selections (need >= 1, non-null array)", n);
    if (H_kv < 1)
        return fail(CRKV_E_INVAL, "H_kv = %d < 1", H_kv);
    if (d != 64 && d != 128)
        return fail(CRKV_E_UNSUPPORTED, "d = %d: only 64 and 128 are supported", d);
    for (int p = 0; p < n; ++p) {
        const crkv_kv_select &q = sel[p];
        if (q.m < 0)
            return fail(CRKV_E_INVAL, "selection %d: m = %d < 0", p, q.m);
        if (!q.chunk_K || !q.chunk_V || !q.chunk_len)
            return fail(CRKV_E_INVAL, "selection %d: chunk_K, chunk_V and chunk_len must be non-null", p);
        if (q.k < 0)
            return fail(CRKV_E_INVAL, "selection %d: k = %d < 0", p, q.k);
        if (q.k > 0 && (!q.idx || !q.K_sel || !q.V_sel))
            return fail(CRKV_E_INVAL, "selection %d: idx, K_sel and V_sel must be non-null", p);
        if (q.k > 0 && (!aligned16(q.K_sel) || !aligned16(q.V_sel)))
            return fail(CRKV_E_INVAL, "selection %d: K_sel and V_sel must be 16-byte aligned", p);
        int64_t total = 0;
        for (int c = 0; c <= q.m; ++c) {
            const int32_t len = q.chunk_len[c];
            if (len < 0)
                return fail(CRKV_E_INVAL, "selection %d: chunk_len[%d] = %d < 0", p, c, len);
            if (len > 0 && (!q.chunk_K[c] || !q.chunk_V[c]))
                return fail(CRKV_E_INVAL, "selection %d: chunk %d has %d keys but a null K or V", p, c, len);
            if (len > 0 && (!aligned16(q.chunk_K[c]) || !aligned16(q.chunk_V[c])))
                return fail(CRKV_E_INVAL, "selection %d: chunk %d K/V must be 16-byte aligned", p, c);
            total += len;
        }
        if (total >= (int64_t(1) << 30))
            return fail(CRKV_E_UNSUPPORTED, "selection %d: %lld keys (limit 2^30)", p, (long long)total);
    }
    return CRKV_OK;
}

int run_sel(bool scatter, const crkv_kv_select *sel, int n, int H_kv, int d, const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    int rc = validate_sel(sel, n, H_kv, d, o);
    if (rc)
        return rc;
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    std::vector<SelProb> probs(n);
    std::vector<SelSeg> segs;
    std::vector<SelItem> items;
    std::vector<size_t> seg_base(n);
    for (int p = 0; p < n; ++p) {
        const crkv_kv_select &q = sel[p];
        seg_base[p] = segs.size();
        int32_t start = 0;
        for (int c = 0; c <= q.m; ++c) {
            SelSeg sg{};
            sg.K = q.chunk_K[c];
            sg.V = q.chunk_V[c];
            sg.start = start;
            sg.len = q.chunk_len[c];
            segs.push_back(sg);
            start += q.chunk_len[c];
        }
        SelProb &pr = probs[p];
        pr = SelProb{};
        pr.idx = q.idx;
        pr.K_sel = q.K_sel;
        pr.V_sel = q.V_sel;
        pr.n_seg = q.m + 1;
        pr.k = q.k;
        for (int j0 = 0; j0 < q.k; j0 += kSelKeysPerItem)
            items.push_back(SelItem{p, j0});
    }
    if (items.empty())
        return CRKV_OK;
    const size_t off_probs = 0;
    const size_t off_segs = align_up(probs.size() * sizeof(SelProb), 256);
    const size_t off_items = align_up(off_segs + segs.size() * sizeof(SelSeg), 256);
    const size_t bytes = align_up(off_items + items.size() * sizeof(SelItem), 256);
    PlanLease lease;
    rc = plan_acquire(lease, bytes);
    if (rc)
        return rc;
    for (int p = 0; p < n; ++p)
        probs[p].segs = reinterpret_cast<const SelSeg *>(lease.dev + off_segs) + seg_base[p];
    memset(lease.host, 0, bytes);
    memcpy(lease.host + off_probs, probs.data(), probs.size() * sizeof(SelProb));
    memcpy(lease.host + off_segs, segs.data(), segs.size() * sizeof(SelSeg));
    memcpy(lease.host + off_items, items.data(), items.size() * sizeof(SelItem));
    rc = plan_commit(lease, bytes, stream);
    hipError_t e = hipSuccess;
    if (rc == CRKV_OK) {
        SelArgs args{};
        args.probs = reinterpret_cast<const SelProb *>(lease.dev + off_probs);
        args.items = reinterpret_cast<const SelItem *>(lease.dev + off_items);
        args.H_kv = H_kv;
        args.row_bytes = d * (o.dtype == CRKV_BF16 ? 2 : 4);
        if (o.timing_events[0])
            e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[0]), stream);
        if (e == hipSuccess)
            e = launch_kvsel(scatter, args, (int)items.size(), stream);
        if (e == hipSuccess && o.timing_events[1])
            e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[1]), stream);
    }
    plan_release(lease, stream);
    if (rc)
        return rc;
    return e == hipSuccess ? CRKV_OK : hip_fail(e, scatter ? "scatter launch" : "gather launch");
}

// ------------------------------------------------------------ key re-positioning
int run_rope(const crkv_rope_seg *segs, int n, int H_kv, int d, double base, const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    int rc = check_opts(o);
    if (rc)
        return rc;
    if (n < 1 || !segs)
        return fail(CRKV_E_INVAL, "n = %d segments (need >= 1, non-null array)", n);
    if (H_kv < 1)
        return fail(CRKV_E_INVAL, "H_kv = %d < 1", H_kv);
    if (d != 64 && d != 128)
        return fail(CRKV_E_UNSUPPORTED, "d = %d: only 64 and 128 are supported", d);
    if (!(base > 1.0) || !std::isfinite(base))
        return fail(CRKV_E_INVAL, "base = %g must be finite and > 1", base);
    for (int i = 0; i < n; ++i) {
        if (segs[i].len < 0)
            return fail(CRKV_E_INVAL, "segment %d: len = %d < 0", i, segs[i].len);
        if ((int64_t)segs[i].len * H_kv >= (int64_t(1) << 31))
            return fail(CRKV_E_UNSUPPORTED, "segment %d: %lld rows (limit 2^31)", i,
                        (long long)segs[i].len * H_kv);
        if (segs[i].len > 0 && segs[i].delta != 0 && (!segs[i].K || !aligned16(segs[i].K)))
            return fail(CRKV_E_INVAL, "segment %d: K must be non-null and 16-byte aligned", i);
    }
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    const int half = d / 2;
    std::vector<double> theta(half);   // base^(-2j/d), in double
    for (int j = 0; j < half; ++j)
        theta[j] = std::pow(base, -2.0 * j / d);
    std::vector<RopeSeg> rs;
    std::vector<size_t> table_of;      // per RopeSeg: its cos/sin table
    std::vector<RopeItem> items;
    std::vector<float> cs;
    std::map<int, size_t> tables;      // one table per distinct shift
    for (int i = 0; i < n; ++i) {
        if (segs[i].len == 0 || segs[i].delta == 0)   // nothing moves
            continue;
        auto t = tables.find(segs[i].delta);
        if (t == tables.end()) {
            const size_t at = cs.size() / d;
            cs.resize(cs.size() + d);
            for (int j = 0; j < half; ++j) {   // angle delta * theta_j
                const double ang = (double)segs[i].delta * theta[j];
                cs[at * d + j] = (float)std::cos(ang);
                cs[at * d + half + j] = (float)std::sin(ang);
            }
            t = tables.emplace(segs[i].delta, at).first;
        }
        const int idx = (int)rs.size();
        RopeSeg r{};
        r.K = segs[i].K;
        r.rows = segs[i].len * H_kv;
        rs.push_back(r);
        table_of.push_back(t->second);
        for (int r0 = 0; r0 < r.rows; r0 += kRopeRowsPerItem)
            items.push_back(RopeItem{idx, r0});
    }
    if (items.empty())
        return CRKV_OK;
    const size_t off_segs = 0;
    const size_t off_items = align_up(rs.size() * sizeof(RopeSeg), 256);
    const size_t off_cs = align_up(off_items + items.size() * sizeof(RopeItem), 256);
    const size_t bytes = align_up(off_cs + cs.size() * sizeof(float), 256);
    PlanLease lease;
    rc = plan_acquire(lease, bytes);
    if (rc)
        return rc;
    for (size_t i = 0; i < rs.size(); ++i)
        rs[i].cs = reinterpret_cast<const float *>(lease.dev + off_cs) + table_of[i] * d;
    memset(lease.host, 0, bytes);
    memcpy(lease.host + off_segs, rs.data(), rs.size() * sizeof(RopeSeg));
    memcpy(lease.host + off_items, items.data(), items.size() * sizeof(RopeItem));
    memcpy(lease.host + off_cs, cs.data(), cs.size() * sizeof(float));
    rc = plan_commit(lease, bytes, stream);
    hipError_t e = hipSuccess;
    if (rc == CRKV_OK) {
        RopeArgs args{};
        args.segs = reinterpret_cast<const RopeSeg *>(lease.dev + off_segs);
        args.items = reinterpret_cast<const RopeItem *>(lease.dev + off_items);
        args.d = d;
        args.bf16 = o.dtype == CRKV_BF16;
        if (o.timing_events[0])
            e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[0]), stream);
        if (e == hipSuccess)
            e = launch_rope_shift(d, o.dtype == CRKV_BF16, args, (int)items.size(), stream);
        if (e == hipSuccess && o.timing_events[1])
            e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[1]), stream);
    }
    plan_release(lease, stream);
    if (rc)
        return rc;
    return e == hipSuccess ? CRKV_OK : hip_fail(e, "key re-positioning launch");
}

// ------------------------------------------------------------ prepared plans
// A batched attention (and top-k) call planned once: its tables, impact
// partials and top-k descriptors live in device memory owned by the plan, so
// a launch only enqueues kernels (capturable in a hipGraph).
struct crkv_plan {
    int device = 0;
    int n_problems = 0;
    int d = 0;
    int dtype = CRKV_F32;
    int max_keys = 0;
    LaunchArgs args{};
    unsigned char *tables = nullptr;          // device plan tables
    void *scratch = nullptr;                  // device impact partials
    bool own_scratch = false;
    std::vector<TopkDesc> topk;               // one per selecting problem (may be empty)
    TopkDesc *topk_dev = nullptr;             // the same, on the device, past kTopkInline
};

void plan_free(crkv_plan *p)
{
    if (!p)
        return;
    if (p->tables)
        (void)hipFree(p->tables);
    if (p->own_scratch && p->scratch)
        (void)hipFree(p->scratch);
    if (p->topk_dev)
        (void)hipFree(p->topk_dev);
    delete p;
}

int plan_create(const crkv_problem *problems, int n_problems, int H, int H_kv, int d, const int32_t *k,
                int32_t *const *idx, const crkv_opts *opts, crkv_plan **out)
{
    if (!out)
        return fail(CRKV_E_INVAL, "plan output pointer must be non-null");
    *out = nullptr;
    const crkv_opts o = resolve(opts);
    int rc = validate_batch(problems, n_problems, H, H_kv, d, o);
    if (rc)
        return rc;
    std::vector<TopkDesc> descs;
    if (k) {
        if (!idx)
            return fail(CRKV_E_INVAL, "k given without idx");
        for (int i = 0; i < n_problems; ++i) {
            int64_t n_doc = 0;
            for (int c = 0; c < problems[i].m; ++c)
                n_doc += problems[i].chunk_len[c];
            if (k[i] == 0)
                continue;   // this problem selects nothing
            rc = check_topk_args(problems[i].impact, (int)n_doc, k[i], idx[i], i);
            if (rc)
                return rc;
            descs.push_back(TopkDesc{problems[i].impact, idx[i], (int32_t)n_doc, k[i]});
        }
    }
    Plan pl;
    build_plan(pl, problems, n_problems, H, H_kv, d, o);
    if (o.workspace && o.workspace_bytes < pl.scratch_bytes)
        return fail(CRKV_E_INVAL, "workspace too small: %zu bytes given, %zu needed", o.workspace_bytes,
                    pl.scratch_bytes);
    std::unique_ptr<crkv_plan, void (*)(crkv_plan *)> p(new crkv_plan(), plan_free);
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    e = hipMalloc(reinterpret_cast<void **>(&p->tables), pl.table_bytes);
    if (e != hipSuccess) {
        p->tables = nullptr;
        return hip_fail(e, "hipMalloc(plan tables)");
    }
    if (o.workspace) {
        p->scratch = o.workspace;
    } else {
        e = hipMalloc(&p->scratch, pl.scratch_bytes);
        if (e != hipSuccess) {
            p->scratch = nullptr;
            return hip_fail(e, "hipMalloc(plan scratch)");
        }
        p->own_scratch = true;
    }
    std::vector<unsigned char> host(pl.table_bytes);
    fill_tables(pl, problems, host.data(), p->tables, static_cast<float *>(p->scratch));
    e = hipMemcpy(p->tables, host.data(), pl.table_bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpy(plan tables)");
    if (descs.size() > (size_t)kTopkInline) {
        e = hipMalloc(reinterpret_cast<void **>(&p->topk_dev), descs.size() * sizeof(TopkDesc));
        if (e != hipSuccess) {
            p->topk_dev = nullptr;
            return hip_fail(e, "hipMalloc(plan top-k)");
        }
        e = hipMemcpy(p->topk_dev, descs.data(), descs.size() * sizeof(TopkDesc), hipMemcpyHostToDevice);
        if (e != hipSuccess)
            return hip_fail(e, "hipMemcpy(plan top-k)");
    }
    p->n_problems = n_problems;
    p->d = d;
    p->dtype = o.dtype;
    p->max_keys = pl.max_keys;
    p->topk = std::move(descs);
    p->args = make_args(pl, H, H_kv, d, o, p->tables, p->scratch);
    *out = p.release();
    return CRKV_OK;
}

int plan_launch(const crkv_plan *p, void *stream_ptr, void *const *timing_events)
{
    if (!p)
        return fail(CRKV_E_INVAL, "plan must be non-null");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev != p->device)
        return fail(CRKV_E_INVAL, "plan was made on device %d, the current device is %d", p->device, dev);
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    if (timing_events && timing_events[0])
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(timing_events[0]), stream);
    if (e == hipSuccess)
        e = launch_attn_kernels(p->args, stream);
    if (e == hipSuccess && timing_events && timing_events[1])
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(timing_events[1]), stream);
    if (e == hipSuccess)
        e = launch_combine(p->args.attn.probs, p->n_problems, p->max_keys, stream);
    if (e == hipSuccess && !p->topk.empty()) {
        if (p->topk.size() == 1)
            e = launch_topk_one(p->topk[0], stream);
        else if (p->topk.size() <= (size_t)kTopkInline)
            e = launch_topk_inline(p->topk.data(), (int)p->topk.size(), stream);
        else
            e = launch_topk_batched(p->topk_dev, (int)p->topk.size(), stream);
    }
    return e == hipSuccess ? CRKV_OK : hip_fail(e, "plan launch");
}

// ------------------------------------------------------------ 8-bit segments
size_t q8_bytes(int H_kv, int len, int d, int kind)
{
    if (H_kv < 0 || len < 0 || (d != 64 && d != 128) || (kind != CRKV_Q8_K && kind != CRKV_Q8_V))
        return 0;
    if (len == 0)
        return 0;
    return (size_t)H_kv * len * d + (size_t)H_kv * (kind == CRKV_Q8_K ? d : len) * sizeof(float);
}

int run_quantize(const crkv_q8_seg *segs, int n, int H_kv, int d, const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    int rc = check_opts(o);
    if (rc)
        return rc;
    if (o.dtype != CRKV_BF16)
        return fail(CRKV_E_UNSUPPORTED, "quantize: the input must be CRKV_BF16");
    if (n < 1 || !segs)
        return fail(CRKV_E_INVAL, "n = %d segments (need >= 1, non-null array)", n);
    if (H_kv < 1)
        return fail(CRKV_E_INVAL, "H_kv = %d < 1", H_kv);
    if (d != 64 && d != 128)
        return fail(CRKV_E_UNSUPPORTED, "d = %d: only 64 and 128 are supported", d);
    for (int i = 0; i < n; ++i) {
        if (segs[i].len < 0)
            return fail(CRKV_E_INVAL, "segment %d: len = %d < 0", i, segs[i].len);
        if ((int64_t)segs[i].len * H_kv >= (int64_t(1) << 31))
            return fail(CRKV_E_UNSUPPORTED, "segment %d: %lld rows (limit 2^31)", i,
                        (long long)segs[i].len * H_kv);
        if (segs[i].kind != CRKV_Q8_K && segs[i].kind != CRKV_Q8_V)
            return fail(CRKV_E_INVAL, "segment %d: kind %d is not CRKV_Q8_K or CRKV_Q8_V", i, segs[i].kind);
        if (segs[i].len == 0)
            continue;
        if (!segs[i].x || !segs[i].q8 || !aligned16(segs[i].x) || !aligned16(segs[i].q8))
            return fail(CRKV_E_INVAL, "segment %d: x and q8 must be non-null and 16-byte aligned", i);
        const uintptr_t x0 = reinterpret_cast<uintptr_t>(segs[i].x);
        const uintptr_t q0 = reinterpret_cast<uintptr_t>(segs[i].q8);
        const size_t xb = (size_t)H_kv * segs[i].len * d * 2, qb = q8_bytes(H_kv, segs[i].len, d, segs[i].kind);
        if (x0 < q0 + qb && q0 < x0 + xb)
            return fail(CRKV_E_INVAL, "segment %d: q8 overlaps x", i);
    }
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    std::vector<Q8Seg> qs;
    std::vector<Q8Item> v_items, k_items;   // V: blocks of rows; K: one per (segment, KV head)
    for (int i = 0; i < n; ++i) {
        if (segs[i].len == 0)
            continue;
        Q8Seg q{};
        q.x = segs[i].x;
        q.q8 = segs[i].q8;
        q.rows = segs[i].len * H_kv;
        q.len = segs[i].len;
        const int idx = (int)qs.size();
        qs.push_back(q);
        if (segs[i].kind == CRKV_Q8_V) {
            for (int r0 = 0; r0 < q.rows; r0 += kQ8RowsPerItem)
                v_items.push_back(Q8Item{idx, r0});
        } else {
            for (int h = 0; h < H_kv; ++h)
                k_items.push_back(Q8Item{idx, h});
        }
    }
    if (qs.empty())
        return CRKV_OK;
    std::vector<Q8Item> items(v_items);
    items.insert(items.end(), k_items.begin(), k_items.end());
    const size_t off_items = align_up(qs.size() * sizeof(Q8Seg), 256);
    const size_t bytes = align_up(off_items + items.size() * sizeof(Q8Item), 256);
    PlanLease lease;
    rc = plan_acquire(lease, bytes);
    if (rc)
        return rc;
    memset(lease.host, 0, bytes);
    memcpy(lease.host, qs.data(), qs.size() * sizeof(Q8Seg));
    memcpy(lease.host + off_items, items.data(), items.size() * sizeof(Q8Item));
    rc = plan_commit(lease, bytes, stream);
    hipError_t e = hipSuccess;
    if (rc == CRKV_OK) {
        Q8Args va{}, ka{};
        va.segs = ka.segs = reinterpret_cast<const Q8Seg *>(lease.dev);
        va.items = reinterpret_cast<const Q8Item *>(lease.dev + off_items);
        ka.items = va.items + v_items.size();
        if (o.timing_events[0])
            e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[0]), stream);
        if (e == hipSuccess)
            e = launch_quantize_q8(d, va, (int)v_items.size(), ka, (int)k_items.size(), stream);
        if (e == hipSuccess && o.timing_events[1])
            e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[1]), stream);
    }
    plan_release(lease, stream);
    if (rc)
        return rc;
    return e == hipSuccess ? CRKV_OK : hip_fail(e, "quantize launch");
}

extern "C" {

int crkv_plan_create(const crkv_problem *problems, int n_problems, int H, int H_kv, int d, const int32_t *k,
                     int32_t *const *idx, const crkv_opts *opts, crkv_plan **plan)
{
    return plan_create(problems, n_problems, H, H_kv, d, k, idx, opts, plan);
}

int crkv_plan_launch(const crkv_plan *plan, void *stream, void *const *timing_events)
{
    return plan_launch(plan, stream, timing_events);
}

int crkv_plan_destroy(crkv_plan *plan)
{
    if (!plan)
        return CRKV_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    const bool other = e == hipSuccess && dev != plan->device;
    if (other)
        e = hipSetDevice(plan->device);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();   // no launch of the plan may still read its memory
    plan_free(plan);
    if (other)
        (void)hipSetDevice(dev);
    return e == hipSuccess ? CRKV_OK : hip_fail(e, "plan destroy");
}

size_t crkv_q8_bytes(int H_kv, int len, int d, int kind) { return q8_bytes(H_kv, len, d, kind); }

int crkv_quantize_q8(const crkv_q8_seg *segs, int n, int H_kv, int d, const crkv_opts *opts)
{
    return run_quantize(segs, n, H_kv, d, opts);
}

void crkv_opts_init(crkv_opts *opts)
{
    if (!opts)
        return;
    memset(opts, 0, sizeof *opts);
    opts->dtype = CRKV_F32;
    opts->mode = CRKV_IMPACT_QUERY_ROWS;
    opts->deterministic = 1;
}

int crkv_version(void) { return CRKV_VERSION; }

const char *crkv_last_error(void) { return g_last_error.c_str(); }

size_t crkv_decode_workspace_size(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                                  const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    if (validate_decode(problems, n_problems, H, H_kv, d, o) != CRKV_OK)
        return 0;
    DecodePlan pl;
    build_decode_plan(pl, problems, n_problems, H, H_kv, d, o.dtype == CRKV_KV_Q8 ? 1 : 2);
    return pl.scratch_bytes;
}

int crkv_decode_chunks_batched(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                               const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    int rc = validate_decode(problems, n_problems, H, H_kv, d, o);
    if (rc)
        return rc;
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    DecodePlan pl;
    const bool q8 = o.dtype == CRKV_KV_Q8;
    build_decode_plan(pl, problems, n_problems, H, H_kv, d, q8 ? 1 : 2);
    Scratch sc;
    rc = scratch_get(sc, pl.scratch_bytes, o, stream);
    if (rc)
        return rc;
    PlanLease lease;
    rc = plan_acquire(lease, pl.table_bytes);
    if (rc) {
        scratch_release(sc, stream);
        return rc;
    }
    unsigned char *dev = lease.dev;
    for (int pi = 0; pi < n_problems; ++pi) {
        ProbDesc &pd = pl.probs[pi];
        pd.Q = problems[pi].Q;
        pd.out = problems[pi].out;
        pd.tiles = reinterpret_cast<const KTile *>(dev + pl.off_tiles) + pl.tile_base[pi];
    }
    unsigned char *host = lease.host;
    memset(host, 0, pl.table_bytes);
    memcpy(host + pl.off_probs, pl.probs.data(), pl.probs.size() * sizeof(ProbDesc));
    memcpy(host + pl.off_items, pl.items.data(), pl.items.size() * sizeof(DecodeItem));
    memcpy(host + pl.off_pairs, pl.pairs.data(), pl.pairs.size() * sizeof(DecodePair));
    memcpy(host + pl.off_tiles, pl.tiles.data(), pl.tiles.size() * sizeof(KTile));
    rc = plan_commit(lease, pl.table_bytes, stream);
    if (rc) {
        plan_release(lease, stream);
        scratch_release(sc, stream);
        return rc;
    }
    DecodeArgs args{};
    args.probs = reinterpret_cast<const ProbDesc *>(dev + pl.off_probs);
    args.items = reinterpret_cast<const DecodeItem *>(dev + pl.off_items);
    args.pairs = reinterpret_cast<const DecodePair *>(dev + pl.off_pairs);
    args.part = static_cast<float *>(sc.ptr);
    args.G = H / H_kv;
    args.c_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    args.H_kv = H_kv;
    hipError_t e = hipSuccess;
    if (o.timing_events[0])
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[0]), stream);
    if (e == hipSuccess)
        e = q8 ? launch_decode_q8(d, args, (int)pl.items.size(), (int)pl.pairs.size(), stream)
               : launch_decode_bf16(d, args, (int)pl.items.size(), (int)pl.pairs.size(), stream);
    if (e == hipSuccess && o.timing_events[1])
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(o.timing_events[1]), stream);
    plan_release(lease, stream);
    scratch_release(sc, stream);
    if (e != hipSuccess)
        return hip_fail(e, "decode launch");
    return CRKV_OK;
}

const char *crkv_status_string(int status)
{
    switch (status) {
    case CRKV_OK: return "ok";
    case CRKV_E_INVAL: return "invalid argument";
    case CRKV_E_UNSUPPORTED: return "unsupported configuration";
    case CRKV_E_HIP: return "HIP runtime error";
    case CRKV_E_NOMEM: return "out of memory";
    default: return "unknown status";
    }
}

int64_t crkv_budget(int64_t n_doc, double r)
{
    if (n_doc < 0 || !(r >= 0.0 && r <= 1.0))
        return -1;
    const double x = std::floor(r * (double)n_doc);
    const int64_t k = (int64_t)x;
    return k < 1 ? 1 : k;
}

size_t crkv_workspace_size(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                           const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    if (validate_batch(problems, n_problems, H, H_kv, d, o) != CRKV_OK)
        return 0;
    Plan pl;
    build_plan(pl, problems, n_problems, H, H_kv, d, o);
    return pl.scratch_bytes;
}

int crkv_plan_info(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                   const crkv_opts *opts, int *kernel, int *row_tiles, int *workgroups)
{
    if (!kernel || !row_tiles || !workgroups)
        return fail(CRKV_E_INVAL, "crkv_plan_info: NULL output pointer");
    const crkv_opts o = resolve(opts);
    const int rc = validate_batch(problems, n_problems, H, H_kv, d, o);
    if (rc)
        return rc;
    Plan pl;
    build_plan(pl, problems, n_problems, H, H_kv, d, o);
    *kernel = (o.dtype != CRKV_BF16 && o.dtype != CRKV_KV_Q8) ? 0 : pl.kernel == kBf16Wave ? 1 : 2;
    *row_tiles = pl.rt;
    *workgroups = (int)pl.items.size();
    return CRKV_OK;
}

int crkv_plan_stats(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                    const crkv_opts *opts, crkv_plan_stat *st)
{
    if (!st)
        return fail(CRKV_E_INVAL, "crkv_plan_stats: NULL output pointer");
    const crkv_opts o = resolve(opts);
    const int rc = validate_batch(problems, n_problems, H, H_kv, d, o);
    if (rc)
        return rc;
    Plan pl;
    build_plan(pl, problems, n_problems, H, H_kv, d, o);
    memset(st, 0, sizeof *st);
    st->kernel = (o.dtype != CRKV_BF16 && o.dtype != CRKV_KV_Q8) ? 0 : pl.kernel == kBf16Wave ? 1 : 2;
    st->row_tiles = pl.rt;
    st->workgroups = (int)pl.items.size();
    st->pass1_separate = pl.lse_kernel ? 1 : 0;
    st->split_blocks = pl.split_blocks;
    st->max_ranges = pl.max_ranges;
    st->combine_workgroups = (int)pl.comb.size();
    st->model_cycles = (double)pl.model_cycles;
    st->work_cycles = (double)pl.work_cycles;
    st->scratch_bytes = pl.scratch_bytes;
    return CRKV_OK;
}

int crkv_attn_chunks_batched(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                             const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    int rc = validate_batch(problems, n_problems, H, H_kv, d, o);
    if (rc)
        return rc;
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    Plan pl;
    build_plan(pl, problems, n_problems, H, H_kv, d, o);

    Scratch sc;
    rc = scratch_get(sc, pl.scratch_bytes, o, stream);
    if (rc)
        return rc;
    PlanLease lease;
    rc = plan_acquire(lease, pl.table_bytes);
    if (rc) {
        scratch_release(sc, stream);
        return rc;
    }
    unsigned char *dev = lease.dev;
    fill_tables(pl, problems, lease.host, dev, static_cast<float *>(sc.ptr));
    rc = plan_commit(lease, pl.table_bytes, stream);
    if (rc) {
        plan_release(lease, stream);
        scratch_release(sc, stream);
        return rc;
    }
    const hipError_t e = launch_planned(pl, n_problems, H, H_kv, d, o, dev, sc.ptr, stream);
    plan_release(lease, stream);
    scratch_release(sc, stream);
    if (e != hipSuccess)
        return hip_fail(e, "attention launch");
    return CRKV_OK;
}

int crkv_attn_chunks_batched_static(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                                    const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    int rc = validate_batch(problems, n_problems, H, H_kv, d, o);
    if (rc)
        return rc;
    if (o.workspace)
        return fail(CRKV_E_INVAL, "crkv_attn_chunks_batched_static uses the library's static scratch: "
                                  "opts.workspace must be NULL (pass a workspace to crkv_attn_chunks_batched)");
    Plan pl;
    build_plan(pl, problems, n_problems, H, H_kv, d, o);
    // tables first, then the impact partials (and pass-1 states and output
    // partials), each 256-byte aligned; a plan with key ranges whose output
    // partials do not fit is made again without them
    size_t partial_off = align_up(pl.table_bytes, 256);
    if (partial_off + pl.scratch_bytes > kStaticScratchBytes && pl.split_blocks) {
        pl = Plan();
        build_plan(pl, problems, n_problems, H, H_kv, d, o, false);
        partial_off = align_up(pl.table_bytes, 256);
    }
    const size_t need = partial_off + pl.scratch_bytes;
    if (need > kStaticScratchBytes)
        return fail(CRKV_E_UNSUPPORTED,
                    "crkv_attn_chunks_batched_static: the call needs %zu bytes of scratch (tables %zu, impact "
                    "partials %zu), above the static scratch of %zu bytes",
                    need, pl.table_bytes, pl.scratch_bytes, kStaticScratchBytes);
    unsigned char *base = nullptr;
    rc = static_scratch(&base);
    if (rc)
        return rc;
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    std::vector<unsigned char> host(pl.table_bytes);
    fill_tables(pl, problems, host.data(), base, reinterpret_cast<float *>(base + partial_off));
    // from pageable memory: the call returns once `host` has been read
    hipError_t e = hipMemcpyAsync(base, host.data(), pl.table_bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpyAsync(static tables)");
    e = launch_planned(pl, n_problems, H, H_kv, d, o, base, base + partial_off, stream);
    if (e != hipSuccess)
        return hip_fail(e, "attention launch");
    return CRKV_OK;
}

size_t crkv_static_scratch_bytes(void) { return kStaticScratchBytes; }

int crkv_attn_chunks(const void *Q, const void *const *chunk_K, const void *const *chunk_V,
                     const int32_t *chunk_len, int m, int q_len, int H, int H_kv, int d, void *out,
                     float *impact, const crkv_opts *opts)
{
    crkv_problem p;
    p.Q = Q;
    p.chunk_K = chunk_K;
    p.chunk_V = chunk_V;
    p.chunk_len = chunk_len;
    p.m = m;
    p.q_len = q_len;
    p.out = out;
    p.impact = impact;
    return crkv_attn_chunks_batched(&p, 1, H, H_kv, d, opts);
}

int crkv_topk(const float *impact, int n, int k, int32_t *idx, const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    if (o.deterministic != 0 && o.deterministic != 1)
        return fail(CRKV_E_INVAL, "opts.deterministic %d is not 0 or 1", o.deterministic);
    int rc = check_topk_args(impact, n, k, idx, 0);
    if (rc)
        return rc;
    TopkDesc td{impact, idx, n, k};
    hipError_t e = launch_topk_one(td, reinterpret_cast<hipStream_t>(o.stream));
    if (e != hipSuccess)
        return hip_fail(e, "top-k launch");
    return CRKV_OK;
}

int crkv_topk_batched(const float *const *impact, const int32_t *n, const int32_t *k,
                      int32_t *const *idx, int n_problems, const crkv_opts *opts)
{
    const crkv_opts o = resolve(opts);
    if (o.deterministic != 0 && o.deterministic != 1)
        return fail(CRKV_E_INVAL, "opts.deterministic %d is not 0 or 1", o.deterministic);
    if (n_problems < 1)
        return fail(CRKV_E_INVAL, "n_problems = %d < 1", n_problems);
    if (!impact || !n || !k || !idx)
        return fail(CRKV_E_INVAL, "impact, n, k and idx arrays must be non-null");
    if (o.workspace && (reinterpret_cast<uintptr_t>(o.workspace) & 255u))
        return fail(CRKV_E_INVAL, "workspace must be 256-byte aligned");
    std::vector<TopkDesc> descs(n_problems);
    for (int i = 0; i < n_problems; ++i) {
        int rc = check_topk_args(impact[i], n[i], k[i], idx[i], i);
        if (rc)
            return rc;
        descs[i] = TopkDesc{impact[i], idx[i], n[i], k[i]};
    }
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    if (n_problems == 1) {
        hipError_t e = launch_topk_one(descs[0], stream);
        return e == hipSuccess ? CRKV_OK : hip_fail(e, "top-k launch");
    }
    if (n_problems <= kTopkInline) {   // descriptors travel as kernel arguments
        hipError_t e = launch_topk_inline(descs.data(), n_problems, stream);
        return e == hipSuccess ? CRKV_OK : hip_fail(e, "top-k launch");
    }
    const size_t bytes = descs.size() * sizeof(TopkDesc);
    PlanLease lease;
    int rc = plan_acquire(lease, bytes);
    if (rc)
        return rc;
    memcpy(lease.host, descs.data(), bytes);
    rc = plan_commit(lease, bytes, stream);
    hipError_t e = hipSuccess;
    if (rc == CRKV_OK)
        e = launch_topk_batched(reinterpret_cast<const TopkDesc *>(lease.dev), n_problems, stream);
    plan_release(lease, stream);
    if (rc)
        return rc;
    return e == hipSuccess ? CRKV_OK : hip_fail(e, "top-k launch");
}

int crkv_gather_kv(const crkv_kv_select *sel, int n, int H_kv, int d, const crkv_opts *opts)
{
    return run_sel(false, sel, n, H_kv, d, opts);
}

int crkv_scatter_kv(const crkv_kv_select *sel, int n, int H_kv, int d, const crkv_opts *opts)
{
    return run_sel(true, sel, n, H_kv, d, opts);
}

int crkv_rope_shift(const crkv_rope_seg *segs, int n, int H_kv, int d, double base, const crkv_opts *opts)
{
    return run_rope(segs, n, H_kv, d, base, opts);
}

}  // extern "C"
