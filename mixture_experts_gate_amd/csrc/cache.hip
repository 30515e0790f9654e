// Expert cache: device slots fed from pinned host memory by hipMemcpyAsync on
// a copy stream, a least-recently-used order over (layer, expert) keys, and a
// per-layer device table of moe_expert_w that the expert FFN reads.
//
// The pages' design keeps most experts in host memory and loads them on
// demand (winzheng.com page, "Why Now of All Times"), reuses frequently used
// experts through a global LRU expert cache and overlaps weight movement with
// computation by double-buffered full-layer streaming in prefill (winzheng.com
// page, "FreeToken's Three-Layer Mechanism"; aimodeling.com/en page, "Three
// Engineering Cores").
//
// Release protocol (what makes the overlap safe): every prefetch call is a
// generation g and records an event ev[g] on the compute stream at entry, so
// ev[g] covers all compute enqueued before call g. A slot last handed out by
// call g is read only by compute enqueued after call g and before call g+1,
// hence is free once ev[g+1] has completed. A miss reuses the least recently
// used slot not handed out by the current call; the copy stream waits on
// ev[last_gen + 1] of that slot before overwriting it. With room for two
// layers of experts, prefetching layer l+1 evicts layer l-1 and overlaps the
// compute of layer l.
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <deque>
#include <new>
#include <vector>

#include "common.hpp"

namespace moe {

// Test knobs (MOE_OPT_CACHE_FAULT, MOE_OPT_CACHE_DELAY_US): the n-th
// host-to-device copy of the cache from now fails without being issued; every
// prefetch with copies first holds its copy stream for this many microseconds
// (a host function that sleeps).
static std::atomic<long long> g_fault_at{0};     // remaining copies before the fault, 0 = off
static std::atomic<int> g_delay_us{0};
static std::atomic<int> g_throttle_mbs{0};       // MOE_OPT_CACHE_THROTTLE_MBS, 0 = off

int cache_set_fault(int n) {
    if (n < 0) return MOE_EINVAL;
    g_fault_at.store(n);
    return MOE_OK;
}
int cache_get_fault() { return (int)g_fault_at.load(); }
int cache_set_delay(int us) {
    if (us < 0 || us > 10000000) return MOE_EINVAL;
    g_delay_us.store(us);
    return MOE_OK;
}
int cache_get_delay() { return g_delay_us.load(); }
int cache_set_throttle(int mbs) {
    if (mbs < 0) return MOE_EINVAL;
    g_throttle_mbs.store(mbs);
    return MOE_OK;
}
int cache_get_throttle() { return g_throttle_mbs.load(); }

// True if this copy is the one the fault knob designates (counts it down).
static bool copy_fault_now() {
    long long v = g_fault_at.load();
    while (v > 0) {
        if (g_fault_at.compare_exchange_weak(v, v - 1)) return v == 1;
    }
    return false;
}

static void sleep_host_fn(void *arg) { usleep((useconds_t)(uintptr_t)arg); }

constexpr int kTableBatch = 240;

struct TableUpdate {
    int n;
    int key[kTableBatch];
    int slot[kTableBatch];
};

__global__ void cache_table_kernel(moe_expert_w *table, const char *pool, size_t slot_bytes,
                                   size_t o_w13, size_t o_s13, size_t o_w2, size_t o_s2,
                                   TableUpdate up) {
    for (int i = threadIdx.x; i < up.n; i += blockDim.x) {
        const char *b = pool + (size_t)up.slot[i] * slot_bytes;
        moe_expert_w w;
        w.w13 = b + o_w13;
        w.s13 = reinterpret_cast<const uint8_t *>(b + o_s13);
        w.w2 = b + o_w2;
        w.s2 = reinterpret_cast<const uint8_t *>(b + o_s2);
        table[up.key[i]] = w;
    }
}

// Slot moves of a resize, by value: move i copies slot src[i] of the old pool
// to slot dst[i] of the new one (sources and destinations never overlap).
constexpr int kMoveBatch = 240;
struct SlotMoves {
    int n;
    int src[kMoveBatch];
    int dst[kMoveBatch];
};

// grid (chunks per slot, moves): each workgroup copies 64 KB of one slot with
// 16-byte non-temporal loads and stores, 16 in flight per lane.
constexpr int kMoveChunk = 65536;
__global__ __launch_bounds__(256) void cache_move_kernel(const char *old_pool, char *new_pool,
                                                         size_t slot_bytes, SlotMoves mv) {
    const int i = blockIdx.y;
    const size_t base = (size_t)blockIdx.x * kMoveChunk;
    if (i >= mv.n || base >= slot_bytes) return;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(old_pool + (size_t)mv.src[i] * slot_bytes + base);
    u32x4 *dst = reinterpret_cast<u32x4 *>(new_pool + (size_t)mv.dst[i] * slot_bytes + base);
    const size_t left = slot_bytes - base;
    const int n16 = (int)((left < (size_t)kMoveChunk ? left : (size_t)kMoveChunk) / 16);
    constexpr int kUnroll = kMoveChunk / 16 / 256;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int j = u * 256 + (int)threadIdx.x;
        if (j < n16) v[u] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int j = u * 256 + (int)threadIdx.x;
        if (j < n16) __builtin_nontemporal_store(v[u], dst + j);
    }
}

}  // namespace moe

using namespace moe;

struct moe_cache {
    char *pool = nullptr;
    size_t slot_bytes = 0, expert_bytes = 0;
    int L = 0, E = 0, nslots = 0;
    size_t lay[4] = {0, 0, 0, 0};
    std::vector<const void *> src;      // [L*E] pinned host blobs
    hipStream_t copy_stream = nullptr;
    moe_expert_w *d_table = nullptr;    // [L*E]
    hipEvent_t ready = nullptr;

    std::vector<int> slot_of;           // key -> slot or -1
    std::vector<int> key_of;            // slot -> key or -1
    std::vector<int> prev, next;        // LRU list over slots; head = most recent
    int head = -1, tail = -1;
    std::vector<long long> last_gen;    // slot -> generation that last handed it out (0 = never)
    std::vector<long long> pick_gen;    // slot -> generation whose plan took it (scratch)
    long long gen = 0;
    std::deque<hipEvent_t> entry_ev;    // entry_ev[i] belongs to generation ev_front_gen + i
    long long ev_front_gen = 1;
    long long done_gen = 0;             // every generation <= done_gen has its entry event complete
    std::vector<hipEvent_t> spare_ev;

    long long hits = 0, misses = 0, h2d_bytes = 0;

    // Live host-to-device rate: timing events around each call's copies,
    // folded into an exponentially weighted mean once they have completed.
    struct Timed {
        hipEvent_t a, b;
        double bytes;
    };
    std::deque<Timed> timed;
    std::vector<hipEvent_t> spare_timing_ev;
    double bw_gbs = 0.0;
    long long bw_samples = 0;
    hipEvent_t timing_event() {
        if (!spare_timing_ev.empty()) {
            hipEvent_t e = spare_timing_ev.back();
            spare_timing_ev.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    void retire_timing() {
        while (!timed.empty() && hipEventQuery(timed.front().b) == hipSuccess) {
            const Timed t = timed.front();
            timed.pop_front();
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, t.a, t.b) == hipSuccess && ms > 0.0f) {
                const double r = t.bytes / (ms * 1e-3) / 1e9;
                bw_gbs = bw_samples ? 0.75 * bw_gbs + 0.25 * r : r;
                ++bw_samples;
            }
            spare_timing_ev.push_back(t.a);
            spare_timing_ev.push_back(t.b);
        }
    }

    void unlink(int s) {
        if (prev[s] >= 0) next[prev[s]] = next[s]; else head = next[s];
        if (next[s] >= 0) prev[next[s]] = prev[s]; else tail = prev[s];
        prev[s] = next[s] = -1;
    }
    void push_front(int s) {
        prev[s] = -1;
        next[s] = head;
        if (head >= 0) prev[head] = s;
        head = s;
        if (tail < 0) tail = s;
    }
    void push_back(int s) {
        next[s] = -1;
        prev[s] = tail;
        if (tail >= 0) next[tail] = s;
        tail = s;
        if (head < 0) head = s;
    }
    hipEvent_t get_event() {
        if (!spare_ev.empty()) {
            hipEvent_t e = spare_ev.back();
            spare_ev.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
        return e;
    }
    // Drop entry events that have completed, advancing done_gen.
    void retire_events() {
        while (!entry_ev.empty() && hipEventQuery(entry_ev.front()) == hipSuccess) {
            spare_ev.push_back(entry_ev.front());
            entry_ev.pop_front();
            done_gen = ev_front_gen;
            ++ev_front_gen;
        }
    }
};

extern "C" int expert_cache_reserve(moe_cache **cache, void *pool, size_t pool_bytes,
                                    size_t expert_bytes, int n_layers, int n_experts,
                                    const void *const *host_src, size_t lay_w13, size_t lay_s13,
                                    size_t lay_w2, size_t lay_s2, void *copy_stream) {
    if (!cache || !pool || !host_src || expert_bytes == 0 || n_layers < 1 || n_experts < 1)
        return MOE_EINVAL;
    if (lay_w13 >= expert_bytes || lay_w2 >= expert_bytes || lay_s13 > expert_bytes ||
        lay_s2 > expert_bytes)
        return MOE_EINVAL;
    const size_t slot_bytes = (expert_bytes + 255) & ~(size_t)255;
    const size_t nslots = pool_bytes / slot_bytes;
    if (nslots < (size_t)n_experts) return MOE_ENOMEM;
    if (nslots > 0x7FFFFFFF || (long long)n_layers * n_experts > 0x7FFFFFFF) return MOE_EINVAL;
    const long nkeys = (long)n_layers * n_experts;
    for (long i = 0; i < nkeys; ++i)
        if (!host_src[i]) return MOE_EINVAL;

    moe_cache *c = new (std::nothrow) moe_cache();
    if (!c) return MOE_ENOMEM;
    c->pool = reinterpret_cast<char *>(pool);
    c->slot_bytes = slot_bytes;
    c->expert_bytes = expert_bytes;
    c->L = n_layers;
    c->E = n_experts;
    c->nslots = (int)nslots;
    c->lay[0] = lay_w13;
    c->lay[1] = lay_s13;
    c->lay[2] = lay_w2;
    c->lay[3] = lay_s2;
    c->copy_stream = (hipStream_t)copy_stream;
    try {
        c->src.assign(host_src, host_src + nkeys);
        c->slot_of.assign(nkeys, -1);
        c->key_of.assign(nslots, -1);
        c->prev.assign(nslots, -1);
        c->next.assign(nslots, -1);
        c->last_gen.assign(nslots, 0);
        c->pick_gen.assign(nslots, 0);
    } catch (...) {
        delete c;
        return MOE_ENOMEM;
    }
    // free slots at the least recently used end, the lowest index taken first
    for (int s = c->nslots - 1; s >= 0; --s) c->push_back(s);
    int rc = check_hip(hipMalloc(&c->d_table, sizeof(moe_expert_w) * (size_t)nkeys));
    if (!rc) rc = check_hip(hipMemset(c->d_table, 0, sizeof(moe_expert_w) * (size_t)nkeys));
    if (!rc) rc = check_hip(hipEventCreateWithFlags(&c->ready, hipEventDisableTiming));
    if (rc) {
        if (c->d_table) (void)hipFree(c->d_table);
        delete c;
        return rc;
    }
    *cache = c;
    return MOE_OK;
}

extern "C" int expert_cache_prefetch(moe_cache *c, int layer, const int32_t *ids, int n,
                                     void *compute_stream, const moe_expert_w **table_out) {
    if (!c || layer < 0 || layer >= c->L || (ids && n < 0)) return MOE_EINVAL;
    const int E = c->E;
    std::vector<int> want;
    if (ids) {
        want.reserve(n);
        for (int i = 0; i < n; ++i) {
            if (ids[i] < 0 || ids[i] >= E) return MOE_EINVAL;
            want.push_back(ids[i]);
        }
        std::sort(want.begin(), want.end());
        want.erase(std::unique(want.begin(), want.end()), want.end());
    } else {
        want.resize(E);
        for (int e = 0; e < E; ++e) want[e] = e;
    }
    if ((int)want.size() > c->nslots) return MOE_ENOMEM;
    hipStream_t cs = (hipStream_t)compute_stream;

    // new generation: mark everything enqueued on the compute stream so far
    c->retire_events();
    hipEvent_t ev = c->get_event();
    if (!ev) return MOE_EHIP;
    int rc = check_hip(hipEventRecord(ev, cs));
    if (rc) {
        c->spare_ev.push_back(ev);
        return rc;
    }
    const long long g = ++c->gen;
    c->entry_ev.push_back(ev);      // generation g == ev_front_gen + index

    const long base_key = (long)layer * E;
    // Plan, without changing anything: the hits, and for each miss (ascending
    // expert) the least recently used slot that neither a hit nor an earlier
    // miss of this call takes.
    std::vector<int> hit_slot, miss, victim;
    for (int e : want) {
        const int s = c->slot_of[base_key + e];
        if (s >= 0) {
            hit_slot.push_back(s);
            c->pick_gen[s] = g;
        } else {
            miss.push_back(e);
        }
    }
    for (int s = c->tail; victim.size() < miss.size(); s = c->prev[s]) {
        while (s >= 0 && c->pick_gen[s] == g) s = c->prev[s];
        if (s < 0) return MOE_ENOMEM;    // cannot happen: want.size() <= nslots
        victim.push_back(s);
        c->pick_gen[s] = g;
    }
    // Issue the copies. A copy that cannot be enqueued ends the call: the
    // misses copied before it are committed below (their copies are in
    // flight), the rest of the call is not, so a failure at the first copy
    // leaves the cache, its table and its counters as they were.
    size_t issued = 0;
    c->retire_timing();
    hipEvent_t t_a = nullptr, t_b = nullptr;
    if (!miss.empty()) {
        t_a = c->timing_event();
        t_b = c->timing_event();
        if (t_a && t_b && hipEventRecord(t_a, c->copy_stream) != hipSuccess) {
            c->spare_timing_ev.push_back(t_a);
            c->spare_timing_ev.push_back(t_b);
            t_a = t_b = nullptr;
        }
        // test knobs: a fixed hold, or a hold that makes the link look slower
        long long hold_us = g_delay_us.load();
        const int thr = g_throttle_mbs.load();
        if (thr > 0) hold_us += (long long)((double)miss.size() * c->expert_bytes / thr);
        if (hold_us > 0) {
            rc = check_hip(hipLaunchHostFunc(c->copy_stream, sleep_host_fn,
                                             (void *)(uintptr_t)hold_us));
            if (rc) return rc;
        }
    }
    // A victim's readers are covered by the entry event of generation
    // last_gen + 1; the copy stream waits for it before the copy. A wait
    // covers every later copy on the stream and entry events complete in
    // generation order, so one wait per larger generation suffices.
    // Consecutive misses whose blobs sit back to back in host memory and whose
    // slots are adjacent go in one copy (a whole layer into the slots of the
    // layer before it is then a few large copies).
    long long waited = c->done_gen;
    while (issued < miss.size() && !rc) {
        size_t run = 1;
        while (issued + run < miss.size() &&
               victim[issued + run] == victim[issued + run - 1] + 1 &&
               miss[issued + run] == miss[issued + run - 1] + 1 &&
               (const char *)c->src[base_key + miss[issued + run]] ==
                   (const char *)c->src[base_key + miss[issued + run - 1]] + c->slot_bytes)
            ++run;
        long long need = 0;
        for (size_t i = issued; i < issued + run; ++i) {
            const long long lg = c->last_gen[victim[i]];
            if (lg > 0 && lg + 1 > need) need = lg + 1;
        }
        if (need > waited) {
            const long long idx = need - c->ev_front_gen;
            if (idx >= 0 && idx < (long long)c->entry_ev.size()) {
                rc = check_hip(hipStreamWaitEvent(c->copy_stream, c->entry_ev[(size_t)idx], 0));
                if (rc) break;
            }
            waited = need;
        }
        // the fault knob counts experts: a run stops short of the designated one
        size_t ok = 0;
        while (ok < run && !copy_fault_now()) ++ok;
        if (ok > 0) {
            rc = check_hip(hipMemcpyAsync(c->pool + (size_t)victim[issued] * c->slot_bytes,
                                          c->src[base_key + miss[issued]],
                                          (ok - 1) * c->slot_bytes + c->expert_bytes,
                                          hipMemcpyHostToDevice, c->copy_stream));
            if (rc) break;
            issued += ok;
        }
        if (ok < run) {
            set_last_hip_error(hipErrorUnknown);
            rc = MOE_EHIP;
        }
    }
    // Commit: hits (only when the whole call succeeded), then the issued misses.
    if (!rc) {
        for (int s : hit_slot) {
            ++c->hits;
            c->unlink(s);
            c->push_front(s);
            c->last_gen[s] = g;
        }
    }
    TableUpdate up;
    up.n = 0;
    int rc_table = MOE_OK;
    auto flush = [&]() {
        if (up.n == 0) return;
        MOE_LAUNCH(K_CACHE_TABLE, cache_table_kernel, dim3(1), dim3(256), 0, c->copy_stream,
                   c->d_table, (const char *)c->pool, c->slot_bytes, c->lay[0], c->lay[1],
                   c->lay[2], c->lay[3], up);
        up.n = 0;
        if (!rc_table) rc_table = check_launch();
    };
    for (size_t i = 0; i < issued; ++i) {
        const int s = victim[i], e = miss[i];
        const int old = c->key_of[s];
        if (old >= 0) c->slot_of[old] = -1;
        c->key_of[s] = (int)(base_key + e);
        c->slot_of[base_key + e] = s;
        c->unlink(s);
        c->push_front(s);
        c->last_gen[s] = g;
        ++c->misses;
        c->h2d_bytes += (long long)c->expert_bytes;
        up.key[up.n] = (int)(base_key + e);
        up.slot[up.n] = s;
        if (++up.n == kTableBatch) flush();
    }
    flush();
    if (!rc) rc = rc_table;
    if (t_a && t_b) {
        if (issued > 0 && hipEventRecord(t_b, c->copy_stream) == hipSuccess) {
            c->timed.push_back({t_a, t_b, (double)issued * (double)c->expert_bytes});
        } else {
            c->spare_timing_ev.push_back(t_a);
            c->spare_timing_ev.push_back(t_b);
        }
    }
    if (issued > 0 || !rc) {
        // the compute stream waits for whatever was enqueued on the copy stream
        const int rc2 = check_hip(hipEventRecord(c->ready, c->copy_stream));
        const int rc3 = rc2 ? rc2 : check_hip(hipStreamWaitEvent(cs, c->ready, 0));
        if (!rc) rc = rc3;
    }
    if (rc) return rc;
    if (table_out) *table_out = c->d_table + base_key;
    return MOE_OK;
}

// Elastic resize (the expert-cache half of re-allocating device memory between
// the expert cache and other uses at run time, aimodeling.com/en page, "Three
// Engineering Cores"; winzheng.com page, "FreeToken's Three-Layer Mechanism"):
// the most recently used residents that fit move to the new pool by
// device-to-device copies, the rest are dropped; nothing is read from the host.
// A kept resident keeps its slot index when it is below the new slot count;
// the others take the lowest free indices, most recent first. Free slots go
// to the least recently used end, the lowest index to be taken first.
extern "C" int expert_cache_resize(moe_cache *c, void *new_pool, size_t new_pool_bytes,
                                   void *compute_stream, int *moved) {
    if (!c || !new_pool) return MOE_EINVAL;
    const size_t n2 = new_pool_bytes / c->slot_bytes;
    if (n2 > 0x7FFFFFFF) return MOE_EINVAL;
    if (n2 < (size_t)c->E) return MOE_ENOMEM;
    char *np = reinterpret_cast<char *>(new_pool);
    const bool same = np == c->pool;
    if (!same) {
        const char *o0 = c->pool, *o1 = c->pool + (size_t)c->nslots * c->slot_bytes;
        const char *n0 = np, *n1 = np + n2 * c->slot_bytes;
        if (n0 < o1 && o0 < n1) return MOE_EINVAL;     // partial overlap
    }
    const int N2 = (int)n2;
    // residents from most to least recently used; keep the first N2
    std::vector<int> kept;
    for (int s = c->head; s >= 0; s = c->next[s])
        if (c->key_of[s] >= 0) kept.push_back(s);
    std::vector<int> drop;
    if ((int)kept.size() > N2) {
        drop.assign(kept.begin() + N2, kept.end());
        kept.resize(N2);
    }
    // new slot of every kept resident
    std::vector<char> used(N2, 0);
    for (int s : kept)
        if (s < N2) used[s] = 1;
    std::vector<int> dst(kept.size());
    int freep = 0;
    for (size_t i = 0; i < kept.size(); ++i) {
        const int s = kept[i];
        if (s < N2) {
            dst[i] = s;
        } else {
            while (used[freep]) ++freep;
            used[freep] = 1;
            dst[i] = freep;
        }
    }
    hipStream_t cs = (hipStream_t)compute_stream;
    // compute enqueued before this call may still read the old slots
    c->retire_events();
    hipEvent_t ev = c->get_event();
    if (!ev) return MOE_EHIP;
    int rc = check_hip(hipEventRecord(ev, cs));
    if (!rc) rc = check_hip(hipStreamWaitEvent(c->copy_stream, ev, 0));
    c->spare_ev.push_back(ev);      // reusable: the wait is enqueued
    if (rc) return rc;
    // dropped residents leave first: their slots may be copy destinations
    for (int s : drop) {
        c->slot_of[c->key_of[s]] = -1;
        c->key_of[s] = -1;
        c->unlink(s);
        c->push_back(s);
    }
    int nmoved = 0;
    SlotMoves mv;
    mv.n = 0;
    const unsigned chunks = (unsigned)((c->slot_bytes + kMoveChunk - 1) / kMoveChunk);
    for (size_t i = 0; i < kept.size(); ++i) {
        if (!(same && dst[i] == kept[i])) {
            mv.src[mv.n] = kept[i];
            mv.dst[mv.n] = dst[i];
            ++mv.n;
            ++nmoved;
        }
        if (mv.n > 0 && (mv.n == kMoveBatch || i + 1 == kept.size())) {
            MOE_LAUNCH(K_CACHE_MOVE, cache_move_kernel, dim3(chunks, (unsigned)mv.n), dim3(256), 0,
                       c->copy_stream, (const char *)c->pool, np, c->slot_bytes, mv);
            // on failure the cache stays on the old pool: sources are never destinations
            if ((rc = check_launch())) return rc;
            mv.n = 0;
        }
    }
    // metadata of the new pool
    std::vector<int> key2(N2, -1);
    for (size_t i = 0; i < kept.size(); ++i) key2[dst[i]] = c->key_of[kept[i]];
    c->pool = np;
    c->nslots = N2;
    c->key_of = key2;
    c->prev.assign(N2, -1);
    c->next.assign(N2, -1);
    c->last_gen.assign(N2, 0);
    c->pick_gen.assign(N2, 0);
    c->head = c->tail = -1;
    for (size_t i = 0; i < kept.size(); ++i) {
        c->slot_of[key2[dst[i]]] = dst[i];
        c->push_back(dst[i]);
    }
    for (int s = N2 - 1; s >= 0; --s)
        if (!used[s]) c->push_back(s);
    // table entries of the residents point into the new pool
    TableUpdate up;
    up.n = 0;
    for (size_t i = 0; i < kept.size(); ++i) {
        up.key[up.n] = key2[dst[i]];
        up.slot[up.n] = dst[i];
        if (++up.n == kTableBatch || i + 1 == kept.size()) {
            MOE_LAUNCH(K_CACHE_TABLE, cache_table_kernel, dim3(1), dim3(256), 0, c->copy_stream,
                       c->d_table, (const char *)c->pool, c->slot_bytes, c->lay[0], c->lay[1],
                       c->lay[2], c->lay[3], up);
            if ((rc = check_launch())) return rc;
            up.n = 0;
        }
    }
    rc = check_hip(hipEventRecord(c->ready, c->copy_stream));
    if (!rc) rc = check_hip(hipStreamWaitEvent(cs, c->ready, 0));
    if (rc) return rc;
    if (moved) *moved = nmoved;
    return MOE_OK;
}

extern "C" int expert_cache_evict(moe_cache *c, int layer, const int32_t *ids, int n) {
    if (!c || layer < 0 || layer >= c->L || (ids && n < 0)) return MOE_EINVAL;
    const long base_key = (long)layer * c->E;
    const int cnt = ids ? n : c->E;
    for (int i = 0; i < cnt; ++i) {
        const int e = ids ? ids[i] : i;
        if (e < 0 || e >= c->E) return MOE_EINVAL;
    }
    for (int i = 0; i < cnt; ++i) {
        const int e = ids ? ids[i] : i;
        const int s = c->slot_of[base_key + e];
        if (s < 0) continue;
        c->slot_of[base_key + e] = -1;
        c->key_of[s] = -1;
        c->unlink(s);
        c->push_back(s);     // first in line for reuse; last_gen keeps its readers safe
    }
    return MOE_OK;
}

extern "C" int expert_cache_stats(const moe_cache *c, long long *hits, long long *misses,
                                  long long *h2d_bytes) {
    if (!c) return MOE_EINVAL;
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (h2d_bytes) *h2d_bytes = c->h2d_bytes;
    return MOE_OK;
}

extern "C" int expert_cache_slots(const moe_cache *c) { return c ? c->nslots : MOE_EINVAL; }

extern "C" int expert_cache_slot_of(const moe_cache *c, int layer, int expert) {
    if (!c || layer < 0 || layer >= c->L || expert < 0 || expert >= c->E) return MOE_EINVAL;
    return c->slot_of[(long)layer * c->E + expert];
}

extern "C" int expert_cache_destroy(moe_cache *c) {
    if (!c) return MOE_EINVAL;
    int rc = check_hip(hipStreamSynchronize(c->copy_stream));
    for (hipEvent_t e : c->entry_ev) (void)hipEventSynchronize(e), (void)hipEventDestroy(e);
    for (hipEvent_t e : c->spare_ev) (void)hipEventDestroy(e);
    for (auto &t : c->timed) (void)hipEventSynchronize(t.b), (void)hipEventDestroy(t.a),
                                   (void)hipEventDestroy(t.b);
    for (hipEvent_t e : c->spare_timing_ev) (void)hipEventDestroy(e);
    if (c->ready) (void)hipEventDestroy(c->ready);
    if (c->d_table) {
        const int rc2 = check_hip(hipFree(c->d_table));
        if (!rc) rc = rc2;
    }
    delete c;
    return rc;
}

extern "C" int expert_cache_bandwidth(moe_cache *c, double *gbs, long long *samples) {
    if (!c) return MOE_EINVAL;
    c->retire_timing();
    if (gbs) *gbs = c->bw_gbs;
    if (samples) *samples = c->bw_samples;
    return MOE_OK;
}

// Bandwidth-adaptive placement (the pages' q* policy: the system keeps
// measuring the bandwidth it actually gets and decides per expert whether the
// GPU or the host CPU computes it; winzheng.com page, "FreeToken's Three-Layer
// Mechanism"; aimodeling.com/en page, "Three Engineering Cores"). A resident
// expert always stays on the GPU. A missing one costs expert_bytes / rate on
// the link, or host_s_per_expert + rows x host_s_per_row on the host (decoding
// its weights, then its rows), plus host_s_fixed once for using the host at
// all (reading the inputs back, sending the rows), and the two sides work at
// the same time; so misses move to the host, fewest rows first, while the
// host's summed time stays within the copy time still left to the link.
extern "C" int expert_cache_prefetch_qstar(moe_cache *c, int layer, const int32_t *ids,
                                           const int32_t *rows, int n, double host_s_fixed,
                                           double host_s_per_expert, double host_s_per_row,
                                           double link_gbs, void *compute_stream,
                                           const moe_expert_w **table_out, uint8_t *host_mask,
                                           int *n_host) {
    if (!c || layer < 0 || layer >= c->L || !ids || !rows || n < 0 || !host_mask ||
        host_s_fixed < 0.0 || host_s_per_row < 0.0 || host_s_per_expert < 0.0)
        return MOE_EINVAL;
    const int E = c->E;
    std::vector<long long> want_rows(E, 0);
    std::vector<char> wanted(E, 0);
    for (int i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= E || rows[i] < 0) return MOE_EINVAL;
        want_rows[ids[i]] += rows[i];
        wanted[ids[i]] = 1;
    }
    c->retire_timing();
    const double gbs = link_gbs > 0.0 ? link_gbs : c->bw_gbs;
    const long base_key = (long)layer * E;
    std::vector<int> host;
    if (gbs > 0.0) {
        std::vector<int> miss;
        for (int e = 0; e < E; ++e)
            if (wanted[e] && c->slot_of[base_key + e] < 0) miss.push_back(e);
        std::stable_sort(miss.begin(), miss.end(),
                         [&](int a, int b) { return want_rows[a] < want_rows[b]; });
        // moving one more miss leaves (misses - moved - 1) copies to the link
        const double t_copy = (double)c->expert_bytes / (gbs * 1e9);
        double host_t = host_s_fixed;     // paid once if any expert goes to the host
        for (int e : miss) {
            const double h = host_t + host_s_per_expert + (double)want_rows[e] * host_s_per_row;
            if (h > t_copy * (double)(miss.size() - host.size() - 1)) break;
            host_t = h;
            host.push_back(e);
        }
    }
    std::vector<int32_t> dev_ids(1, 0);    // (never empty: a NULL list means every expert)
    dev_ids.clear();
    std::vector<char> on_host(E, 0);
    for (int e : host) on_host[e] = 1;
    for (int e = 0; e < E; ++e)
        if (wanted[e] && !on_host[e]) dev_ids.push_back(e);
    const int32_t none = 0;
    const int rc = expert_cache_prefetch(c, layer, dev_ids.empty() ? &none : dev_ids.data(),
                                         (int)dev_ids.size(), compute_stream, table_out);
    if (rc) return rc;
    for (int e = 0; e < E; ++e) host_mask[e] = (uint8_t)on_host[e];
    if (n_host) *n_host = (int)host.size();
    return MOE_OK;
}
