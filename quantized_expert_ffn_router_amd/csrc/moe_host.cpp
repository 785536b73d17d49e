// moe_host.cpp -- host half of libmoe: errors, expert sizes, the repacker
// into the slot layout, and the expert slot-pool cache.
//
// Slot-pool cache (T4 MoE-cache report, kongchang.com, sections "What the
// MoE cache caches" and "Size your experts before configuring"): experts
// are grouped by (type, shape); each group owns one pool of fixed-size slots
// in HBM shared by all of its layers, so a hot expert of one layer can push
// out a cold expert of another; hits are read from HBM, misses are uploaded
// over PCIe; eviction is least-recently-used.  One hipMalloc per pool (one
// large allocation instead of one per tensor, as the GPU-offload research
// notes, kwkr.cn, section 3, recommend).  Uploads are hipMemcpyAsync from
// pinned host memory on a caller-given copy stream (pinned memory and
// asynchronous copies: laptop 16B MoE post, lpnh.cn, section 5.2).
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "moe_internal.h"

namespace moe {

static thread_local char g_err[512] = "no error";

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

namespace {

// Copy one canonical matrix [n, k] into tiles.
void repack_matrix(int qt, const uint8_t *src, int n, int k, uint8_t *dst)
{
    const int S = k / kTileCols;
    const size_t TB = (size_t)tile_bytes(qt);
    const size_t row_bytes = (size_t)(k / block_weights(qt)) * block_bytes(qt);
    for (int r = 0; r < n; r++) {
        const int rt = r / kTileRows, lt = r % kTileRows;
        const uint8_t *row = src + row_bytes * r;
        for (int s = 0; s < S; s++) {
            uint8_t *tile = dst + ((size_t)rt * S + s) * TB;
            if (qt == MOE_Q4_K) {
                const uint8_t *b = row + (size_t)s * 144;
                memcpy(tile + lt * 16, b, 16);  // d, dmin, scales[12]
                for (int j = 0; j < 8; j++) memcpy(tile + 1024 + j * 1024 + lt * 16, b + 16 + 16 * j, 16);
            } else if (qt == MOE_Q6_K) {
                const uint8_t *b = row + (size_t)s * 210;
                for (int j = 0; j < 8; j++) memcpy(tile + j * 1024 + lt * 16, b + 16 * j, 16);        // ql
                for (int j = 0; j < 4; j++) memcpy(tile + 8192 + j * 1024 + lt * 16, b + 128 + 16 * j, 16);  // qh
                memcpy(tile + 12288 + lt * 16, b + 192, 16);  // sc
                memcpy(tile + 13312 + lt * 2, b + 208, 2);    // d
            } else {
                for (int bb = 0; bb < 8; bb++) {
                    const uint8_t *b = row + (size_t)(8 * s + bb) * 34;
                    memcpy(tile + (2 * bb) * 1024 + lt * 16, b + 2, 16);
                    memcpy(tile + (2 * bb + 1) * 1024 + lt * 16, b + 18, 16);
                    memcpy(tile + 16384 + lt * 16 + bb * 2, b, 2);
                }
            }
        }
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_last_error(void) { return g_err; }

int64_t moe_expert_bytes(const moe_expert_desc *d)
{
    ExpertGeom g;
    if (!d || !geom(*d, &g)) return -1;
    return (int64_t)g.bytes;
}

int32_t moe_down_k(const moe_expert_desc *d)
{
    ExpertGeom g;
    if (!d || !geom(*d, &g)) return -1;
    return g.kd;
}

moe_status moe_repack_expert(const moe_expert_desc *d, const void *gate, const void *up, const void *down,
                             void *slot, size_t slot_bytes)
{
    ExpertGeom g;
    if (!d || !gate || !up || !down || !slot) { set_error("moe_repack_expert: null argument"); return MOE_ERR_ARG; }
    if (!qtype_ok(d->gate) || !qtype_ok(d->up) || !qtype_ok(d->down)) { set_error("moe_repack_expert: bad qtype"); return MOE_ERR_QTYPE; }
    if (!geom(*d, &g)) { set_error("moe_repack_expert: bad shape H=%d I=%d", d->H, d->I); return MOE_ERR_SHAPE; }
    if (slot_bytes < g.bytes) { set_error("moe_repack_expert: slot of %zu bytes < %zu", slot_bytes, g.bytes); return MOE_ERR_ARG; }
    uint8_t *dst = (uint8_t *)slot;
    repack_matrix(d->gate, (const uint8_t *)gate, d->I, d->H, dst + g.gate_off);
    repack_matrix(d->up, (const uint8_t *)up, d->I, d->H, dst + g.up_off);
    repack_matrix(d->down, (const uint8_t *)down, d->H, g.kd, dst + g.down_off);
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// slot-pool cache

moe_status moe_cache_plan(const moe_expert_desc *groups, const int32_t *layers_per_group, int32_t n_groups,
                          uint64_t budget_bytes, int32_t top_k, int32_t *slots_out)
{
    if (!groups || !layers_per_group || !slots_out || n_groups < 1 || top_k < 1) {
        set_error("moe_cache_plan: bad argument");
        return MOE_ERR_ARG;
    }
    unsigned __int128 denom = 0;
    for (int g = 0; g < n_groups; g++) {
        ExpertGeom eg;
        if (!geom(groups[g], &eg) || layers_per_group[g] < 1) {
            set_error("moe_cache_plan: bad group %d", g);
            return MOE_ERR_SHAPE;
        }
        denom += (unsigned __int128)eg.bytes * (uint64_t)layers_per_group[g];
    }
    bool any = false;
    for (int g = 0; g < n_groups; g++) {
        unsigned __int128 q = ((unsigned __int128)budget_bytes * (uint64_t)layers_per_group[g]) / denom;
        long long s = (long long)q - 1;
        if (s < top_k) s = 0;
        if (s > 0x7fffffff) s = 0x7fffffff;
        slots_out[g] = (int32_t)s;
        any = any || s > 0;
    }
    if (!any) {
        set_error("cache budget of %llu bytes leaves every group below %d slots", (unsigned long long)budget_bytes, top_k);
        return MOE_ERR_BUDGET;
    }
    return MOE_OK;
}

moe_status moe_placement_plan(const moe_expert_desc *groups, int32_t n_groups, const int32_t *layer_group,
                              int32_t n_layers, int32_t E, uint64_t vram_bytes, uint64_t cache_bytes,
                              int32_t top_k, int32_t mode, int32_t *layer_state, int32_t *slots_out)
{
    if (!groups || !layer_group || !layer_state || !slots_out || n_groups < 1 || n_layers < 1 || E < 1 || top_k < 1 ||
        (mode != MOE_PLACE_FIT && mode != MOE_PLACE_ALL_CACHED) || (mode == MOE_PLACE_FIT && cache_bytes > vram_bytes)) {
        set_error("moe_placement_plan: bad argument");
        return MOE_ERR_ARG;
    }
    std::vector<uint64_t> layer_bytes(n_layers);
    for (int l = 0; l < n_layers; l++) {
        ExpertGeom eg;
        const int g = layer_group[l];
        if (g < 0 || g >= n_groups || !geom(groups[g], &eg)) {
            set_error("moe_placement_plan: layer %d has a bad group", l);
            return MOE_ERR_ARG;
        }
        layer_bytes[l] = (uint64_t)eg.bytes * (uint64_t)E;
    }
    // resident layers first (FIT: whole layers, in layer order, first fit)
    uint64_t avail = mode == MOE_PLACE_FIT ? vram_bytes - cache_bytes : 0;
    const uint64_t pool = mode == MOE_PLACE_FIT ? cache_bytes : vram_bytes;
    std::vector<int32_t> cached(n_groups, 0);
    for (int l = 0; l < n_layers; l++) {
        const int g = layer_group[l];
        if (mode == MOE_PLACE_FIT && layer_bytes[l] <= avail) {
            avail -= layer_bytes[l];
            layer_state[l] = -(g + 1);
        } else {
            layer_state[l] = g;
            cached[g]++;
        }
    }
    // the cache's slots over the cached layers alone (the planner's formula)
    unsigned __int128 denom = 0;
    for (int g = 0; g < n_groups; g++) {
        ExpertGeom eg;
        geom(groups[g], &eg);
        denom += (unsigned __int128)eg.bytes * (uint64_t)cached[g];
    }
    int short_group = -1;
    for (int g = 0; g < n_groups; g++) {
        long long sl = 0;
        if (cached[g] > 0) {
            sl = (long long)(((unsigned __int128)pool * (uint64_t)cached[g]) / denom) - 1;
            if (sl < top_k) {
                sl = 0;
                short_group = g;
            }
            if (sl > 0x7fffffff) sl = 0x7fffffff;
        }
        slots_out[g] = (int32_t)sl;
    }
    if (short_group >= 0) {
        set_error("moe_placement_plan: a pool of %llu bytes leaves group %d (%d cached layers) below %d slots",
                  (unsigned long long)pool, short_group, cached[short_group], top_k);
        return MOE_ERR_BUDGET;
    }
    return MOE_OK;
}

}  // extern "C"

struct moe_cache {
    struct Group {
        moe_expert_desc desc;
        size_t slot_bytes = 0;
        int n_slots = 0;                // 0: below the budget floor, its layers resident
        uint8_t *pool = nullptr;        // the slots
        uint8_t *res = nullptr;         // the group's resident layers' experts, layer-major
        std::vector<int64_t> slot_key;  // key = layer*E + expert, -1 free
        std::vector<int> prev, next;    // recency list over slots, head = most recent
        int head = -1, tail = -1, next_free = 0;
    };
    // One decision of a host lookup, kept until the layer's upload so that a
    // failed upload can undo the lookup from a miss on (in reverse order).
    struct Op {
        int slot, old_prev;   // the slot, and its predecessor in the recency list before the decision
        int64_t key, victim;  // the key looked up; the key evicted, or -1
        uint8_t kind;         // 0 hit, 1 miss into a never-used slot, 2 miss with eviction
    };
    struct Pending { int slot; const void *src; int op; };
    int n_layers = 0, E = 0, device = 0;
    bool custom = false;                 // caller-supplied (synchronous) backend
    moe_cache_backend be{};
    std::vector<Group> groups;
    std::vector<int> layer_group;        // group of each layer (its shape, resident or not)
    std::vector<char> resident;          // the layer's experts stay resident, no lookups
    std::vector<int> layer_rank;         // position of a resident layer among its group's resident layers
    std::vector<const void *> host;      // [L*E] pinned sources
    std::vector<int> where;              // [L*E] slot of a key, -1 absent
    const void **htab = nullptr;         // host [L*E] slot addresses (pinned with the default backend)
    void **dtab = nullptr;               // device [L*E]
    std::vector<hipEvent_t> table_done;  // per layer: last copy of its table row
    std::vector<char> table_pending;     // that copy may still be reading htab
    std::vector<char> dirty;             // row changed since its last upload
    std::vector<std::vector<Pending>> pending;  // per layer: misses of its last lookup
    std::vector<std::vector<Op>> ops;           // per layer: decisions of its last lookup
    std::vector<int> lookup_T;
    std::vector<char> looked_up;
    int open_lookup = -1;                // layer whose lookup awaits its upload, -1 none
    moe_cache_stats_t st{};
    // device-side lookup (moe_cache_device_enable): the LRU state in device
    // memory, one stamp and key per slot per group
    bool dev = false;
    struct DevGroup { uint32_t *stamp = nullptr; int32_t *key = nullptr; };
    std::vector<DevGroup> dgroups;
    int32_t *d_where = nullptr;       // [L*E]
    const void **d_src = nullptr;     // [L*E] device addresses of the host copies
    int32_t *d_counters = nullptr;    // [n_groups] next_free, then clock, njobs, ntrace
    CacheJob *d_jobs = nullptr;       // [E]
    int32_t *d_jwait = nullptr;       // [E] moe_cache_ffn_device: each selected id's copy job + 1
    uint32_t *d_done = nullptr;       // [E] its jobs' completion counts
    unsigned long long *d_stats = nullptr;  // moe_cache_stats_t
    int32_t *d_trace = nullptr;
    // prefetch (moe_cache_prefetch_device): per layer a list of miss copies
    // run on the caller's copy stream and the event that ends them, and the
    // slot touches of the layer's group since the prefetch (-1: none pending)
    CacheJob *d_pjobs = nullptr;      // [L][E]
    int32_t *d_pnjobs = nullptr;      // [L]
    hipEvent_t ev_fork = nullptr;
    std::vector<hipEvent_t> ev_pref;  // [L]
    std::vector<int> pend_touch;      // [L]
    // per group: slot touches since (and including) its latest device lookup,
    // whose experts the FFN that follows is reading; -1 before the first
    std::vector<int> recent_touch;
    int trace_cap = 0;
    // large-batch staging: the host-LRU path's table row (pinned; its last copy
    // ends at stage_done), the device path's copy jobs
    const void **stage_row = nullptr;
    hipEvent_t stage_done = nullptr;
    bool stage_pending = false;
    CacheJob *d_sjobs = nullptr;     // [E]
    int32_t *d_snjobs = nullptr;
};

namespace {

using Group = moe_cache::Group;

void unlink(Group &g, int s)
{
    int p = g.prev[s], n = g.next[s];
    if (p >= 0) g.next[p] = n; else g.head = n;
    if (n >= 0) g.prev[n] = p; else g.tail = p;
    g.prev[s] = g.next[s] = -1;
}

void push_front(Group &g, int s)
{
    g.prev[s] = -1;
    g.next[s] = g.head;
    if (g.head >= 0) g.prev[g.head] = s;
    g.head = s;
    if (g.tail < 0) g.tail = s;
}

// Put s back right after p (p = -1: at the head).
void insert_after(Group &g, int p, int s)
{
    if (p < 0) { push_front(g, s); return; }
    const int n = g.next[p];
    g.next[p] = s;
    g.prev[s] = p;
    g.next[s] = n;
    if (n >= 0) g.prev[n] = s; else g.tail = s;
}

// The default backend: HBM from hipMalloc, copies by hipMemcpyAsync.
int32_t hip_alloc(void *, size_t bytes, void **out) { return hipMalloc(out, bytes) == hipSuccess ? 0 : 1; }
void hip_release(void *, void *p) { (void)hipFree(p); }

void destroy(moe_cache *c)
{
    if (!c) return;
    if (!c->custom) {
        (void)hipSetDevice(c->device);
        (void)hipDeviceSynchronize();
    }
    for (auto &g : c->groups) {
        if (g.pool) c->be.release(c->be.user, g.pool);
        if (g.res) c->be.release(c->be.user, g.res);
    }
    if (c->dtab) c->be.release(c->be.user, c->dtab);
    if (c->htab) {
        if (c->custom) free((void *)c->htab);
        else (void)hipHostFree((void *)c->htab);
    }
    for (auto ev : c->table_done)
        if (ev) (void)hipEventDestroy(ev);
    for (auto &dg : c->dgroups) {
        if (dg.stamp) (void)hipFree(dg.stamp);
        if (dg.key) (void)hipFree(dg.key);
    }
    for (void *p : {(void *)c->d_where, (void *)c->d_src, (void *)c->d_counters, (void *)c->d_jobs,
                    (void *)c->d_stats, (void *)c->d_trace, (void *)c->d_pjobs, (void *)c->d_pnjobs,
                    (void *)c->d_jwait, (void *)c->d_done})
        if (p) (void)hipFree(p);
    for (auto ev : c->ev_pref)
        if (ev) (void)hipEventDestroy(ev);
    if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
    if (c->stage_row) {
        if (c->custom) free((void *)c->stage_row);
        else (void)hipHostFree((void *)c->stage_row);
    }
    if (c->stage_done) (void)hipEventDestroy(c->stage_done);
    if (c->d_sjobs) (void)hipFree(c->d_sjobs);
    if (c->d_snjobs) (void)hipFree(c->d_snjobs);
    delete c;
}

bool resident_layer(const moe_cache *c, int layer) { return c->resident[layer] != 0; }

// A prefetch's copies run beside the lookups that follow it.  The slots it
// filled were touched last by the prefetch, so a later lookup can take one
// of them as its victim only once every other slot of the group has been
// touched since.  A call that could reach that count while the prefetch may
// still be copying is refused (`skip`: the layer whose own wait comes first).
moe_status prefetch_guard(moe_cache *c, int g, int n, int skip, const char *who)
{
    for (int m = 0; m < c->n_layers; m++)
        if (m != skip && c->pend_touch[m] >= 0 && c->layer_group[m] == g && c->pend_touch[m] + n >= c->groups[g].n_slots) {
            set_error("%s: %d more slot touches could evict the experts prefetched for layer %d (group of %d slots)",
                      who, n, m, c->groups[g].n_slots);
            return MOE_ERR_CAPACITY;
        }
    return MOE_OK;
}

void prefetch_count(moe_cache *c, int g, int n)
{
    for (int m = 0; m < c->n_layers; m++)
        if (c->pend_touch[m] >= 0 && c->layer_group[m] == g) c->pend_touch[m] += n;
}

CacheDevArgs device_args(moe_cache *c, int layer, const int32_t *idx, int T, int k)
{
    const int g = c->layer_group[layer], ng = (int)c->groups.size();
    auto &G = c->groups[g];
    CacheDevArgs a{};
    a.idx = idx; a.T = T; a.k = k; a.layer = layer; a.E = c->E;
    a.where = c->d_where; a.src = c->d_src; a.dtab = c->dtab;
    a.stamp = c->dgroups[g].stamp; a.key = c->dgroups[g].key;
    a.next_free = c->d_counters + g;
    a.clock = (uint32_t *)(c->d_counters + ng);
    a.njobs = c->d_counters + ng + 1;
    a.pool = G.pool; a.slot_bytes = G.slot_bytes; a.n_slots = G.n_slots;
    a.jobs = c->d_jobs;
    a.stats = c->d_stats;
    a.trace = c->d_trace; a.ntrace = c->d_counters + ng + 2; a.trace_cap = c->trace_cap;
    return a;
}

void count_lookup(moe_cache_stats_t &st, int T, bool hit, int sign)
{
    const uint64_t d = (uint64_t)(int64_t)sign;  // +1 or -1 (mod 2^64)
    st.lookups += d;
    if (T <= 8) st.lookups_le8 += d; else st.lookups_9_32 += d;
    if (hit) {
        st.hits += d;
        if (T <= 8) st.hits_le8 += d; else st.hits_9_32 += d;
    } else {
        st.misses += d;
    }
}

// Undo one decision of a host lookup.  Called in reverse order over a suffix
// of the lookup's decisions, with no other lookup since, so the decision's
// slot is at the head of the recency list.
void undo_op(moe_cache *c, Group &G, const moe_cache::Op &op, int T)
{
    const int s = op.slot;
    const int64_t E = c->E;
    unlink(G, s);
    count_lookup(c->st, T, op.kind == 0, -1);
    if (op.kind != 0) {
        c->where[op.key] = -1;
        c->htab[op.key] = nullptr;
        c->dirty[op.key / E] = 1;
        if (op.kind == 1) {  // the never-used slot is free again
            G.slot_key[s] = -1;
            G.next_free--;
            return;
        }
        c->st.evictions--;
        G.slot_key[s] = op.victim;
        c->where[op.victim] = s;
        c->htab[op.victim] = G.pool + (size_t)s * G.slot_bytes;
        c->dirty[op.victim / E] = 1;
    }
    insert_after(G, op.old_prev, s);
}

// Copy one table row to the device (default backend: on `s`, recording the
// row's event; a custom backend: synchronously).
moe_status upload_row(moe_cache *c, int r, hipStream_t s)
{
    const size_t off = (size_t)r * c->E, bytes = sizeof(void *) * (size_t)c->E;
    if (c->custom) {
        if (c->be.copy(c->be.user, c->dtab + off, c->htab + off, bytes) != 0) {
            set_error("slot table upload of layer %d failed (backend copy)", r);
            return MOE_ERR_HIP;
        }
        c->dirty[r] = 0;
        return MOE_OK;
    }
    hipError_t e = hipMemcpyAsync(c->dtab + off, c->htab + off, bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(c->table_done[r], s);
    if (e != hipSuccess) { set_error("slot table upload of layer %d failed: %s", r, hipGetErrorString(e)); return MOE_ERR_HIP; }
    c->table_pending[r] = 1;
    c->dirty[r] = 0;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_cache_create_ex(const moe_expert_desc *groups, int32_t n_groups, const int32_t *slots,
                               const int32_t *layer_group, int32_t n_layers, int32_t E,
                               const void *const *host_experts, const moe_cache_backend *backend,
                               moe_cache **out)
{
    if (!groups || !slots || !layer_group || !host_experts || !out || n_groups < 1 || n_layers < 1 || E < 1) {
        set_error("moe_cache_create: bad argument");
        return MOE_ERR_ARG;
    }
    if (backend && (!backend->alloc || !backend->release || !backend->copy)) {
        set_error("moe_cache_create_ex: the backend needs alloc, release and copy");
        return MOE_ERR_ARG;
    }
    *out = nullptr;
    bool any = false, wants_cache = false;
    for (int g = 0; g < n_groups; g++) {
        if (slots[g] < 0) { set_error("group %d: negative slot count %d", g, slots[g]); return MOE_ERR_ARG; }
        any = any || slots[g] > 0;
    }
    for (int l = 0; l < n_layers; l++) {
        const int g = layer_group[l] < 0 ? -layer_group[l] - 1 : layer_group[l];
        if (g < 0 || g >= n_groups) { set_error("layer %d: bad group", l); return MOE_ERR_ARG; }
        wants_cache = wants_cache || layer_group[l] >= 0;
    }
    if (!any && wants_cache) {
        set_error("every group has 0 slots (the budget is below the floor of each)");
        return MOE_ERR_BUDGET;
    }
    for (size_t i = 0; i < (size_t)n_layers * E; i++) {
        if (!host_experts[i]) { set_error("host expert %zu is null", i); return MOE_ERR_ARG; }
    }
    moe_cache *c = new moe_cache();
    c->n_layers = n_layers;
    c->E = E;
    c->custom = backend != nullptr;
    c->be = backend ? *backend : moe_cache_backend{nullptr, hip_alloc, hip_release, nullptr};
    if (!c->custom && hipGetDevice(&c->device) != hipSuccess) { delete c; set_error("hipGetDevice failed"); return MOE_ERR_HIP; }
    // a layer is resident when asked to be (negative group) or when its group
    // has no slots; layer_rank: its position among its group's resident layers
    c->layer_group.assign(n_layers, 0);
    c->resident.assign(n_layers, 0);
    c->layer_rank.assign(n_layers, 0);
    std::vector<int> per_group(n_groups, 0);
    for (int l = 0; l < n_layers; l++) {
        const int g = layer_group[l] < 0 ? -layer_group[l] - 1 : layer_group[l];
        c->layer_group[l] = g;
        c->resident[l] = layer_group[l] < 0 || slots[g] == 0;
        if (c->resident[l]) c->layer_rank[l] = per_group[g]++;
    }
    c->groups.resize(n_groups);
    for (int g = 0; g < n_groups; g++) {
        ExpertGeom eg;
        if (!geom(groups[g], &eg)) { destroy(c); set_error("group %d: bad expert desc", g); return MOE_ERR_SHAPE; }
        auto &G = c->groups[g];
        G.desc = groups[g];
        G.slot_bytes = eg.bytes;
        G.n_slots = slots[g];
        G.slot_key.assign(G.n_slots, -1);
        G.prev.assign(G.n_slots, -1);
        G.next.assign(G.n_slots, -1);
        for (int pass = 0; pass < 2; pass++) {
            // the slots, then the group's resident layers' experts
            const size_t n = pass == 0 ? (size_t)G.n_slots : (size_t)per_group[g] * E;
            if (n == 0) continue;
            void *p = nullptr;
            if (c->be.alloc(c->be.user, G.slot_bytes * n, &p) != 0 || !p) {
                destroy(c);
                set_error("allocation of %zu bytes for group %d failed", G.slot_bytes * n, g);
                return MOE_ERR_HIP;
            }
            (pass == 0 ? G.pool : G.res) = (uint8_t *)p;
        }
    }
    c->host.assign(host_experts, host_experts + (size_t)n_layers * E);
    c->where.assign((size_t)n_layers * E, -1);
    size_t tb = sizeof(void *) * (size_t)n_layers * E;
    void *dt = nullptr;
    bool ok = c->be.alloc(c->be.user, tb, &dt) == 0 && dt;
    c->dtab = (void **)dt;
    if (ok) {
        if (c->custom) ok = (c->htab = (const void **)calloc((size_t)n_layers * E, sizeof(void *))) != nullptr;
        else ok = hipHostMalloc((void **)&c->htab, tb, hipHostMallocDefault) == hipSuccess;
    }
    if (!ok) {
        destroy(c);
        set_error("allocation of the slot tables failed");
        return MOE_ERR_HIP;
    }
    memset((void *)c->htab, 0, tb);
    if (!c->custom) {
        c->table_done.assign(n_layers, nullptr);
        for (int l = 0; l < n_layers; l++) {
            if (hipEventCreateWithFlags(&c->table_done[l], hipEventDisableTiming) != hipSuccess) {
                destroy(c);
                set_error("hipEventCreate failed");
                return MOE_ERR_HIP;
            }
        }
    }
    c->table_pending.assign(n_layers, 0);
    c->dirty.assign(n_layers, 1);  // every row goes up once (resident rows are final)
    c->pending.assign(n_layers, {});
    c->ops.assign(n_layers, {});
    c->lookup_T.assign(n_layers, 0);
    c->looked_up.assign(n_layers, 0);
    // groups below the floor: their layers' experts resident, uploaded once
    int n_res = 0;
    size_t res_bytes = 0;
    for (int l = 0; l < n_layers; l++) {
        auto &G = c->groups[c->layer_group[l]];
        if (!c->resident[l]) continue;
        n_res++;
        for (int e = 0; e < E; e++) {
            uint8_t *dst = G.res + ((size_t)c->layer_rank[l] * E + e) * G.slot_bytes;
            const void *src = c->host[(size_t)l * E + e];
            const bool cp = c->custom ? c->be.copy(c->be.user, dst, src, G.slot_bytes) == 0
                                      : hipMemcpy(dst, src, G.slot_bytes, hipMemcpyHostToDevice) == hipSuccess;
            if (!cp) { destroy(c); set_error("upload of resident expert (%d, %d) failed", l, e); return MOE_ERR_HIP; }
            c->htab[(size_t)l * E + e] = dst;
            res_bytes += G.slot_bytes;
        }
    }
    for (int l = 0; l < n_layers; l++) {
        const size_t off = (size_t)l * E;
        const bool cp = c->custom ? c->be.copy(c->be.user, c->dtab + off, c->htab + off, sizeof(void *) * (size_t)E) == 0
                                  : hipMemcpy(c->dtab + off, c->htab + off, sizeof(void *) * (size_t)E,
                                              hipMemcpyHostToDevice) == hipSuccess;
        if (!cp) { destroy(c); set_error("upload of the slot tables failed"); return MOE_ERR_HIP; }
        c->dirty[l] = 0;
    }
    if (n_res) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "moe cache: %d of %d layers keep their experts resident (%zu bytes) and are not cached (placed "
                 "resident, or their group is below the budget floor)", n_res, n_layers, res_bytes);
        fprintf(stderr, "%s\n", msg);
        set_error("%s", msg);
    }
    *out = c;
    return MOE_OK;
}

moe_status moe_cache_create(const moe_expert_desc *groups, int32_t n_groups, const int32_t *slots,
                            const int32_t *layer_group, int32_t n_layers, int32_t E,
                            const void *const *host_experts, moe_cache **out)
{
    return moe_cache_create_ex(groups, n_groups, slots, layer_group, n_layers, E, host_experts, nullptr, out);
}

moe_status moe_cache_lookup(moe_cache *c, int32_t layer, int32_t T, int32_t k, const int32_t *idx,
                            int32_t *experts_out, int32_t *n_out, int32_t *slot_out, uint8_t *hit_out,
                            int32_t *victim_layer, int32_t *victim_expert)
{
    if (!c || !idx || !experts_out || !n_out || !slot_out || !hit_out || k < 1 || layer < 0 || layer >= c->n_layers) {
        set_error("moe_cache_lookup: bad argument");
        return MOE_ERR_ARG;
    }
    if (c->dev) { set_error("moe_cache_lookup: the cache looks up on the device (moe_cache_lookup_device)"); return MOE_ERR_STATE; }
    if (T < 1 || T > kMaxT) { set_error("moe_cache_lookup: T=%d outside [1, 32]; larger batches bypass the slots", T); return MOE_ERR_BATCH; }
    const int64_t E = c->E;
    std::vector<char> sel((size_t)E, 0);
    for (int p = 0; p < T * k; p++) {
        if (idx[p] < 0 || idx[p] >= E) { set_error("moe_cache_lookup: id %d outside [0, %d)", idx[p], (int)E); return MOE_ERR_ARG; }
        sel[idx[p]] = 1;
    }
    int n = 0;
    for (int e = 0; e < E; e++)
        if (sel[e]) experts_out[n++] = e;
    *n_out = n;
    auto &G = c->groups[c->layer_group[layer]];
    if (resident_layer(c, layer)) {
        for (int i = 0; i < n; i++) {
            slot_out[i] = -1;
            hit_out[i] = 1;
            if (victim_layer) victim_layer[i] = -1;
            if (victim_expert) victim_expert[i] = -1;
        }
        return MOE_OK;
    }
    if (n > G.n_slots) {
        set_error("moe_cache_lookup: %d distinct experts exceed the %d slots of the group", n, G.n_slots);
        return MOE_ERR_CAPACITY;
    }
    if (c->open_lookup >= 0) {
        set_error("moe_cache_lookup: the lookup of layer %d has not been uploaded", c->open_lookup);
        return MOE_ERR_STATE;
    }
    // table rows of this group still being copied must be read before this
    // lookup rewrites them (in the usual flow they finished long ago)
    if (!c->custom)
        for (int l = 0; l < c->n_layers; l++)
            if (c->table_pending[l] && c->layer_group[l] == c->layer_group[layer]) {
                if (hipEventSynchronize(c->table_done[l]) != hipSuccess) { set_error("hipEventSynchronize failed"); return MOE_ERR_HIP; }
                c->table_pending[l] = 0;
            }
    auto &ops = c->ops[layer];
    auto &pend = c->pending[layer];
    ops.clear();
    pend.clear();
    for (int i = 0; i < n; i++) {
        const int64_t key = layer * E + experts_out[i];
        int s = c->where[key];
        moe_cache::Op op{};
        op.key = key;
        op.victim = -1;
        if (s >= 0) {
            op.kind = 0;
            op.old_prev = G.prev[s];
            unlink(G, s);
        } else if (G.next_free < G.n_slots) {
            op.kind = 1;
            op.old_prev = -1;
            s = G.next_free++;
        } else {
            op.kind = 2;
            s = G.tail;
            op.old_prev = G.prev[s];
            op.victim = G.slot_key[s];
            c->where[op.victim] = -1;
            c->htab[op.victim] = nullptr;  // the evicted expert is no longer resident
            c->dirty[op.victim / E] = 1;
            unlink(G, s);
            c->st.evictions++;
        }
        op.slot = s;
        count_lookup(c->st, T, op.kind == 0, +1);
        if (op.kind != 0) {
            G.slot_key[s] = key;
            c->where[key] = s;
            c->htab[key] = G.pool + (size_t)s * G.slot_bytes;
            c->dirty[layer] = 1;
            pend.push_back({s, c->host[key], (int)ops.size()});
        }
        push_front(G, s);
        ops.push_back(op);
        slot_out[i] = s;
        hit_out[i] = op.kind == 0;
        if (victim_layer) victim_layer[i] = op.victim >= 0 ? (int)(op.victim / E) : -1;
        if (victim_expert) victim_expert[i] = op.victim >= 0 ? (int)(op.victim % E) : -1;
    }
    c->lookup_T[layer] = T;
    c->looked_up[layer] = 1;
    c->open_lookup = layer;
    return MOE_OK;
}

moe_status moe_cache_upload(moe_cache *c, int32_t layer, hipStream_t copy_stream, hipEvent_t done)
{
    if (!c || layer < 0 || layer >= c->n_layers) { set_error("moe_cache_upload: bad argument"); return MOE_ERR_ARG; }
    if (c->dev) { set_error("moe_cache_upload: the cache looks up on the device (moe_cache_lookup_device)"); return MOE_ERR_STATE; }
    if (c->custom && done) { set_error("moe_cache_upload: a backend cache has no events (done must be NULL)"); return MOE_ERR_ARG; }
    if (resident_layer(c, layer)) {
        if (done && hipEventRecord(done, copy_stream) != hipSuccess) { set_error("hipEventRecord failed"); return MOE_ERR_HIP; }
        return MOE_OK;
    }
    if (!c->looked_up[layer]) { set_error("moe_cache_upload: layer %d has no lookup", layer); return MOE_ERR_STATE; }
    auto &G = c->groups[c->layer_group[layer]];
    auto &pend = c->pending[layer];
    for (size_t j = 0; j < pend.size(); j++) {
        uint8_t *dst = G.pool + (size_t)pend[j].slot * G.slot_bytes;
        bool ok;
        char why[160] = "";
        if (c->custom) {
            ok = c->be.copy(c->be.user, dst, pend[j].src, G.slot_bytes) == 0;
            if (!ok) snprintf(why, sizeof why, "the backend's copy failed");
        } else {
            hipError_t e = hipMemcpyAsync(dst, pend[j].src, G.slot_bytes, hipMemcpyHostToDevice, copy_stream);
            ok = e == hipSuccess;
            if (!ok) snprintf(why, sizeof why, "%s", hipGetErrorString(e));
        }
        if (!ok) {
            // undo the lookup from this miss on, newest decision first
            auto &ops = c->ops[layer];
            const int from = pend[j].op;
            for (int o = (int)ops.size() - 1; o >= from; o--) undo_op(c, G, ops[o], c->lookup_T[layer]);
            ops.resize(from);
            pend.clear();
            c->looked_up[layer] = 0;
            c->open_lookup = -1;
            set_error("expert upload %zu of layer %d failed (%s); the lookup was rolled back to its first %d decisions",
                      j, layer, why, from);
            return MOE_ERR_HIP;
        }
        c->st.upload_bytes += G.slot_bytes;
    }
    pend.clear();
    c->ops[layer].clear();
    c->looked_up[layer] = 0;
    c->open_lookup = -1;
    for (int r = 0; r < c->n_layers; r++)
        if (c->dirty[r])
            if (moe_status st = upload_row(c, r, copy_stream)) return st;
    if (done && hipEventRecord(done, copy_stream) != hipSuccess) { set_error("hipEventRecord failed"); return MOE_ERR_HIP; }
    return MOE_OK;
}

const void *const *moe_cache_expert_ptrs(moe_cache *c, int32_t layer)
{
    if (!c || layer < 0 || layer >= c->n_layers) { set_error("moe_cache_expert_ptrs: bad argument"); return nullptr; }
    return (const void *const *)(c->dtab + (size_t)layer * c->E);
}

moe_status moe_cache_stats(const moe_cache *c, moe_cache_stats_t *out)
{
    if (!c || !out) { set_error("moe_cache_stats: null argument"); return MOE_ERR_ARG; }
    if (c->dev) {
        if (hipSetDevice(c->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipMemcpy(out, c->d_stats, sizeof *out, hipMemcpyDeviceToHost) != hipSuccess) {
            set_error("moe_cache_stats: reading the device counters failed");
            return MOE_ERR_HIP;
        }
        return MOE_OK;
    }
    *out = c->st;
    return MOE_OK;
}

moe_status moe_cache_reset_stats(moe_cache *c)
{
    if (!c) { set_error("moe_cache_reset_stats: null cache"); return MOE_ERR_ARG; }
    if (c->dev) {
        if (hipSetDevice(c->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipMemset(c->d_stats, 0, sizeof(moe_cache_stats_t)) != hipSuccess) {
            set_error("moe_cache_reset_stats: clearing the device counters failed");
            return MOE_ERR_HIP;
        }
        return MOE_OK;
    }
    c->st = moe_cache_stats_t{};
    return MOE_OK;
}

moe_status moe_cache_device_enable(moe_cache *c, int32_t trace_capacity)
{
    if (!c || trace_capacity < 0) { set_error("moe_cache_device_enable: bad argument"); return MOE_ERR_ARG; }
    if (c->custom) { set_error("moe_cache_device_enable: a cache with a caller-supplied backend looks up on the host"); return MOE_ERR_STATE; }
    if (c->dev) { set_error("moe_cache_device_enable: already enabled"); return MOE_ERR_STATE; }
    if (c->st.lookups || c->open_lookup >= 0) { set_error("moe_cache_device_enable: the cache has host lookups already"); return MOE_ERR_STATE; }
    for (size_t g = 0; g < c->groups.size(); g++)
        if (c->groups[g].n_slots > kCacheMaxSlots) {
            set_error("moe_cache_device_enable: group %zu has %d slots, above the %d the device lookup holds", g,
                      c->groups[g].n_slots, kCacheMaxSlots);
            return MOE_ERR_CAPACITY;
        }
    if (hipSetDevice(c->device) != hipSuccess) { set_error("hipSetDevice failed"); return MOE_ERR_HIP; }
    const size_t LE = (size_t)c->n_layers * c->E, ng = c->groups.size();
    std::vector<const void *> src(LE);
    for (size_t i = 0; i < LE; i++) {
        void *dp = nullptr;
        if (hipHostGetDevicePointer(&dp, const_cast<void *>(c->host[i]), 0) != hipSuccess || !dp) {
            set_error("moe_cache_device_enable: host expert %zu is not pinned memory the device can read", i);
            return MOE_ERR_ARG;
        }
        src[i] = dp;
    }
    std::vector<int32_t> minus1(LE, -1);
    bool ok = hipMalloc((void **)&c->d_where, LE * 4) == hipSuccess &&
              hipMalloc((void **)&c->d_src, LE * sizeof(void *)) == hipSuccess &&
              hipMalloc((void **)&c->d_counters, (ng + 3) * 4) == hipSuccess &&
              hipMalloc((void **)&c->d_jobs, (size_t)c->E * sizeof(CacheJob)) == hipSuccess &&
              hipMalloc((void **)&c->d_jwait, (size_t)c->E * 4) == hipSuccess &&
              hipMalloc((void **)&c->d_done, (size_t)c->E * 4) == hipSuccess &&
              hipMalloc((void **)&c->d_stats, sizeof(moe_cache_stats_t)) == hipSuccess &&
              hipMalloc((void **)&c->d_pjobs, LE * sizeof(CacheJob)) == hipSuccess &&
              hipMalloc((void **)&c->d_pnjobs, (size_t)c->n_layers * 4) == hipSuccess &&
              hipMemset(c->d_pnjobs, 0, (size_t)c->n_layers * 4) == hipSuccess &&
              hipMemcpy(c->d_where, minus1.data(), LE * 4, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(c->d_src, src.data(), LE * sizeof(void *), hipMemcpyHostToDevice) == hipSuccess &&
              hipMemset(c->d_counters, 0, (ng + 3) * 4) == hipSuccess &&
              hipMemset(c->d_stats, 0, sizeof(moe_cache_stats_t)) == hipSuccess;
    if (ok && trace_capacity > 0)
        ok = hipMalloc((void **)&c->d_trace, (size_t)trace_capacity * 16) == hipSuccess;
    c->dgroups.assign(ng, {});
    for (size_t g = 0; ok && g < ng; g++) {
        const int n = c->groups[g].n_slots;
        if (n == 0) continue;  // resident group: no LRU state
        std::vector<int32_t> keys(n, -1);
        ok = hipMalloc((void **)&c->dgroups[g].stamp, (size_t)n * 4) == hipSuccess &&
             hipMalloc((void **)&c->dgroups[g].key, (size_t)n * 4) == hipSuccess &&
             hipMemset(c->dgroups[g].stamp, 0, (size_t)n * 4) == hipSuccess &&
             hipMemcpy(c->dgroups[g].key, keys.data(), (size_t)n * 4, hipMemcpyHostToDevice) == hipSuccess;
    }
    if (!ok) {
        // leave the cache as it was (host lookups, nothing allocated)
        for (auto &dg : c->dgroups) {
            if (dg.stamp) (void)hipFree(dg.stamp);
            if (dg.key) (void)hipFree(dg.key);
        }
        c->dgroups.clear();
        for (void **pp : {(void **)&c->d_where, (void **)&c->d_src, (void **)&c->d_counters, (void **)&c->d_jobs,
                          (void **)&c->d_stats, (void **)&c->d_trace, (void **)&c->d_pjobs, (void **)&c->d_pnjobs,
                          (void **)&c->d_jwait, (void **)&c->d_done}) {
            if (*pp) (void)hipFree(*pp);
            *pp = nullptr;
        }
        set_error("moe_cache_device_enable: device allocation failed");
        return MOE_ERR_HIP;
    }
    // the host table is no longer refreshed; the device lookup writes dtab
    c->trace_cap = trace_capacity;
    c->pend_touch.assign(c->n_layers, -1);
    c->ev_pref.assign(c->n_layers, nullptr);
    c->recent_touch.assign(ng, -1);
    c->dev = true;
    return MOE_OK;
}

moe_status moe_cache_lookup_device(moe_cache *c, int32_t layer, const int32_t *idx, int32_t T, int32_t k,
                                   hipStream_t stream)
{
    if (!c || !idx || layer < 0 || layer >= c->n_layers || k < 1 || k > c->E) {
        set_error("moe_cache_lookup_device: bad argument");
        return MOE_ERR_ARG;
    }
    if (!c->dev) { set_error("moe_cache_lookup_device: moe_cache_device_enable was not called"); return MOE_ERR_STATE; }
    if (T < 1 || T > kMaxT) { set_error("moe_cache_lookup_device: T=%d outside [1, 32]", T); return MOE_ERR_BATCH; }
    if (resident_layer(c, layer)) return MOE_OK;  // its table row is final
    const int g = c->layer_group[layer];
    auto &G = c->groups[g];
    if (T * k > G.n_slots) {
        set_error("moe_cache_lookup_device: %d selections may exceed the %d slots of the group", T * k, G.n_slots);
        return MOE_ERR_CAPACITY;
    }
    if (moe_status st = prefetch_guard(c, g, T * k, layer, "moe_cache_lookup_device")) return st;
    if (c->pend_touch[layer] >= 0) {
        // the layer's prefetched copies end before its lookup
        if (hipStreamWaitEvent(stream, c->ev_pref[layer], 0) != hipSuccess) {
            set_error("moe_cache_lookup_device: hipStreamWaitEvent failed");
            return MOE_ERR_HIP;
        }
        c->pend_touch[layer] = -1;
    }
    moe_status st = launch_cache_device(device_args(c, layer, idx, T, k), stream);
    if (st != MOE_OK) return st;
    prefetch_count(c, g, T * k);
    c->recent_touch[g] = T * k;  // the slots the FFN after this lookup reads
    return MOE_OK;
}

moe_status moe_cache_lookup_device_route(moe_cache *c, int32_t layer, const void *ws, size_t ws_bytes, int32_t k,
                                         hipStream_t stream)
{
    if (!c || !ws || layer < 0 || layer >= c->n_layers || k < 1 || k > c->E || ws_bytes < kDlog + (size_t)c->E * 4) {
        set_error("moe_cache_lookup_device_route: bad argument");
        return MOE_ERR_ARG;
    }
    if (!c->dev) { set_error("moe_cache_lookup_device_route: moe_cache_device_enable was not called"); return MOE_ERR_STATE; }
    if (resident_layer(c, layer)) return MOE_OK;  // its table row is final
    const int g = c->layer_group[layer];
    auto &G = c->groups[g];
    if (!route_defers(G.desc, 1, c->E)) {
        set_error("moe_cache_lookup_device_route: this group's route launch does not leave the logit keys "
                  "(E <= 128 and the dot-product path at T=1 are needed); use moe_cache_lookup_device");
        return MOE_ERR_ARG;
    }
    if (k > G.n_slots) {
        set_error("moe_cache_lookup_device_route: %d selections may exceed the %d slots of the group", k, G.n_slots);
        return MOE_ERR_CAPACITY;
    }
    if (moe_status st = prefetch_guard(c, g, k, layer, "moe_cache_lookup_device_route")) return st;
    if (c->pend_touch[layer] >= 0) {
        if (hipStreamWaitEvent(stream, c->ev_pref[layer], 0) != hipSuccess) {
            set_error("moe_cache_lookup_device_route: hipStreamWaitEvent failed");
            return MOE_ERR_HIP;
        }
        c->pend_touch[layer] = -1;
    }
    CacheDevArgs a = device_args(c, layer, nullptr, 1, k);
    a.keys = (const uint32_t *)((const uint8_t *)ws + kDlog);
    moe_status st = launch_cache_device(a, stream);
    if (st != MOE_OK) return st;
    prefetch_count(c, g, k);
    c->recent_touch[g] = k;
    return MOE_OK;
}

moe_status moe_cache_ffn_device(moe_cache *c, int32_t layer, const moe_expert_desc *d, float *h, int32_t k,
                                const void *const *shared_ptrs, int32_t n_shared, const float *bias, float eps,
                                int32_t chain_in, const float *next_router, int32_t next_E, int32_t parity,
                                void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!c || !d || !h || !ws || layer < 0 || layer >= c->n_layers || k < 1 || k > c->E ||
        ws_bytes < kDlog + (size_t)c->E * 4 || (n_shared > 0 && !shared_ptrs)) {
        set_error("moe_cache_ffn_device: bad argument");
        return MOE_ERR_ARG;
    }
    if (!c->dev) { set_error("moe_cache_ffn_device: moe_cache_device_enable was not called"); return MOE_ERR_STATE; }
    const bool chain = chain_in || next_router;
    if (chain) {
        if (!moe_layer_chain_supported(d, 1, c->E)) {
            set_error("moe_cache_ffn_device: chaining takes the single-token kernels (E <= %d, H <= %d)", kChainE,
                      kChainMaxH);
            return MOE_ERR_ARG;
        }
        if ((next_router && (next_E < 1 || next_E > kChainE)) || (parity != 0 && parity != 1)) {
            set_error("moe_cache_ffn_device: next_E=%d or parity=%d out of range", next_E, parity);
            return MOE_ERR_ARG;
        }
    }
    Chain ch{};
    ch.rp_in = chain_in ? chain_buf(ws, parity) : nullptr;
    ch.rp_out = next_router ? chain_buf(ws, parity ^ 1) : nullptr;
    ch.wn = next_router;
    ch.En = next_E;
    ch.bias = bias;
    ch.eps = eps;
    const void *const *table = moe_cache_expert_ptrs(c, layer);
    if (resident_layer(c, layer))  // its table row is final: no lookup, nothing to copy
        return launch_ffn_copy(d, h, c->E, k, table, shared_ptrs, n_shared, ws, ws_bytes, stream, nullptr,
                               chain ? &ch : nullptr);
    const int g = c->layer_group[layer];
    auto &G = c->groups[g];
    if (!route_defers(G.desc, 1, c->E)) {
        set_error("moe_cache_ffn_device: this group's route launch does not leave the logit keys "
                  "(E <= 128 and the dot-product path at T=1 are needed)");
        return MOE_ERR_ARG;
    }
    if (k > G.n_slots) {
        set_error("moe_cache_ffn_device: %d selections may exceed the %d slots of the group", k, G.n_slots);
        return MOE_ERR_CAPACITY;
    }
    if (moe_status st = prefetch_guard(c, g, k, layer, "moe_cache_ffn_device")) return st;
    if (c->pend_touch[layer] >= 0) {
        if (hipStreamWaitEvent(stream, c->ev_pref[layer], 0) != hipSuccess) {
            set_error("moe_cache_ffn_device: hipStreamWaitEvent failed");
            return MOE_ERR_HIP;
        }
        c->pend_touch[layer] = -1;
    }
    uint32_t *keys = (uint32_t *)((uint8_t *)ws + kDlog);
    CacheDevArgs a = device_args(c, layer, nullptr, 1, k);
    if (chain_in) {
        // the keys are formed by the lookup from the previous layer's partials,
        // and stored where the FFN launch ranks them
        a.rp_in = ch.rp_in; a.hs = h; a.bias = bias; a.eps = eps; a.H = d->H; a.keys_out = keys;
    } else {
        a.keys = keys;
    }
    a.jwait = c->d_jwait;
    a.done = c->d_done;
    moe_status st = launch_cache_device(a, stream);  // the lookup alone
    if (st != MOE_OK) return st;
    prefetch_count(c, g, k);
    c->recent_touch[g] = k;
    CacheCopy cc{a.jobs, a.njobs, a.jwait, a.done, a.slot_bytes};
    ch.dlog_keys = true;  // the FFN ranks the keys the lookup ranked
    return launch_ffn_copy(d, h, c->E, k, table, shared_ptrs, n_shared, ws, ws_bytes, stream, &cc,
                           chain ? &ch : nullptr);
}

moe_status moe_cache_prefetch_device(moe_cache *c, int32_t layer, const int32_t *idx, int32_t T, int32_t k,
                                     hipStream_t stream, hipStream_t copy_stream)
{
    if (!c || !idx || layer < 0 || layer >= c->n_layers || k < 1 || k > c->E || copy_stream == stream) {
        set_error("moe_cache_prefetch_device: bad argument");
        return MOE_ERR_ARG;
    }
    if (!c->dev) { set_error("moe_cache_prefetch_device: moe_cache_device_enable was not called"); return MOE_ERR_STATE; }
    if (T < 1 || T > kMaxT) { set_error("moe_cache_prefetch_device: T=%d outside [1, 32]", T); return MOE_ERR_BATCH; }
    if (resident_layer(c, layer)) return MOE_OK;  // nothing to fetch
    if (c->pend_touch[layer] >= 0) {
        set_error("moe_cache_prefetch_device: layer %d has a prefetch that its lookup has not taken yet", layer);
        return MOE_ERR_STATE;
    }
    const int g = c->layer_group[layer];
    const int n_slots = c->groups[g].n_slots;
    if (T * k >= n_slots) {
        set_error("moe_cache_prefetch_device: %d selections need more than the %d slots of the group", T * k, n_slots);
        return MOE_ERR_CAPACITY;
    }
    // The copies overlap the FFN that follows the group's latest lookup.  A
    // miss can evict one of that lookup's slots only once every slot of the
    // group has been touched since the lookup, so the prefetch is refused
    // when the touches since it plus this prefetch's could reach the slots.
    if (c->recent_touch[g] >= 0 && c->recent_touch[g] + T * k >= n_slots) {
        set_error("moe_cache_prefetch_device: %d slot touches since the group's latest lookup plus %d more could evict "
                  "experts that its FFN is reading (group of %d slots)", c->recent_touch[g], T * k, n_slots);
        return MOE_ERR_CAPACITY;
    }
    if (moe_status st = prefetch_guard(c, g, T * k, -1, "moe_cache_prefetch_device")) return st;
    if (!c->ev_fork && hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess) {
        c->ev_fork = nullptr;
        set_error("moe_cache_prefetch_device: hipEventCreate failed");
        return MOE_ERR_HIP;
    }
    if (!c->ev_pref[layer] && hipEventCreateWithFlags(&c->ev_pref[layer], hipEventDisableTiming) != hipSuccess) {
        c->ev_pref[layer] = nullptr;
        set_error("moe_cache_prefetch_device: hipEventCreate failed");
        return MOE_ERR_HIP;
    }
    CacheDevArgs a = device_args(c, layer, idx, T, k);
    a.jobs = c->d_pjobs + (size_t)layer * c->E;
    a.njobs = c->d_pnjobs + layer;
    moe_status st = launch_cache_device(a, stream, copy_stream, c->ev_fork, c->ev_pref[layer]);
    if (st != MOE_OK) return st;
    prefetch_count(c, g, T * k);
    if (c->recent_touch[g] >= 0) c->recent_touch[g] += T * k;
    c->pend_touch[layer] = T * k;
    return MOE_OK;
}

moe_status moe_cache_trace_read(moe_cache *c, int32_t *out, int32_t capacity, int32_t *n)
{
    if (!c || !n || capacity < 0 || (capacity && !out)) { set_error("moe_cache_trace_read: bad argument"); return MOE_ERR_ARG; }
    if (!c->dev || !c->d_trace) { set_error("moe_cache_trace_read: no device trace (moe_cache_device_enable with a capacity)"); return MOE_ERR_STATE; }
    const int ng = (int)c->groups.size();
    int32_t total = 0;
    if (hipSetDevice(c->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&total, c->d_counters + ng + 2, 4, hipMemcpyDeviceToHost) != hipSuccess) {
        set_error("moe_cache_trace_read: reading the trace failed");
        return MOE_ERR_HIP;
    }
    *n = total;
    const int m = total < c->trace_cap ? total : c->trace_cap;
    const int cp = m < capacity ? m : capacity;
    if (cp > 0 && hipMemcpy(out, c->d_trace, (size_t)cp * 16, hipMemcpyDeviceToHost) != hipSuccess) {
        set_error("moe_cache_trace_read: reading the trace failed");
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

moe_status moe_cache_stage_large(moe_cache *c, int32_t layer, int32_t T, int32_t k, const int32_t *idx,
                                 void *staging, size_t staging_bytes, void **table_out, hipStream_t s)
{
    if (!c || !idx || !table_out || k < 1 || layer < 0 || layer >= c->n_layers) {
        set_error("moe_cache_stage_large: bad argument");
        return MOE_ERR_ARG;
    }
    if (c->dev) { set_error("moe_cache_stage_large: the cache looks up on the device (moe_cache_stage_large_device)"); return MOE_ERR_STATE; }
    if (T <= kMaxT || T > kMaxTLarge) { set_error("moe_cache_stage_large: T=%d outside [33, %d]", T, kMaxTLarge); return MOE_ERR_BATCH; }
    if (c->open_lookup >= 0) {
        set_error("moe_cache_stage_large: the lookup of layer %d has not been uploaded (its slots are not filled)", c->open_lookup);
        return MOE_ERR_STATE;
    }
    const int E = c->E;
    auto &G = c->groups[c->layer_group[layer]];
    const size_t need = (size_t)std::min(E, T * k) * G.slot_bytes;
    if (!resident_layer(c, layer) && (!staging || staging_bytes < need)) {
        set_error("moe_cache_stage_large: staging of %zu bytes, %zu needed", staging_bytes, need);
        return MOE_ERR_ARG;
    }
    std::vector<char> sel(E, 0);
    for (int p = 0; p < T * k; p++) {
        if (idx[p] < 0 || idx[p] >= E) { set_error("moe_cache_stage_large: id %d outside [0, %d)", idx[p], E); return MOE_ERR_ARG; }
        sel[idx[p]] = 1;
    }
    if (!c->stage_row) {
        if (c->custom) c->stage_row = (const void **)calloc(E, sizeof(void *));
        else if (hipHostMalloc((void **)&c->stage_row, sizeof(void *) * E, hipHostMallocDefault) != hipSuccess) c->stage_row = nullptr;
        if (!c->stage_row || (!c->custom && hipEventCreateWithFlags(&c->stage_done, hipEventDisableTiming) != hipSuccess)) {
            set_error("moe_cache_stage_large: allocation failed");
            return MOE_ERR_HIP;
        }
    }
    if (c->stage_pending) {  // the previous call's table copy must have read the row
        if (hipEventSynchronize(c->stage_done) != hipSuccess) { set_error("hipEventSynchronize failed"); return MOE_ERR_HIP; }
        c->stage_pending = false;
    }
    const size_t off = (size_t)layer * E;
    int u = 0, copies = 0;
    for (int e = 0; e < E; e++) {
        if (resident_layer(c, layer)) { c->stage_row[e] = c->htab[off + e]; continue; }
        if (!sel[e]) { c->stage_row[e] = nullptr; continue; }
        uint8_t *dst = (uint8_t *)staging + (size_t)u * G.slot_bytes;
        const int sl = c->where[off + e];
        const void *src = sl >= 0 ? (const void *)(G.pool + (size_t)sl * G.slot_bytes) : c->host[off + e];
        bool ok;
        if (c->custom) ok = c->be.copy(c->be.user, dst, src, G.slot_bytes) == 0;
        else ok = hipMemcpyAsync(dst, src, G.slot_bytes, sl >= 0 ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, s) == hipSuccess;
        if (!ok) { set_error("moe_cache_stage_large: copy of expert %d failed", e); return MOE_ERR_HIP; }
        c->stage_row[e] = dst;
        copies += sl >= 0;
        u++;
    }
    bool ok;
    if (c->custom) ok = c->be.copy(c->be.user, table_out, c->stage_row, sizeof(void *) * E) == 0;
    else ok = hipMemcpyAsync(table_out, c->stage_row, sizeof(void *) * E, hipMemcpyHostToDevice, s) == hipSuccess &&
              hipEventRecord(c->stage_done, s) == hipSuccess;
    if (!ok) { set_error("moe_cache_stage_large: table copy failed"); return MOE_ERR_HIP; }
    c->stage_pending = !c->custom;
    c->st.large_copies += copies;
    c->st.large_uploads += u - copies;
    return MOE_OK;
}

moe_status moe_cache_stage_large_device(moe_cache *c, int32_t layer, int32_t T, int32_t k, const int32_t *idx,
                                        void *staging, size_t staging_bytes, void **table_out, hipStream_t s)
{
    if (!c || !idx || !table_out || k < 1 || k > (c ? c->E : 0) || layer < 0 || layer >= c->n_layers) {
        set_error("moe_cache_stage_large_device: bad argument");
        return MOE_ERR_ARG;
    }
    if (!c->dev) { set_error("moe_cache_stage_large_device: moe_cache_device_enable was not called"); return MOE_ERR_STATE; }
    if (T <= kMaxT || T > kMaxTLarge) { set_error("moe_cache_stage_large_device: T=%d outside [33, %d]", T, kMaxTLarge); return MOE_ERR_BATCH; }
    const int E = c->E;
    auto &G = c->groups[c->layer_group[layer]];
    if (resident_layer(c, layer)) {
        if (hipMemcpyAsync(table_out, c->dtab + (size_t)layer * E, sizeof(void *) * E, hipMemcpyDeviceToDevice, s) != hipSuccess) {
            set_error("moe_cache_stage_large_device: table copy failed");
            return MOE_ERR_HIP;
        }
        return MOE_OK;
    }
    const size_t need = (size_t)std::min(E, T * k) * G.slot_bytes;
    if (!staging || staging_bytes < need) {
        set_error("moe_cache_stage_large_device: staging of %zu bytes, %zu needed", staging_bytes, need);
        return MOE_ERR_ARG;
    }
    if (!c->d_sjobs && (hipMalloc((void **)&c->d_sjobs, sizeof(CacheJob) * (size_t)E) != hipSuccess ||
                        hipMalloc((void **)&c->d_snjobs, 4) != hipSuccess)) {
        set_error("moe_cache_stage_large_device: allocation failed");
        return MOE_ERR_HIP;
    }
    if (c->pend_touch[layer] >= 0 && hipStreamWaitEvent(s, c->ev_pref[layer], 0) != hipSuccess) {
        set_error("moe_cache_stage_large_device: hipStreamWaitEvent failed");  // a prefetch into this layer's slots
        return MOE_ERR_HIP;
    }
    StageDevArgs a{};
    a.idx = idx; a.T = T; a.k = k; a.layer = layer; a.E = E;
    a.where = c->d_where; a.src = c->d_src; a.pool = G.pool; a.slot_bytes = G.slot_bytes;
    a.staging = (uint8_t *)staging; a.table = table_out;
    a.jobs = c->d_sjobs; a.njobs = c->d_snjobs; a.stats = c->d_stats;
    return launch_stage_device(a, s);
}

void moe_cache_destroy(moe_cache *c) { destroy(c); }

}  // extern "C"
