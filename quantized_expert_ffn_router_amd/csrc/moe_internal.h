// moe_internal.h -- private definitions shared by the libmoe sources.
//
// Slot layout.  A quantized matrix [N, K] (N a multiple of 64, K a multiple
// of 256) is cut into tiles of 64 rows x 256 columns, stored tile after tile
// with the column index fastest: tile (rt, s) starts at (rt*S + s)*tile_bytes,
// S = K/256.  Inside a tile each 16-byte piece ("granule") of the 64 rows'
// blocks is stored side by side (row 0's granule, row 1's, ...), so that a
// wavefront in which lane r owns row r reads each granule of the tile as
// 1 KiB of consecutive bytes.  The bytes are the canonical block bytes,
// permuted; no byte is added or dropped.
//
//   Q4_K tile (9216 B):  [meta 64x16: d,dmin,scales[12]] [qs granule j=0..7: 64x16]
//   Q6_K tile (13440 B): [ql granule j=0..7: 64x16] [qh granule j=0..3: 64x16]
//                        [sc 64x16] [d 64x2]
//   Q8_0 tile (17408 B): [q granule j=0..15: 64x16 (block j/2, half j%2)] [d 64x16 (8 fp16)]
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kTileRows = 64;
constexpr int kTileCols = 256;
constexpr int kMaxT = 32;        // batch of the layer path and the slot-pool cache
constexpr int kMaxTLarge = 256;  // batch of moe_route_topk and moe_expert_ffn (prompt-sized batches)
constexpr int kMaxE = 1024;
constexpr int kMaxShared = 8;
constexpr int kMaxH = 8192;
constexpr int kPieces = 3;  // activations are encoded as 3 int8 pieces

inline int tile_bytes(int qtype)
{
    switch (qtype) {
    case MOE_Q4_K: return 64 * 144;
    case MOE_Q6_K: return 64 * 210;
    case MOE_Q8_0: return 64 * 8 * 34;
    default: return 0;
    }
}

inline int block_weights(int qtype) { return qtype == MOE_Q8_0 ? 32 : 256; }
inline int block_bytes(int qtype)
{
    return qtype == MOE_Q8_0 ? 34 : qtype == MOE_Q4_K ? 144 : qtype == MOE_Q6_K ? 210 : 0;
}
inline bool qtype_ok(int q) { return q == MOE_Q8_0 || q == MOE_Q4_K || q == MOE_Q6_K; }

// Down-row length after padding to whole 256-column tiles.
inline int down_k(const moe_expert_desc &d) { return (d.I + kTileCols - 1) / kTileCols * kTileCols; }

inline size_t mat_bytes(int qtype, int n, int k)
{
    return (size_t)(n / kTileRows) * (size_t)(k / kTileCols) * (size_t)tile_bytes(qtype);
}

struct ExpertGeom {
    size_t gate_off, up_off, down_off, bytes;
    int kd;  // padded down row length
};

inline bool geom(const moe_expert_desc &d, ExpertGeom *g)
{
    if (!qtype_ok(d.gate) || !qtype_ok(d.up) || !qtype_ok(d.down)) return false;
    if (d.H <= 0 || d.I <= 0 || d.H % kTileCols || d.H % kTileRows || d.I % kTileRows) return false;
    if (d.H > kMaxH || d.I > kMaxH) return false;
    g->kd = down_k(d);
    g->gate_off = 0;
    g->up_off = mat_bytes(d.gate, d.I, d.H);
    g->down_off = g->up_off + mat_bytes(d.up, d.I, d.H);
    g->bytes = g->down_off + mat_bytes(d.down, d.H, g->kd);
    return true;
}


// Device-side slot-pool lookup (see k_cache_lookup): the LRU state of one
// group, the layer's selected ids, and where the results go.
struct CacheJob {
    uint8_t *dst;        // slot
    const uint8_t *src;  // device address of the expert's pinned host copy
};
struct CacheDevArgs {
    const int32_t *idx;  // [T][k] selected ids of the layer-step (device), or null:
    const uint32_t *keys;  // [E] (T = 1) the route launch's logit keys, whose k largest are the ids
    int T, k, layer, E;
    int32_t *where;              // [L*E] slot of each key, -1 absent
    const void *const *src;      // [L*E] device addresses of the host copies
    void **dtab;                 // [L*E] slot addresses (the layer's row is written)
    uint32_t *stamp;             // [n_slots] last use of each slot (group)
    int32_t *key;                // [n_slots] key held by each slot, -1 free (group)
    int32_t *next_free;          // group's first never-used slot
    uint32_t *clock;             // last stamp handed out (all groups)
    uint8_t *pool;
    unsigned long long slot_bytes;
    int n_slots;
    CacheJob *jobs;              // [E] misses of this call
    int32_t *njobs;
    unsigned long long *stats;   // moe_cache_stats_t fields, in order
    int32_t *trace;              // [trace_cap][4] (layer, expert, hit, victim key) or null
    int32_t *ntrace;
    int trace_cap;
    // copies left to the FFN launch (moe_cache_ffn_device), or null: each
    // selected id's job + 1 (0: a hit), and the jobs' completion counts
    // (cleared here); no copy kernel is launched
    int32_t *jwait;              // [E]
    uint32_t *done;              // [E]
    // T = 1 of a chained layer (keys null): the logits from the previous
    // layer's tile partials rp_in [H/64][kChainE], the state hs [H], bias
    // [E] (or null) and eps, as the chained gate/up kernel forms them
    const float *rp_in, *hs, *bias;
    float eps;
    int H;
    uint32_t *keys_out;          // [E] the keys formed from rp_in, for the FFN's rank
};
constexpr int kCacheMaxSlots = 16384;  // slots per group that the device lookup holds in LDS
// True when moe_layer_route leaves a single token's routing to the FFN (only
// the logit keys at kDlog are written unless the caller asks for the ids).
bool route_defers(const moe_expert_desc &d, int T, int E);
// The lookup on s, then the miss copies: on s, or with a side stream cs on cs
// after `fork` (recorded on s), recording `done` on cs after them.
moe_status launch_cache_device(const CacheDevArgs &a, hipStream_t s, hipStream_t cs = nullptr,
                               hipEvent_t fork = nullptr, hipEvent_t done = nullptr);
// A cached single token's FFN whose gate/up launch also copies the misses
// that a lookup with jwait/done left (moe_cache_ffn_device).
struct CacheCopy {
    const CacheJob *jobs;
    const int32_t *njobs;
    const int32_t *jwait;
    uint32_t *done;
    unsigned long long slot_bytes;
};


// Staging of a large batch's experts on the device (moe_cache_stage_large_device):
// the layer's distinct ids, each copied from its slot or its host copy.
struct StageDevArgs {
    const int32_t *idx;          // [T][k] (device)
    int T, k, layer, E;
    const int32_t *where;        // [L*E] slot of each key, -1 absent
    const void *const *src;      // [L*E] device addresses of the host copies
    const uint8_t *pool;
    unsigned long long slot_bytes;
    uint8_t *staging;
    void **table;                // [E] out
    CacheJob *jobs;              // [E]
    int32_t *njobs;
    unsigned long long *stats;   // moe_cache_stats_t fields, in order
};
moe_status launch_stage_device(const StageDevArgs &a, hipStream_t s);

// The router's hand-over of logit keys sits at a fixed offset at the start of
// every workspace, sized for the largest batch and expert count, so that calls
// of different sizes can share one workspace: the route launch finds it zero
// (as moe_workspace_init leaves it) and leaves it zero.
constexpr size_t kKeys = 0;
constexpr size_t kKeysBytes = (size_t)kMaxT * kMaxE * 4;
// After them, the per-token top-k workgroups' hand-over of each token's k
// selections to the route tail (64-bit, never zero), same protocol.
constexpr size_t kTkBytes = (size_t)kMaxT * 64 * 8;
// Then the workspace's status word (a 256-byte region): bits that the route
// launch sets when a bounded wait gives up (MOE_WS_* in moe.h), sticky until
// moe_workspace_init clears the workspace.
constexpr size_t kStatus = kKeys + kKeysBytes + kTkBytes;
constexpr size_t kStatusBytes = 256;
static_assert(kStatus == MOE_WS_STATUS_OFFSET, "status word offset published in moe.h");
// Then the logit keys of up to kDlogTok tokens, [T][E], written by the route
// launch for routing in the FFN kernels (or, for a single token, in the
// cache's device lookup), at a fixed offset.
constexpr int kDlogTok = 8;
constexpr size_t kDlog = kStatus + kStatusBytes;
constexpr size_t kDlogBytes = (size_t)kDlogTok * kMaxE * 4;
// Then the router dot products that chained single-token layers hand on:
// two buffers (the layer's parity picks the one it reads; it writes the
// other) of partial sums over 64-position tiles of the state, [H/64][kChainE]
// (E <= kChainE, H <= kChainMaxH).
constexpr int kChainE = 128;
constexpr int kChainMaxH = 4096;
constexpr size_t kChainBufBytes = (size_t)(kChainMaxH / 64) * kChainE * 4;
constexpr size_t kChain = kDlog + kDlogBytes;
constexpr size_t kChainBytes = 2 * kChainBufBytes;

// Workspace map (byte offsets, 256-aligned regions) for a batch of T tokens.
//
// Activations are stored encoded, one contiguous record of 4K bytes per
// vector of K positions: pieces q[3][K] (int8, piece-major), per-32-position
// block scales bs[K/32] and exact fp32 block sums bsum[K/32] (float), and
// per-16-position integer sums of each piece ps[3][K/16] (int32).
constexpr size_t enc_bytes(int K) { return (size_t)4 * K; }

// Pairs per work item of the VALU FFN kernels: an expert with more pairs is
// cut into several items, so that its row tiles' token passes run in
// parallel workgroups.
constexpr int kItemTok = 4;

// Half-precision records of the MFMA path, one per (vector, 256-position
// super-block): the positions times 2^e (e brings the super-block's largest
// magnitude to [0.5, 1)) split into fp16 hi + lo, [hi 256][lo 256] halves,
// the 32-position block sums of the scaled values as fp16 hi [8] and lo [8],
// then 2^-e as fp32 and padding.
constexpr int kX16Bytes = 1072;

struct WsLayout {
    int T, k, E, ns, H, kd, P, U, UI;  // U: distinct experts, UI: work items (both at most)
    size_t keys, tk, status, xenc, x16, idx, w, nuniq, wt, ptok, inv, pw, henc, hf, dlog, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline WsLayout ws_layout(const moe_expert_desc &d, int T, int k, int E, int ns)
{
    WsLayout L{};
    L.T = T; L.k = k; L.E = E; L.ns = ns; L.H = d.H; L.kd = down_k(d);
    L.P = T * (k + ns);
    int ur = E < T * k ? E : T * k;
    L.U = ur + ns;
    L.UI = L.U + (L.P + kItemTok - 1) / kItemTok;
    L.keys = kKeys;
    L.tk = kKeys + kKeysBytes;
    L.status = kStatus;
    L.dlog = kDlog;
    size_t o = kChain + kChainBytes;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    L.xenc = take((size_t)T * enc_bytes(d.H));
    L.x16 = take((size_t)T * (d.H / 256) * kX16Bytes);
    L.idx = take((size_t)T * k * 4);
    L.w = take((size_t)T * k * 4);
    L.nuniq = take(4);
    L.wt = take((size_t)L.UI * 32);
    L.ptok = take((size_t)L.P * 4);
    L.inv = take((size_t)L.P * 4);
    L.pw = take((size_t)L.P * 4);
    L.henc = take((size_t)L.P * enc_bytes(L.kd));
    L.hf = take((size_t)L.P * L.kd * 4);
    L.total = o;
    return L;
}

// Chained single-token layers (moe_layer_forward_chain, moe_cache_ffn_device):
// where this layer's router dots come from (rp_in, or null: the route launch
// ran) and where the next layer's go.
struct Chain {
    const float *rp_in;
    float *rp_out;
    const float *wn;  // the next layer's router [En][H]
    int En;
    const float *bias;
    float eps;
    bool dlog_keys;   // with rp_in: rank the keys at kDlog (formed by the cache lookup), not the partials
};
// The chain's hand-off buffer of the given parity in a workspace
inline float *chain_buf(void *ws, int parity)
{
    return (float *)((uint8_t *)ws + kChain) + (size_t)parity * (kChainBufBytes / 4);
}
moe_status launch_ffn_copy(const moe_expert_desc *d, float *h, int E, int k, const void *const *eptr,
                           const void *const *sptr, int n_shared, void *ws, size_t ws_bytes, hipStream_t s,
                           const CacheCopy *cc, const Chain *ch);

// Error reporting (thread-local message).
void set_error(const char *fmt, ...);

}  // namespace moe
