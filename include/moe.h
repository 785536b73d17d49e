/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) decode-time MoE expert FFN.
 *
 * The library computes one Mixture-of-Experts FFN layer for a small decode
 * batch (T <= 32 tokens for the fused layer calls and the cache; the
 * stand-alone router and FFN calls also take prompt-sized batches of up to
 * 256) whose experts are stored as GGUF-style quantized
 * blocks: router GEMV, softmax top-k with renormalised weights, grouping of
 * (token, expert) pairs, gate/up quantized matvecs with SiLU(gate)*up, the
 * down matvec and the weighted combine (plus always-active shared experts
 * and the residual add).  Beside it sits a slot-pool expert cache that keeps
 * hot experts in HBM and uploads misses from pinned host memory.
 *
 * Sources (pages on the method): the gating step and its softmax top-k are
 * described in the MoE offload blog (mhpn.cn, sections 3.1 and 5.2); the
 * slot-pool cache, its grouping of experts by tensor type and shape, the LRU
 * eviction, the 32-token batch limit and the budget planner are described in
 * the T4 MoE-cache report (kongchang.com, sections "What the MoE cache
 * caches" and "Size your experts before configuring"); a GPU matvec that
 * keeps weights in their quantized blocks is described in the GPU-offload
 * research notes (kwkr.cn, section 1.2).
 *
 * Conventions for every call:
 *  - Pointers documented as "device" must point to GPU memory of the current
 *    HIP device; "host" pointers to host memory; "pinned" to memory from
 *    hipHostMalloc.  The caller owns every buffer it passes in.
 *  - GPU work is enqueued on the given stream and the call returns at once.
 *    Argument and shape errors are detected on the host before anything is
 *    enqueued and returned synchronously; nothing is enqueued then.  Launch
 *    failures return MOE_ERR_HIP.  No exception crosses the ABI.
 *  - On any error, moe_last_error() returns a message (thread-local).
 *  - Layouts are row-major and tightly packed unless stated otherwise.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_ARG = -1,      /* null pointer, negative size, k > E, ... */
    MOE_ERR_SHAPE = -2,    /* row length not a whole number of tiles/blocks */
    MOE_ERR_QTYPE = -3,    /* unknown quantization type */
    MOE_ERR_BUDGET = -4,   /* cache budget below the floor for some group */
    MOE_ERR_CAPACITY = -5, /* more distinct experts in one layer-step than slots */
    MOE_ERR_HIP = -6,      /* a HIP runtime call failed */
    MOE_ERR_BATCH = -7,    /* T outside [1, 32] */
    MOE_ERR_STATE = -8     /* call out of order (e.g. upload before lookup) */
} moe_status;

/* Block formats (public GGUF layouts; the pages name them but print no bit
 * packing -- T4 MoE-cache report, section "What the MoE cache caches", names
 * Q4_K/Q6_K; the GPU-offload research notes, section 1.2, give the 34-byte
 * q8_0 block):
 *   MOE_Q8_0: 32 weights / 34 B: fp16 d, int8 q[32];            w = d*q
 *   MOE_Q4_K: 256 weights / 144 B: fp16 d, fp16 dmin, 12 B of packed 6-bit
 *             scales and mins of 8 sub-blocks, 128 B of 4-bit q;  w = d*sc*q - dmin*m
 *   MOE_Q6_K: 256 weights / 210 B: 128 B low 4 bits, 64 B high 2 bits,
 *             int8 sc[16] (one per 16 weights), fp16 d;         w = d*sc*(q-32) */
typedef enum { MOE_Q8_0 = 1, MOE_Q4_K = 2, MOE_Q6_K = 3 } moe_qtype;

/* One expert's shape: gate and up are [I, H] (rows of H weights), down is
 * [H, Ipad] with Ipad = I rounded up to a multiple of 256 (the tile width,
 * for every type; the padded columns multiply zeros).  Requirements: H a
 * multiple of 256, I a multiple of 64, the three qtypes valid. */
typedef struct {
    int32_t gate, up, down; /* moe_qtype of each matrix */
    int32_t H, I;
} moe_expert_desc;

/* Thread-local text of the last error (never NULL). */
const char *moe_last_error(void);

/* ---------------------------------------------------------------------- */
/* Expert storage.                                                         */

/* Bytes of one expert (gate + up + down) in either layout; the slot layout
 * permutes the canonical bytes and adds nothing.  Returns -1 on a bad desc. */
int64_t moe_expert_bytes(const moe_expert_desc *d);

/* Padded down-row length Ipad of the desc (see moe_expert_desc), -1 on error. */
int32_t moe_down_k(const moe_expert_desc *d);

/* Repack one expert from canonical GGUF blocks (row-major rows of whole
 * blocks: gate [I,H], up [I,H], down [H,Ipad]; host memory) into the slot
 * layout read by moe_expert_ffn (host memory, moe_expert_bytes(d) bytes).
 * The slot layout groups 64 rows x 256 columns into one contiguous tile and
 * inside a tile stores each 16-byte piece of a block for all 64 rows side by
 * side, so that 64 lanes reading the same piece of 64 rows read 1 KiB of
 * consecutive bytes.  Pure host function, no GPU. */
moe_status moe_repack_expert(const moe_expert_desc *d, const void *gate, const void *up,
                             const void *down, void *slot, size_t slot_bytes);

/* ---------------------------------------------------------------------- */
/* Steps of the decode path.                                               */

/* xhat[t] = h[t] / sqrt(mean(h[t]^2) + eps), per token.  h, xhat: device
 * fp32 [T, H].  (Weightless pre-norm of the layer stack; the pages give no
 * stack composition, so the residual pre-norm block is this library's
 * reading.) */
moe_status moe_rmsnorm(const float *h, int32_t T, int32_t H, float eps, float *xhat, hipStream_t s);

/* Router and top-k (MoE offload blog, section 3.1: router logits, softmax,
 * pick the k best experts; the batched form is section 5.2).
 *   x        device fp32 [T, H], the normalised token states
 *   w_router device fp32 [E, H]
 *   bias     device fp32 [E] or NULL (added to the logits)
 *   idx      device int32 [T, k]: expert ids by descending logit, ties to
 *            the lower id
 *   w        device fp32 [T, k]: softmax over the k selected logits (equal
 *            to the full softmax renormalised over the k winners)
 *   logits   device fp32 [T, E] or NULL
 * 1 <= T <= 256 (prompt-sized batches too), 1 <= k <= E <= 1024, k <= 64,
 * H a multiple of 256. */
moe_status moe_route_topk(const float *x, int32_t T, int32_t H, const float *w_router,
                          const float *bias, int32_t E, int32_t k, int32_t *idx, float *w,
                          float *logits, hipStream_t s);

/* Stable counting sort of the T*k (token, slot) pairs by expert.
 *   idx    device int32 [T, k], values in [0, E)
 *   count  device int32 [E]
 *   offset device int32 [E+1], exclusive prefix sum of count
 *   pairs  device int32 [T*k], entries t*k+j ordered by (expert, token, slot) */
moe_status moe_group_tokens(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *count,
                            int32_t *offset, int32_t *pairs, hipStream_t s);

/* Device scratch needed by moe_expert_ffn / moe_layer_forward for batches
 * of up to T tokens (counters, grouped pairs, activation encodings,
 * per-pair outputs).  Returns 0 on a bad argument. */
size_t moe_workspace_bytes(const moe_expert_desc *d, int32_t T, int32_t k, int32_t E, int32_t n_shared);

/* Zero a workspace (a fill kernel on stream s, no hipMemset) before its
 * first use.  The kernels leave their counters at zero when they finish, so
 * a workspace is reusable by any later call of the same or smaller sizes.
 * Calls that share one workspace must be ordered (same stream or events).
 * ws == NULL (ws_bytes ignored) clears the static scratch array of
 * moe_layer_forward_noalloc on the current device instead (no allocation).
 * This is also the one way to clear a workspace's status word (below). */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t s);

/* Status word of a workspace.  The route launch of moe_layer_route,
 * moe_layer_forward and moe_layer_forward_noalloc hands logit keys (and,
 * above 16 tokens, each token's top-k) between its workgroups through the
 * workspace, and the receiving workgroup waits for them with a bounded poll.
 * A poll that gives up -- never seen in normal operation: it means the
 * sending workgroups were not scheduled within about a million polling
 * rounds -- sets a bit here and routes that launch with NaN weights (idx_out
 * ids stay in [0, E)), so the routing outputs and the updated state are NaN
 * and no caller can miss it.  The bits are sticky: since late senders may
 * still write into the hand-off arrays, every later route launch on the
 * workspace that would read them routes with NaN weights too (without
 * waiting) until moe_workspace_init clears the workspace.  Exceptions: a
 * single token on the dot-product path with E <= 128 and H <= 4096 is ranked
 * again inside moe_layer_ffn's gate/up kernel from plainly stored logits, not
 * from the hand-off: its updated state stays exact (only idx_out / w_out, when
 * requested, show the NaN weights).  2 to 8 tokens on the integer-MFMA path
 * (all-Q4_K experts) with E <= 256 are ranked there too; without idx_out and
 * w_out the route launch then hands nothing over and waits for nothing, but
 * that gate/up kernel still routes with NaN weights while a bit is set, as the
 * route launch would. */
enum {
    MOE_WS_KEYS_TIMEOUT = 1, /* the wait for the router's logit keys gave up */
    MOE_WS_TOPK_TIMEOUT = 2, /* a wait on the per-token top-k hand-off gave up */
    MOE_WS_COPY_TIMEOUT = 4  /* moe_cache_ffn_device: a wait for a missed expert's copy gave up */
};
/* Byte offset of the status word (uint32) in every workspace, for callers
 * that check it on the device or from a captured graph. */
#define MOE_WS_STATUS_OFFSET 147456u

/* Read a workspace's status word (0: no wait has given up).  Waits for the
 * work queued on s (stream-synchronous).  ws == NULL reads the static scratch
 * array of moe_layer_forward_noalloc on the current device (0 if no call has
 * used it yet).  MOE_ERR_ARG for a null status or a workspace too small to
 * hold the word; MOE_ERR_HIP if the copy fails. */
moe_status moe_workspace_status(const void *ws, size_t ws_bytes, uint32_t *status, hipStream_t s);

/* Test hook for the give-up path above, for the route launches (and the
 * waits for missed experts' copies of moe_cache_ffn_device) that follow
 * this call in the process.  rounds: polling rounds after which a wait gives
 * up (0 restores the default of 2^20; 1 makes a give-up likely whenever a
 * sender is late).  withhold_keys != 0: the router workgroups store no logit
 * keys into the hand-off, so every wait for them gives up after `rounds`
 * (the plainly stored single-token logits are still written).  Production
 * code never calls this; (0, 0) restores normal operation. */
void moe_set_spin_limit(uint32_t rounds, int32_t withhold_keys);

/* Expert FFN and weighted combine for one layer:
 *   y[t] = (accumulate ? y[t] : 0) + sum_j w[t,j] * FFN_{idx[t,j]}(x[t]) + sum_s FFN_shared_s(x[t])
 *   FFN_e(x) = down_e( SiLU(gate_e x) * (up_e x) )
 * (gate/up/down expert tensors: T4 MoE-cache report, section "What the MoE
 * cache caches"; shared experts of weight one: laptop 16B MoE post, lpnh.cn,
 * section 2.1.)
 *   d           expert shape, shared by all experts of the layer
 *   x           device fp32 [T, H] normalised states
 *   idx, w      device int32 / fp32 [T, k] routing (ids distinct per token)
 *   expert_ptrs device array [E] of device addresses of each expert in the
 *               slot layout (only the selected entries are read)
 *   shared_ptrs device array [n_shared] of slot-layout addresses, or NULL
 *               when n_shared == 0
 *   y           device fp32 [T, H]
 *   act_out     NULL, or device fp32 [T*(k+n_shared), Ipad]: SiLU(g)*u of
 *               every pair, in grouped order (routed experts by ascending
 *               id then token; then each shared expert by token); columns
 *               [I, Ipad) are not written
 *   ws          workspace from moe_workspace_bytes(d, >=T, >=k, >=E, >=n_shared),
 *               initialised once with moe_workspace_init
 * 1 <= T <= 256 (batches above 32 tokens, prompt-sized, are grouped by a
 * one-workgroup kernel into work entries of at most 32 pairs on the MFMA
 * path, 4 otherwise).  The experts' contributions are added into y with float
 * atomics, so the order of the sum over a token's experts follows the
 * order in which workgroups finish: results agree with any fixed order to
 * fp32 rounding, but their last bits can differ from run to run.  The same
 * holds for moe_layer_ffn and moe_layer_forward.  All-Q4_K experts with
 * T > 8 run on matrix cores (fp16 MFMA with fp32 accumulation of exact
 * integer weights and a two-part activation split). */
moe_status moe_expert_ffn(const moe_expert_desc *d, const float *x, int32_t T, int32_t k,
                          int32_t E, const int32_t *idx, const float *w,
                          const void *const *expert_ptrs, const void *const *shared_ptrs,
                          int32_t n_shared, float *y, int32_t accumulate, float *act_out,
                          void *ws, size_t ws_bytes, hipStream_t s);

/* First half of moe_layer_forward (one kernel): RMSNorm of h, router
 * logits (+ bias), softmax top-k, grouping of the (token, expert) pairs and
 * the encoding of the normalised states, all left in the workspace for the
 * moe_layer_ffn that follows on the same stream and workspace.
 *   expert_ptrs / shared_ptrs  NULL, or the expert address tables when their
 *       entries are final when this kernel runs (resident experts): the
 *       grouping then records each selected expert's address and the FFN
 *       kernels skip one dependent load.  With a slot cache, whose table is
 *       refreshed after the routing is known, pass NULL.
 *   idx_out / w_out as in moe_layer_forward. */
moe_status moe_layer_route(const moe_expert_desc *d, const float *h, int32_t T, const float *w_router,
                           const float *bias, int32_t E, int32_t k, const void *const *expert_ptrs,
                           const void *const *shared_ptrs, int32_t n_shared, float eps,
                           int32_t *idx_out, float *w_out, void *ws, size_t ws_bytes, hipStream_t s);

/* Second half (two kernels): the expert FFN of the pairs grouped by the
 * preceding moe_layer_route in `ws`, weighted combine, h += result.  T, E,
 * k and n_shared must equal those of that moe_layer_route. */
moe_status moe_layer_ffn(const moe_expert_desc *d, float *h, int32_t T, int32_t E, int32_t k,
                         const void *const *expert_ptrs, const void *const *shared_ptrs, int32_t n_shared,
                         void *ws, size_t ws_bytes, hipStream_t s);

/* One whole pre-norm residual MoE layer, fused into three kernels:
 *   xhat = RMSNorm(h); idx, w = top-k(router(xhat) + bias); h += MoE(xhat)
 *   h           device fp32 [T, H], updated in place
 *   idx_out     NULL or device int32 [T, k]; w_out NULL or device fp32 [T, k]
 * Other arguments as for moe_route_topk and moe_expert_ffn. */
moe_status moe_layer_forward(const moe_expert_desc *d, float *h, int32_t T, const float *w_router,
                             const float *bias, int32_t E, int32_t k,
                             const void *const *expert_ptrs, const void *const *shared_ptrs,
                             int32_t n_shared, float eps, int32_t *idx_out, float *w_out,
                             void *ws, size_t ws_bytes, hipStream_t s);

/* moe_layer_forward for consecutive single-token layers of a stack (the
 * decode step of the MoE offload blog, section 3.1, layer after layer):
 * the same update of h, with the next layer's router dot products started
 * in this layer's FFN kernels, so that the next layer needs no route launch
 * (two kernels per layer instead of three).  The router logits are linear in
 * the state, so the next router's dots with this layer's output are the
 * dots with its input (computed by the gate/up kernel) plus the dots with
 * each expert's weighted contribution (added by the down kernel's
 * workgroups, 64 positions each, with float atomics); the next layer's
 * gate/up kernel sums them, applies 1/RMS and the bias, ranks them and
 * encodes the normalised state itself.
 *   chain_in     nonzero: the previous call on this workspace and stream was
 *                given this layer's router as next_router (w_router is then
 *                not read; bias and eps are); zero: this call routes with a
 *                route launch as moe_layer_forward does
 *   next_router  NULL (last layer of the chain), or the next layer's router,
 *                device fp32 [next_E, H]; the next call must use the same h
 *   next_E       rows of next_router, 1 .. 128
 *   parity       0 or 1: which of the workspace's two hand-off buffers this
 *                call reads (chain_in); it writes the other one, so
 *                consecutive calls alternate (the layer index mod 2)
 * Chaining needs T == 1 on the single-token kernels: E <= 128, H <= 4096,
 * the dot-product path (moe_layer_chain_supported); otherwise MOE_ERR_ARG
 * (nothing enqueued).  With chain_in == 0 and next_router == NULL this is
 * moe_layer_forward without idx_out / w_out.  The logits are the same sums in
 * another order (fp32 rounding; the last bits vary from run to run, as the
 * combine's do).  Other arguments as for moe_layer_forward. */
moe_status moe_layer_forward_chain(const moe_expert_desc *d, float *h, int32_t T, const float *w_router,
                                   const float *bias, int32_t E, int32_t k, const void *const *expert_ptrs,
                                   const void *const *shared_ptrs, int32_t n_shared, float eps, int32_t chain_in,
                                   const float *next_router, int32_t next_E, int32_t parity, void *ws,
                                   size_t ws_bytes, hipStream_t s);

/* 1 if a layer of this desc, T tokens and E experts can be chained with
 * moe_layer_forward_chain, else 0.  Pure host function. */
int32_t moe_layer_chain_supported(const moe_expert_desc *d, int32_t T, int32_t E);

/* moe_layer_forward without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the layer runs in a library-owned static scratch array of 8 MiB per GPU,
 * held from the first call on that GPU until the process ends (the first
 * call also clears it on stream s).  Arguments as for moe_layer_forward.
 * MOE_ERR_CAPACITY (nothing enqueued) when the layer needs more scratch than
 * the array holds (moe_workspace_bytes of the same sizes; every
 * configuration of up to 32 tokens with H, I <= 4096 and E <= 256 fits).  Every call on
 * a GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams without ordering) race. */
moe_status moe_layer_forward_noalloc(const moe_expert_desc *d, float *h, int32_t T, const float *w_router,
                                     const float *bias, int32_t E, int32_t k, const void *const *expert_ptrs,
                                     const void *const *shared_ptrs, int32_t n_shared, float eps,
                                     int32_t *idx_out, float *w_out, hipStream_t s);

/* ---------------------------------------------------------------------- */
/* Expert slot-pool cache (T4 MoE-cache report, sections "What the MoE cache
 * caches" and "Size your experts before configuring").  Experts are grouped
 * by (type, shape) -- one moe_expert_desc per group -- and each group owns
 * one pool of fixed-size slots in HBM shared by all of its layers.  A
 * lookup of a layer-step's distinct experts hits (the expert is in a slot)
 * or misses (the least recently used key of the group is evicted and its
 * slot reassigned); misses are then uploaded from pinned host memory with
 * hipMemcpyAsync on a copy stream.  Only batches of up to 32 tokens use the
 * cache. */

/* Slots per group for a byte budget: each group gets the same share of its
 * (layer, expert) keys,
 *     slots[g] = floor(budget * layers[g] / sum_h layers[h] * bytes[h]) - 1,
 * and a group below top_k slots is disabled (0).  This reproduces the
 * report's printed figures (1,834 slots per group at 10,000 MiB for
 * Qwen3-30B-A3B Q4_K_M; 50 MiB accepted, 49 MiB refused).
 *   groups [n_groups] host, layers_per_group [n_groups] host, slots_out
 *   [n_groups] host.  Returns MOE_ERR_BUDGET when every group is disabled
 *   (slots_out still filled). */
moe_status moe_cache_plan(const moe_expert_desc *groups, const int32_t *layers_per_group,
                          int32_t n_groups, uint64_t budget_bytes, int32_t top_k,
                          int32_t *slots_out);

/* Placement of a stack's experts in a VRAM budget (T4 MoE-cache report,
 * section "Two ways to run: automatic placement vs manual takeover"):
 *   MOE_PLACE_FIT         layer granularity, as --fit with a cache: the
 *                         cache reserves cache_bytes, layers are made
 *                         resident whole in layer order while they fit in
 *                         the rest of vram_bytes (a layer that does not fit
 *                         is skipped, a later smaller one may still fit), and
 *                         the layers left over are served by the cache, whose
 *                         slots are planned over them alone;
 *   MOE_PLACE_ALL_CACHED  expert granularity, as --cpu-moe with a cache:
 *                         no layer resident, all of vram_bytes to the cache.
 *   groups [n_groups]; layer_group [n_layers] the group of each layer (>= 0);
 *   E experts per layer; vram_bytes the budget for expert bytes (resident
 *   layers plus pools); cache_bytes the pool budget (FIT only); top_k the
 *   slot floor per group.
 *   layer_state [n_layers] out: the group g of a cached layer, or -(g+1) for
 *   a resident one -- the layer_group argument of moe_cache_create;
 *   slots_out [n_groups] out (0 for a group with no cached layer).
 * MOE_ERR_BUDGET when a group with cached layers gets fewer than top_k
 * slots (the outputs are still filled); MOE_ERR_ARG for bad arguments.
 * (Computing missed experts on the host CPU, as --cpu-moe without a cache
 * does, is not offered: every step of the path runs in this library's GPU
 * kernels.)  Pure host function. */
enum { MOE_PLACE_FIT = 1, MOE_PLACE_ALL_CACHED = 2 };
moe_status moe_placement_plan(const moe_expert_desc *groups, int32_t n_groups, const int32_t *layer_group,
                              int32_t n_layers, int32_t E, uint64_t vram_bytes, uint64_t cache_bytes,
                              int32_t top_k, int32_t mode, int32_t *layer_state, int32_t *slots_out);

typedef struct moe_cache moe_cache;

/* Create a cache.
 *   groups [n_groups], slots [n_groups] as moe_cache_plan gives them.  A
 *   group with 0 slots is below the budget floor and is not cached: its
 *   layers keep all of their experts resident in HBM (uploaded here, once),
 *   their lookups are answered without touching any pool and count in no
 *   statistic, and a warning goes to stderr and to moe_last_error() (the
 *   T4 MoE-cache report, section "Size your experts before configuring":
 *   a group below the floor is left out with a warning; only a budget that
 *   disables every group is refused).  MOE_ERR_BUDGET when every group has 0
 *   slots while some layer asks for caching, MOE_ERR_ARG for a negative
 *   count.
 *   layer_group [n_layers]: the group g of each layer, or -(g+1) for a
 *   layer whose experts stay resident (shape of group g; see
 *   moe_placement_plan), host_experts [n_layers * E]
 *   pinned host addresses of each expert in the slot layout (the pinned
 *   memory stays owned by the caller and must outlive the cache).  Allocates
 *   one device pool per group (hipMalloc) and one device pointer table per
 *   layer. */
moe_status moe_cache_create(const moe_expert_desc *groups, int32_t n_groups, const int32_t *slots,
                            const int32_t *layer_group, int32_t n_layers, int32_t E,
                            const void *const *host_experts, moe_cache **out);

/* Where a cache keeps its pools and how it fills them.  The default
 * (moe_cache_create) is hipMalloc'd HBM and hipMemcpyAsync from pinned host
 * memory on the caller's copy stream.  A caller-supplied backend is
 * synchronous: alloc returns memory for the pools and the slot tables,
 * copy must have read src and written dst when it returns, and a non-zero
 * return from copy is an upload failure (moe_cache_upload then rolls the
 * lookup back, see there).  Such a cache runs the host LRU only (no
 * moe_cache_device_enable), makes no HIP call, and serves hit-rate
 * simulation of a budget without a GPU and the failure tests of the LRU. */
typedef struct {
    void *user;
    int32_t (*alloc)(void *user, size_t bytes, void **out); /* 0 on success */
    void (*release)(void *user, void *p);
    int32_t (*copy)(void *user, void *dst, const void *src, size_t bytes); /* 0 on success */
} moe_cache_backend;

/* moe_cache_create with an explicit backend (NULL: the default). */
moe_status moe_cache_create_ex(const moe_expert_desc *groups, int32_t n_groups, const int32_t *slots,
                               const int32_t *layer_group, int32_t n_layers, int32_t E,
                               const void *const *host_experts, const moe_cache_backend *backend,
                               moe_cache **out);

/* Look up one layer-step (T4 MoE-cache report, section "What the MoE cache
 * caches": LRU over (layer, expert) keys in the group's pool).
 *   idx        host int32 [T*k], the selected ids of the step's T tokens,
 *              each in [0, E); repeats allowed
 * The step's distinct ids are looked up once each in ascending order; they
 * go to experts_out (host int32 [T*k]), their number to *n_out.  Per
 * distinct expert: slot_out (host int32 [T*k]), hit_out (host uint8 [T*k]),
 * victim_layer / victim_expert (host int32 [T*k], -1 when nothing was
 * evicted; either may be NULL).  A hit refreshes the expert's recency; a
 * miss takes the group's next never-used slot, else evicts the least
 * recently used key of the group, whose entry in its layer's slot table
 * becomes NULL (the cleared rows reach the device with the next
 * moe_cache_upload).  The misses are recorded for the next moe_cache_upload
 * of this layer.  For a layer of a group with 0 slots (resident, see
 * moe_cache_create) every expert is reported as a hit in slot -1 and nothing
 * is recorded.  Returns MOE_ERR_CAPACITY when the distinct ids exceed the
 * group's slots and MOE_ERR_BATCH when T > 32 (state unchanged in both
 * cases). */
moe_status moe_cache_lookup(moe_cache *c, int32_t layer, int32_t T, int32_t k, const int32_t *idx,
                            int32_t *experts_out, int32_t *n_out, int32_t *slot_out, uint8_t *hit_out,
                            int32_t *victim_layer, int32_t *victim_expert);

/* Enqueue the misses recorded by the last lookup of `layer` as copies from
 * pinned host memory into their slots (hipMemcpyAsync on copy_stream), then
 * the slot-table rows that changed since their last upload (this layer's
 * and those of evicted keys), then record `done` (may be NULL; must be NULL
 * with a caller-supplied backend, which ignores copy_stream) on copy_stream.
 * The compute stream waits on `done` before the FFN reads the slots.  If a
 * copy cannot be enqueued (or a backend's copy fails), the lookup is rolled
 * back from that miss on: the misses already enqueued stay (their slots are
 * being filled), and the rest of the lookup's decisions are undone in
 * reverse order (keys, recency order, free-slot count, evicted keys put back
 * in their untouched slots, table entries, statistics), as if the lookup had
 * stopped before that miss; MOE_ERR_HIP is returned and the layer may be
 * looked up again. */
moe_status moe_cache_upload(moe_cache *c, int32_t layer, hipStream_t copy_stream, hipEvent_t done);

/* Device array [E] of slot addresses of `layer` (NULL for experts that are
 * not resident: never looked up, or evicted).  The array is owned by the
 * cache and is valid after the upload of the layer completes (with the
 * device lookup: after moe_cache_lookup_device).  Pass it as expert_ptrs. */
const void *const *moe_cache_expert_ptrs(moe_cache *c, int32_t layer);

typedef struct {
    uint64_t lookups, hits, misses, evictions, upload_bytes;
    uint64_t lookups_le8, hits_le8;     /* steps with T <= 8 */
    uint64_t lookups_9_32, hits_9_32;   /* steps with 9 <= T <= 32 */
    /* batches above 32 tokens (moe_cache_stage_large): experts copied from
     * their slots into the caller's staging area, and experts uploaded there
     * from host memory because no slot held them */
    uint64_t large_copies, large_uploads;
} moe_cache_stats_t;

moe_status moe_cache_stats(const moe_cache *c, moe_cache_stats_t *out);

/* Reset statistics (not the cache contents). */
moe_status moe_cache_reset_stats(moe_cache *c);

/* Switch the cache to lookups on the device (before any host lookup): the
 * LRU state moves to device memory (a last-use stamp and a key per slot per
 * group, from one clock, and the key->slot map), so that a layer-step's
 * lookup and miss uploads run on a stream with no host synchronization (and
 * can be captured in a HIP graph).  Same policy as moe_cache_lookup (T4
 * MoE-cache report, sections "What the MoE cache caches" and "Size your
 * experts before configuring"): the distinct selected ids in ascending
 * order; a hit refreshes its slot; a miss takes the group's next never-used
 * slot, else the least recently used one (smallest stamp).  The host
 * copies must be pinned memory the device can read (hipHostMalloc; torch
 * pin_memory); their device addresses are taken here.  trace_capacity > 0
 * keeps the first trace_capacity lookups (see moe_cache_trace_read).  After
 * this call moe_cache_lookup and moe_cache_upload return MOE_ERR_STATE;
 * moe_cache_stats and moe_cache_reset_stats synchronize the device.
 * Returns MOE_ERR_CAPACITY when a group has more than 16384 slots. */
moe_status moe_cache_device_enable(moe_cache *c, int32_t trace_capacity);

/* Device lookup of one layer-step on `stream`: idx (device int32 [T][k],
 * the layer's selected ids as moe_layer_route writes them) -> the LRU
 * update, the layer's row of moe_cache_expert_ptrs, and the misses' copies
 * from pinned host memory into their slots (a kernel reading the host
 * memory over the bus).  Work on `stream` after this call sees the
 * experts in their slots.  Calls on one cache must be ordered (one stream,
 * or the caller's events).  MOE_ERR_CAPACITY when T*k exceeds the layer's
 * group's slots, MOE_ERR_BATCH when T > 32. */
moe_status moe_cache_lookup_device(moe_cache *c, int32_t layer, const int32_t *idx, int32_t T, int32_t k,
                                   hipStream_t stream);

/* moe_cache_lookup_device for a single token whose routing the layer calls
 * leave to the FFN kernels: the lookup kernel itself selects the k largest
 * of the logit keys that the moe_layer_route before it on `stream`, on
 * workspace ws, wrote (called without idx_out / w_out, so that its launch
 * has no routing tail), ties to the lower id, as moe_layer_route's top-k
 * does; then as moe_cache_lookup_device with those ids.  This saves the
 * route launch's tail on the cached decode path.  MOE_ERR_ARG when the
 * layer's group would not leave the keys (its route launch routes itself:
 * E > 128, or experts off the dot-product path at T=1). */
moe_status moe_cache_lookup_device_route(moe_cache *c, int32_t layer, const void *ws, size_t ws_bytes, int32_t k,
                                         hipStream_t stream);

/* moe_cache_lookup_device_route followed by the layer's FFN (moe_layer_ffn
 * on the cache's table of the layer), with the misses copied inside the FFN's
 * gate/up launch instead of by a launch of their own (Laptop post §2.3: the
 * copies overlap the compute): that launch's first workgroups copy each
 * missed expert from its pinned host copy into its slot, while the hit
 * experts' workgroups start at once; a missed expert's workgroups wait for
 * their copy (bounded; a wait that gives up sets MOE_WS_COPY_TIMEOUT in the
 * workspace's status word and makes the layer's outputs NaN).  One token (T=1)
 * after a moe_layer_route on the same stream and workspace, as for
 * moe_cache_lookup_device_route; h, d, shared_ptrs, n_shared, ws as for
 * moe_layer_ffn.  A layer kept resident runs its FFN alone.
 * Chained layers, as in moe_layer_forward_chain (single-token kernels: E <=
 * 128, H <= 4096): next_router (NULL: none) [next_E, H] makes this call leave
 * the next layer's router dots in the workspace's hand-off buffer parity^1;
 * chain_in != 0 takes this layer's from buffer `parity` (left by the previous
 * call, given this layer's router), so that no moe_layer_route precedes the
 * call: the lookup forms the logit keys from them (with bias [E] or NULL and
 * eps, the layer's RMSNorm) and stores them where the FFN ranks them.
 * With chain_in == 0 and next_router == NULL, bias and eps are not read.
 * Errors as for the two calls it replaces; MOE_ERR_ARG for a chain outside
 * the single-token kernels or a bad next_E / parity. */
moe_status moe_cache_ffn_device(moe_cache *c, int32_t layer, const moe_expert_desc *d, float *h, int32_t k,
                                const void *const *shared_ptrs, int32_t n_shared, const float *bias, float eps,
                                int32_t chain_in, const float *next_router, int32_t next_E, int32_t parity,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* Cross-layer prefetch (Laptop post, section 2.3: the experts of the next
 * layers are fetched while the current one computes).  idx (device int32
 * [T][k]): the ids predicted for `layer`, e.g. its router applied to an
 * earlier layer's state.  The lookup runs on `stream`, the stream of every
 * other lookup of the cache, and counts in the statistics and the trace
 * like any lookup; the misses' copies run on `copy_stream` (which must
 * differ from `stream`) after the work queued on `stream` so far, so they
 * overlap what `stream` does next.  The next moe_cache_lookup_device of
 * `layer` makes its stream wait for those copies.  Because the copies are
 * still running, the library refuses (MOE_ERR_CAPACITY) a lookup or
 * prefetch that touches so many slots of the group that a prefetched slot
 * could become the victim before that wait; MOE_ERR_STATE when `layer`
 * already has a prefetch not yet taken by its lookup, MOE_ERR_BATCH when
 * T > 32. */
moe_status moe_cache_prefetch_device(moe_cache *c, int32_t layer, const int32_t *idx, int32_t T, int32_t k,
                                     hipStream_t stream, hipStream_t copy_stream);

/* Copy the device trace (synchronizes): records of 4 int32 (layer, expert,
 * hit 1/0, evicted key layer*E+expert or -1), in lookup order; *n gets the
 * number of lookups made (the device keeps the first trace_capacity). */
moe_status moe_cache_trace_read(moe_cache *c, int32_t *out, int32_t capacity, int32_t *n);

/* Batches above 32 tokens (prompt processing) leave the slots alone (T4
 * MoE-cache report, section "What the MoE cache caches": larger batches do
 * not go through the cache; the experts they need that the cache holds are
 * copied from it, its log counts them).  The layer's distinct selected
 * experts are staged in a caller-owned device area instead: an expert that a
 * slot holds is copied from the slot device to device (statistic
 * large_copies), any other is read from its pinned host copy
 * (large_uploads).  The LRU state, its statistics and its trace are not
 * touched.  A resident layer stages nothing: its table is its own.
 *   idx          host int32 [T*k] (moe_cache_stage_large) or device int32
 *                [T*k] (moe_cache_stage_large_device), ids in [0, E)
 *   staging      device area of at least min(E, T*k) * expert bytes of the
 *                layer's group; the u-th distinct id (ascending) lands at
 *                staging + u * expert bytes
 *   table_out    device array [E] (caller-owned): the staged address of each
 *                selected expert, NULL for the others; pass it as the
 *                expert_ptrs of moe_expert_ffn
 *   s            the stream of the FFN; work queued on it after this call sees
 *                the staged experts.  With the host LRU, s must already be
 *                ordered after the uploads of earlier lookups (their slots are
 *                read); with a caller-supplied backend the copies are done on
 *                return and s is ignored.
 * 33 <= T <= 256 (MOE_ERR_BATCH otherwise), MOE_ERR_ARG when staging is too
 * small.  moe_cache_stage_large needs the host LRU, moe_cache_stage_large_device
 * the device one (MOE_ERR_STATE otherwise). */
moe_status moe_cache_stage_large(moe_cache *c, int32_t layer, int32_t T, int32_t k, const int32_t *idx,
                                 void *staging, size_t staging_bytes, void **table_out, hipStream_t s);
moe_status moe_cache_stage_large_device(moe_cache *c, int32_t layer, int32_t T, int32_t k, const int32_t *idx,
                                        void *staging, size_t staging_bytes, void **table_out, hipStream_t s);

/* Drain outstanding copies and free the pools and tables. */
void moe_cache_destroy(moe_cache *c);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
