// moe_kernels.hip -- gfx950 kernels and compute entry points of libmoe.
//
// Decode path of one MoE layer (T <= 32 tokens), three launches:
//
//   k_route    router GEMV, 2 router rows per workgroup against a group of up
//              to 8 tokens (the 8 waves split H; the sum of squares of the
//              state rides along for the RMSNorm), each logit handed to the
//              tail as an order-preserving 32-bit key; encoding workgroups
//              write each token's normalised state as activation records;
//              above 16 tokens one top-k workgroup per token; the last
//              workgroup (the tail) polls the keys (bounded), takes the
//              softmax top-k and groups the (token, expert) pairs into a work
//              table of items of at most 4 pairs, largest first.  A single
//              token has no tail (unless the caller asks for its routing):
//              the router workgroups also store the keys plainly and every
//              k_gate_up workgroup ranks them itself after the launch
//              boundary.  For 2 .. 8 tokens on the integer-MFMA kernels the
//              tail stops after the softmax and k_gate_up_i8 groups the pairs.
//              Consecutive single-token layers can be chained
//              (moe_layer_forward_chain): only the first runs k_route; each
//              layer's k_gate_up and k_down also leave the next layer's
//              router dots as partial sums over 64-position tiles, and the
//              next k_gate_up forms the logits, ranks them and encodes the
//              normalised state itself.
//   k_gate_up  one workgroup per (work item, 32-row tile): the gate and up
//              rows of the item's expert against its tokens, SiLU(g)*u, and
//              the encoding of those 32 values as one activation block.
//   k_down     one workgroup per (work item, 64-row tile): down rows against
//              SiLU(g)*u; each pair's rows, times its combine weight, are
//              added into the token's rows of y with float atomics (y holds
//              the residual already, so no combine pass follows).
// Batches of 2 to 8 tokens on all-Q4_K experts use k_gate_up_i8 / k_down_i8
// instead (integer MFMA on the int8 activation pieces and the weights' sc*q
// split into two int8 parts), batches of more than 8 k_gate_up_mfma /
// k_down_mfma (fp16 MFMA on the exact integer weights sc*q and a two-part
// split of the activations).  The slot-pool cache's device lookup and miss
// copies are k_cache_lookup and k_cache_copy.
//
// Gating follows the MoE offload blog (mhpn.cn, section 3.1: router logits,
// softmax, top-k; section 5.2: the batched form); matvecs that keep the
// weights in their quantized blocks follow the GPU-offload research notes
// (kwkr.cn, section 1.2); the gate/up/down expert tensors and the 32-token
// batch limit follow the T4 MoE-cache report (kongchang.com, section "What
// the MoE cache caches").
//
// Activation encoding.  Each block of 32 consecutive activation values v is
// stored as three int8 pieces with one fp32 scale s = m/127:
//     v ~= s * (x0 + x1/254 + x2/254^2),   |xi| <= 127,
// an error below s * 7.8e-6 = m * 6.1e-8, i.e. fp32 class.  m is the largest
// magnitude of the 256-position super-block for the normalised input states
// of batches on the integer-MFMA path (one scale per Q4_K super-block) and of
// the 32-value block itself otherwise.  Quantized
// weights are small integers times per-block scales, so the product of a
// weight block with an activation block is three exact integer dot products
// (v_dot4 on 4 int8 lanes) and a few fp32 operations per block.  This keeps
// the matvec near 1.3 VALU operations per weight, well under the ~2.7 that
// 8 TB/s of Q4_K leaves on 256 CUs, while the result stays within fp32
// rounding of the exact product.  The records are staged in LDS and read by
// broadcast (every lane of a wave owns a weight row and reads the same
// activation words).
//
// Cross-workgroup hand-off (router -> tail, top-k workgroups -> tail) uses
// relaxed agent-scope atomic stores and loads of words that are never zero
// once written (coherent across the XCDs' L2 caches without whole-cache
// write-back or invalidation); the tail polls them with a bounded loop and
// clears them for the next launch.  There is no arrival counter.  A wait that
// gives up sets a sticky bit in the workspace's status word (see RouteArgs).
#include <hip/hip_runtime.h>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <hip/hip_fp16.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr float kC1 = 1.0f / 254.0f;
constexpr float kC2 = 1.0f / 64516.0f;
constexpr int kChunk = 8;  // tokens per pass of the matvec kernels
constexpr int kRouteThreads = 256;
constexpr int kRouteRows = 2;                   // router rows per workgroup
constexpr int kRouteTok = 8;                    // tokens per pass of a router workgroup
constexpr int kRouteWG = 512;                   // threads of a k_route workgroup
constexpr int kEncPos = 512;                    // positions encoded per k_route encoding workgroup
constexpr int kMaxK = 64;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
// A value that is the same in every lane, moved to a scalar register.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Cross-lane exchanges without LDS: DPP quad permutes and row mirrors move
// data inside 16-lane rows, v_permlane16_swap / v_permlane32_swap (gfx950)
// between rows.  xchg_*(v) returns the value of a partner lane such that a
// symmetric reduction over (v, partner) pairs at steps 1, 2, 4, 8, 16, 32
// reduces 2, 4, 8, 16, 32, 64 lanes; every lane of a group ends with the
// same result.
template <int CTRL> __device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int STEP> __device__ __forceinline__ int xchg(int v)
{
    if constexpr (STEP == 1) return dpp_i<0xB1>(v);        // quad_perm [1,0,3,2]
    else if constexpr (STEP == 2) return dpp_i<0x4E>(v);   // quad_perm [2,3,0,1]
    else if constexpr (STEP == 4) return dpp_i<0x141>(v);  // row_half_mirror
    else if constexpr (STEP == 8) return dpp_i<0x140>(v);  // row_mirror
    else if constexpr (STEP == 16) {
        auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (int)((threadIdx.x & 16) ? r[0] : r[1]);
    } else {
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (int)((threadIdx.x & 32) ? r[0] : r[1]);
    }
}
template <int STEP> __device__ __forceinline__ float xchg(float v) { return __int_as_float(xchg<STEP>(__float_as_int(v))); }

template <int N, class T> __device__ __forceinline__ T group_sum(T v)
{
    v += xchg<1>(v);
    v += xchg<2>(v);
    if constexpr (N > 4) v += xchg<4>(v);
    if constexpr (N > 8) v += xchg<8>(v);
    if constexpr (N > 16) v += xchg<16>(v);
    if constexpr (N > 32) v += xchg<32>(v);
    return v;
}

template <int N> __device__ __forceinline__ float group_max(float v)
{
    v = fmaxf(v, xchg<1>(v));
    v = fmaxf(v, xchg<2>(v));
    if constexpr (N > 4) v = fmaxf(v, xchg<4>(v));
    if constexpr (N > 8) v = fmaxf(v, xchg<8>(v));
    if constexpr (N > 16) v = fmaxf(v, xchg<16>(v));
    if constexpr (N > 32) v = fmaxf(v, xchg<32>(v));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Wave sums of N values at once (N a multiple of 8), written to dst[0, nv):
// three exchange steps across lanes 32, 16 and 8 apart each keep half of
// the values per lane (the half given away is added into the partner's),
// then an 8-lane sum finishes the N/8 values each lane group holds.
// 1.25 N exchanges instead of the 6 N of N separate wave sums.
template <int N> __device__ __forceinline__ void wave_sums_to(const float (&v)[N], float *dst, int nv)
{
    static_assert(N % 8 == 0, "N must be a multiple of 8");
    const int lane = lane_id();
    float a[N / 2], b[N / 4], c[N / 8];
    const bool u5 = lane & 32, u4 = lane & 16, u3 = lane & 8;
#pragma unroll
    for (int i = 0; i < N / 2; i++) a[i] = (u5 ? v[i + N / 2] : v[i]) + xchg<32>(u5 ? v[i] : v[i + N / 2]);
#pragma unroll
    for (int i = 0; i < N / 4; i++) b[i] = (u4 ? a[i + N / 4] : a[i]) + xchg<16>(u4 ? a[i] : a[i + N / 4]);
#pragma unroll
    for (int i = 0; i < N / 8; i++) c[i] = group_sum<8>((u3 ? b[i + N / 8] : b[i]) + xchg<8>(u3 ? b[i] : b[i + N / 8]));
    if ((lane & 7) == 0) {
        const int base = (u5 ? N / 2 : 0) + (u4 ? N / 4 : 0) + (u3 ? N / 8 : 0);
#pragma unroll
        for (int i = 0; i < N / 8; i++)
            if (base + i < nv) dst[base + i] = c[i];
    }
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps
// inside 16-lane rows (row_shr 1, 2, 4, 8), then the row totals carried
// across rows with row_bcast:15 and row_bcast:31.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
    return v;
}

__device__ __forceinline__ uint32_t comp(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float half_lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }

__device__ __forceinline__ int dot4(uint32_t a, int b, int c) { return __builtin_amdgcn_sdot4((int)a, b, c, false); }

__device__ __forceinline__ void st_coh(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_coh(const float *p) { return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t ld_coh_u(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Default bound on the polls of a wait for other workgroups of the same
// launch (moe_set_spin_limit overrides it for tests of the give-up path).
constexpr unsigned kSpinLimit = 1u << 20;

__device__ float block_sum(float v, float *red)
{
    v = wave_sum(v);
    const int nw = blockDim.x >> 6;
    __syncthreads();
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < nw; i++) s += red[i];
    __syncthreads();
    return s;
}

// ---------------------------------------------------------------------------
// Encoded activation records, one per vector of K positions (4K bytes):
//   [0, 3K)          pieces q[3][K], int8, piece-major
//   [3K, 3K+K/8)     block scales bs[K/32], fp32
//   [3K+K/8, 3K+K/4) exact block sums bsum[K/32], fp32
//   [3K+K/4, 4K)     per-16 sums of each piece ps[3][K/16], int32
struct Enc {
    uint8_t *base;  // records back to back
};

__device__ __forceinline__ uint8_t *rec_at(const Enc &e, int vec, int K) { return e.base + (size_t)vec * 4 * K; }

// Encode one 32-value block held by 32 consecutive lanes (lane r of the
// group holds position pos0 + r) into record `rec`, with the scale a/127:
// a = the block's own largest magnitude (amax < 0), or amax, a bound on it
// shared by more blocks (the input states' records share one scale per
// 256-position super-block, which the integer-MFMA kernels need).
__device__ __forceinline__ void encode32(float v, int r, uint8_t *rec, int K, int pos0, float amax = -1.f)
{
    const float a = amax >= 0.f ? amax : group_max<32>(fabsf(v));
    const float sm = group_sum<32>(v);
    const float inv = a > 0.f ? 127.0f / a : 0.f;
    const float r0 = v * inv, f0 = rintf(r0);
    const float r1 = (r0 - f0) * 254.0f, f1 = rintf(r1);
    const float r2 = (r1 - f1) * 254.0f, f2 = rintf(r2);
    const int i0 = (int)f0, i1 = (int)f1, i2 = (int)f2;
    const int sh = 8 * (r & 3);
    // bytes of 4 lanes are disjoint, so their sum is their concatenation
    const int w0 = group_sum<4>((int)((uint32_t)(i0 & 0xff) << sh));
    const int w1 = group_sum<4>((int)((uint32_t)(i1 & 0xff) << sh));
    const int w2 = group_sum<4>((int)((uint32_t)(i2 & 0xff) << sh));
    const int s0 = group_sum<16>(i0), s1 = group_sum<16>(i1), s2 = group_sum<16>(i2);
    if ((r & 3) == 0) {
        *(int *)(rec + pos0 + r) = w0;
        *(int *)(rec + K + pos0 + r) = w1;
        *(int *)(rec + 2 * K + pos0 + r) = w2;
    }
    if ((r & 15) == 0) {
        int *ps = (int *)(rec + 3 * K + K / 4) + (pos0 + r) / 16;
        ps[0] = s0;
        ps[K / 16] = s1;
        ps[K / 8] = s2;
    }
    if (r == 0) {
        float *bs = (float *)(rec + 3 * K);
        bs[pos0 / 32] = a / 127.0f;
        bs[K / 32 + pos0 / 32] = sm;
    }
}

// Largest of v over the 256 consecutive threads (4 whole waves: the waves
// 4g .. 4g+3 of the caller's group g) of a workgroup; every thread calls it
// (barriers inside).  redm: LDS of one float per wave.
__device__ __forceinline__ float group256_max(float v, float *redm)
{
    const float am = group_max<64>(v);
    if (lane_id() == 0) redm[wave_id()] = am;
    __syncthreads();
    const int g0 = wave_id() & ~3;
    const float cm = fmaxf(fmaxf(redm[g0], redm[g0 + 1]), fmaxf(redm[g0 + 2], redm[g0 + 3]));
    __syncthreads();  // redm is free again
    return cm;
}

// One position of a half-precision (MFMA) record: 256 consecutive threads
// (a quarter or half of the workgroup, whole waves) hold positions p =
// 0..255 of one super-block, v their value (0 past the vector's end); rec is
// the super-block's record (kX16Bytes), cm the super-block's largest
// magnitude (group256_max).
__device__ __forceinline__ void encode_x16(float v, uint8_t *rec, int p, bool live, float cm)
{
    if (!live) return;
    const int e = cm > 0.f ? -ilogbf(cm) - 1 : 0;  // cm * 2^e in [0.5, 1)
    const float x = v * ldexpf(1.0f, e);           // exact (power of two)
    const _Float16 xh = (_Float16)x;
    ((_Float16 *)rec)[p] = xh;
    ((_Float16 *)(rec + 512))[p] = (_Float16)(x - (float)xh);
    const float s32 = group_sum<32>(x);
    if ((p & 31) == 0) {
        const _Float16 sh = (_Float16)s32;
        ((_Float16 *)(rec + 1024))[p >> 5] = sh;
        ((_Float16 *)(rec + 1040))[p >> 5] = (_Float16)(s32 - (float)sh);
    }
    if (p == 0) *(float *)(rec + 1056) = ldexpf(1.0f, -e);
}

// Zero blocks [b0, b1) of a record (padding columns of the down rows).
__device__ void zero_blocks(uint8_t *rec, int K, int b0, int b1, int tid, int nthr)
{
    for (int b = b0 + tid; b < b1; b += nthr) {
        float *bs = (float *)(rec + 3 * K);
        int *ps = (int *)(rec + 3 * K + K / 4);
        for (int p = 0; p < kPieces; p++) {
            int *q = (int *)(rec + (size_t)p * K + 32 * b);
            for (int i = 0; i < 8; i++) q[i] = 0;
            ps[p * (K / 16) + 2 * b] = 0;
            ps[p * (K / 16) + 2 * b + 1] = 0;
        }
        bs[b] = 0.f;
        bs[K / 32 + b] = 0.f;
    }
}

// ---------------------------------------------------------------------------
// Grouping (stable counting sort) of the T*k routed pairs plus T*ns shared
// pairs, run by one workgroup.  Routed pairs of expert e come first in
// ascending e, each expert's pairs by ascending token; shared expert s is
// pseudo-expert E+s with one pair per token.  Ids outside [0, E) are dropped.
constexpr int kInlineTok = 8;
struct WorkEntry {
    int e, p0, p1, pad;          // expert (E+s for shared s), grouped pairs [p0, p1)
    const void *ptr;             // expert's slot address, or null: read it from the pointer table
    uint8_t tok[kInlineTok];     // tokens of the first kInlineTok pairs
};

// A work-table entry read whole by one scalar load: the table is written by
// an earlier launch and only read in this one, so it may be read as
// constant memory (a uniform index then gives one s_load_dwordx8 instead of
// two loads split around the early exit for an empty entry).
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ WorkEntry load_entry(const WorkEntry *wt, int u)
{
    typedef const __attribute__((address_space(4))) uint8_t cbyte;
    const i32x8 v = *(const __attribute__((address_space(4))) i32x8 *)((cbyte *)wt + (size_t)u * sizeof(WorkEntry));
    WorkEntry we;
    static_assert(sizeof(WorkEntry) == sizeof(i32x8), "work entry size");
    __builtin_memcpy(&we, &v, sizeof(we));
    return we;
}

struct GroupOut {
    int *nuniq;           // work-table entries in use (workspace)
    WorkEntry *wt;        // [Umax]; entries past nuniq are empty (p0 == p1)
    int Umax;
    int *ptok;            // [P] token of each grouped pair
    int *inv;             // [T][k+ns] grouped position of (t, j), -1 if dropped
    const void *const *eptr, *const *sptr;  // pointer tables to resolve, or null
    int *count, *offset, *pairs;  // moe_group_tokens outputs (may be null)
    float *pw;            // [P] combine weight of each grouped pair, or null
    const float *wsrc;    // [T][k] routing weights the pair weights are taken from
    int chunk;            // kItemTok: work items of at most kItemTok pairs; 0: one entry per expert
};

// Expert-table entries that the route tail's wave 0 loads before the top-k,
// so that the grouping does not wait on them: for a single token, entries
// lane and 64 + lane; for group_block, entries EPL*lane and EPL*lane + 1,
// EPL = ceil(E / 64) (the first two experts of the lane).
struct PrePtr { const void *p0, *p1; bool valid; };

// Waits for the loads of pre here, before the caller issues stores: a later
// wait for them would also wait for those stores (one counter for both).
__device__ __forceinline__ void settle(const PrePtr &pre) { asm volatile("" ::"v"(pre.p0), "v"(pre.p1)); }

// Grouping by token masks.  Ids are distinct within a token, so an expert
// is chosen at most once per token and its pairs, in (token, slot) order,
// are described by a T-bit mask (T <= 32) of the tokens that chose it:
//   count(e) = popc(mask_e),  rank of token t's pair = popc(mask_e & ((1<<t)-1)),
//   offset(e) = sum of counts of experts below e (wave scan),
//   distinct-expert index = number of non-empty experts below e (wave scan).
// Shared expert s follows as pseudo-expert E+s with pair nvalid + s*T + t.
// A token that names one expert in two slots gets one pair, which both slots
// point at (its output then carries the sum of their weights).
// `lmask` is LDS of at least E ints; wave 0 scans.
__device__ __forceinline__ void group_block(const int *sidx, int T, int k, int E, int ns, GroupOut g, int *lmask,
                            PrePtr pre /* this lane's table entries lane and 64 + lane, if valid */)
{
    __shared__ int s_nu, s_valid;
    __shared__ const void *lptr[kMaxE];  // slot addresses of the chosen experts
    const int P = T * k;
    for (int e = threadIdx.x; e < E; e += blockDim.x) lmask[e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int ep = sidx[p];
        if ((unsigned)ep < (unsigned)E) atomicOr((unsigned *)&lmask[ep], 1u << (p / k));
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        // lane l takes experts [EPL*l, EPL*l + EPL): one scan of the lanes' totals
        const int lane = lane_id();
        const int EPL = (E + 63) >> 6;
        const int eb = lane * EPL;
        // Counts, and the slot addresses of the chosen experts into LDS: the
        // table loads stay in this loop, so that the store loop below has no
        // load to wait for (a wait for a load also waits for every store
        // issued before it).
        // Work items go to the table largest first (items of kItemTok pairs,
        // then kItemTok-1, ...), so that the FFN launches, which take them in
        // table order, start the long ones first; pairs stay in expert order.
        // nb[c]: this lane's items of class c (class c holds items of
        // kItemTok - c pairs; with one entry per expert, class 0 only).
        int lc = 0, nb[kItemTok];
#pragma unroll
        for (int c = 0; c < kItemTok; c++) nb[c] = 0;
        for (int j = 0; j < EPL; j++) {
            const int e = eb + j;
            const int cnt = e < E ? __popc((uint32_t)lmask[e]) : 0;
            lc += cnt;
            if (g.chunk > 0) {
                nb[0] += cnt / kItemTok;
                const int rem = cnt % kItemTok;
#pragma unroll
                for (int c = 1; c < kItemTok; c++) nb[c] += rem == kItemTok - c;
            } else {
                nb[0] += cnt > 0;
            }
            if (cnt > 0 && g.wt && g.eptr) {
                if (pre.valid && j < 2) lptr[e] = j == 0 ? pre.p0 : pre.p1;
                else lptr[e] = g.eptr[e];
            }
        }
        const int incl = wave_incl_scan(lc);
        int off = incl - lc, ui[kItemTok], nu = 0;
#pragma unroll
        for (int c = 0; c < kItemTok; c++) {
            const int ic = wave_incl_scan(nb[c]);
            ui[c] = nu + ic - nb[c];
            nu += __shfl(ic, 63, 64);
        }
        for (int j = 0; j < EPL; j++) {
            const int e = eb + j;
            if (e >= E) break;
            const uint32_t m = (uint32_t)lmask[e];
            const int cnt = __popc(m);
            const int chunk = g.chunk > 0 ? kItemTok : (cnt > 0 ? cnt : 1);
            const int nit = g.chunk > 0 ? (cnt + kItemTok - 1) / kItemTok : cnt > 0;  // work items of the expert
            if (g.count) g.count[e] = cnt;
            if (g.offset) g.offset[e] = off;
            if (cnt > 0 && g.wt) {
                const void *ptr = g.eptr ? lptr[e] : nullptr;
                uint32_t mm = m;  // the expert's tokens, ascending
                for (int it = 0; it < nit; it++) {
                    WorkEntry we{};
                    we.e = e; we.p0 = off + it * chunk; we.p1 = min(off + (it + 1) * chunk, off + cnt);
                    we.ptr = ptr;
                    uint64_t toks = 0;
                    if (g.chunk > 0) {
                        // the item's (at most kItemTok) tokens, a fixed count of steps
#pragma unroll
                        for (int i = 0; i < kItemTok; i++) {
                            const uint32_t t = (uint32_t)__builtin_ctz(mm | 0x80000000u);  // 31 once empty
                            toks |= (uint64_t)(mm ? t : 0u) << (8 * i);
                            mm &= mm - 1;
                        }
                    } else {
                        // the first kInlineTok tokens inline; the rest are read from ptok
                        for (int i = 0; i < kInlineTok && mm; i++) {
                            const int t = __ffs(mm) - 1;
                            toks |= (uint64_t)t << (8 * i);
                            mm &= mm - 1;
                        }
                    }
                    __builtin_memcpy(we.tok, &toks, sizeof(toks));
                    // the item's class: full items class 0, the last one by its size
                    const int c = g.chunk > 0 ? kItemTok - (we.p1 - we.p0) : 0;
                    int at = ui[0];
#pragma unroll
                    for (int c2 = 1; c2 < kItemTok; c2++) at = c == c2 ? ui[c2] : at;
                    g.wt[at] = we;
#pragma unroll
                    for (int c2 = 0; c2 < kItemTok; c2++) ui[c2] += c == c2;
                }
            }
            lmask[E + e] = off;
            off += cnt;
        }
        if (lane == 63) { s_nu = nu; s_valid = off; }
    }
    __syncthreads();
    const int nu = s_nu, nvalid = s_valid;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int ep = sidx[p];
        const int t = p / k, j = p - t * k;
        if ((unsigned)ep >= (unsigned)E) {
            if (g.inv) g.inv[t * (k + ns) + j] = -1;
            continue;
        }
        const int pos = lmask[E + ep] + __popc((uint32_t)lmask[ep] & ((1u << t) - 1u));
        if (g.pairs) g.pairs[pos] = p;
        if (g.ptok) {
            g.ptok[pos] = t;
            g.inv[t * (k + ns) + j] = pos;
        }
        if (g.pw) g.pw[pos] = g.wsrc[p];
    }
    if (g.offset && threadIdx.x == 0) g.offset[E] = nvalid;
    if (g.wt) {
        // shared expert s2: pairs nvalid + s2*T + t, cut into items like the routed ones
        const int sc = g.chunk > 0 ? kItemTok : T;
        const int sit = (T + sc - 1) / sc;
        for (int i = threadIdx.x; i < ns * sit; i += blockDim.x) {
            const int s2 = i / sit, it = i - s2 * sit;
            WorkEntry we{};
            we.e = E + s2; we.p0 = nvalid + s2 * T + it * sc; we.p1 = nvalid + s2 * T + min((it + 1) * sc, T);
            we.ptr = g.eptr ? g.sptr[s2] : nullptr;
            for (int q = 0; q < kInlineTok; q++) we.tok[q] = (uint8_t)(it * sc + q);
            g.wt[nu + i] = we;
        }
        for (int u = nu + ns * sit + threadIdx.x; u < g.Umax; u += blockDim.x) g.wt[u] = WorkEntry{};
        if (threadIdx.x == 0) *g.nuniq = nu + ns * sit;
    }
    if (g.ptok) {
        for (int i = threadIdx.x; i < ns * T; i += blockDim.x) {
            const int s2 = i / T, t = i - s2 * T;
            const int pos = nvalid + s2 * T + t;
            if (g.pw) g.pw[pos] = 1.0f;  // shared experts have weight one
            g.ptok[pos] = t;
            g.inv[t * (k + ns) + k + s2] = pos;
        }
    }
}

// Stable counting sort of the T*k (token, slot) pairs by expert, for the
// stand-alone grouping entry point (which also admits repeated ids in a
// token): pair p goes to (valid ids below idx[p]) + (earlier pairs with the
// same id).
__device__ void group_sort(const int *sidx, int T, int k, int E, int *count, int *offset, int *pairs)
{
    const int P = T * k;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int ep = sidx[p];
        if ((unsigned)ep >= (unsigned)E) continue;
        int below = 0, rank = 0;
        for (int q = 0; q < P; q++) {
            const int eq = sidx[q];
            below += (unsigned)eq < (unsigned)ep;
            rank += q < p && eq == ep;
        }
        pairs[below + rank] = p;
    }
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        int below = 0, cnt = 0;
        for (int q = 0; q < P; q++) {
            const int eq = sidx[q];
            below += (unsigned)eq < (unsigned)e;
            cnt += eq == e;
        }
        if (e < E) count[e] = cnt;
        offset[e] = below;
    }
}

// A float's bits mapped to an unsigned integer of the same order (every
// non-NaN value maps above 0).
__device__ __forceinline__ uint32_t ord_bits(float v)
{
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_bits(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ int below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
__device__ __forceinline__ int ballot_count(bool p) { return __popcll(__ballot(p)); }

// Routing key of a logit: its order-preserving bits.  Keys are never zero
// (NaN is taken as the canonical positive NaN), so that zero can mark a
// key not yet written.
__device__ __forceinline__ uint32_t logit_key(float v)
{
    return ord_bits(v != v ? __uint_as_float(0x7fc00000u) : v);
}

// Top-k of one token by one wave, E <= 64*NVL keys (lane l holds experts
// l + 64i), read from LDS or (GLOBAL) with coherent loads.  A radix select
// finds the k-th largest key v from the most significant bit down (bit b is
// kept when at least k keys are >= the candidate); the keys above v and,
// among those equal to v, the lowest ids make up the selection.  A selected
// key's rank is the number of keys above it plus the equal keys of lower id
// (logit descending, ties to the lower id); selection j goes to sidx[j],
// skey[j].
template <int NVL, bool GLOBAL>
__device__ __forceinline__ void topk_wave(const uint32_t *keys, int E, int k, int *sidx, uint32_t *skey)
{
    const int lane = lane_id();
    uint32_t key[NVL];
#pragma unroll
    for (int i = 0; i < NVL; i++) {
        const int e = lane + 64 * i;
        key[i] = e >= E ? 0u : GLOBAL ? ld_coh_u(keys + e) : keys[e];
    }
    uint32_t thr = 0;
    for (int b = 31; b >= 0; b--) {
        const uint32_t cand = thr | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NVL; i++) cnt += ballot_count(key[i] >= cand);
        if (cnt >= k) thr = cand;
    }
    int need = k;  // keys equal to thr taken, lowest ids first
#pragma unroll
    for (int i = 0; i < NVL; i++) need -= ballot_count(key[i] > thr);
    uint64_t sel[NVL];
    int before = 0;
#pragma unroll
    for (int i = 0; i < NVL; i++) {
        const uint64_t eq = __ballot(key[i] == thr && lane + 64 * i < E);
        const bool take = key[i] > thr || ((eq >> lane) & 1ull && before + below(eq) < need);
        sel[i] = __ballot(take);
        before += __popcll(eq);
    }
#pragma unroll
    for (int i = 0; i < NVL; i++) {
        uint64_t m = sel[i];
        while (m) {
            const int l = __builtin_ctzll(m);
            m &= m - 1;
            const uint32_t kx = (uint32_t)__builtin_amdgcn_readlane((int)key[i], l);
            const int id = l + 64 * i;
            int r = 0;
#pragma unroll
            for (int i2 = 0; i2 < NVL; i2++)
                r += ballot_count(key[i2] > kx || (key[i2] == kx && lane + 64 * i2 < id));
            if (lane == r) {
                sidx[r] = id;
                skey[r] = kx;
            }
        }
    }
}

template <bool GLOBAL>
__device__ __forceinline__ void topk_wave_any(const uint32_t *keys, int E, int k, int *sidx, uint32_t *skey)
{
    if (E <= 64) topk_wave<1, GLOBAL>(keys, E, k, sidx, skey);
    else if (E <= 128) topk_wave<2, GLOBAL>(keys, E, k, sidx, skey);
    else if (E <= 256) topk_wave<4, GLOBAL>(keys, E, k, sidx, skey);
    else if (E <= 512) topk_wave<8, GLOBAL>(keys, E, k, sidx, skey);
    else topk_wave<16, GLOBAL>(keys, E, k, sidx, skey);
}

constexpr int kStageKeys = 4096;  // keys the route tail keeps in LDS
constexpr int kWaveTopE = 256;    // experts for the per-wave topk_multi (4 keys per lane)
constexpr int kCandSlots = kWaveTopE + 9 + kMaxK + 1;  // candidate slots of one token
constexpr int kTopkBlocksMinT = 16;  // batches above this rank their tokens in top-k workgroups

// floor(i / d) for 0 <= i < 2^16, 1 <= d <= 2^16, with r = 1.0f/d: (i + 0.5)/d
// is at least 0.5/d away from an integer, far more than the float error.
__device__ __forceinline__ int fdiv(int i, float r) { return (int)(((float)i + 0.5f) * r); }

// ---------------------------------------------------------------------------
// k_route

struct RouteArgs {
    const float *h;  // [T][H]
    int T, H;
    const float *wr;    // [E][H]
    const float *bias;  // [E] or null
    int E, k;
    float eps;
    int normalize;          // scale logits (and the encoding) by 1/rms(h[t])
    unsigned *keys;         // [T][E] hand-over of logit keys; zero = not yet written
    int *idx;               // [T][k]
    float *w;               // [T][k]
    int *idx2;              // optional copies
    float *w2;
    float *logits2;
    Enc x;                  // [T] vectors of H
    uint8_t *x16;           // [T][H/256] half-precision records of the normalised states, or null
    int group;
    int ns;
    GroupOut go;
    Enc hpad;               // [P] vectors of kd: padding blocks zeroed here
    int P, I, kd;
    int n_expert_blocks;    // router workgroups (row pair, token group); then T * ceil(H/kEncPos) encoding workgroups,
                            // then topk_blocks top-k workgroups, then the tail
    int topk_blocks;        // 0, or T: a workgroup per token ranks its keys and hands them to the tail
    unsigned long long *tk; // [T][k] hand-over of those selections (key << 32 | ~id, never zero)
    int tail;               // 1: the last workgroup routes (keys handed over); 0: no tail
    uint32_t *dlog;         // [T][E] the logit keys for routing in the FFN (plain stores), or null
    int sb_scale;           // 1: the input records share one scale per 256-position super-block
    uint32_t *status;       // the workspace's status word: nonzero = a wait gave up earlier (sticky)
    unsigned spin;          // polling rounds before a wait gives up
    int withhold;           // 1: the router workgroups store no keys (forced give-up, for tests)
};

// Sets bit b of the status word (a vector atomic; lane 0 of the calling wave).
__device__ __forceinline__ void flag_status(uint32_t *status, uint32_t b)
{
    if (lane_id() == 0) __hip_atomic_fetch_or(status, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Top-k of NT tokens' E keys each by one wave (no barriers), keys in
// registers (lane l holds experts l + 64i of token t in key[t][i], zero past
// E); the NT tokens' steps are interleaved, so that their latencies overlap.
// tau, the k-th largest of the 64 per-lane maxima (bitonic sort across the
// lanes), bounds the top k from below: at least k keys are >= tau, so the
// top k are among them, and usually only a few more.  Those candidates, as
// 64-bit C = key << 32 | ~e (unique, ordered like the key with ties to the
// lower id), are ranked against each other in LDS.  Returns in out[t], in
// lane j < k, the C of token t's selection j (logit descending, ties to the
// lower id), 0 in the other lanes.
// cand: LDS of NT regions of cstride >= E + 9 + k + ... 64-bit slots (see
// kCandSlots), 16-byte aligned.
template <int NVL, int NT>
__device__ __forceinline__ void topk_multi(const uint32_t (&key)[NT][NVL], int E, int k, uint64_t *cand, int cstride,
                                           uint64_t (&out)[NT])
{
    const int lane = lane_id();
    uint32_t v[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        v[t] = 0;
#pragma unroll
        for (int i = 0; i < NVL; i++) v[t] = max(v[t], key[t][i]);
    }
#pragma unroll
    for (int k2 = 2; k2 <= 64; k2 <<= 1)
#pragma unroll
        for (int j = k2 >> 1; j > 0; j >>= 1) {
            const bool up = ((lane & j) == 0) == ((lane & k2) == 0);
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const uint32_t p = (uint32_t)__shfl_xor((int)v[t], j, 64);
                v[t] = up ? max(v[t], p) : min(v[t], p);
            }
        }
    // candidates >= tau, compacted into the token's cand[0, m), zero padding after
    int m[NT], mp[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const uint32_t tau = (uint32_t)__shfl((int)v[t], k - 1, 64);
        uint64_t *ct = cand + t * cstride;
        m[t] = 0;
#pragma unroll
        for (int i = 0; i < NVL; i++) {
            const int e = lane + 64 * i;
            const bool c = e < E && key[t][i] >= tau;
            const uint64_t bal = __ballot(c);
            if (c) ct[m[t] + below(bal)] = (uint64_t)key[t][i] << 32 | (uint32_t)~e;
            m[t] += __popcll(bal);
        }
        if (lane < 8) ct[m[t] + lane] = 0ull;
        mp[t] = (m[t] + 7) & ~7;
    }
    // exact ranks among the candidates; selection r goes to sel[r]
    const int soff = (E + 8 + 1) & ~1;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        uint64_t *ct = cand + t * cstride;
        for (int c = lane; c < m[t]; c += 64) {
            const uint64_t ci = ct[c];
            int r0 = 0, r1 = 0;
            for (int c2 = 0; c2 < mp[t]; c2 += 8) {
                const ulonglong2 *q = (const ulonglong2 *)(ct + c2);
                const ulonglong2 x0 = q[0], x1 = q[1], x2 = q[2], x3 = q[3];
                r0 += (x0.x > ci) + (x0.y > ci) + (x1.x > ci) + (x1.y > ci);
                r1 += (x2.x > ci) + (x2.y > ci) + (x3.x > ci) + (x3.y > ci);
            }
            if (r0 + r1 < k) ct[soff + r0 + r1] = ci;
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = lane < k ? cand[t * cstride + soff + lane] : 0ull;
}

// Top-k of one token's keys by one wave for k <= 8: lane l holds experts
// l + 64 i in key[i] (zero past E).  tau, the smallest of the eight 8-lane
// groups' largest keys, bounds the top k from below (each group holds a key
// >= tau, so at least 8 >= k keys reach it); six lane exchanges find it,
// where topk_multi sorts the 64 lane maxima.  The candidates >= tau, as
// 64-bit C = key << 32 | ~e, are ranked against each other in LDS as there:
// the same result, lane j < k returning selection j (key descending, ties to
// the lower id), the other lanes 0.  cand: LDS of E + 23 64-bit slots,
// 16-byte aligned.
template <int NVL>
__device__ __forceinline__ uint64_t topk_few(const uint32_t (&key)[NVL], int E, int k, uint64_t *cand)
{
    const int lane = lane_id();
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < NVL; i++) v = max(v, key[i]);
    v = max(v, (uint32_t)xchg<1>((int)v));
    v = max(v, (uint32_t)xchg<2>((int)v));
    v = max(v, (uint32_t)xchg<4>((int)v));
    v = min(v, (uint32_t)xchg<8>((int)v));
    v = min(v, (uint32_t)xchg<16>((int)v));
    v = min(v, (uint32_t)xchg<32>((int)v));
    const uint32_t tau = (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
    int m = 0;
#pragma unroll
    for (int i = 0; i < NVL; i++) {
        const int e = lane + 64 * i;
        const bool c = e < E && key[i] >= tau;
        const uint64_t bal = __ballot(c);
        if (c) cand[m + below(bal)] = (uint64_t)key[i] << 32 | (uint32_t)~e;
        m += __popcll(bal);
    }
    if (lane < 8) cand[m + lane] = 0ull;
    const int mp = (m + 7) & ~7, soff = mp + 8;
    for (int c = lane; c < m; c += 64) {
        const uint64_t ci = cand[c];
        int r0 = 0, r1 = 0;
        for (int c2 = 0; c2 < mp; c2 += 8) {
            const ulonglong2 *q = (const ulonglong2 *)(cand + c2);
            const ulonglong2 x0 = q[0], x1 = q[1], x2 = q[2], x3 = q[3];
            r0 += (x0.x > ci) + (x0.y > ci) + (x1.x > ci) + (x1.y > ci);
            r1 += (x2.x > ci) + (x2.y > ci) + (x3.x > ci) + (x3.y > ci);
        }
        if (r0 + r1 < k) cand[soff + r0 + r1] = ci;
    }
    return lane < k ? cand[soff + lane] : 0ull;
}

// Top-k of a single token: topk_few for k <= 8, else topk_multi.  cand:
// E + 9 + k + 1 slots, and at least E + 23.
template <int NVL>
__device__ __forceinline__ uint64_t topk_one(const uint32_t (&key)[NVL], int E, int k, uint64_t *cand)
{
    if (k <= 8) return topk_few<NVL>(key, E, k, cand);
    uint32_t kk[1][NVL];
#pragma unroll
    for (int i = 0; i < NVL; i++) kk[0][i] = key[i];
    uint64_t out[1];
    topk_multi<NVL, 1>(kk, E, k, cand, 0, out);
    return out[0];
}

// Single-token routing tail, by wave 0 alone (no barriers): polls the keys
// into registers, topk_one, softmax over the k selected logits, and the
// grouping (selection j is pair and distinct expert pos_j, its position
// among the k ids in ascending order).
template <int NVL>
__device__ __forceinline__ void route_tail_one(const RouteArgs &a, uint64_t *cand, PrePtr pre)
{
    const int E = a.E, k = a.k, ns = a.ns, lane = lane_id();
    uint32_t key[NVL];
    // a workspace whose status word is set may hold stale keys: no wait
    const bool dead = *a.status != 0u;
    int ok = !dead;
    for (unsigned it = 0;; it++) {
        bool missing = false;
#pragma unroll
        for (int i = 0; i < NVL; i++) {
            const int e = lane + 64 * i;
            key[i] = e < E ? ld_coh_u(a.keys + e) : 0u;
            missing |= e < E && key[i] == 0u;
        }
        if (!__ballot(missing)) break;
        if (dead || it >= a.spin) {
            if (!dead) flag_status(a.status, MOE_WS_KEYS_TIMEOUT);
            ok = 0;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    const uint64_t cs = topk_one<NVL>(key, E, k, cand);
    settle(pre);
    const int id = (int)~(uint32_t)cs;
    // softmax over the k selected logits
    const float lg = lane < k ? unord_bits((uint32_t)(cs >> 32)) : 0.f;
    const float top = __shfl(lg, 0, 64);
    const float ex = lane < k ? expf(lg - top) : 0.f;
    const float wsum = wave_sum(ex);
    const float wj = ok ? ex / wsum : __builtin_nanf("");
    // clear the keys for the next launch (plain stores: the launch boundary
    // makes them visible)
#pragma unroll
    for (int i = 0; i < NVL; i++)
        if (lane + 64 * i < E) a.keys[lane + 64 * i] = 0u;
    // grouping: position of each id among the k ids in ascending order
    const int idl = lane < k ? id : 0x7fffffff;
    int pos = 0;
    for (int q = 0; q < k; q++) pos += __shfl(idl, q, 64) < idl;
    const long long q0 = __shfl((long long)pre.p0, id & 63, 64);
    const long long q1 = __shfl((long long)pre.p1, id & 63, 64);
    GroupOut g = a.go;
    if (lane < k) {
        a.idx[lane] = id;
        a.w[lane] = wj;
        if (a.idx2) a.idx2[lane] = id;
        if (a.w2) a.w2[lane] = wj;
        WorkEntry we{};
        we.e = id; we.p0 = pos; we.p1 = pos + 1;
        we.ptr = !g.eptr                 ? nullptr
                 : (pre.valid && id < 64)  ? (const void *)q0
                 : (pre.valid && id < 128) ? (const void *)q1
                                           : g.eptr[id];
        g.wt[pos] = we;  // tok[] all zero: token 0
        g.ptok[pos] = 0;
        g.inv[lane] = pos;
        g.pw[pos] = wj;
    }
    if (lane < ns) {
        WorkEntry we{};
        we.e = E + lane; we.p0 = k + lane; we.p1 = k + lane + 1;
        we.ptr = g.eptr ? g.sptr[lane] : nullptr;
        g.wt[k + lane] = we;
        g.ptok[k + lane] = 0;
        g.inv[k + lane] = k + lane;
        g.pw[k + lane] = 1.0f;
    }
    for (int u = k + ns + lane; u < g.Umax; u += 64) g.wt[u] = WorkEntry{};
    if (lane == 0) *g.nuniq = k + ns;
}

// Top-k workgroup of token t (batches with topk_blocks): wave 0 polls the
// token's E keys into registers (bounded, as the tail does), ranks them with
// topk_one and hands the k selections to the tail with coherent 64-bit
// stores (key << 32 | ~id: the key half is never zero).  A poll that gives
// up sets the status word and hands over selections with a zero key half,
// which the tail never accepts: it gives up too and routes with NaN weights.
template <int NVL>
__device__ __forceinline__ void route_topk_token(const RouteArgs &a, int t, uint64_t *cand)
{
    const int E = a.E, k = a.k, lane = lane_id();
    const unsigned *kt = a.keys + (size_t)t * E;
    uint32_t key[NVL];
    const bool dead = *a.status != 0u;
    bool ok = !dead;
    for (unsigned it = 0;; it++) {
        bool missing = false;
#pragma unroll
        for (int i = 0; i < NVL; i++) {
            const int e = lane + 64 * i;
            key[i] = e < E ? ld_coh_u(kt + e) : 0u;
            missing |= e < E && key[i] == 0u;
        }
        if (!__ballot(missing)) break;
        if (dead || it >= a.spin) {
            if (!dead) flag_status(a.status, MOE_WS_TOPK_TIMEOUT);
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    uint64_t cs = topk_one<NVL>(key, E, k, cand);
    if (!ok) cs = 0xffffffffull;  // zero key half: never accepted
    if (lane < k)
        __hip_atomic_store(a.tk + (size_t)t * k + lane, (unsigned long long)cs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void route_topk_role(const RouteArgs &a, int t)
{
    __shared__ __align__(16) uint64_t tcand[kCandSlots];
    if (wave_id() != 0) return;
    if (a.E <= 64) route_topk_token<1>(a, t, tcand);
    else if (a.E <= 128) route_topk_token<2>(a, t, tcand);
    else route_topk_token<4>(a, t, tcand);  // E <= kWaveTopE (the host's condition)
}

// The tail workgroup: a single token goes to route_tail_one; otherwise the
// workgroup polls the keys until every one is written, then top-k (clearing
// the keys for the next launch), softmax and grouping.  A poll that
// gives up after a.spin rounds sets the status word and routes with NaN
// weights, which no caller can miss; a set status word (from an earlier
// launch) means no wait at all and NaN weights again, since senders that came
// late may have left stale words behind.
__device__ __forceinline__ void route_tail(const RouteArgs &a)
{
    __shared__ __align__(16) uint32_t lk[kStageKeys];
    __shared__ __align__(16) union {
        uint64_t cand[kRouteWG / 64][kCandSlots];  // top-k, per wave
        int lstart[2 * kMaxE];                             // grouping, after the top-k
    } u;
    int *lstart = u.lstart;
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ uint32_t skey[kMaxT * kMaxK];
    __shared__ float sw[kMaxT * kMaxK];
    const int T = a.T, E = a.E, k = a.k, n = T * E;
    const int tid = (int)threadIdx.x, lane = lane_id();
    const bool staged = n <= kStageKeys;  // keys kept in LDS by the poll

    // pointer table entries for the grouping (layouts: see PrePtr)
    PrePtr pre{nullptr, nullptr, a.go.eptr != nullptr};
    if (a.go.eptr && wave_id() == 0) {
        const int EPL = (E + 63) >> 6;
        const int i0 = T == 1 ? lane : EPL * lane, i1 = T == 1 ? 64 + lane : (EPL > 1 ? EPL * lane + 1 : E);
        if (i0 < E) pre.p0 = a.go.eptr[i0];
        if (i1 < E) pre.p1 = a.go.eptr[i1];
    }
    if (T == 1 && a.group) {
        if (wave_id() != 0) return;
        static_assert(kMaxE + 9 + kMaxK <= kStageKeys / 2, "candidate slots");
        uint64_t *cand = (uint64_t *)lk;  // E + 9 + k slots
        if (E <= 64) route_tail_one<1>(a, cand, pre);
        else if (E <= 128) route_tail_one<2>(a, cand, pre);
        else if (E <= 256) route_tail_one<4>(a, cand, pre);
        else if (E <= 512) route_tail_one<8>(a, cand, pre);
        else route_tail_one<16>(a, cand, pre);
        return;
    }
    // a workspace whose status word is set may hold stale hand-offs: no wait
    const bool dead = *a.status != 0u;
    int ok = !dead;
    constexpr int kPollQ = 8;
    if (a.topk_blocks) {
        // the top-k workgroups' selections, polled like the keys
        const int nk = T * k;
        for (unsigned it = 0;; it++) {
            int missing = 0;
            for (int i = tid; i < nk; i += kRouteWG) {
                const unsigned long long c = __hip_atomic_load(a.tk + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sidx[i] = (int)~(uint32_t)c;
                skey[i] = (uint32_t)(c >> 32);
                missing |= (c >> 32) == 0ull;  // not yet written (or given up on)
            }
            if (!__ballot(missing)) break;
            if (dead || it >= a.spin) {
                if (!dead) flag_status(a.status, MOE_WS_TOPK_TIMEOUT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        ok = __syncthreads_and(ok);
        // selections that never arrived (zero) or were given up on carry no
        // valid id: route with ids 0..k-1 (distinct, in range; NaN weights)
        if (!ok)
            for (int i = tid; i < nk; i += kRouteWG) {
                sidx[i] = i % k;
                skey[i] = 0u;
            }
        // clear both hand-overs for the next launch (the top-k workgroups are
        // done with the keys once their selections are all here)
        for (int i = tid; i < n; i += kRouteWG) a.keys[i] = 0u;
        for (int i = tid; i < nk; i += kRouteWG) a.tk[i] = 0ull;
        settle(pre);
        __syncthreads();
    } else {
    // each wave polls its own share of the keys, then the workgroup meets
    // once; a thread's keys of a round are all loaded before any is checked
    // (one round trip per round, not one per key)
    for (unsigned it = 0;; it++) {
        int missing = 0;
        for (int i0 = tid; i0 < n; i0 += kPollQ * kRouteWG) {
            uint32_t v[kPollQ];
#pragma unroll
            for (int q = 0; q < kPollQ; q++) v[q] = ld_coh_u(a.keys + min(i0 + q * kRouteWG, n - 1));
#pragma unroll
            for (int q = 0; q < kPollQ; q++) {
                const int i = i0 + q * kRouteWG;
                if (i < n) {
                    if (staged) lk[i] = v[q];
                    missing |= v[q] == 0u;
                }
            }
        }
        if (!__ballot(missing)) break;
        if (dead || it >= a.spin) {
            if (!dead) flag_status(a.status, MOE_WS_KEYS_TIMEOUT);
            ok = 0;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    ok = __syncthreads_and(ok);
    if (staged && E <= kWaveTopE) {
        // a wave per token: topk_multi on the token's staged keys
        constexpr int NVL = kWaveTopE / 64;
        for (int t = wave_id(); t < T; t += kRouteWG / 64) {
            uint32_t key[1][NVL];
#pragma unroll
            for (int i = 0; i < NVL; i++) {
                const int e = lane + 64 * i;
                key[0][i] = e < E ? lk[t * E + e] : 0u;
            }
            uint64_t cs[1];
            cs[0] = topk_one<NVL>(key[0], E, k, u.cand[wave_id()]);
            if (lane < k) {
                sidx[t * k + lane] = (int)~(uint32_t)cs[0];
                skey[t * k + lane] = (uint32_t)(cs[0] >> 32);
            }
        }
    } else if (staged) {
        for (int t = wave_id(); t < T; t += kRouteWG / 64)
            topk_wave_any<false>(lk + t * E, E, k, sidx + t * k, skey + t * k);
    } else {
        for (int t = wave_id(); t < T; t += kRouteWG / 64)
            topk_wave_any<true>(a.keys + (size_t)t * E, E, k, sidx + t * k, skey + t * k);
    }
    settle(pre);
    __syncthreads();
    // clear the keys for the next launch (plain stores: the launch boundary
    // makes them visible); nothing reads them again in this launch
    for (int i = tid; i < n; i += kRouteWG) a.keys[i] = 0u;
    }
    // softmax over the k selected logits of each token (selection 0 is the
    // largest): for k <= 8, eight tokens per wave, lane 8q + j holding
    // selection j of token 8w + q; else a token per wave, lane j selection j
    const bool narrow = k <= 8;
    for (int t0 = narrow ? 8 * wave_id() : wave_id(); t0 < T; t0 += narrow ? 8 * (kRouteWG / 64) : kRouteWG / 64) {
        const int t = narrow ? t0 + (lane >> 3) : t0, j = narrow ? lane & 7 : lane;
        const bool live = j < k && t < T;
        const float lg = live ? unord_bits(skey[t * k + j]) : 0.f;
        const float top = __shfl(lg, narrow ? lane & ~7 : 0, 64);
        const float ex = live ? expf(lg - top) : 0.f;
        const float s = narrow ? group_sum<8>(ex) : wave_sum(ex);
        if (live) {
            const float wj = ok ? ex / s : __builtin_nanf("");
            const int id = sidx[t * k + j];
            sw[t * k + j] = wj;
            a.idx[t * k + j] = id;
            a.w[t * k + j] = wj;
            if (a.idx2) a.idx2[t * k + j] = id;
            if (a.w2) a.w2[t * k + j] = wj;
        }
    }
    if (!a.group) return;
    GroupOut go = a.go;
    go.wsrc = sw;
    __syncthreads();
    group_block(sidx, T, k, E, a.ns, go, lstart, pre);
}

// Router rows [e0, e0 + nr) against all tokens, NT tokens per pass; wave w
// takes the 256-column chunks w, w+8, ... of H, and the partial sums meet in
// LDS.  Loads are unconditional (row and token indices clamped; results for
// clamped tokens are dropped), so that each pass issues all of its loads at
// once.
template <int NT>
__device__ __forceinline__ void router_rows(const RouteArgs &a, int e0, int nr, int tb, int te)
{
    __shared__ float part[kRouteWG / 64][kRouteRows + 1][NT];
    const int H = a.H, T = a.T, E = a.E, nv = H >> 8;
    const int w = wave_id(), lane = lane_id();
    const float4 *wrow[kRouteRows];
#pragma unroll
    for (int r = 0; r < kRouteRows; r++) wrow[r] = (const float4 *)(a.wr + (size_t)(r < nr ? e0 + r : e0) * H);
    for (int t0 = tb; t0 < te; t0 += NT) {
        const float4 *hrow[NT];
#pragma unroll
        for (int tt = 0; tt < NT; tt++) hrow[tt] = (const float4 *)(a.h + (size_t)min(t0 + tt, T - 1) * H);
        float acc[kRouteRows][NT], ss[NT];
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            ss[tt] = 0.f;
#pragma unroll
            for (int r = 0; r < kRouteRows; r++) acc[r][tt] = 0.f;
        }
#pragma unroll 2
        for (int c = w; c < nv; c += kRouteWG / 64) {
            float4 wv[kRouteRows], hv[NT];
#pragma unroll
            for (int r = 0; r < kRouteRows; r++) wv[r] = wrow[r][c * 64 + lane];
#pragma unroll
            for (int tt = 0; tt < NT; tt++) hv[tt] = hrow[tt][c * 64 + lane];
#pragma unroll
            for (int tt = 0; tt < NT; tt++) {
                const float4 x = hv[tt];
                ss[tt] += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
#pragma unroll
                for (int r = 0; r < kRouteRows; r++)
                    acc[r][tt] += wv[r].x * x.x + wv[r].y * x.y + wv[r].z * x.z + wv[r].w * x.w;
            }
        }
        // the wave's partial dots and sums of squares, all reduced at once
        constexpr int NV = (kRouteRows + 1) * NT, N8 = (NV + 7) / 8 * 8;
        float vals[N8];
#pragma unroll
        for (int i = 0; i < N8; i++) vals[i] = 0.f;
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
#pragma unroll
            for (int r = 0; r < kRouteRows; r++) vals[r * NT + tt] = acc[r][tt];
            vals[kRouteRows * NT + tt] = ss[tt];
        }
        wave_sums_to<N8>(vals, &part[w][0][0], NV);
        __syncthreads();
        if ((int)threadIdx.x < nr * NT) {
            const int r = threadIdx.x / NT, tt = threadIdx.x % NT, t = t0 + tt;
            if (t < T) {
                float d = 0.f, q = 0.f;
#pragma unroll
                for (int ww = 0; ww < kRouteWG / 64; ww++) {
                    d += part[ww][r][tt];
                    q += part[ww][kRouteRows][tt];
                }
                const float rr = a.normalize ? 1.0f / sqrtf(q / (float)H + a.eps) : 1.0f;
                const float lg = d * rr + (a.bias ? a.bias[e0 + r] : 0.f);
                if (a.dlog) a.dlog[(size_t)t * E + e0 + r] = logit_key(lg);  // read after the launch boundary
                if (a.tail && !a.withhold)
                    __hip_atomic_store(a.keys + (size_t)t * E + e0 + r, logit_key(lg), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (a.logits2) a.logits2[(size_t)t * E + e0 + r] = lg;
            }
        }
        __syncthreads();
    }
}

// Router workgroup: 2 router rows against all T tokens, the 8 waves
// splitting H; the logits go to the tail as keys.  Encoding workgroup (t, c):
// RMS of token t, then positions [kEncPos c, kEncPos c + kEncPos).  The last
// workgroup is the tail.
__global__ __launch_bounds__(kRouteWG) void k_route(RouteArgs a)
{
    __shared__ float red[kRouteWG / 64], redx[kRouteWG / 64];

    const int H = a.H, T = a.T, E = a.E;
    const int blk = blockIdx.x;
    const int lane = lane_id();
    if (a.tail && blk == (int)gridDim.x - 1) {
        route_tail(a);
        return;
    }
    if (a.tail && blk >= (int)gridDim.x - 1 - a.topk_blocks) {
        route_topk_role(a, blk - ((int)gridDim.x - 1 - a.topk_blocks));
        return;
    }
    if (blk >= a.n_expert_blocks) {
        // encoding workgroup (t, c): positions [kEncPos c, kEncPos c + kEncPos) of token t
        const int ne = (H + kEncPos - 1) / kEncPos;
        const int g = blk - a.n_expert_blocks;
        const int t = g / ne, c = g - t * ne;
        const float4 *hr = (const float4 *)(a.h + (size_t)t * H);
        float ss = 0.f;
        for (int i = threadIdx.x; i < H / 4; i += blockDim.x) {
            const float4 v = hr[i];
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wave_id()] = ss;
        __syncthreads();
        ss = 0.f;
        for (int i = 0; i < kRouteWG / 64; i++) ss += red[i];
        const float r = a.normalize ? 1.0f / sqrtf(ss / (float)H + a.eps) : 1.0f;
        const int pos = c * kEncPos + threadIdx.x;
        const float xv = pos < H ? a.h[(size_t)t * H + pos] * r : 0.f;
        // one scale per 256-position super-block (4 whole waves) when the
        // integer-MFMA or half-precision records need it, else per block
        const float sbmax = a.sb_scale || a.x16 ? group256_max(fabsf(xv), redx) : -1.f;
        if (pos < H) {  // whole waves (H is a multiple of 256)
            encode32(xv, threadIdx.x & 31, rec_at(a.x, t, H), H, pos & ~31, a.sb_scale ? sbmax : -1.f);
        }
        if (a.x16)
            encode_x16(xv, a.x16 + ((size_t)t * (H >> 8) + (pos >> 8)) * kX16Bytes, pos & 255, pos < H, sbmax);
        if (a.kd > a.I) {
            const int nenc = T * ne;
            for (int p = g; p < a.P; p += nenc)
                zero_blocks(rec_at(a.hpad, p, a.kd), a.kd, a.I / 32, a.kd / 32, threadIdx.x, blockDim.x);
        }
        return;
    }

    // router workgroup (row pair, token group of kRouteTok)
    const int npair = (E + kRouteRows - 1) / kRouteRows;
    const int grp = blk / npair;
    const int e0 = (blk - grp * npair) * kRouteRows;
    const int nr = E - e0 < kRouteRows ? E - e0 : kRouteRows;
    if (T == 1) router_rows<1>(a, e0, nr, 0, 1);
    else if (T == 2) router_rows<2>(a, e0, nr, 0, 2);
    else if (T <= 4) router_rows<4>(a, e0, nr, 0, T);
    else router_rows<kRouteTok>(a, e0, nr, grp * kRouteTok, min(T, grp * kRouteTok + kRouteTok));
}

// k_route_token: stand-alone routing, one workgroup per token (16 waves
// share the E router rows; the keys stay in LDS).
constexpr int kRouteTokThreads = 1024;
__global__ __launch_bounds__(kRouteTokThreads) void k_route_token(const float *x, int H, const float *wr,
                                                                  const float *bias, int E, int k, int *idx,
                                                                  float *w, float *logits)
{
    __shared__ uint32_t lk[kMaxE];
    __shared__ int sidx[kMaxK];
    __shared__ uint32_t skey[kMaxK];
    const int t = blockIdx.x, lane = lane_id();
    const float4 *xr = (const float4 *)(x + (size_t)t * H);
    const int nv = H >> 8;
    for (int e = wave_id(); e < E; e += kRouteTokThreads / 64) {
        const float4 *wrow = (const float4 *)(wr + (size_t)e * H);
        float acc = 0.f;
        for (int i = 0; i < nv; i++) {
            const float4 a = wrow[i * 64 + lane], b = xr[i * 64 + lane];
            acc += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            const float l = acc + (bias ? bias[e] : 0.f);
            lk[e] = logit_key(l);
            if (logits) logits[(size_t)t * E + e] = l;
        }
    }
    __syncthreads();
    if (wave_id() != 0) return;
    topk_wave_any<false>(lk, E, k, sidx, skey);
    // softmax over the k selected logits, lane j holding selection j
    const float lg = lane < k ? unord_bits(skey[lane]) : 0.f;
    const float top = __shfl(lg, 0, 64);
    const float ex = lane < k ? expf(lg - top) : 0.f;
    const float sum = wave_sum(ex);
    if (lane < k) {
        idx[t * k + lane] = sidx[lane];
        w[t * k + lane] = ex / sum;
    }
}

// ---------------------------------------------------------------------------
// k_prep: encode given token states (no normalisation), and group given
// routing (workgroup 0).
struct PrepArgs {
    const float *x;
    int T, H, k, E, ns;
    const int *idx;
    const float *w;  // [T][k] routing weights
    float *yzero;    // [T][H] cleared here (the FFN adds into it), or null
    Enc xe;
    uint8_t *x16;    // [T][H/256] half-precision records of x, or null
    int sb_scale;    // 1: one record scale per 256-position super-block
    GroupOut go;
    Enc hpad;
    int P, I, kd;
};

__global__ __launch_bounds__(kRouteThreads) void k_prep(PrepArgs a)
{
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ int lstart[2 * kMaxE];
    __shared__ float redm[kRouteThreads / 64];
    const int t = blockIdx.x;
    for (int pos = threadIdx.x; pos < a.H; pos += blockDim.x) {
        const float v = a.x[(size_t)t * a.H + pos];
        // blockDim = 256: one super-block per pass (H is a multiple of 256)
        const float sbmax = a.sb_scale || a.x16 ? group256_max(fabsf(v), redm) : -1.f;
        encode32(v, threadIdx.x & 31, rec_at(a.xe, t, a.H), a.H, pos & ~31, a.sb_scale ? sbmax : -1.f);
        if (a.yzero) a.yzero[(size_t)t * a.H + pos] = 0.f;
        if (a.x16) encode_x16(v, a.x16 + ((size_t)t * (a.H >> 8) + (pos >> 8)) * kX16Bytes, pos & 255, true, sbmax);
    }
    if (a.kd > a.I)
        for (int p = t; p < a.P; p += a.T)
            zero_blocks(rec_at(a.hpad, p, a.kd), a.kd, a.I / 32, a.kd / 32, threadIdx.x, blockDim.x);
    if (t != 0 || a.T > kMaxT) return;  // larger batches are grouped by k_group_large
    for (int p = threadIdx.x; p < a.T * a.k; p += blockDim.x) sidx[p] = a.idx[p];
    __syncthreads();
    GroupOut go = a.go;
    go.wsrc = a.w;
    group_block(sidx, a.T, a.k, a.E, a.ns, go, lstart, PrePtr{nullptr, nullptr, false});
}

// k_group_large: the grouping of group_block for batches of up to
// kMaxTLarge tokens (one workgroup of 1024 threads), with a bitmap of
// tokens per expert instead of one 32-bit mask: ids are distinct per token,
// so pair (t, j) of expert e sits at offset[e] + (tokens below t that chose
// e).  Work entries cover at most `chunk` consecutive pairs of one expert
// (kItemTok for the dot-product kernels, kMfmaCols for the MFMA ones),
// in expert order, then the shared experts' pairs (token order) in the same
// chunks; entries past them are cleared.
constexpr int kGroupLargeThreads = 1024;
constexpr int kBmWords = kMaxTLarge / 32;

struct GroupLargeArgs {
    const int *idx;
    const float *w;
    int T, k, E, ns, chunk;
    GroupOut go;
};

// Exclusive scans of two values over the 1024 threads; totals in tot[2].
__device__ __forceinline__ void block_excl_scan2(int &a, int &b, int *lds /* 2 * 16 */, int *tot)
{
    const int lane = lane_id(), wv = wave_id();
    const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    if (lane == 63) { lds[wv] = ia; lds[16 + wv] = ib; }
    __syncthreads();
    int pa = 0, pb = 0, ta = 0, tb = 0;
    for (int w = 0; w < kGroupLargeThreads / 64; w++) {
        if (w < wv) { pa += lds[w]; pb += lds[16 + w]; }
        ta += lds[w];
        tb += lds[16 + w];
    }
    a = pa + ia - a;
    b = pb + ib - b;
    if (threadIdx.x == 0) { tot[0] = ta; tot[1] = tb; }
    __syncthreads();
}

__global__ __launch_bounds__(kGroupLargeThreads) void k_group_large(GroupLargeArgs a)
{
    __shared__ uint32_t bm[kMaxE * kBmWords];  // tokens of each expert
    __shared__ int cnt[kMaxE], off[kMaxE], iof[kMaxE];
    __shared__ int scan[32], tot[2];
    const int tid = (int)threadIdx.x, T = a.T, k = a.k, E = a.E, ns = a.ns, P = T * k, chunk = a.chunk;
    const int nw = (T + 31) >> 5;
    GroupOut g = a.go;
    for (int i = tid; i < E * kBmWords; i += kGroupLargeThreads) bm[i] = 0u;
    for (int e = tid; e < E; e += kGroupLargeThreads) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += kGroupLargeThreads) {
        const int e = a.idx[p], t = p / k;
        if ((unsigned)e < (unsigned)E) {
            atomicOr(&bm[e * kBmWords + (t >> 5)], 1u << (t & 31));
            atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    // pair offsets and entry offsets by expert (E <= kMaxE = 1024: one per thread)
    int c = tid < E ? cnt[tid] : 0;
    int it = (c + chunk - 1) / chunk;
    block_excl_scan2(c, it, scan, tot);
    if (tid < E) { off[tid] = c; iof[tid] = it; }
    __syncthreads();
    const int nvalid = tot[0], nitems = tot[1];
    for (int p = tid; p < P; p += kGroupLargeThreads) {
        const int e = a.idx[p], t = p / k, j = p - t * k;
        if ((unsigned)e >= (unsigned)E) {
            g.inv[t * (k + ns) + j] = -1;
            continue;
        }
        const uint32_t *row = bm + e * kBmWords;
        int r = __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
        for (int wd = 0; wd < (t >> 5); wd++) r += __popc(row[wd]);
        const int pos = off[e] + r;
        g.ptok[pos] = t;
        g.inv[t * (k + ns) + j] = pos;
        if (g.pw) g.pw[pos] = a.w[p];
    }
    for (int i = tid; i < ns * T; i += kGroupLargeThreads) {
        const int s2 = i / T, t = i - s2 * T, pos = nvalid + s2 * T + t;
        g.ptok[pos] = t;
        g.inv[t * (k + ns) + k + s2] = pos;
        if (g.pw) g.pw[pos] = 1.0f;  // shared experts have weight one
    }
    // routed entries: expert e's pairs [off, off + cnt) in chunks; the first
    // kInlineTok tokens of each chunk inline (the set bits of the bitmap from
    // rank it*chunk on)
    for (int e = tid; e < E; e += kGroupLargeThreads) {
        const int ce = cnt[e];
        if (ce == 0) continue;
        const uint32_t *row = bm + e * kBmWords;
        int wd = 0;
        uint32_t m = row[0];
        for (int i0 = 0, u = iof[e]; i0 < ce; i0 += chunk, u++) {
            WorkEntry we{};
            we.e = e; we.p0 = off[e] + i0; we.p1 = off[e] + min(i0 + chunk, ce);
            we.ptr = g.eptr ? g.eptr[e] : nullptr;
            // walk the bitmap to the chunk's tokens (bits consumed in order)
            for (int q = 0; q < chunk && i0 + q < ce; q++) {
                while (m == 0u && wd + 1 < nw) m = row[++wd];
                const int t = wd * 32 + __builtin_ctz(m);
                m &= m - 1u;
                if (q < kInlineTok) we.tok[q] = (uint8_t)t;  // t < kMaxTLarge = 256
            }
            g.wt[u] = we;
        }
    }
    const int sit = (T + chunk - 1) / chunk;
    for (int i = tid; i < ns * sit; i += kGroupLargeThreads) {
        const int s2 = i / sit, itn = i - s2 * sit;
        WorkEntry we{};
        we.e = E + s2;
        we.p0 = nvalid + s2 * T + itn * chunk;
        we.p1 = nvalid + s2 * T + min((itn + 1) * chunk, T);
        we.ptr = g.eptr ? g.sptr[s2] : nullptr;
        for (int q = 0; q < kInlineTok; q++) we.tok[q] = (uint8_t)(itn * chunk + q);
        g.wt[nitems + i] = we;
    }
    for (int u = nitems + ns * sit + tid; u < g.Umax; u += kGroupLargeThreads) g.wt[u] = WorkEntry{};
    if (tid == 0) *g.nuniq = nitems + ns * sit;
}

// k_group: moe_group_tokens (one workgroup).
__global__ __launch_bounds__(kRouteThreads) void k_group(const int *idx, int T, int k, int E, int *count,
                                                          int *offset, int *pairs)
{
    __shared__ int sidx[kMaxT * kMaxK];
    for (int p = threadIdx.x; p < T * k; p += blockDim.x) sidx[p] = idx[p];
    __syncthreads();
    group_sort(sidx, T, k, E, count, offset, pairs);
}

// k_rmsnorm: one workgroup per token.
__global__ __launch_bounds__(256) void k_rmsnorm(const float *h, int H, float eps, float *out)
{
    __shared__ float red[16];
    const float *ht = h + (size_t)blockIdx.x * H;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += blockDim.x) ss += ht[i] * ht[i];
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    for (int i = threadIdx.x; i < H; i += blockDim.x) out[(size_t)blockIdx.x * H + i] = ht[i] * r;
}

// ---------------------------------------------------------------------------
// Per-lane K-group dot products.  A lane owns one row of a 64-row tile (two
// rows, of two matrices sharing the activation, in k_gate_up) and one
// 256-column K-group.  The token's encoded record is staged in LDS; every
// lane of a half-wave reads the same 16-byte words (broadcast ds_read_b128),
// which feed v_dot4 directly.

struct XL {  // one encoded K-group in LDS
    const int4 *q0, *q1, *q2;        // 16 int4 (64 words) of each piece
    const float *bs, *bsum;          // 8 block scales, 8 block sums
    const int *p0, *p1, *p2;         // 16 per-16 sums of each piece
};

__device__ __forceinline__ XL xl(const uint8_t *rec, int K, int s)
{
    XL X;
    X.q0 = (const int4 *)(rec + s * 256);
    X.q1 = (const int4 *)(rec + K + s * 256);
    X.q2 = (const int4 *)(rec + 2 * K + s * 256);
    X.bs = (const float *)(rec + 3 * K) + s * 8;
    X.bsum = X.bs + K / 32;
    const int *ps = (const int *)(rec + 3 * K + K / 4) + s * 16;
    X.p0 = ps;
    X.p1 = ps + K / 16;
    X.p2 = ps + K / 8;
    return X;
}

__device__ __forceinline__ int w4(const int4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Q4KRegs { uint4 meta; uint4 q[8]; };
struct Q6KRegs { uint4 ql[8]; uint4 qh[4]; uint4 sc; uint32_t d; };
struct Q80Regs { uint4 q[16]; uint4 d; };

// Loads from expert slots.  Slot addresses come from tables in memory, whose
// address space the compiler cannot infer; these loads name the global
// space, so that they compile to global (not flat) loads, which need not
// wait for LDS traffic (flat loads may address LDS).
typedef const __attribute__((address_space(1))) uint8_t gbyte;
template <class T> __device__ __forceinline__ T ldg(const uint8_t *p, int off)
{
    return *(const __attribute__((address_space(1))) T *)((gbyte *)p + off);
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <> __device__ __forceinline__ uint2 ldg<uint2>(const uint8_t *p, int off)
{
    const u32x2 v = *(const __attribute__((address_space(1))) u32x2 *)((gbyte *)p + off);
    return make_uint2(v.x, v.y);
}
template <> __device__ __forceinline__ uint4 ldg<uint4>(const uint8_t *p, int off)
{
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)((gbyte *)p + off);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void load_regs(Q4KRegs &r, const uint8_t *tile, int lt)
{
    r.meta = ldg<uint4>(tile, lt * 16);
#pragma unroll
    for (int j = 0; j < 8; j++) r.q[j] = ldg<uint4>(tile, 1024 + j * 1024 + lt * 16);
}

__device__ __forceinline__ void load_regs(Q6KRegs &r, const uint8_t *tile, int lt)
{
#pragma unroll
    for (int j = 0; j < 8; j++) r.ql[j] = ldg<uint4>(tile, j * 1024 + lt * 16);
#pragma unroll
    for (int j = 0; j < 4; j++) r.qh[j] = ldg<uint4>(tile, 8192 + j * 1024 + lt * 16);
    r.sc = ldg<uint4>(tile, 12288 + lt * 16);
    r.d = ldg<unsigned short>(tile, 13312 + lt * 2);
}

__device__ __forceinline__ void load_regs(Q80Regs &r, const uint8_t *tile, int lt)
{
#pragma unroll
    for (int j = 0; j < 16; j++) r.q[j] = ldg<uint4>(tile, j * 1024 + lt * 16);
    r.d = ldg<uint4>(tile, 16384 + lt * 16);
}

__device__ __forceinline__ float fpieces(int a0, int a1, int a2)
{
    return (float)a0 + (float)a1 * kC1 + (float)a2 * kC2;
}

// Q4_K: sum_b bs_b*(d*sc_b*D_b) - dmin*m_b*bsum_b, D_b = piece dots of sub-block b.
template <int NM>
__device__ __forceinline__ void kgroup_dot(const Q4KRegs (&r)[NM], const XL &X, float (&out)[NM])
{
    uint32_t sclo[NM], mlo[NM], schi[NM], mhi[NM];
    float acc[NM], accm[NM];
#pragma unroll
    for (int m = 0; m < NM; m++) {
        const uint32_t W0 = r[m].meta.y, W1 = r[m].meta.z, W2 = r[m].meta.w;
        sclo[m] = W0 & 0x3F3F3F3Fu;
        mlo[m] = W1 & 0x3F3F3F3Fu;
        schi[m] = (W2 & 0x0F0F0F0Fu) | ((W0 >> 2) & 0x30303030u);
        mhi[m] = ((W2 >> 4) & 0x0F0F0F0Fu) | ((W1 >> 2) & 0x30303030u);
        acc[m] = 0.f;
        accm[m] = 0.f;
    }
#pragma unroll
    for (int sb = 0; sb < 8; sb++) {
        // sub-block sb: the low (even sb) or high (odd sb) nibbles of q words
        // 8(sb/2) .. 8(sb/2)+7, against words 8sb .. 8sb+7 of each piece
        const int c = sb >> 1;
        const int4 x0a = X.q0[2 * sb], x0b = X.q0[2 * sb + 1];
        const int4 x1a = X.q1[2 * sb], x1b = X.q1[2 * sb + 1];
        const int4 x2a = X.q2[2 * sb], x2b = X.q2[2 * sb + 1];
        const float bsv = X.bs[sb], bmv = X.bsum[sb];
#pragma unroll
        for (int m = 0; m < NM; m++) {
            const uint32_t scw = c < 2 ? sclo[m] : schi[m];
            const uint32_t mw = c < 2 ? mlo[m] : mhi[m];
            const int sh = 8 * (sb & 3);
            const int sc = (scw >> sh) & 0xff, mn = (mw >> sh) & 0xff;
            int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t qd = comp(r[m].q[2 * c + (i >> 2)], i & 3);
                const uint32_t nib = (sb & 1) ? (qd >> 4) & 0x0F0F0F0Fu : qd & 0x0F0F0F0Fu;
                a0 = dot4(nib, i < 4 ? w4(x0a, i) : w4(x0b, i - 4), a0);
                a1 = dot4(nib, i < 4 ? w4(x1a, i) : w4(x1b, i - 4), a1);
                a2 = dot4(nib, i < 4 ? w4(x2a, i) : w4(x2b, i - 4), a2);
            }
            acc[m] += (float)sc * (bsv * fpieces(a0, a1, a2));
            accm[m] += (float)mn * bmv;
        }
    }
#pragma unroll
    for (int m = 0; m < NM; m++) out[m] = half_lo(r[m].meta.x) * acc[m] - half_hi(r[m].meta.x) * accm[m];
}

// Q4_K against nt <= NT vectors at once: each sub-block's nibbles and
// scales are unpacked once for all of them.
template <int NT>
__device__ __forceinline__ void kgroup_dot_n(const Q4KRegs &r, const XL (&X)[NT], int nt, float (&out)[NT])
{
    const uint32_t W0 = r.meta.y, W1 = r.meta.z, W2 = r.meta.w;
    const uint32_t sclo = W0 & 0x3F3F3F3Fu, mlo = W1 & 0x3F3F3F3Fu;
    const uint32_t schi = (W2 & 0x0F0F0F0Fu) | ((W0 >> 2) & 0x30303030u);
    const uint32_t mhi = ((W2 >> 4) & 0x0F0F0F0Fu) | ((W1 >> 2) & 0x30303030u);
    float acc[NT], accm[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = accm[t] = 0.f;
#pragma unroll
    for (int sb = 0; sb < 8; sb++) {
        const int c = sb >> 1, sh = 8 * (sb & 3);
        const float fsc = (float)(((c < 2 ? sclo : schi) >> sh) & 0xff);
        const float fmn = (float)(((c < 2 ? mlo : mhi) >> sh) & 0xff);
        uint32_t nib[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t qd = comp(r.q[2 * c + (i >> 2)], i & 3);
            nib[i] = (sb & 1) ? (qd >> 4) & 0x0F0F0F0Fu : qd & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int t = 0; t < NT; t++) {
            if (t >= nt) break;
            const int4 x0a = X[t].q0[2 * sb], x0b = X[t].q0[2 * sb + 1];
            const int4 x1a = X[t].q1[2 * sb], x1b = X[t].q1[2 * sb + 1];
            const int4 x2a = X[t].q2[2 * sb], x2b = X[t].q2[2 * sb + 1];
            int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                a0 = dot4(nib[i], i < 4 ? w4(x0a, i) : w4(x0b, i - 4), a0);
                a1 = dot4(nib[i], i < 4 ? w4(x1a, i) : w4(x1b, i - 4), a1);
                a2 = dot4(nib[i], i < 4 ? w4(x2a, i) : w4(x2b, i - 4), a2);
            }
            acc[t] += fsc * (X[t].bs[sb] * fpieces(a0, a1, a2));
            accm[t] += fmn * X[t].bsum[sb];
        }
    }
    const float d = half_lo(r.meta.x), dmin = half_hi(r.meta.x);
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = d * acc[t] - dmin * accm[t];
}

// Q6_K: d * sum_b bs_b * sum_{j in b} sc_j * (Q_j - 32*S_j), Q_j / S_j piece dots / sums of sub-block j.
template <int NM>
__device__ __forceinline__ void kgroup_dot(const Q6KRegs (&r)[NM], const XL &X, float (&out)[NM])
{
    float acc[NM];
#pragma unroll
    for (int m = 0; m < NM; m++) acc[m] = 0.f;
#pragma unroll
    for (int n = 0; n < 2; n++) {
#pragma unroll
        for (int mq = 0; mq < 4; mq++) {
            // activation block b = 4n+mq: words 32n+8mq .. +8 of each piece (sub-blocks 2b, 2b+1)
            const int b = 4 * n + mq;
            const int4 x0a = X.q0[(32 * n + 8 * mq) / 4], x0b = X.q0[(32 * n + 8 * mq) / 4 + 1];
            const int4 x1a = X.q1[(32 * n + 8 * mq) / 4], x1b = X.q1[(32 * n + 8 * mq) / 4 + 1];
            const int4 x2a = X.q2[(32 * n + 8 * mq) / 4], x2b = X.q2[(32 * n + 8 * mq) / 4 + 1];
            const int s00 = X.p0[2 * b], s01 = X.p0[2 * b + 1];
            const int s10 = X.p1[2 * b], s11 = X.p1[2 * b + 1];
            const int s20 = X.p2[2 * b], s21 = X.p2[2 * b + 1];
            const float bsb = X.bs[b];
#pragma unroll
            for (int m = 0; m < NM; m++) {
                int I0 = 0, I1 = 0, I2 = 0;
#pragma unroll
                for (int ih = 0; ih < 2; ih++) {
                    int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
                    for (int i4 = 0; i4 < 4; i4++) {
                        const int i = 4 * ih + i4;
                        const uint32_t qlA = comp(r[m].ql[4 * n + (i >> 2)], i & 3);
                        const uint32_t qlB = comp(r[m].ql[4 * n + 2 + (i >> 2)], i & 3);
                        const uint32_t qhw = comp(r[m].qh[2 * n + (i >> 2)], i & 3);
                        uint32_t qv;
                        if (mq == 0) qv = (qlA & 0x0F0F0F0Fu) | ((qhw << 4) & 0x30303030u);
                        else if (mq == 1) qv = (qlB & 0x0F0F0F0Fu) | ((qhw << 2) & 0x30303030u);
                        else if (mq == 2) qv = ((qlA >> 4) & 0x0F0F0F0Fu) | (qhw & 0x30303030u);
                        else qv = ((qlB >> 4) & 0x0F0F0F0Fu) | ((qhw >> 2) & 0x30303030u);
                        const int xw0 = ih ? w4(x0b, i4) : w4(x0a, i4);
                        const int xw1 = ih ? w4(x1b, i4) : w4(x1a, i4);
                        const int xw2 = ih ? w4(x2b, i4) : w4(x2a, i4);
                        a0 = dot4(qv, xw0, a0);
                        a1 = dot4(qv, xw1, a1);
                        a2 = dot4(qv, xw2, a2);
                    }
                    const int j = 2 * b + ih;
                    const int sc = (int)(int8_t)((comp(r[m].sc, j >> 2) >> (8 * (j & 3))) & 0xff);
                    I0 += __mul24(sc, a0 - 32 * (ih ? s01 : s00));
                    I1 += __mul24(sc, a1 - 32 * (ih ? s11 : s10));
                    I2 += __mul24(sc, a2 - 32 * (ih ? s21 : s20));
                }
                acc[m] += bsb * fpieces(I0, I1, I2);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < NM; m++) out[m] = half_lo(r[m].d) * acc[m];
}

// Q8_0: sum_b d_b * bs_b * D_b over the 8 blocks of 32.
template <int NM>
__device__ __forceinline__ void kgroup_dot(const Q80Regs (&r)[NM], const XL &X, float (&out)[NM])
{
    float acc[NM];
#pragma unroll
    for (int m = 0; m < NM; m++) acc[m] = 0.f;
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const int4 x0a = X.q0[2 * b], x0b = X.q0[2 * b + 1];
        const int4 x1a = X.q1[2 * b], x1b = X.q1[2 * b + 1];
        const int4 x2a = X.q2[2 * b], x2b = X.q2[2 * b + 1];
        const float bsb = X.bs[b];
#pragma unroll
        for (int m = 0; m < NM; m++) {
            int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int D = 8 * b + i;
                const uint32_t qd = comp(r[m].q[D >> 2], D & 3);
                a0 = dot4(qd, i < 4 ? w4(x0a, i) : w4(x0b, i - 4), a0);
                a1 = dot4(qd, i < 4 ? w4(x1a, i) : w4(x1b, i - 4), a1);
                a2 = dot4(qd, i < 4 ? w4(x2a, i) : w4(x2b, i - 4), a2);
            }
            const uint32_t dw = comp(r[m].d, b >> 1);
            const float db = (b & 1) ? half_hi(dw) : half_lo(dw);
            acc[m] += db * (bsb * fpieces(a0, a1, a2));
        }
    }
#pragma unroll
    for (int m = 0; m < NM; m++) out[m] = acc[m];
}

// An empty asm that claims to modify the weight registers: the nibble
// unpacking then stays inside each dot product instead of being hoisted out
// of the token loop, where its unpacked copies would not fit in registers.
// Uses v, so that a load into it stays ahead of the branch it is issued
// before (the compiler would otherwise sink it into the one path using it).
__device__ __forceinline__ void use(const u32x4 &v) { asm volatile("" ::"v"(v)); }

template <class R> __device__ __forceinline__ void opaque(R &r)
{
    uint32_t *w = reinterpret_cast<uint32_t *>(&r);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(R) / 4); i++) asm volatile("" : "+v"(w[i]));
}

template <int QT> struct RegsOf;
template <> struct RegsOf<MOE_Q4_K> { using T = Q4KRegs; };
template <> struct RegsOf<MOE_Q6_K> { using T = Q6KRegs; };
template <> struct RegsOf<MOE_Q8_0> { using T = Q80Regs; };

template <int QT> constexpr int kTileBytes = QT == MOE_Q4_K ? 9216 : QT == MOE_Q6_K ? 13440 : 17408;

// Copy n bytes (multiple of 16) from global to LDS with the whole workgroup.
__device__ __forceinline__ void stage16(uint8_t *dst, const uint8_t *src, size_t n)
{
    const uint4 *s4 = (const uint4 *)src;
    uint4 *d4 = (uint4 *)dst;
    for (size_t i = threadIdx.x; i < n / 16; i += blockDim.x) d4[i] = s4[i];
}

__device__ __forceinline__ int token_of(const WorkEntry &we, const int *ptok, int p)
{
    const int i = p - we.p0;
    uint64_t toks;
    __builtin_memcpy(&toks, we.tok, sizeof(toks));
    return i < kInlineTok ? (int)((toks >> (8 * i)) & 0xff) : ptok[p];
}

// ---------------------------------------------------------------------------
// k_gate_up: workgroup (u, rt) = distinct expert u, rows [32rt, 32rt+32) of
// gate and up.  Thread 256m + 32j + r owns row 32rt+r of matrix m (0: gate,
// 1: up) for K-groups j, j+8, ...; the expert's tokens are staged in LDS
// `tpass` at a time.

struct GateUpArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const WorkEntry *wt;
    const int *ptok;
    Enc x;            // token records, K = H
    int H, I, kd;
    unsigned long long up_off;
    Enc h;            // pair records, K = kd
    float *act_out;   // [P][kd] or null
    int ntile;        // I/32
    int tpass;        // tokens staged per pass
    int T;            // tokens (records of x)
    // single-token routing done here (DEFER): the router's logit keys [E],
    // and the grouping that workgroup (0, 0) records for k_down
    const uint32_t *dlog;
    int k, ns, Umax;
    WorkEntry *wt_out;
    int *ptok_out, *inv, *nuniq;
    float *pw;
    // chained single-token layers (CH): this layer's router dots as partial
    // sums over 64-position tiles of the state (rp_in [H/64][kChainE]; null:
    // the route launch left its keys in dlog and its record in x), the state
    // hs [H], the router's bias [E] (or null) and eps; the next layer's router
    // wn [En][H], whose dots with the input state go to rp_out as tile
    // partials (or null: no next layer) for the down launch to add to
    const float *rp_in, *hs, *bias;
    float eps;
    const float *wn;
    int En;
    float *rp_out;
    int P;  // pair records in h (with rp_in their padding blocks are cleared here)
    int dlog_keys;  // with rp_in: rank the keys in dlog (a cache lookup formed them), not the partials
    // a cached single token whose missed experts are copied in this launch
    // (ncopy > 0, DEFER): the first ncopy workgroups copy the jobs' experts
    // from their pinned host copies into their slots, each adding its finished
    // share of job j to done[j] (with release semantics); a routed workgroup
    // whose expert e has jwait[e] = j + 1 (a miss) waits for done[j] = ncopy
    // (bounded by spin; a give-up sets the status word and NaN outputs)
    int ncopy;
    const CacheJob *jobs;
    const int32_t *njobs;
    const int32_t *jwait;
    uint32_t *done;
    unsigned long long slot_bytes;
    uint32_t *status;
    unsigned spin;
};

constexpr int kGUThreadsC = 512;  // the gate/up kernels' workgroup size

// One copying workgroup's share (16-byte words w*512 + tid, + ncopy*512, ...)
// of every miss job of the call, then the count of that share in done[j]:
// each thread's stores complete, the workgroup meets, and one release add
// (which writes the workgroup's data back to the device level first).
__device__ void cache_copy_share(const GateUpArgs &a, int w)
{
    const int nj = *a.njobs;
    const size_t n16 = a.slot_bytes / 16, stride = (size_t)a.ncopy * kGUThreadsC;
    for (int j = 0; j < nj; j++) {
        const CacheJob jb = a.jobs[j];
        const uint4 *src = (const uint4 *)jb.src;
        uint4 *dst = (uint4 *)jb.dst;
        size_t i = (size_t)w * kGUThreadsC + threadIdx.x;
        // four words in flight per thread
        for (; i + 3 * stride < n16; i += 4 * stride) {
            const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
            dst[i] = v0; dst[i + stride] = v1; dst[i + 2 * stride] = v2; dst[i + 3 * stride] = v3;
        }
        for (; i < n16; i += stride) dst[i] = src[i];
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(a.done + j, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One item j of the next router's dots with the state (chained layers): the
// 16 lanes of a 64-position tile of one router row each hold a float4 pair;
// their sum is the tile's partial of that row, stored by the first of them.
// Items past n4 (whole 16-lane groups) store nothing.
__device__ __forceinline__ void chain_item(float4 w, float4 x, int j, int n4, int H, float *rp_out)
{
    float d = w.x * x.x + w.y * x.y + w.z * x.z + w.w * x.w;
    d = group_sum<16>(d);
    if ((lane_id() & 15) == 0 && j < n4) {
        const int q4 = H >> 2, row = j / q4, c4 = j - row * q4;
        rp_out[(c4 >> 4) * kChainE + row] = d;
    }
}

// The items j0, j0 + stride, ... (stride a multiple of 16), four in flight
__device__ void chain_dots(const float *wn, const float *hs, int En, int H, float *rp_out, int j0, int stride)
{
    const int n4 = En * (H >> 2), q4 = H >> 2;
    for (int j = j0; j < n4; j += 4 * stride) {
        float4 w[4], x[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int jj = min(j + i * stride, n4 - 1);
            w[i] = ((const float4 *)wn)[jj];
            x[i] = ((const float4 *)hs)[jj % q4];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) chain_item(w[i], x[i], j + i * stride, n4, H, rp_out);
    }
}

// Encoding of positions pos .. pos+3 (v) of a record, the 8 consecutive
// lanes of a 32-position block holding 4 positions each: the arithmetic of
// encode32 (block scale a/127 from the block's largest magnitude, three
// int8 pieces, exact block sum, per-16 piece sums) in that layout.
__device__ __forceinline__ void encode32_x4(float4 v, uint8_t *rec, int K, int pos)
{
    const int r = lane_id() & 7;
    const float a = group_max<8>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    const float sm = group_sum<8>((v.x + v.y) + (v.z + v.w));
    const float inv = a > 0.f ? 127.0f / a : 0.f;
    const float vv[4] = {v.x, v.y, v.z, v.w};
    uint32_t w0 = 0, w1 = 0, w2 = 0;
    int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float r0 = vv[i] * inv, f0 = rintf(r0);
        const float r1 = (r0 - f0) * 254.0f, f1 = rintf(r1);
        const float r2 = (r1 - f1) * 254.0f, f2 = rintf(r2);
        const int i0 = (int)f0, i1 = (int)f1, i2 = (int)f2;
        w0 |= (uint32_t)(i0 & 0xff) << (8 * i);
        w1 |= (uint32_t)(i1 & 0xff) << (8 * i);
        w2 |= (uint32_t)(i2 & 0xff) << (8 * i);
        s0 += i0; s1 += i1; s2 += i2;
    }
    *(uint32_t *)(rec + pos) = w0;
    *(uint32_t *)(rec + K + pos) = w1;
    *(uint32_t *)(rec + 2 * K + pos) = w2;
    s0 = group_sum<4>(s0); s1 = group_sum<4>(s1); s2 = group_sum<4>(s2);
    if ((r & 3) == 0) {
        int *ps = (int *)(rec + 3 * K + K / 4) + pos / 16;
        ps[0] = s0;
        ps[K / 16] = s1;
        ps[K / 8] = s2;
    }
    if (r == 0) {
        float *bs = (float *)(rec + 3 * K);
        bs[pos / 32] = a / 127.0f;
        bs[K / 32 + pos / 32] = sm;
    }
}

// Ranks of one token's E <= 128 logit keys by a whole 512-thread workgroup:
// key i's rank is the number of keys that beat it (a larger key, or an equal
// key of lower id), i.e. of larger 64-bit composites key << 32 | ~id.  The
// lane quad 4i..4i+3 counts for key i, lane q over the quarter q of the
// composites (ids 32q .. 32q+31), all 16 reads issued at once, and the quad
// sums its counts with DPP.  The quarters sit 272 bytes apart in LDS, so that
// the four quarters' 16-byte reads of one instruction fall in different
// banks.  key: the composite of id tid/4 in lanes with tid % 4 == 0.
// Returns the rank of id tid/4 in every lane of its quad (ids past E: more
// than any k).  Holds one barrier.
constexpr int kRankStride = 34;  // 64-bit keys per quarter in LDS, with padding (272 B)
__device__ __forceinline__ int rank_keys_128(uint64_t key, int E, uint64_t *lk)
{
    const int tid = (int)threadIdx.x, i = tid >> 2, q = tid & 3;
    const int at = (i >> 5) * kRankStride + (i & 31);
    if (q == 0) lk[at] = i < E ? key : 0ull;
    __syncthreads();
    const uint64_t ki = lk[at];
    const ulonglong2 *src = (const ulonglong2 *)(lk + kRankStride * q);
    ulonglong2 v[16];
#pragma unroll
    for (int j = 0; j < 16; j++) v[j] = src[j];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) cnt += (v[j].x > ki) + (v[j].y > ki);
    cnt += xchg<1>(cnt);
    cnt += xchg<2>(cnt);
    return i < E ? cnt : 0x7fffffff;
}

constexpr int kGUThreads = kGUThreadsC;
constexpr int kTokPass = 4;  // <= kInlineTok
constexpr int kGUPre = 2;     // record words per thread loaded before the weights
constexpr int kGULds = 32768;   // staged token records per pass
constexpr int kDnLds = 24576;   // staged pair records per pass
constexpr int kDnPre = 4;       // record words per thread loaded before the weights

// NTOK: tokens per pass at most (1, 2 or kTokPass).  NTOK <= 2 (ALL):
// every token's record fits the first pass and the prefetch words (T <= 2,
// T * RB <= kGUPre * kGUThreads * 16); the records are then loaded before
// the work entry arrives, token t to LDS slot t.
// CP: a cached single token whose misses this launch copies (ncopy > 0); the
// copy role and the waits are compiled only into these instantiations
template <int QT, int NTOK, bool DEFER, bool CH = false, bool CP = false>
__global__ __launch_bounds__(kGUThreads) __attribute__((amdgpu_waves_per_eu(QT == MOE_Q4_K && !CH ? 4 : 2))) void k_gate_up(GateUpArgs a)
{
    extern __shared__ __align__(16) uint8_t xs[];
    __shared__ float part[8][kTokPass][32][2];
    constexpr bool ALL = NTOK <= 2;
    static_assert(!DEFER || NTOK == 1, "routing in the FFN is for a single token");
    static_assert(!CH || DEFER, "chained layers route in the FFN");
    static_assert(!CP || DEFER, "the copies are a single token's");

    int bid = (int)blockIdx.x;
    if constexpr (CP) {
        if (bid < a.ncopy) {  // a copying workgroup (the first ones, dispatched first)
            cache_copy_share(a, bid);
            return;
        }
        bid -= a.ncopy;
    }
    const int u = bid / a.ntile;
    const int rt = bid - u * a.ntile;
    const int H = a.H, S = H >> 8;
    const size_t RB = enc_bytes(H);
    const int q16 = (int)(RB / 16);  // 16-byte words per record
    const bool cin = CH && a.rp_in;
    const bool ckeys = cin && !a.dlog_keys;  // the keys formed here from the partials
    // CH loads first: with rp_in, this layer's router partials (id tid/4:
    // tiles tid%4, tid%4 + 4, ..., summed in the lane quad later), its bias
    // and the state (positions 4 tid + 2048 q)
    float4 hst[kChainMaxH / 2048];
    float pv[kChainMaxH / 256];
    float dsum = 0.f, dbias = 0.f;
    if constexpr (CH) {
        if (cin) {
            // every load issued before any is used (clamped indices; the
            // partials past the state's tiles are loaded and dropped)
            const int i = (int)(threadIdx.x >> 2), q4 = (int)(threadIdx.x & 3), nct = H >> 6;
            dbias = a.bias ? a.bias[min(i, a.E - 1)] : 0.f;
#pragma unroll
            for (int q = 0; q < kChainMaxH / 2048; q++)
                hst[q] = ((const float4 *)a.hs)[min((int)threadIdx.x + kGUThreads * q, (H >> 2) - 1)];
            // (loaded even when the keys come from dlog)
#pragma unroll
            for (int n = 0; n < kChainMaxH / 256; n++) pv[n] = a.rp_in[min(q4 + 4 * n, nct - 1) * kChainE + i];
        }
    }
    // DEFER: the logit key (unless CH computes it) and expert address of id
    // tid/4, loaded first by lane 0 of each quad
    uint32_t dkey = 0;
    const void *dptr = nullptr;
    int djw = 0;  // ncopy: the id's copy job + 1 (0: no copy to wait for)
    if (DEFER && u < a.k && (threadIdx.x & 3) == 0 && (int)(threadIdx.x >> 2) < a.E) {
        if (!ckeys) dkey = a.dlog[threadIdx.x >> 2];
        dptr = a.eptr[threadIdx.x >> 2];
        if (CP) djw = a.jwait[threadIdx.x >> 2];
    }
    u32x4 xr[kGUPre] = {};
    if (ALL && !cin) {
        // the records are back to back: word i is word i % q16 of token i / q16
#pragma unroll
        for (int q = 0; q < kGUPre; q++)
            xr[q] = ((const u32x4 *)a.x.base)[min((int)threadIdx.x + q * kGUThreads, a.T * q16 - 1)];
    }
    int e, p0, p1;
    const uint8_t *base;
    uint64_t toks = 0;
    bool gave = false;  // ncopy: the wait for this expert's copy gave up (NaN outputs)
    if constexpr (DEFER) {
        // Routing of the single token from the router's logit keys, in every
        // workgroup (E <= 128): the ranks of the keys; the expert of rank u is
        // work item and pair u (ranks order the pairs here: the layer calls
        // never expose the grouped order).  Workgroup (0, 0) records the
        // grouping and the softmax weights for k_down.  Items k .. k+ns-1 are
        // the shared experts, items past them are empty.
        __shared__ __align__(16) uint64_t lk[4 * kRankStride];
        __shared__ int lsel_e[kMaxK];
        __shared__ const void *lsel_p[kMaxK];
        __shared__ int lsel_w[kMaxK];
        __shared__ int lgave;
        __shared__ uint32_t lkey_r[kMaxK];
        const int k = a.k, ns = a.ns, tid = (int)threadIdx.x;
        if (u >= k + ns) {
#pragma unroll
            for (int q = 0; q < kGUPre; q++) use(xr[q]);
            if constexpr (CH) {
                // the workgroups without a work item (the last ones) take
                // the next router's dots with the input state
                const int i0 = (k + ns) * a.ntile;
                if (a.rp_out)
                    chain_dots(a.wn, a.hs, a.En, H, a.rp_out, (bid - i0) * kGUThreads + tid,
                               ((int)gridDim.x - (CP ? a.ncopy : 0) - i0) * kGUThreads);
                // the route launch, which did not run, cleared the pair
                // records' padding blocks
                if (cin && u == k + ns && a.kd > a.I)
                    for (int p = rt; p < a.P; p += a.ntile)
                        zero_blocks(rec_at(a.h, p, a.kd), a.kd, a.I / 32, a.kd / 32, tid, kGUThreads);
            }
            return;
        }
        if constexpr (CH) {
            if (cin) {
                // the RMS of the state, then the logit key of id tid/4
                __shared__ float lred[kGUThreads / 64];
                float ss = 0.f;
#pragma unroll
                for (int q = 0; q < kChainMaxH / 2048; q++)
                    if (tid + kGUThreads * q < (H >> 2))
                        ss += hst[q].x * hst[q].x + hst[q].y * hst[q].y + hst[q].z * hst[q].z + hst[q].w * hst[q].w;
                ss = wave_sum(ss);
                if (lane_id() == 0) lred[wave_id()] = ss;
                __syncthreads();
                ss = 0.f;
#pragma unroll
                for (int w = 0; w < kGUThreads / 64; w++) ss += lred[w];
                const float rms = 1.0f / sqrtf(ss / (float)H + a.eps);
#pragma unroll
                for (int q = 0; q < kChainMaxH / 2048; q++) {
                    hst[q].x *= rms; hst[q].y *= rms; hst[q].z *= rms; hst[q].w *= rms;
                }
                if (ckeys) {
#pragma unroll
                    for (int n = 0; n < kChainMaxH / 256; n++) dsum += (tid & 3) + 4 * n < (H >> 6) ? pv[n] : 0.f;
                    dsum += xchg<1>(dsum);
                    dsum += xchg<2>(dsum);
                    dkey = logit_key(dsum * rms + dbias);
                }
            }
        }
        if (u >= k) {
            e = a.E + (u - k);
            base = (const uint8_t *)a.sptr[u - k];
        } else {
            const int r = rank_keys_128((uint64_t)dkey << 32 | (uint32_t)~(threadIdx.x >> 2), a.E, lk);
            if (r < k && (tid & 3) == 0) {
                lsel_e[r] = tid >> 2;
                lsel_p[r] = dptr;
                lsel_w[r] = djw;
                lkey_r[r] = dkey;
            }
            __syncthreads();
            e = lsel_e[u];
            base = (const uint8_t *)lsel_p[u];
            if constexpr (CP) {
                const int jw = lsel_w[u];
                if (jw > 0) {
                    // a missed expert: thread 0 waits for its copy, then an
                    // acquire, so that no line of the slot read before the
                    // copy is used; the workgroup meets after it
                    if (tid == 0) {
                        int ok = 0;
                        for (unsigned it = 0;; it++) {
                            if (__hip_atomic_load(a.done + jw - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                                (uint32_t)a.ncopy) {
                                ok = 1;
                                break;
                            }
                            if (it >= a.spin) break;
                            __builtin_amdgcn_s_sleep(2);
                        }
                        if (!ok) flag_status(a.status, MOE_WS_COPY_TIMEOUT);
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                        lgave = !ok;
                    }
                    __syncthreads();
                    gave = lgave != 0;
                }
            }
        }
        p0 = u;
        p1 = u + 1;
        if (u == 0 && rt == 0 && tid < 64) {
            // softmax over the k selected logits (selection j = rank j) and
            // the grouping: pair j = selection j
            const int lane = tid;
            const float lg = lane < k ? unord_bits(lkey_r[lane]) : 0.f;
            const float top = unord_bits(lkey_r[0]);
            const float ex = lane < k ? expf(lg - top) : 0.f;
            const float wsum = wave_sum(ex);
            if (lane < k) {
                WorkEntry we{};
                we.e = lsel_e[lane]; we.p0 = lane; we.p1 = lane + 1;
                we.ptr = lsel_p[lane];
                a.wt_out[lane] = we;
                a.ptok_out[lane] = 0;
                a.inv[lane] = lane;
                a.pw[lane] = ex / wsum;
            }
            if (lane < ns) {
                WorkEntry we{};
                we.e = a.E + lane; we.p0 = k + lane; we.p1 = k + lane + 1;
                we.ptr = a.sptr[lane];
                a.wt_out[k + lane] = we;
                a.ptok_out[k + lane] = 0;
                a.inv[k + lane] = k + lane;
                a.pw[k + lane] = 1.0f;
            }
            for (int u2 = k + ns + lane; u2 < a.Umax; u2 += 64) a.wt_out[u2] = WorkEntry{};
            if (lane == 0) *a.nuniq = k + ns;
        }
    } else {
        const WorkEntry we = load_entry(a.wt, u);
        e = we.e; p0 = we.p0; p1 = we.p1;
        if (p0 >= p1) {
            if (ALL)
#pragma unroll
                for (int q = 0; q < kGUPre; q++) use(xr[q]);
            return;
        }
        base = (const uint8_t *)(we.ptr ? we.ptr : e < a.E ? a.eptr[e] : a.sptr[e - a.E]);
        __builtin_memcpy(&toks, we.tok, sizeof(toks));
    }
    (void)e;
    const int lane = lane_id();
    const int m = (int)(threadIdx.x >> 8);              // 0: gate, 1: up
    const int slot = (int)((threadIdx.x >> 5) & 7), r = lane & 31;
    const int row = rt * 32 + r;
    const int tile64 = row >> 6, lt = row & 63;
    const uint8_t *mat = base + (m ? a.up_off : 0);

    // The first pass's token records (kGUPre words per thread into registers,
    // the rest by LDS DMA) are loaded before the weights: loads complete in
    // order, so when the registers suffice the barrier after staging them
    // does not wait for the weights, and each wave starts its dots as soon as
    // its own weights arrive.
    const int nt0 = p1 - p0 < a.tpass ? p1 - p0 : a.tpass;
    const float rq16 = 1.0f / (float)q16;
    if (!ALL) {
#pragma unroll
        for (int q = 0; q < kGUPre; q++) {
            // unconditional loads (clamped index): no per-word branches, whose
            // merges would wait for each load
            const int i = min((int)threadIdx.x + q * kGUThreads, nt0 * q16 - 1);
            const int tt = fdiv(i, rq16);  // < tpass <= kInlineTok: an inline token
            const int tok = (int)((toks >> (8 * tt)) & 0xff);
            xr[q] = ((const u32x4 *)rec_at(a.x, tok, H))[i - tt * q16];
        }
        // Words past the prefetch go straight to LDS (a 16-byte LDS DMA per
        // lane, 64 consecutive words per wave, which never straddle two
        // records: q16 is a multiple of 64).  Their wait then also waits for
        // the weights issued below, which the dots need first anyway.
        const int w0 = (int)(threadIdx.x & ~63u);
#pragma unroll
        for (int q = kGUPre; q < kGULds / 16 / kGUThreads; q++) {
            const int i0 = w0 + q * kGUThreads;  // wave-uniform
            if (i0 < nt0 * q16) {
                const int tt = fdiv(i0, rq16);
                const int tok = (int)((toks >> (8 * tt)) & 0xff);
                const uint8_t *src = rec_at(a.x, tok, H) + (size_t)(i0 + lane - tt * q16) * 16;
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                                 (__attribute__((address_space(3))) void *)(xs + (size_t)i0 * 16), 16, 0, 0);
            }
        }
    }
    // the first K-group's weights, loaded unconditionally (slots past S
    // load K-group 0 and leave it unused) so that the waits for the records
    // above count these loads as still in flight
    typename RegsOf<QT>::T rg[1];
    load_regs(rg[0], mat + ((size_t)tile64 * S + (slot < S ? slot : 0)) * kTileBytes<QT>, lt);
    int loaded = slot < S ? slot : -1;
    for (int c0 = p0; c0 < p1; c0 += a.tpass) {
        const int nt = p1 - c0 < a.tpass ? p1 - c0 : a.tpass;
        if (cin && c0 == p0) {
            // the state's record (normalised above), encoded here
#pragma unroll
            for (int q = 0; q < kChainMaxH / 2048; q++) {
                const int pos = 4 * ((int)threadIdx.x + kGUThreads * q);
                if (pos < H) encode32_x4(hst[q], xs, H, pos);  // whole waves
            }
        } else if (c0 == p0) {
            const int n16 = (ALL ? a.T : nt0) * q16;
#pragma unroll
            for (int q = 0; q < kGUPre; q++) {
                const int i = (int)threadIdx.x + q * kGUThreads;
                if (i < n16) ((u32x4 *)xs)[i] = xr[q];
            }
        } else {
            __syncthreads();  // the previous pass is done with xs
            for (int tt = 0; tt < nt; tt++) {
                const int i = c0 + tt - p0;
                const int tok = i < kInlineTok ? (int)((toks >> (8 * i)) & 0xff) : a.ptok[c0 + tt];
                stage16(xs + tt * RB, rec_at(a.x, tok, H), RB);
            }
        }
        __syncthreads();
        // each lane owns part[slot][*][r]: plain writes for its first K-group, sums after
        for (int s = slot; s < S; s += 8) {
            if (s != loaded) {
                load_regs(rg[0], mat + ((size_t)tile64 * S + s) * kTileBytes<QT>, lt);
                loaded = s;
            }
            if constexpr (QT == MOE_Q4_K) {
                // all nt <= kTokPass tokens of the pass at once (ALL: a
                // single pass, its tokens inline)
                XL X[kTokPass];
#pragma unroll
                for (int tt = 0; tt < kTokPass; tt++)
                    X[tt] = xl(xs + (ALL ? (int)((toks >> (8 * tt)) & 0xff) : tt) * RB, H, s);
                float o[kTokPass];
                opaque(rg[0]);
                if constexpr (NTOK < kTokPass) {
                    XL Xn[NTOK];
                    float on[NTOK];
#pragma unroll
                    for (int tt = 0; tt < NTOK; tt++) Xn[tt] = X[tt];
                    kgroup_dot_n<NTOK>(rg[0], Xn, nt, on);
#pragma unroll
                    for (int tt = 0; tt < NTOK; tt++) o[tt] = on[tt];
                } else {
                    kgroup_dot_n<kTokPass>(rg[0], X, nt, o);
                }
#pragma unroll
                for (int tt = 0; tt < kTokPass; tt++)
                    if (tt < nt) {
                        if (s == slot) part[slot][tt][r][m] = o[tt];
                        else part[slot][tt][r][m] += o[tt];
                    }
            } else {
#pragma unroll 1
                for (int tt = 0; tt < nt; tt++) {
                    float o[1];
                    opaque(rg[0]);
                    const int xslot = ALL ? (int)((toks >> (8 * tt)) & 0xff) : tt;
                    kgroup_dot<1>(rg, xl(xs + xslot * RB, H, s), o);
                    if (s == slot) part[slot][tt][r][m] = o[0];
                    else part[slot][tt][r][m] += o[0];
                }
            }
        }
        if (slot >= S)
            for (int tt = 0; tt < nt; tt++) part[slot][tt][r][m] = 0.f;
        __syncthreads();
        // SiLU(g)*u of rows [32rt, 32rt+32) and their encoding as block rt
        for (int i = threadIdx.x; i < nt * 32; i += blockDim.x) {
            const int tt = i >> 5, rr = i & 31;
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int sl = 0; sl < 8; sl++) {
                gs += part[sl][tt][rr][0];
                us += part[sl][tt][rr][1];
            }
            const float hv = CP && gave ? __builtin_nanf("") : gs / (1.0f + expf(-gs)) * us;
            encode32(hv, rr, rec_at(a.h, c0 + tt, a.kd), a.kd, rt * 32);
            if (a.act_out) a.act_out[(size_t)(c0 + tt) * a.kd + rt * 32 + rr] = hv;
        }
    }
}

// ---------------------------------------------------------------------------
// k_down: workgroup (u, rt) = distinct expert u, down rows [64rt, 64rt+64);
// wave w takes K-groups w, w+nw, ...  The expert's pair records are staged
// in LDS `tpass` at a time.  Each pair's rows, times the pair's combine
// weight, are added to its token's rows of y with float atomics, so the
// experts of a token are summed in whatever order their workgroups finish
// (the sum is exact up to fp32 rounding; its last bits can vary from run to
// run).

struct DownArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const int *nuniq;
    const WorkEntry *wt;
    Enc h;           // pair records, K = kd
    int H, kd;
    unsigned long long down_off;
    int nrt;
    const int *ptok; // [P] token of each grouped pair
    const float *pw; // [P] combine weight of each grouped pair
    float *y;        // [T][H], added into
    int tpass;
    int P;           // pair records in h
    // chained single-token layers (CH): the next layer's router wn [En][H];
    // each workgroup adds the dots of its rows' contribution with wn's
    // columns of the tile to rp_out [H/64][kChainE]
    const float *wn;
    int En;
    float *rp_out;
};

// next-router float4 per thread held through the dots (CH; fewer for the
// types whose dots need more registers)
template <int QT> constexpr int kDnChainPre = QT == MOE_Q4_K ? 12 : 6;

// y[t][row] += v, relaxed agent-scope float atomic (no return value).
__device__ __forceinline__ void add_to(float *p, float v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ONE: a single token, whose work item u is pair u (one pair per item, in
// pair order); the pair's record is then loaded before the work entry
// arrives (it must fit the prefetch words).
template <int QT, bool ONE, bool CH = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(CH ? 2 : QT == MOE_Q4_K ? 4 : 3))) void k_down(DownArgs a)
{
    static_assert(!CH || ONE, "chained layers carry a single token");
    extern __shared__ __align__(16) uint8_t hsl[];
    __shared__ __align__(16) float part[8][kItemTok][64];
    __shared__ int lptok[kItemTok];   // the item's pairs' tokens and combine weights
    __shared__ float lpw[kItemTok];

    const int u = blockIdx.x / a.nrt;
    const int rt = blockIdx.x - u * a.nrt;
    u32x4 hr[kDnPre];
    int tok1 = 0;
    float pw1 = 0.f;
    if (ONE) {
        // item u is pair u: its record, token and weight are loaded before
        // the work entry arrives (their addresses do not depend on it)
        const int pp = min(u, a.P - 1);
        const u32x4 *h16 = (const u32x4 *)rec_at(a.h, pp, a.kd);
        const int n16 = (int)(enc_bytes(a.kd) / 16);
#pragma unroll
        for (int q = 0; q < kDnPre; q++) hr[q] = h16[min((int)threadIdx.x + q * (int)blockDim.x, n16 - 1)];
        tok1 = a.ptok[pp];
        pw1 = a.pw[pp];
    }
    const WorkEntry we = load_entry(a.wt, u);
    const int e = we.e, p0 = we.p0, p1 = we.p1;
    if (p0 >= p1) {
        if (ONE) {
#pragma unroll
            for (int q = 0; q < kDnPre; q++) use(hr[q]);
            asm volatile("" ::"v"(tok1), "v"(pw1));
        }
        return;
    }
    if (ONE && (p0 != u || p1 != u + 1)) {
        // not the one-pair-per-item grouping the records were loaded for
        for (int i = threadIdx.x; i < (p1 - p0) * 64; i += blockDim.x)
            add_to(a.y + (size_t)a.ptok[p0 + (i >> 6)] * a.H + rt * 64 + (i & 63), __builtin_nanf(""));
        return;
    }
    const uint8_t *base =
        (const uint8_t *)(we.ptr ? we.ptr : e < a.E ? a.eptr[e] : a.sptr[e - a.E]) + a.down_off;
    const int kd = a.kd, S = kd >> 8;
    const size_t RB = enc_bytes(kd);
    const int nwv = (int)(blockDim.x >> 6);
    const int wv = wave_id(), lane = lane_id();

    // The first pass's pair records (contiguous), up to kDnPre words per
    // thread, are loaded before the weights, as in k_gate_up: the wait for
    // them before the barrier then leaves the weights in flight, and each
    // wave starts its dots as soon as its own weights arrive.  Words past
    // kDnPre are staged after the barrier.
    const int n16 = (int)((p1 - p0 < a.tpass ? p1 - p0 : a.tpass) * RB / 16);
    const u32x4 *h16 = (const u32x4 *)rec_at(a.h, p0, kd);
    if (!ONE) {
#pragma unroll
        for (int q = 0; q < kDnPre; q++) hr[q] = h16[min((int)threadIdx.x + q * (int)blockDim.x, n16 - 1)];
        // an item has at most kItemTok pairs
        if ((int)threadIdx.x < p1 - p0) {
            lptok[threadIdx.x] = a.ptok[p0 + threadIdx.x];
            lpw[threadIdx.x] = a.pw[p0 + threadIdx.x];
        }
    }
    // blockDim = 64 * min(S, 8): every wave has a K-group (loaded
    // unconditionally, for the same reason as in k_gate_up)
    typename RegsOf<QT>::T rg[1];
    load_regs(rg[0], base + ((size_t)rt * S + wv) * kTileBytes<QT>, lane);
    int loaded = wv;
    // CH: the next router's columns of this tile (item j: row j/16, float4
    // j%16 of the 64 positions), issued after the weights, so that the dots'
    // waits for those do not wait for these
    float4 cwv[kDnChainPre<QT>];
    int cn4 = 0;
    if constexpr (CH) {
        cn4 = a.En * 16;
#pragma unroll
        for (int q = 0; q < kDnChainPre<QT>; q++) {
            const int j = min((int)threadIdx.x + q * (int)blockDim.x, cn4 - 1);
            cwv[q] = ((const float4 *)(a.wn + (size_t)(j >> 4) * a.H + rt * 64))[j & 15];
        }
    }
    for (int c0 = p0; c0 < p1; c0 += a.tpass) {
        const int nt = p1 - c0 < a.tpass ? p1 - c0 : a.tpass;
        if (c0 == p0) {
#pragma unroll
            for (int q = 0; q < kDnPre; q++) {
                const int i = (int)threadIdx.x + q * (int)blockDim.x;
                if (i < n16) ((u32x4 *)hsl)[i] = hr[q];
            }
            for (int i = (int)threadIdx.x + kDnPre * (int)blockDim.x; i < n16; i += blockDim.x)
                ((u32x4 *)hsl)[i] = h16[i];
        } else {
            __syncthreads();
            stage16(hsl, rec_at(a.h, c0, kd), nt * RB);  // the expert's pairs are contiguous
        }
        __syncthreads();
        for (int s = wv; s < S; s += nwv) {
            if (s != loaded) {
                load_regs(rg[0], base + ((size_t)rt * S + s) * kTileBytes<QT>, lane);
                loaded = s;
            }
            if constexpr (QT == MOE_Q4_K) {
                // all nt <= kItemTok pairs of the pass at once (tpass <= kItemTok)
                XL X[kItemTok];
#pragma unroll
                for (int tt = 0; tt < kItemTok; tt++) X[tt] = xl(hsl + tt * RB, kd, s);
                float v[kItemTok];
                opaque(rg[0]);
                if constexpr (ONE) {
                    XL X1[1] = {X[0]};
                    float v1[1];
                    kgroup_dot_n<1>(rg[0], X1, 1, v1);
                    v[0] = v1[0];
                } else {
                    kgroup_dot_n<kItemTok>(rg[0], X, nt, v);
                }
#pragma unroll
                for (int tt = 0; tt < kItemTok; tt++)
                    if (tt < nt) {
                        if (s == wv) part[wv][tt][lane] = v[tt];
                        else part[wv][tt][lane] += v[tt];
                    }
            } else {
#pragma unroll 1
                for (int tt = 0; tt < nt; tt++) {
                    float v[1];
                    opaque(rg[0]);
                    kgroup_dot<1>(rg, xl(hsl + tt * RB, kd, s), v);
                    if (s == wv) part[wv][tt][lane] = v[0];
                    else part[wv][tt][lane] += v[0];
                }
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nt * 64; i += blockDim.x) {
            const int tt = i >> 6, ln = i & 63;
            float sum = 0.f;
            for (int w = 0; w < nwv; w++) sum += part[w][tt][ln];
            const int q = c0 - p0 + tt;  // < kItemTok
            const int tok = ONE ? tok1 : lptok[q];
            const float pw = ONE ? pw1 : lpw[q];
            add_to(a.y + (size_t)tok * a.H + rt * 64 + ln, pw * sum);
        }
    }
    if constexpr (CH) {
        // The dots of the tile's contribution with the next router's rows,
        // without a barrier: every wave forms the contribution's columns
        // 4(lane%16) .. +3 from the waves' partial sums (complete since the
        // barrier before the sums above, and summed in the same order), 16
        // lanes take a row, and the wave's row sums are gathered into lanes
        // 4q + i (row 4w + q*blockDim/16 + i) for one atomic instruction.
        const int c4 = 4 * (lane & 15);
        float4 cv = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int w = 0; w < nwv; w++) {
            cv.x += part[w][0][c4];
            cv.y += part[w][0][c4 + 1];
            cv.z += part[w][0][c4 + 2];
            cv.w += part[w][0][c4 + 3];
        }
        cv.x *= pw1; cv.y *= pw1; cv.z *= pw1; cv.w *= pw1;
        float mine = 0.f;
#pragma unroll
        for (int q = 0; q < kDnChainPre<QT>; q++) {
            const float d = group_sum<16>(cwv[q].x * cv.x + cwv[q].y * cv.y + cwv[q].z * cv.z + cwv[q].w * cv.w);
            const float v = __shfl(d, 16 * (lane & 3), 64);
            if ((lane >> 2) == q) mine = v;
        }
        {
            const int q = lane >> 2, i = lane & 3;
            const int j = 64 * wv + q * (int)blockDim.x + 16 * i;
            if (q < kDnChainPre<QT> && j < cn4) add_to(a.rp_out + rt * kChainE + (j >> 4), mine);
        }
        // rows past the held ones (small workgroups, or types holding fewer)
        for (int j = (int)threadIdx.x + kDnChainPre<QT> * (int)blockDim.x; j < cn4; j += blockDim.x) {
            const float4 w = ((const float4 *)(a.wn + (size_t)(j >> 4) * a.H + rt * 64))[j & 15];
            const float d = group_sum<16>(w.x * cv.x + w.y * cv.y + w.z * cv.z + w.w * cv.w);
            if ((lane & 15) == 0) add_to(a.rp_out + rt * kChainE + (j >> 4), d);
        }
    }
}

// ---------------------------------------------------------------------------
// MFMA path for Q4_K experts with many tokens (the batched form of the
// expert FFN, T4 MoE-cache report, "What the MoE cache caches": batches of
// up to 32 tokens).  Per 256-wide super-block of a weight row the Q4_K value
// is  d * sc_b * q - dmin * m_b  (b = 32-wide sub-block), so
//     row . x = d * sum_b sc_b (q . x)_b  -  dmin * sum_b m_b S_b,
// S_b the block sums of x.  sc_b * q <= 63 * 15 = 945 and m_b <= 63 are
// integers exact in fp16; x is split into fp16 hi + lo parts (22 bits) after
// scaling the column's super-block by a power of two.  One super-block of
// one 32-row block against up to 32 columns is then 16 v_mfma_f32_32x32x16_f16
// per part for the first term and one v_mfma_f32_32x32x8_f16 per part for
// the second, both accumulated in fp32 (products exact), and an epilogue
//     acc[t][r] += 2^-e_t * (d_r * C1[t][r] - dmin_r * C2[t][r]).
// MFMA operand layouts (v_mfma_f32_32x32x16_f16): A lane l holds row l%32,
// K (l/32)*8 + [0,8); B lane l holds column l%32, the same K; D lane l holds
// column l%32, rows 8j + 4*(l/32) + i in element 4j+i.  Here A = activations
// (rows = the expert's columns, i.e. tokens or pairs), B = weights (columns
// = weight rows), so each lane owns one weight row of the output.

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaCols = 32;  // columns (tokens or pairs) per expert
// LDS of one staged super-block: hi and lo [16 K-steps][2 halves][32 cols][8]
// (for one column, its 256 positions in order, in 32 chunks of 8 that lie
// 32 columns apart), block sums [hi, lo][32 cols][8 blocks], column scales
// [32] (+32 unused, the second half-wave's target when staged by DMA).
constexpr int kStageHalf = 16 * 2 * kMfmaCols * 8;  // halves per part
constexpr int kStageSum = 2 * kMfmaCols * 8;       // halves
constexpr size_t kStageBytes = (size_t)(2 * kStageHalf + kStageSum) * 2 + 2 * kMfmaCols * 4;

struct Stage {
    _Float16 *hi, *lo, *sum;
    float *esc;
};
__device__ __forceinline__ Stage stage_at(uint8_t *base)
{
    Stage st;
    st.hi = (_Float16 *)base;
    st.lo = st.hi + kStageHalf;
    st.sum = st.lo + kStageHalf;
    st.esc = (float *)(st.sum + kStageSum);
    return st;
}

// Staging of super-block sb of n columns (column c = row rowof(c) of src,
// fp32, row length K, positions >= valid read as zero), in two halves so
// that the loads of the next super-block are in flight during the MFMAs of
// the current one: stage_load fills the registers, stage_store converts them
// into LDS.  The 256 items (column c, 32-wide block b) go to the NT threads
// in turn, NI = 256/NT each, columns fastest (neighbouring threads store
// neighbouring 16-byte chunks: no LDS bank conflicts).  A column's scale is
// a power of two bringing its largest magnitude in the super-block to
// [0.5, 1).
template <int NT> struct StageRegs {
    float v[256 / NT][32];
};

template <int NT, class RowOf>
__device__ __forceinline__ void stage_load(StageRegs<NT> &r, const float *src, int K, int valid, int sb, int n,
                                           RowOf rowof)
{
    constexpr int NI = 256 / NT;
#pragma unroll
    for (int it = 0; it < NI; it++) {
        const int item = threadIdx.x + it * NT, c = item & (kMfmaCols - 1), b = item / kMfmaCols;
        const int pos0 = sb * 256 + b * 32;
        if (c < n) {
            const float *row = src + (size_t)rowof(c) * K;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int p = pos0 + 4 * i;
                float4 q;
                if (p + 3 < valid) {
                    q = *(const float4 *)(row + p);
                } else {  // ragged end of the valid positions
                    q.x = p < valid ? row[p] : 0.f;
                    q.y = p + 1 < valid ? row[p + 1] : 0.f;
                    q.z = p + 2 < valid ? row[p + 2] : 0.f;
                    q.w = 0.f;
                }
                r.v[it][4 * i] = q.x; r.v[it][4 * i + 1] = q.y; r.v[it][4 * i + 2] = q.z; r.v[it][4 * i + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; i++) r.v[it][i] = 0.f;
        }
    }
}

// lmax: LDS [kMfmaCols] ints, zero on entry and left zero on exit.  Every
// thread of the workgroup calls this (it holds barriers).
template <int NT>
__device__ __forceinline__ void stage_store(const StageRegs<NT> &r, Stage st, int *lmax)
{
    constexpr int NI = 256 / NT;
#pragma unroll
    for (int it = 0; it < NI; it++) {
        const int c = (threadIdx.x + it * NT) & (kMfmaCols - 1);
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 32; i++) m = fmaxf(m, fabsf(r.v[it][i]));
        if (m > 0.f) atomicMax(&lmax[c], __float_as_int(m));  // order of magnitudes = order of their bits
    }
    __syncthreads();
    int cms[NI];
#pragma unroll
    for (int it = 0; it < NI; it++) cms[it] = lmax[(threadIdx.x + it * NT) & (kMfmaCols - 1)];
    __syncthreads();
    if (threadIdx.x < kMfmaCols) lmax[threadIdx.x] = 0;  // for the next call
#pragma unroll
    for (int it = 0; it < NI; it++) {
        const int item = threadIdx.x + it * NT, c = item & (kMfmaCols - 1), b = item / kMfmaCols;
        const float cm = __int_as_float(cms[it]);
        const int e = cm > 0.f ? -ilogbf(cm) - 1 : 0;  // cm * 2^e in [0.5, 1)
        const float sc = ldexpf(1.0f, e);
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {  // 8 positions: K-step 2b + j/2, half j%2
            f16x8 h, l;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float x = r.v[it][8 * j + i] * sc;  // exact (power of two)
                const _Float16 xh = (_Float16)x;
                h[i] = xh;
                l[i] = (_Float16)(x - (float)xh);
                sum += x;
            }
            const int s = 2 * b + (j >> 1), kh = j & 1;
            *(f16x8 *)(st.hi + ((s * 2 + kh) * kMfmaCols + c) * 8) = h;
            *(f16x8 *)(st.lo + ((s * 2 + kh) * kMfmaCols + c) * 8) = l;
        }
        // block sums
        const _Float16 sh = (_Float16)sum;
        st.sum[c * 8 + b] = sh;
        st.sum[(kMfmaCols + c) * 8 + b] = (_Float16)(sum - (float)sh);
        if (b == 0) st.esc[c] = ldexpf(1.0f, -e);
    }
}

// Staging of one super-block of up to 32 columns from their half-precision
// records by LDS DMA (16 bytes per lane, 34 wave instructions spread over
// the workgroup's nw waves).  rec: this lane's column's record of the
// super-block (column lane%32).  Instruction i < 32 copies chunks 2i' and
// 2i'+1 (i' = i%16) of hi (i < 16) or lo: lane l takes chunk 2i' + l/32 of
// column l%32, which lies at LDS offset 1024i' + 16l; instruction 32 the
// block sums (lane l: part l/32 of column l%32), 33 the column scales.
__device__ __forceinline__ void stage_dma(const uint8_t *rec, Stage st, int nw)
{
    typedef const __attribute__((address_space(1))) void *gsrc;
    typedef __attribute__((address_space(3))) void *ldst;
    const int wv = wave_id(), half = lane_id() >> 5;
    for (int job = wv; job < 34; job += nw) {
        if (job < 32) {
            const int part = job >> 4, i = job & 15;
            __builtin_amdgcn_global_load_lds((gsrc)(rec + part * 512 + (2 * i + half) * 16),
                                             (ldst)((part ? st.lo : st.hi) + i * 2 * kMfmaCols * 8), 16, 0, 0);
        } else if (job == 32) {
            __builtin_amdgcn_global_load_lds((gsrc)(rec + 1024 + half * 16), (ldst)st.sum, 16, 0, 0);
        } else {
            __builtin_amdgcn_global_load_lds((gsrc)(rec + 1056), (ldst)st.esc, 4, 0, 0);
        }
    }
}

// Weight operand of one 32-row block: lane l owns row r (tile row64) of the
// 64-row tile holding it; per super-block it loads the row's meta and, for
// each of the 4 qs chunks and 2 position halves, the 8 bytes of K positions
// 16*half + 8*(l/32) + [0,8) (low nibbles: sub-block 2c, high: 2c+1).
struct Q4KRow {
    uint4 meta;
    uint2 q[8];  // [chunk c][half]
};
__device__ __forceinline__ void load_q4k_row(Q4KRow &w, const uint8_t *tile, int row64, int kh)
{
    w.meta = ldg<uint4>(tile, row64 * 16);
#pragma unroll
    for (int g = 0; g < 8; g++) w.q[g] = ldg<uint2>(tile, 1024 + g * 1024 + row64 * 16 + kh * 8);
}

// 4 bytes of quants -> 4 fp16 (sc * q), q the low (HI=false) or high nibbles.
template <bool HI>
__device__ __forceinline__ void quant_f16(uint32_t w, f16x2 scv, f16x2 &o0, f16x2 &o1)
{
    const uint32_t q = HI ? (w >> 4) & 0x0F0F0F0Fu : w & 0x0F0F0F0Fu;
    // bytes q0 q1 q2 q3 -> halves 1024+q0, 1024+q1 | 1024+q2, 1024+q3
    const uint32_t a = __builtin_amdgcn_perm(0u, q, 0x0c010c00u) | 0x64006400u;
    const uint32_t b = __builtin_amdgcn_perm(0u, q, 0x0c030c02u) | 0x64006400u;
    const f16x2 k1024 = {(_Float16)1024.f, (_Float16)1024.f};
    o0 = (__builtin_bit_cast(f16x2, a) - k1024) * scv;
    o1 = (__builtin_bit_cast(f16x2, b) - k1024) * scv;
}

// One super-block of one 32-row block: acc[j] += 2^-e_t (d C1 - dmin C2).
__device__ __forceinline__ void mfma_super(const Q4KRow &w, Stage st, int lane, float (&acc)[16])
{
    const int kh = lane >> 5, col = lane & 31;
    const uint32_t W0 = w.meta.y, W1 = w.meta.z, W2 = w.meta.w;
    const uint32_t sclo = W0 & 0x3F3F3F3Fu, mlo = W1 & 0x3F3F3F3Fu;
    const uint32_t schi = (W2 & 0x0F0F0F0Fu) | ((W0 >> 2) & 0x30303030u);
    const uint32_t mhi = ((W2 >> 4) & 0x0F0F0F0Fu) | ((W1 >> 2) & 0x30303030u);
    f32x16 c1 = {};
#pragma unroll
    for (int cch = 0; cch < 4; cch++) {
#pragma unroll
        for (int nib = 0; nib < 2; nib++) {
            const int b = 2 * cch + nib;
            const uint32_t scw = b < 4 ? sclo : schi;
            const _Float16 scb = (_Float16)(float)((scw >> (8 * (b & 3))) & 0xff);
            const f16x2 scv = {scb, scb};
#pragma unroll
            for (int half = 0; half < 2; half++) {
                const uint2 qw = w.q[cch * 2 + half];
                f16x2 p0, p1, p2, p3;
                if (nib) {
                    quant_f16<true>(qw.x, scv, p0, p1);
                    quant_f16<true>(qw.y, scv, p2, p3);
                } else {
                    quant_f16<false>(qw.x, scv, p0, p1);
                    quant_f16<false>(qw.y, scv, p2, p3);
                }
                const f16x8 bw = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                const int s = 2 * b + half;
                const f16x8 ah = *(const f16x8 *)(st.hi + ((s * 2 + kh) * kMfmaCols + col) * 8);
                const f16x8 al = *(const f16x8 *)(st.lo + ((s * 2 + kh) * kMfmaCols + col) * 8);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bw, c1, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bw, c1, 0, 0, 0);
            }
        }
    }
    // min term: A'' = block sums (columns x 8 blocks; lane l holds column
    // l%32, blocks (l/32)*4 + [0,4)), B'' = m_b (blocks x rows)
    const uint32_t mw = kh ? mhi : mlo;
    const f16x4 bm = {(_Float16)(float)(mw & 0xff), (_Float16)(float)((mw >> 8) & 0xff),
                      (_Float16)(float)((mw >> 16) & 0xff), (_Float16)(float)(mw >> 24)};
    const f16x4 sh = *(const f16x4 *)(st.sum + col * 8 + kh * 4);
    const f16x4 sl = *(const f16x4 *)(st.sum + (kMfmaCols + col) * 8 + kh * 4);
    f32x16 c2 = {};
    c2 = __builtin_amdgcn_mfma_f32_32x32x8f16(sh, bm, c2, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x8f16(sl, bm, c2, 0, 0, 0);
    const float d = half_lo(w.meta.x), dmin = half_hi(w.meta.x);
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int t = 8 * (j >> 2) + 4 * kh + (j & 3);
        acc[j] += st.esc[t] * (d * c1[j] - dmin * c2[j]);
    }
}

// k_gate_up_mfma: workgroup (u, rb) = distinct expert u, rows [64rb, 64rb+64)
// of gate (waves 0, 1: 32 rows each) and up (waves 2, 3) against the
// expert's tokens (<= 32); super-blocks staged double-buffered.  Writes
// SiLU(g)*u (fp32) per pair.
struct GateUpMfmaArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const WorkEntry *wt;
    const int *nuniq;
    const int *ptok;
    const uint8_t *x16; // [T][H/256] half-precision records of the normalised states
    int H, I, kd;
    unsigned long long up_off;
    float *hf;          // [P][kd] SiLU(g)*u
    float *act_out;     // [P][kd] or null
    int nrb;            // I/64
};

constexpr int kGUMfmaThreads = 256;
constexpr int kDnMfmaThreads = 256;  // 4 waves: 128 down rows share one staging

__global__ __launch_bounds__(kGUMfmaThreads) void k_gate_up_mfma(GateUpMfmaArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float xg[2][kMfmaCols][33];
    const int nitems = uni(*a.nuniq) * a.nrb;
    const int wv = wave_id(), lane = lane_id();
    const int hr = wv & 1;  // 32-row half of the 64-row block
    const int kh = lane >> 5;
    const int S = a.H >> 8;
    // one workgroup per item (u, rb); the grid covers the largest possible
    // number of distinct experts, and workgroups past the actual ones leave
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int u = item / a.nrb, rb = item - u * a.nrb;
        const WorkEntry we = load_entry(a.wt, u);
        const int p0 = we.p0, n = we.p1 - we.p0;
        const uint8_t *base = (const uint8_t *)(we.ptr ? we.ptr : we.e < a.E ? a.eptr[we.e] : a.sptr[we.e - a.E]);
        const int row64 = hr * 32 + (lane & 31), row = rb * 64 + row64;
        const uint8_t *mat = base + (wv >= 2 ? a.up_off : 0);
        // this lane's column's records (columns past the item's repeat its
        // last token; their results are dropped)
        const uint8_t *rec =
            a.x16 + (size_t)token_of(we, a.ptok, p0 + min(lane & 31, n - 1)) * S * kX16Bytes;
        float acc[16];
#pragma unroll
        for (int j = 0; j < 16; j++) acc[j] = 0.f;
        __syncthreads();  // the previous item is done with the staging buffers and xg
        stage_dma(rec, stage_at(smem), kGUMfmaThreads / 64);
        Q4KRow w;
        load_q4k_row(w, mat + ((size_t)rb * S) * kTileBytes<MOE_Q4_K>, row64, kh);
        for (int sb = 0; sb < S; sb++) {
            __syncthreads();  // stage sb has landed; buffer (sb+1)&1 is free
            Q4KRow wn;
            if (sb + 1 < S) {  // the next super-block's records and weights, in flight during this one's MFMAs
                stage_dma(rec + (size_t)(sb + 1) * kX16Bytes, stage_at(smem + ((sb + 1) & 1) * kStageBytes),
                          kGUMfmaThreads / 64);
                load_q4k_row(wn, mat + ((size_t)rb * S + sb + 1) * kTileBytes<MOE_Q4_K>, row64, kh);
            }
            opaque(w);
            mfma_super(w, stage_at(smem + (sb & 1) * kStageBytes), lane, acc);
            if (sb + 1 < S) w = wn;
        }
        // SiLU(g) * u: the gate waves hand their values over through LDS
        if (wv < 2) {
#pragma unroll
            for (int j = 0; j < 16; j++) xg[hr][8 * (j >> 2) + 4 * kh + (j & 3)][lane & 31] = acc[j];
        }
        __syncthreads();
        if (wv >= 2) {
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const int t = 8 * (j >> 2) + 4 * kh + (j & 3);
                if (t < n) {
                    const float g = xg[hr][t][lane & 31];
                    const float hv = g / (1.0f + expf(-g)) * acc[j];
                    a.hf[(size_t)(p0 + t) * a.kd + row] = hv;
                    if (a.act_out) a.act_out[(size_t)(p0 + t) * a.kd + row] = hv;
                }
            }
        }
    }
}

// k_down_mfma: workgroup (u, rt) = distinct expert u, down rows
// [128rt, 128rt+128) (wave w: rows 32w..32w+31) against the expert's pairs'
// SiLU(g)*u, staged once for the four waves; adds each pair's weighted rows
// into y, as k_down does.
struct DownMfmaArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const int *nuniq;
    const WorkEntry *wt;
    const float *hf;   // [P][kd]
    int H, I, kd;
    unsigned long long down_off;
    int nrt;
    const int *ptok;
    const float *pw;
    float *y;
};

__global__ __launch_bounds__(kDnMfmaThreads) void k_down_mfma(DownMfmaArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int lmax[kMfmaCols];
    __shared__ int lptok[kMfmaCols];  // the expert's pairs' tokens and combine weights
    __shared__ float lpw[kMfmaCols];
    const int u = blockIdx.x / a.nrt, rt = blockIdx.x - u * a.nrt;
    const int nu = uni(*a.nuniq);
    if (u >= nu) return;
    const WorkEntry we = load_entry(a.wt, u);
    const int p0 = we.p0, n = we.p1 - we.p0;
    if ((int)threadIdx.x < n) {  // read in the epilogue, after the loop's barriers
        lptok[threadIdx.x] = a.ptok[p0 + threadIdx.x];
        lpw[threadIdx.x] = a.pw[p0 + threadIdx.x];
    }
    const uint8_t *base =
        (const uint8_t *)(we.ptr ? we.ptr : we.e < a.E ? a.eptr[we.e] : a.sptr[we.e - a.E]) + a.down_off;
    const int wv = wave_id(), lane = lane_id();
    // wave wv: rows 32wv..32wv+31 of the 128-row block rt, in 64-row tile
    // 2rt + wv/2
    const int row64 = (wv & 1) * 32 + (lane & 31), kh = lane >> 5;
    const size_t tile0 = (size_t)(2 * rt + (wv >> 1));
    const int S = a.kd >> 8;
    auto rowof = [&](int c) { return p0 + c; };
    if (threadIdx.x < kMfmaCols) lmax[threadIdx.x] = 0;
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; j++) acc[j] = 0.f;
    StageRegs<kDnMfmaThreads> sr;
    stage_load<kDnMfmaThreads>(sr, a.hf, a.kd, a.I, 0, n, rowof);
    Q4KRow w;
    load_q4k_row(w, base + (tile0 * S) * kTileBytes<MOE_Q4_K>, row64, kh);
    __syncthreads();  // lmax cleared
    stage_store<kDnMfmaThreads>(sr, stage_at(smem), lmax);
    for (int sb = 0; sb < S; sb++) {
        Q4KRow wn;
        if (sb + 1 < S) {  // the next super-block's weights and h, in flight during this one's MFMAs
            load_q4k_row(wn, base + (tile0 * S + sb + 1) * kTileBytes<MOE_Q4_K>, row64, kh);
            stage_load<kDnMfmaThreads>(sr, a.hf, a.kd, a.I, sb + 1, n, rowof);
        }
        __syncthreads();  // stage sb is complete
        opaque(w);
        mfma_super(w, stage_at(smem + (sb & 1) * kStageBytes), lane, acc);
        if (sb + 1 < S) {  // convert the next super-block into the other buffer
            stage_store<kDnMfmaThreads>(sr, stage_at(smem + ((sb + 1) & 1) * kStageBytes), lmax);
            w = wn;
        }
    }
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int t = 8 * (j >> 2) + 4 * kh + (j & 3);
        if (t < n) add_to(a.y + (size_t)lptok[t] * a.H + rt * 128 + wv * 32 + (lane & 31), lpw[t] * acc[j]);
    }
}

// ---------------------------------------------------------------------------
// Integer-MFMA path: batches of 2..8 tokens on all-Q4_K experts.
//
// A Q4_K weight is w_i = d sc_j q_i - dmin m_j (sub-block j of 32 weights,
// 6-bit sc_j and m_j, 4-bit q_i); an input activation is stored as
// x_i = b (p0_i + p1_i/254 + p2_i/254^2) with int8 pieces p and one scale b
// per 256-position super-block, plus the exact sums X_j of each 32-block.
// Over one super-block,
//     sum_i w_i x_i = d b sum_p 254^-p A_p - dmin sum_j m_j X_j,
//     A_p = sum_i (sc_j q_i) p_{p,i}   (exact integers).
// sc_j q_i (<= 945) does not fit int8, but sc_j = 8 sh_j + sl_j with
// sh_j, sl_j <= 7 gives two int8 weight operands (sh q, sl q <= 105) and
// A_p = 8 A_p^h + A_p^l: two v_mfma_i32_32x32x32_i8 per sub-block, whose 32
// K positions are exactly one sub-block.  The 32 rows of the activation
// operand are (token slot t, piece p) = (2 (c >> 3) + ((c >> 2) & 1), c & 3)
// for row c (piece 3 is zero), so each lane of the result holds, for its
// weight row, all pieces of tokens kh, kh+2, kh+4, kh+6 (kh = lane / 32).
// The min term sum_j m_j X_j = b sum_j m_j (X_j / b) is one
// v_mfma_f32_32x32x8_f16 per super-block (K = the 8 sub-blocks, X_j / b <=
// 32 * 127 split into two fp16 parts in the rows of pieces 0 and 1, m_j
// exact in fp16), so that large activations cannot overflow fp16.  Per super-block and lane: 5 weight
// loads, 8 activation loads, 16 integer MFMAs, one fp16 MFMA and about 200
// VALU operations (the nibble masks, 2 packed 16-bit multiplies per 4
// weights, the epilogue) -- against the dot-product kernels' 3 v_dot4 per
// weight per 4 tokens.
//
// MFMA lane layouts (for both operands, lane l: operand row/column l % 32,
// the K half l / 32 holding K positions 16 (l/32) + [0, 16) for the i8 form
// and 4 (l/32) + [0, 4) for the fp16 K=8 form); result element e of lane l:
// row 8 (e >> 2) + 4 (l >> 5) + (e & 3) of the activation operand, column
// l % 32 (the weight row).

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kI8Tok = 8;      // tokens (pairs) per work entry
constexpr int kI8DnKG = 3;     // down K-groups
constexpr int kI8DnRW = 2;     // down 32-row blocks per workgroup
constexpr float kInv254 = 1.0f / 254.0f, kInv254sq = 1.0f / 64516.0f;

// sc and m of the 8 sub-blocks of one Q4_K row (meta = d|dmin, 12 scale bytes)
struct Q4KMeta {
    float d, dmin;
    uint32_t sc03, sc47, m03, m47;  // byte j: sub-block j (and 4 + j)
};
__device__ __forceinline__ Q4KMeta q4k_meta(const uint4 &meta)
{
    Q4KMeta r;
    r.d = half_lo(meta.x);
    r.dmin = half_hi(meta.x);
    const uint32_t W0 = meta.y, W1 = meta.z, W2 = meta.w;
    r.sc03 = W0 & 0x3F3F3F3Fu;
    r.m03 = W1 & 0x3F3F3F3Fu;
    r.sc47 = (W2 & 0x0F0F0F0Fu) | ((W0 >> 2) & 0x30303030u);
    r.m47 = ((W2 >> 4) & 0x0F0F0F0Fu) | ((W1 >> 2) & 0x30303030u);
    return r;
}

// (v, v) in the two 16-bit halves, v = byte b of w
template <int B> __device__ __forceinline__ uint32_t bcast16(uint32_t w)
{
    return __builtin_amdgcn_perm(0u, w, (0x0c0c0c0cu & ~0x00ff00ffu) | ((uint32_t)B << 16) | (uint32_t)B);
}

// 16 nibbles (one u32 per 4 K positions, in K order) times an int8 scale
// (s, s) in both 16-bit halves: q * s <= 105 stays in its byte.
__device__ __forceinline__ i32x4 qscale(const uint32_t (&q)[4], uint32_t ss)
{
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    i32x4 r;
#pragma unroll
    for (int i = 0; i < 4; i++)
        r[i] = (int)__builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, q[i]) * __builtin_bit_cast(s16x2, ss));
    return r;
}

// The activation operand's source for one lane: token slot t and piece p of
// operand row lane % 32; invalid rows read a zero block (stride 0).
struct I8Src {
    const uint8_t *rec;  // the token's record (or the zero block)
    int pstride;         // piece offset (K of the record) or 0
    int valid;           // 1 if this row is (token < n, piece < 3)
    int pcol;            // piece of this row (0..3)
};

// One super-block of one 32-row block: y[jj] += b_t (d sum_p 254^-p A_p -
// dmin M_t) for token slots t = 2 jj + kh.  `aop(s)` returns the activation
// operand of K-step s (sub-block s of the super-block), `sums()` this lane's
// 4 block sums (sub-blocks 4 kh + [0, 4)) of its row's token divided by that
// token's super-block scale b, `scale(jj)` the scale b of token slot 2 jj + kh.
template <class AOp, class Sums, class Scale>
__device__ __forceinline__ void i8_super(const uint4 &meta, const uint4 (&qp)[4], int kh, int prow, AOp aop,
                                         Sums sums, Scale scale, float (&y)[4], int n)
{
    const Q4KMeta mt = q4k_meta(meta);
    const uint32_t sh03 = (mt.sc03 >> 3) & 0x07070707u, sl03 = mt.sc03 & 0x07070707u;
    const uint32_t sh47 = (mt.sc47 >> 3) & 0x07070707u, sl47 = mt.sc47 & 0x07070707u;
    i32x16 ah = {}, al = {};
#pragma unroll
    for (int c = 0; c < 4; c++) {
        // plane 2c + kh: bytes 16 kh + [0, 16) of quant chunk c; low nibbles
        // are sub-block 2c, high nibbles sub-block 2c + 1
        const uint32_t w[4] = {qp[c].x, qp[c].y, qp[c].z, qp[c].w};
#pragma unroll
        for (int nib = 0; nib < 2; nib++) {
            const int sbk = 2 * c + nib;
            uint32_t q[4];
#pragma unroll
            for (int i = 0; i < 4; i++) q[i] = (nib ? w[i] >> 4 : w[i]) & 0x0F0F0F0Fu;
            uint32_t hs, ls;
            switch (sbk) {  // compile-time after unrolling
            case 0: hs = bcast16<0>(sh03); ls = bcast16<0>(sl03); break;
            case 1: hs = bcast16<1>(sh03); ls = bcast16<1>(sl03); break;
            case 2: hs = bcast16<2>(sh03); ls = bcast16<2>(sl03); break;
            case 3: hs = bcast16<3>(sh03); ls = bcast16<3>(sl03); break;
            case 4: hs = bcast16<0>(sh47); ls = bcast16<0>(sl47); break;
            case 5: hs = bcast16<1>(sh47); ls = bcast16<1>(sl47); break;
            case 6: hs = bcast16<2>(sh47); ls = bcast16<2>(sl47); break;
            default: hs = bcast16<3>(sh47); ls = bcast16<3>(sl47); break;
            }
            const i32x4 a = aop(sbk);
            ah = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qscale(q, hs), ah, 0, 0, 0);
            al = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qscale(q, ls), al, 0, 0, 0);
        }
    }
    // min term: rows of piece 0 / 1 carry the high / low fp16 part of X_j
    const float4 xs = sums();
    f16x4 am;
    {
        const float v[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const _Float16 h = (_Float16)v[i];
            am[i] = prow == 0 ? h : prow == 1 ? (_Float16)(v[i] - (float)h) : (_Float16)0.f;
        }
    }
    const uint32_t mw = kh ? mt.m47 : mt.m03;
    const f16x4 bm = {(_Float16)(float)(mw & 0xff), (_Float16)(float)((mw >> 8) & 0xff),
                      (_Float16)(float)((mw >> 16) & 0xff), (_Float16)(float)(mw >> 24)};
    f32x16 cm = {};
    cm = __builtin_amdgcn_mfma_f32_32x32x8f16(am, bm, cm, 0, 0, 0);
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
        if (2 * jj + kh < n) {
            const float A0 = (float)(8 * ah[4 * jj] + al[4 * jj]);
            const float A1 = (float)(8 * ah[4 * jj + 1] + al[4 * jj + 1]);
            const float A2 = (float)(8 * ah[4 * jj + 2] + al[4 * jj + 2]);
            const float v = fmaf(A2, kInv254sq, fmaf(A1, kInv254, A0));
            y[jj] = fmaf(scale(jj), fmaf(mt.d, v, -mt.dmin * (cm[4 * jj] + cm[4 * jj + 1])), y[jj]);
        }
    }
}

// This lane's activation-operand row: token slot and piece of row lane % 32.
__device__ __forceinline__ void i8_row(int lane, int &tslot, int &piece)
{
    const int c = lane & 31;
    tslot = 2 * (c >> 3) + ((c >> 2) & 1);
    piece = c & 3;
}

// k_gate_up_i8: workgroup (u, rb) = distinct expert u, rows [64 rb, 64 rb +
// 64) of gate and up (one 64-row tile of each): wave w takes matrix w & 1,
// 32-row block (w >> 1) & 1 and the super-blocks g, g + kI8GUKG, ... (g =
// w >> 2).
// The entry's token records (pieces, scales, block sums) are first staged in
// LDS (rows of H + 16 bytes, so that the 24 operand rows of one MFMA read
// fall in different banks), while each wave's first weights are in flight;
// the next super-block's weights are loaded during the current one's MFMAs.
// The K-groups' partial sums meet in LDS (over the staged records, once every
// wave is done with them); SiLU(g)*u of each pair goes to hf (fp32).
struct GateUpI8Args {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const WorkEntry *wt;
    const int *nuniq;
    Enc x;              // [T] input records of H
    int H, I, kd;
    unsigned long long up_off;
    float *hf;          // [P][kd]
    float *act_out;     // [P][kd] or null
    int nrb;            // I / 64
    // grouping in these workgroups (idx_in non-null): the routing's ids and
    // weights, or (keys_in non-null) its top-k and softmax here too, from the
    // logit keys, with NaN weights once the status word is set
    const int *idx_in;     // [T][k]
    const float *w_in;     // [T][k]
    const uint32_t *keys_in;  // [T][E] or null
    const uint32_t *status;
    int T, k, ns, Umax;
    WorkEntry *wt_out;  // the down kernel's work table (pair indices inline), its length,
    int *nuniq_out;     // each pair's token and weight, (token, slot) -> pair
    int *ptok_out, *inv_out;
    float *pw_out;
};

constexpr int kI8GUKG = 4;  // gate/up K-groups
constexpr int kGUI8Threads = 2 * 2 * kI8GUKG * 64;
constexpr int kI8MaxH = 2048;  // LDS-staged records of up to this many positions
// dynamic LDS of k_gate_up_i8: 3 kI8Tok piece rows of H + 16 bytes, then
// scales and block sums (kI8Tok x H/32 floats each), then 16 zero bytes
__host__ __device__ constexpr size_t i8_gu_lds(int H)
{
    const size_t st = (size_t)3 * kI8Tok * (H + 16) + (size_t)2 * kI8Tok * (H / 32) * 4 + 16;
    const size_t pt = (size_t)kI8GUKG * 2 * 2 * kI8Tok * 33 * 4;  // the partial sums, after the staging
    return st > pt ? st : pt;
}

__device__ __forceinline__ void load_q4k_plane_row(uint4 &meta, uint4 (&qp)[4], const uint8_t *tile, int row64, int kh)
{
    meta = ldg<uint4>(tile, row64 * 16);
#pragma unroll
    for (int c = 0; c < 4; c++) qp[c] = ldg<uint4>(tile, 1024 + (2 * c + kh) * 1024 + row64 * 16);
}

// LDS bytes of i8_group: the grouping's arrays (i8_group_lds0, 16-byte
// aligned), then the top-k's candidate slots and the ids and weights
__host__ __device__ constexpr size_t i8_group_lds0(int E)
{
    return ((size_t)E * 4 + (size_t)E * kI8Tok + 16 + 15) / 16 * 16;
}
__host__ __device__ constexpr size_t i8_group_lds(int E)
{
    return i8_group_lds0(E) + (size_t)kI8Tok * kCandSlots * 8 + (size_t)2 * kI8Tok * kMaxK * 4;
}

// Grouping of T <= 8 tokens' routing in every workgroup of the integer-MFMA
// gate/up kernel, from the ids and weights the route launch's tail wrote (it
// skips the grouping), or from the logit keys alone (the route launch has no
// tail): then wave t < T first takes token t's top-k (topk_one, as the
// tail's waves do) and its softmax over the k selected
// logits, the same arithmetic in the same order as the tail's.  Workgroup u takes the u-th selected expert in
// ascending id (then the shared experts) with the tokens that selected it
// (ascending) and their pair indices t k + j (j the slot of the expert in
// token t's selection) for routed pairs, T k + s T + t for shared ones: the
// pairs are in (token, slot) order, which the layer calls never expose.
// Workgroup 0 also writes what the down kernel reads: each pair's token and
// combine weight, the (token, slot) -> pair map, the work table (pair
// indices inline) and its length.  Returns the entry's pair count (0: no
// entry u).  lw: LDS of i8_group_lds(E) bytes.
__device__ __forceinline__ int i8_group(const GateUpI8Args &a, int u, int &e, uint64_t &toks, uint64_t &pairs,
                                        uint32_t *lw)
{
    const int T = a.T, E = a.E, k = a.k, ns = a.ns, P = T * k, tid = (int)threadIdx.x, lane = lane_id();
    uint32_t *lmask = lw;                       // [E] tokens selecting each expert
    uint8_t *lslot = (uint8_t *)(lw + E);       // [E][kI8Tok] slot of the expert in each token
    int *lsel = (int *)(lslot + E * kI8Tok);    // [2] the u-th selected expert, selected count
    const int *ids = a.idx_in;
    const float *wts = a.w_in;
    if (a.keys_in) {
        uint64_t *cand = (uint64_t *)((uint8_t *)lw + i8_group_lds0(E));  // [kI8Tok][kCandSlots]
        int *lid = (int *)(cand + kI8Tok * kCandSlots);                     // [T][k]
        float *lwt = (float *)(lid + kI8Tok * kMaxK);                       // [T][k]
        const int w = wave_id();
        if (w < T) {
            const uint32_t *kt = a.keys_in + (size_t)w * E;
            const bool dead = *a.status != 0u;
            uint64_t *cw = cand + w * kCandSlots;
            uint64_t cs;
            if (E <= 128) {
                uint32_t key[2];
#pragma unroll
                for (int i = 0; i < 2; i++) key[i] = lane + 64 * i < E ? kt[lane + 64 * i] : 0u;
                cs = topk_one<2>(key, E, k, cw);
            } else {
                uint32_t key[4];
#pragma unroll
                for (int i = 0; i < 4; i++) key[i] = lane + 64 * i < E ? kt[lane + 64 * i] : 0u;
                cs = topk_one<4>(key, E, k, cw);
            }
            const bool live = lane < k;
            const float lg = live ? unord_bits((uint32_t)(cs >> 32)) : 0.f;
            const float top = __shfl(lg, 0, 64);
            const float ex = live ? expf(lg - top) : 0.f;
            const float sum = k <= 8 ? group_sum<8>(ex) : wave_sum(ex);
            if (live) {
                lid[w * k + lane] = (int)~(uint32_t)cs;
                lwt[w * k + lane] = dead ? __builtin_nanf("") : ex / sum;
            }
        }
        ids = lid;
        wts = lwt;
    }
    for (int j = tid; j < E; j += blockDim.x) lmask[j] = 0u;
    __syncthreads();
    if (tid < P) {
        const int id = ids[tid], t = tid / k;
        if ((unsigned)id < (unsigned)E) {
            atomicOr(&lmask[id], 1u << t);
            lslot[id * kI8Tok + t] = (uint8_t)(tid - t * k);
        }
    }
    __syncthreads();
    const bool w0 = blockIdx.x == 0;
    if (wave_id() == 0) {
        // the selected experts in ascending id: the u-th one (and, in
        // workgroup 0, the work table entries of all of them)
        int base = 0, found = -1;
        for (int j0 = 0; j0 < E; j0 += 64) {
            const int j = j0 + lane;
            const uint32_t mk = j < E ? lmask[j] : 0u;
            const uint64_t b = __ballot(mk != 0u);
            const int r = base + __popcll(b & ((1ull << lane) - 1ull));
            if (mk && r == u) found = j;
            if (w0 && mk) {
                WorkEntry we{};
                we.e = j; we.p0 = 0; we.p1 = __popc(mk);
                we.ptr = a.eptr[j];
                uint64_t pl = 0;
                uint32_t mm = mk;
                for (int q = 0; mm; q++) {
                    const int t = __ffs(mm) - 1;
                    mm &= mm - 1;
                    pl |= (uint64_t)(t * k + lslot[j * kI8Tok + t]) << (8 * q);
                }
                __builtin_memcpy(we.tok, &pl, sizeof(pl));
                a.wt_out[r] = we;
            }
            base += __popcll(b);
        }
        const uint64_t fb = __ballot(found >= 0);
        const int fj = __shfl(found, fb ? __ffsll((long long)fb) - 1 : 0, 64);
        if (lane == 0) {
            lsel[0] = fb ? fj : -1;
            lsel[1] = base;
        }
    }
    __syncthreads();
    const int nsel = lsel[1];
    if (w0) {
        for (int p = tid; p < P; p += blockDim.x) {
            const int t = p / k;
            a.pw_out[p] = wts[p];
            a.ptok_out[p] = t;
            a.inv_out[t * (k + ns) + (p - t * k)] = (unsigned)ids[p] < (unsigned)E ? p : -1;
        }
        for (int i = tid; i < ns * T; i += blockDim.x) {
            const int s2 = i / T, t = i - s2 * T, p = P + s2 * T + t;
            a.pw_out[p] = 1.0f;
            a.ptok_out[p] = t;
            a.inv_out[t * (k + ns) + k + s2] = p;
        }
        for (int s2 = tid; s2 < ns; s2 += blockDim.x) {
            WorkEntry we{};
            we.e = E + s2; we.p0 = 0; we.p1 = T;
            we.ptr = a.sptr[s2];
            uint64_t pl = 0;
            for (int t = 0; t < T; t++) pl |= (uint64_t)(P + s2 * T + t) << (8 * t);
            __builtin_memcpy(we.tok, &pl, sizeof(pl));
            a.wt_out[nsel + s2] = we;
        }
        for (int v = nsel + ns + tid; v < a.Umax; v += blockDim.x) a.wt_out[v] = WorkEntry{};
        if (tid == 0) *a.nuniq_out = nsel + ns;
    }
    int n = 0;
    toks = 0;
    pairs = 0;
    e = -1;
    if (u < nsel) {
        e = lsel[0];
        uint32_t mm = lmask[e];
        for (; mm; n++) {
            const int t = __ffs(mm) - 1;
            mm &= mm - 1;
            toks |= (uint64_t)t << (8 * n);
            pairs |= (uint64_t)(t * k + lslot[e * kI8Tok + t]) << (8 * n);
        }
    } else if (u < nsel + ns) {
        e = E + (u - nsel);
        for (int t = 0; t < T; t++) {
            toks |= (uint64_t)t << (8 * t);
            pairs |= (uint64_t)(P + (u - nsel) * T + t) << (8 * t);
        }
        n = T;
    }
    __syncthreads();  // lw is reused by the caller
    return n;
}

template <bool DEFER>
__global__ __launch_bounds__(kGUI8Threads) __attribute__((amdgpu_waves_per_eu(4))) void k_gate_up_i8(GateUpI8Args a)
{
    extern __shared__ __align__(16) uint8_t lx[];
    const int u = blockIdx.x / a.nrb, rb = blockIdx.x - u * a.nrb;
    uint64_t toks;   // byte t = the token of the entry's slot t (shifts: no indexed private array)
    uint64_t pairs = 0;  // routing here: byte t = the pair of slot t; else the pairs are p0 + t
    int n, p0 = 0;
    const uint8_t *base;
    if constexpr (DEFER) {
        int e;
        n = i8_group(a, u, e, toks, pairs, (uint32_t *)lx);
        if (n == 0) return;
        base = (const uint8_t *)(e < a.E ? a.eptr[e] : a.sptr[e - a.E]);
    } else {
        if (u >= uni(*a.nuniq)) return;
        const WorkEntry we = load_entry(a.wt, u);
        n = we.p1 - we.p0;
        p0 = we.p0;
        __builtin_memcpy(&toks, we.tok, sizeof(toks));
        base = (const uint8_t *)(we.ptr ? we.ptr : we.e < a.E ? a.eptr[we.e] : a.sptr[we.e - a.E]);
    }
    const int wv = wave_id(), lane = lane_id(), kh = lane >> 5, r = lane & 31;
    const int m = wv & 1, rb2 = (wv >> 1) & 1, kg = wv >> 2;
    const int H = a.H, S = H >> 8, RS = H + 16, NB = H / 32;
    const uint8_t *mat = base + (m ? a.up_off : 0);
    const int row64 = rb2 * 32 + r;
    const size_t tile0 = (size_t)rb * S;
    // this wave's first super-block's weights, in flight during the staging
    uint4 meta = make_uint4(0, 0, 0, 0), qp[4] = {};
    if (kg < S) load_q4k_plane_row(meta, qp, mat + (tile0 + kg) * kTileBytes<MOE_Q4_K>, row64, kh);
    // staging: piece rows (16-byte chunks), then scales and block sums
    float *lbs = (float *)(lx + (size_t)3 * kI8Tok * RS);
    float *lsum = lbs + kI8Tok * NB;
    uint8_t *lzero = (uint8_t *)(lsum + kI8Tok * NB);
    {
        const int cpr = H / 16;  // chunks per piece row
        const int nrow = 3 * n, nch = nrow * cpr;
        constexpr int kMaxCh = (3 * kI8Tok * kI8MaxH / 16 + kGUI8Threads - 1) / kGUI8Threads;
        u32x4 v[kMaxCh];
#pragma unroll
        for (int i = 0; i < kMaxCh; i++) {
            const int c = (int)threadIdx.x + i * kGUI8Threads;
            const int row = c / cpr, w = c - row * cpr;
            const int t = row / 3, p = row - 3 * t;
            if (c < nch) v[i] = *(const u32x4 *)(rec_at(a.x, (int)((toks >> (8 * t)) & 0xff), H) + (size_t)p * H + 16 * w);
        }
        const int nsc = n * NB;  // scales and sums: one float each
        constexpr int kMaxSc = (2 * kI8Tok * kI8MaxH / 32 + kGUI8Threads - 1) / kGUI8Threads;
        float sv[kMaxSc];
        int si[kMaxSc];
#pragma unroll
        for (int i = 0; i < kMaxSc; i++) {
            si[i] = -1;
            sv[i] = 0.f;
            const int c = (int)threadIdx.x + i * kGUI8Threads;
            if (c < 2 * nsc) {
                const int which = c >= nsc, cc = c - which * nsc, t = cc / NB, b = cc - t * NB;
                const float *src = (const float *)(rec_at(a.x, (int)((toks >> (8 * t)) & 0xff), H) + 3 * (size_t)H);
                sv[i] = src[which * NB + b];
                si[i] = which * kI8Tok * NB + t * NB + b;
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxCh; i++) {
            const int c = (int)threadIdx.x + i * kGUI8Threads;
            const int row = c / cpr, w = c - row * cpr;
            if (c < nch) *(u32x4 *)(lx + (size_t)row * RS + 16 * w) = v[i];
        }
#pragma unroll
        for (int i = 0; i < kMaxSc; i++)
            if (si[i] >= 0) lbs[si[i]] = sv[i];
        if (threadIdx.x < 4) ((uint32_t *)lzero)[threadIdx.x] = 0u;
    }
    __syncthreads();
    int tslot, piece;
    i8_row(lane, tslot, piece);
    const bool valid = tslot < n && piece < 3;
    const uint8_t *asrc = valid ? lx + (size_t)(tslot * 3 + piece) * RS + 16 * kh : lzero;
    const int astep = valid ? 32 : 0;
    const bool svalid = tslot < n && piece < 2;
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sb = kg; sb < S; sb += kI8GUKG) {
        uint4 nmeta = make_uint4(0, 0, 0, 0), nqp[4] = {};
        if (sb + kI8GUKG < S)
            load_q4k_plane_row(nmeta, nqp, mat + (tile0 + sb + kI8GUKG) * kTileBytes<MOE_Q4_K>, row64, kh);
        const uint8_t *ab = asrc + (valid ? sb * 256 : 0);
        float4 xs = make_float4(0.f, 0.f, 0.f, 0.f);
        if (svalid) {
            xs = *(const float4 *)(lsum + tslot * NB + sb * 8 + 4 * kh);
            const float b = lbs[tslot * NB + sb * 8];
            const float ib = b > 0.f ? 1.0f / b : 0.f;
            xs.x *= ib; xs.y *= ib; xs.z *= ib; xs.w *= ib;
        }
        i8_super(meta, qp, kh, piece, [&](int s) { return *(const i32x4 *)(ab + s * astep); }, [&]() { return xs; },
                 [&](int jj) {
                     const int t = 2 * jj + kh;
                     return lbs[(t < n ? t : 0) * NB + sb * 8];
                 },
                 y, n);
        meta = nmeta;
#pragma unroll
        for (int c = 0; c < 4; c++) qp[c] = nqp[c];
    }
    __syncthreads();  // every wave is done with the staged records
    float(*part)[2][2][kI8Tok][33] = (float(*)[2][2][kI8Tok][33])lx;  // [K-group][matrix][32-row block][token][row]
#pragma unroll
    for (int jj = 0; jj < 4; jj++) part[kg][m][rb2][2 * jj + kh][r] = y[jj];
    __syncthreads();
    for (int i = threadIdx.x; i < n * 64; i += blockDim.x) {
        const int t = i >> 6, rr = i & 63, b2 = rr >> 5, r5 = rr & 31;
        float g = 0.f, uu = 0.f;
#pragma unroll
        for (int q = 0; q < kI8GUKG; q++) {
            g += part[q][0][b2][t][r5];
            uu += part[q][1][b2][t][r5];
        }
        const float hv = g / (1.0f + expf(-g)) * uu;
        const int pr = DEFER ? (int)((pairs >> (8 * t)) & 0xff) : p0 + t;
        const size_t o = (size_t)pr * a.kd + rb * 64 + rr;
        a.hf[o] = hv;
        if (a.act_out) a.act_out[o] = hv;
    }
}

// k_down_i8: workgroup (u, rt) = distinct expert u, down rows [64 rt, 64 rt
// + 64) (kI8DnRW blocks of 32) x kI8DnKG K-groups.  The pairs' SiLU(g)*u
// (fp32, positions >= I zero) are first encoded in LDS with one scale per
// super-block (a wave per (pair, super-block): 4 positions per lane; piece
// rows of kd + 16 bytes, then scales and block sums); then the MFMA loop as
// in k_gate_up_i8; the K-groups' partial sums meet in LDS and each pair's
// rows, times its combine weight, are added into y.
struct DownI8Args {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const int *nuniq;
    const WorkEntry *wt;
    const float *hf;   // [P][kd]
    int H, I, kd;
    unsigned long long down_off;
    int nrt;           // H / 64
    const int *ptok;
    const float *pw;
    float *y;
    int pairlist;      // 1: the entries' tok[] hold their pair indices (routing in the gate/up kernel)
};

constexpr int kDnI8Threads = kI8DnRW * kI8DnKG * 64;
constexpr int kDnI8MaxKd = 1536;  // LDS records of up to this many positions
// one pair's LDS record: 3 piece rows of K + 16 bytes, scales and block sums
__host__ __device__ constexpr int i8_dn_rec(int K) { return 3 * (K + 16) + 2 * (K / 32) * 4; }

__global__ __launch_bounds__(kDnI8Threads) __attribute__((amdgpu_waves_per_eu(5))) void k_down_i8(DownI8Args a)
{
    extern __shared__ __align__(16) uint8_t lrec_base[];  // kI8Tok records of i8_dn_rec(kd) bytes
    __shared__ __align__(16) uint8_t lzero[16];
    __shared__ float part[kI8DnRW][kI8DnKG][kI8Tok][33];
    const int u = blockIdx.x / a.nrt, rt = blockIdx.x - u * a.nrt;
    if (u >= uni(*a.nuniq)) return;
    const WorkEntry we = load_entry(a.wt, u);
    const int p0 = we.p0, n = we.p1 - we.p0;
    uint64_t pl;
    __builtin_memcpy(&pl, we.tok, sizeof(pl));
    auto pair_of = [&](int t) { return a.pairlist ? (int)((pl >> (8 * t)) & 0xff) : p0 + t; };
    const uint8_t *base =
        (const uint8_t *)(we.ptr ? we.ptr : we.e < a.E ? a.eptr[we.e] : a.sptr[we.e - a.E]) + a.down_off;
    const int wv = wave_id(), lane = lane_id(), kh = lane >> 5, r = lane & 31;
    const int rw = wv / kI8DnKG, q = wv - rw * kI8DnKG;
    const int K = a.kd, S = K >> 8, RS = K + 16, RR = i8_dn_rec(K);
    const int row64 = rw * 32 + r;
    const size_t tile0 = (size_t)rt * S;
    // this wave's first super-block's weights, in flight during the encoding
    uint4 meta = make_uint4(0, 0, 0, 0), qp[4];
    if (q < S) {
        const uint8_t *tile = base + (tile0 + q) * kTileBytes<MOE_Q4_K>;
        meta = ldg<uint4>(tile, row64 * 16);
#pragma unroll
        for (int c = 0; c < 4; c++) qp[c] = ldg<uint4>(tile, 1024 + (2 * c + kh) * 1024 + row64 * 16);
    }
    // encode (pair, super-block) units, a wave's units loaded at once
    if (threadIdx.x < 4) ((uint32_t *)lzero)[threadIdx.x] = 0u;
    constexpr int kUnits = 4;  // units per wave per round (loaded at once)
    for (int u0 = wv; u0 < n * S; u0 += kUnits * (kDnI8Threads / 64)) {
    float4 uv[kUnits];
#pragma unroll
    for (int i = 0; i < kUnits; i++) {
        const int unit = u0 + i * (kDnI8Threads / 64);
        const int t = unit / S, pos = (unit - t * S) * 256 + 4 * lane;
        uv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (unit < n * S && pos < a.I) uv[i] = *(const float4 *)(a.hf + (size_t)pair_of(t) * K + pos);  // I: multiple of 32
    }
#pragma unroll
    for (int i = 0; i < kUnits; i++) {
        const int unit = u0 + i * (kDnI8Threads / 64);
        if (unit >= n * S) break;
        const int t = unit / S, sb = unit - t * S;
        const int pos = sb * 256 + 4 * lane;
        const float4 v = uv[i];
        const float am = group_max<64>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        const float inv = am > 0.f ? 127.0f / am : 0.f;
        uint32_t w0 = 0, w1 = 0, w2 = 0;
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float r0 = vv[i] * inv, f0 = rintf(r0);
            const float r1 = (r0 - f0) * 254.0f, f1 = rintf(r1);
            const float r2 = (r1 - f1) * 254.0f, f2 = rintf(r2);
            w0 |= ((uint32_t)(int)f0 & 0xffu) << (8 * i);
            w1 |= ((uint32_t)(int)f1 & 0xffu) << (8 * i);
            w2 |= ((uint32_t)(int)f2 & 0xffu) << (8 * i);
        }
        uint8_t *rec = lrec_base + (size_t)t * RR;
        *(uint32_t *)(rec + pos) = w0;
        *(uint32_t *)(rec + RS + pos) = w1;
        *(uint32_t *)(rec + 2 * RS + pos) = w2;
        const float bs = group_sum<8>(v.x + v.y + v.z + v.w);  // 32 positions = 8 lanes
        if ((lane & 7) == 0) ((float *)(rec + 3 * RS + K / 8))[sb * 8 + (lane >> 3)] = bs;
        if (lane < 8) ((float *)(rec + 3 * RS))[sb * 8 + lane] = am / 127.0f;
    }
    }
    __syncthreads();
    int tslot, piece;
    i8_row(lane, tslot, piece);
    const bool valid = tslot < n && piece < 3;
    const uint8_t *trec = lrec_base + (size_t)(tslot < n ? tslot : 0) * RR;
    const uint8_t *asrc = valid ? trec + (size_t)piece * RS + 16 * kh : lzero;
    const int astep = valid ? 32 : 0;
    const bool svalid = tslot < n && piece < 2;
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sb = q; sb < S; sb += kI8DnKG) {
        if (sb != q) {
            const uint8_t *tile = base + (tile0 + sb) * kTileBytes<MOE_Q4_K>;
            meta = ldg<uint4>(tile, row64 * 16);
#pragma unroll
            for (int c = 0; c < 4; c++) qp[c] = ldg<uint4>(tile, 1024 + (2 * c + kh) * 1024 + row64 * 16);
        }
        const uint8_t *ab = asrc + (valid ? sb * 256 : 0);
        float4 xs = make_float4(0.f, 0.f, 0.f, 0.f);
        if (svalid) {
            xs = *(const float4 *)(trec + 3 * RS + K / 8 + 4 * (sb * 8 + 4 * kh));
            const float b = ((const float *)(trec + 3 * RS))[sb * 8];
            const float ib = b > 0.f ? 1.0f / b : 0.f;
            xs.x *= ib; xs.y *= ib; xs.z *= ib; xs.w *= ib;
        }
        i8_super(meta, qp, kh, piece, [&](int s) { return *(const i32x4 *)(ab + s * astep); },
                 [&]() { return xs; },
                 [&](int jj) {
                     const int t = 2 * jj + kh;
                     return ((const float *)(lrec_base + (size_t)(t < n ? t : 0) * RR + 3 * RS))[sb * 8];
                 },
                 y, n);
    }
#pragma unroll
    for (int jj = 0; jj < 4; jj++) part[rw][q][2 * jj + kh][r] = y[jj];
    __syncthreads();
    for (int i = threadIdx.x; i < n * kI8DnRW * 32; i += blockDim.x) {
        const int t = i / (kI8DnRW * 32), rr = i - t * (kI8DnRW * 32);
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < kI8DnKG; k++) v += part[rr >> 5][k][t][rr & 31];
        const int pr = pair_of(t);
        add_to(a.y + (size_t)a.ptok[pr] * a.H + rt * 64 + rr, a.pw[pr] * v);
    }
}

// ---------------------------------------------------------------------------
// Slot-pool lookup on the device (the same LRU as the host lookup, T4
// MoE-cache report, sections "What the MoE cache caches" and "Size your
// experts before configuring"): the layer-step's distinct selected experts
// are looked up in ascending id; a hit refreshes its slot's recency; a miss
// takes the group's next never-used slot, else the least recently used one.
// Recency is a stamp per slot from one increasing clock, so the least
// recently used slot is the occupied slot with the smallest stamp (the tail
// of the host's recency list).  One workgroup; the group's stamps and keys
// are copied to LDS only when this step can evict.  Misses are written as
// copy jobs for k_cache_copy.

constexpr int kCacheThreads = 1024;

__global__ __launch_bounds__(kCacheThreads) void k_cache_lookup(CacheDevArgs a)
{
    __shared__ int sel[kMaxE];
    __shared__ int list[kMaxE];
    __shared__ int wh[kMaxE];
    __shared__ int s_nd, s_absent;
    __shared__ uint32_t rmin[kCacheThreads / 64];
    __shared__ int rslot[kCacheThreads / 64];
    extern __shared__ uint32_t dyn[];  // lstamp[n_slots], lkey[n_slots]
    uint32_t *lstamp = dyn;
    int *lkey = (int *)(dyn + a.n_slots);
    const int tid = (int)threadIdx.x, lane = lane_id(), E = a.E, P = a.T * a.k;
    const int64_t kbase = (int64_t)a.layer * E;
    // the layer's slot of every id and the group's counters, loaded with the
    // routing (one round trip; E <= kMaxE = kCacheThreads)
    __shared__ int lwhere[kMaxE];
    const int wpre = tid < E ? a.where[kbase + tid] : -1;
    const int nf0 = *a.next_free;
    const uint32_t clk0 = *a.clock;
    for (int e = tid; e < E; e += kCacheThreads) sel[e] = 0;
    if (tid == 0) s_absent = 0;
    if (tid < E) lwhere[tid] = wpre;
    if (a.keys || a.rp_in) {
        // a single token (E <= 128): the k largest logit keys, ties to the
        // lower id (a lane quad ranks each key, as the gate/up kernel does)
        __shared__ __align__(16) uint64_t lrk[(kCacheThreads / 128) * kRankStride];
        const int i = tid >> 2;
        uint32_t kv = 0;
        if (a.rp_in) {
            // a chained layer: the router's dots with the state are the
            // previous layer's tile partials (lane quad i sums tiles q,
            // q+4, ...), times 1/RMS of the state, plus the bias; the keys
            // are stored for the FFN launch, which ranks them as here
            __shared__ float lss[kCacheThreads / 64];
            const int q4 = tid & 3, nct = a.H >> 6, ic = min(i, kChainE - 1);
            float pv[kChainMaxH / 256];
#pragma unroll
            for (int n = 0; n < kChainMaxH / 256; n++) pv[n] = a.rp_in[min(q4 + 4 * n, nct - 1) * kChainE + ic];
            const float4 x = tid < (a.H >> 2) ? ((const float4 *)a.hs)[tid] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float bz = a.bias && i < E ? a.bias[i] : 0.f;
            float ss = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
            ss = wave_sum(ss);
            if (lane == 0) lss[tid >> 6] = ss;
            float d = 0.f;
#pragma unroll
            for (int n = 0; n < kChainMaxH / 256; n++) d += q4 + 4 * n < nct ? pv[n] : 0.f;
            d += xchg<1>(d);
            d += xchg<2>(d);
            __syncthreads();
            ss = 0.f;
#pragma unroll
            for (int w = 0; w < kCacheThreads / 64; w++) ss += lss[w];
            kv = logit_key(d * (1.0f / sqrtf(ss / (float)a.H + a.eps)) + bz);
            if (q4 == 0 && i < E) a.keys_out[i] = kv;
        } else if (i < E) {
            kv = a.keys[i];
        }
        const uint64_t key = i < E ? (uint64_t)kv << 32 | (uint32_t)~i : 0ull;
        const int r = rank_keys_128(key, E, lrk);
        if ((tid & 3) == 0 && i < E) sel[i] = r < a.k;
    } else {
        __syncthreads();
        for (int p = tid; p < P; p += kCacheThreads) {
            const int e = a.idx[p];
            if ((unsigned)e < (unsigned)E) sel[e] = 1;
        }
    }
    __syncthreads();
    // ascending list of the distinct ids: wave 0, EPL consecutive ids per lane
    if (tid < 64) {
        const int EPL = (E + 63) >> 6, e0 = lane * EPL;
        int c = 0;
        for (int j = 0; j < EPL; j++) c += (e0 + j < E) ? sel[e0 + j] : 0;
        int off = wave_incl_scan(c) - c;
        for (int j = 0; j < EPL; j++)
            if (e0 + j < E && sel[e0 + j]) list[off++] = e0 + j;
        if (lane == 63) s_nd = off;
    }
    __syncthreads();
    const int nd = s_nd;
    for (int i = tid; i < nd; i += kCacheThreads) {
        wh[i] = lwhere[list[i]];
        if (wh[i] < 0) atomicAdd(&s_absent, 1);
    }
    __syncthreads();
    int nf = nf0;
    uint32_t clk = clk0;
    // no eviction can happen unless the absent ids outnumber the free slots
    const bool evict = s_absent > a.n_slots - nf;
    if (evict)
        for (int sl = tid; sl < a.n_slots; sl += kCacheThreads) {
            lstamp[sl] = a.stamp[sl];
            lkey[sl] = a.key[sl];
        }
    __syncthreads();
    int nj = 0, nh = 0, nev = 0;
    if (!evict) {
        // no miss can evict: every decision is a hit or the next free slot,
        // so thread 0 walks the ids alone, with no barrier between them
        if (tid == 0) {
            for (int i = 0; i < nd; i++) {
                const int e = list[i];
                const int key = (int)(kbase + e);
                int s = wh[i];
                const bool hit = s >= 0;
                if (hit) nh++;
                else s = nf++;
                ++clk;
                a.stamp[s] = clk;
                uint8_t *slot = a.pool + (size_t)s * a.slot_bytes;
                a.dtab[key] = slot;
                if (!hit) {
                    a.where[key] = s;
                    a.key[s] = key;
                    a.jobs[nj++] = CacheJob{slot, (const uint8_t *)a.src[key]};
                    if (a.jwait) a.done[nj - 1] = 0u;
                }
                if (a.jwait) a.jwait[e] = hit ? 0 : nj;
                if (a.trace) {
                    const int t = a.ntrace[0] + i;
                    if (t < a.trace_cap) {
                        a.trace[4 * t] = a.layer;
                        a.trace[4 * t + 1] = e;
                        a.trace[4 * t + 2] = hit ? 1 : 0;
                        a.trace[4 * t + 3] = -1;
                    }
                }
            }
        }
    } else
    // every thread walks the ids with the same (uniform) decisions; thread 0
    // writes the state, all threads take part in the minimum search
    for (int i = 0; i < nd; i++) {
        const int e = list[i];
        const int key = (int)(kbase + e);
        int s = wh[i];
        const bool hit = s >= 0 && (!evict || lkey[s] == key);
        int victim = -1;
        if (!hit) {
            if (nf < a.n_slots) {
                s = nf++;
            } else {
                // least recently used: the smallest stamp (all slots are in use)
                uint32_t best = 0xffffffffu;
                int bs = 0x7fffffff;
                for (int sl = tid; sl < a.n_slots; sl += kCacheThreads) {
                    const uint32_t v = lstamp[sl];
                    if (v < best) { best = v; bs = sl; }
                }
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) {
                    const uint32_t ov = (uint32_t)__shfl_xor((int)best, o, 64);
                    const int os = __shfl_xor(bs, o, 64);
                    if (ov < best || (ov == best && os < bs)) { best = ov; bs = os; }
                }
                if (lane == 0) { rmin[tid >> 6] = best; rslot[tid >> 6] = bs; }
                __syncthreads();
                best = rmin[0];
                bs = rslot[0];
                for (int w = 1; w < kCacheThreads / 64; w++)
                    if (rmin[w] < best || (rmin[w] == best && rslot[w] < bs)) { best = rmin[w]; bs = rslot[w]; }
                s = bs;
                victim = lkey[s];
                nev++;
            }
        } else {
            nh++;
        }
        ++clk;
        if (tid == 0) {
            if (evict) { lstamp[s] = clk; lkey[s] = key; }
            a.stamp[s] = clk;
            uint8_t *slot = a.pool + (size_t)s * a.slot_bytes;
            a.dtab[key] = slot;
            if (!hit) {
                if (victim >= 0) {
                    a.where[victim] = -1;
                    a.dtab[victim] = nullptr;  // the evicted expert is no longer resident
                }
                a.where[key] = s;
                a.key[s] = key;
                a.jobs[nj] = CacheJob{slot, (const uint8_t *)a.src[key]};
                if (a.jwait) a.done[nj] = 0u;
            }
            if (a.jwait) a.jwait[e] = hit ? 0 : nj + 1;
            if (a.trace) {
                const int t = a.ntrace[0] + i;
                if (t < a.trace_cap) {
                    a.trace[4 * t] = a.layer;
                    a.trace[4 * t + 1] = e;
                    a.trace[4 * t + 2] = hit ? 1 : 0;
                    a.trace[4 * t + 3] = victim;
                }
            }
        }
        if (!hit) nj++;
        __syncthreads();  // the state thread 0 wrote (LDS) before the next id
    }
    if (tid == 0) {
        *a.next_free = nf;
        *a.clock = clk;
        *a.njobs = nj;
        if (a.trace) a.ntrace[0] += nd;
        unsigned long long *st = a.stats;
        st[0] += nd;                    // lookups
        st[1] += nh;                    // hits
        st[2] += nd - nh;               // misses
        st[3] += nev;                   // evictions
        st[4] += (unsigned long long)nj * a.slot_bytes;
        if (a.T <= 8) { st[5] += nd; st[6] += nh; }
        else { st[7] += nd; st[8] += nh; }
    }
}

// The misses' copies from pinned host memory (read over the bus) into their
// slots: every workgroup takes a share of each job's 16-byte words.
constexpr int kCacheCopyThreads = 256;
__global__ __launch_bounds__(kCacheCopyThreads) void k_cache_copy(const CacheJob *jobs, const int32_t *njobs,
                                                                  unsigned long long slot_bytes)
{
    const int nj = *njobs;
    const size_t n16 = slot_bytes / 16, stride = (size_t)gridDim.x * kCacheCopyThreads;
    for (int j = 0; j < nj; j++) {
        const CacheJob jb = jobs[j];
        const uint4 *src = (const uint4 *)jb.src;
        uint4 *dst = (uint4 *)jb.dst;
        size_t i = (size_t)blockIdx.x * kCacheCopyThreads + threadIdx.x;
        // four words in flight per thread
        for (; i + 3 * stride < n16; i += 4 * stride) {
            const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
            dst[i] = v0; dst[i + stride] = v1; dst[i + 2 * stride] = v2; dst[i + 3 * stride] = v3;
        }
        for (; i < n16; i += stride) dst[i] = src[i];
    }
}

// Large-batch staging (T4 MoE-cache report, "What the MoE cache caches":
// batches above 32 tokens bypass the slots, taking the experts the cache
// holds from it): the layer's distinct selected ids in ascending order, the
// u-th staged at staging + u * slot_bytes, copied from its slot when the
// group holds it (large_copies) or from its pinned host copy (large_uploads);
// the table gets the staged addresses, NULL elsewhere.  One workgroup; the
// copies are k_cache_copy's jobs.  The LRU state is only read.
__global__ __launch_bounds__(kCacheThreads) void k_cache_stage(StageDevArgs a)
{
    __shared__ int sel[kMaxE];
    __shared__ int list[kMaxE];
    __shared__ int s_nd, s_cp;
    const int tid = (int)threadIdx.x, lane = lane_id(), E = a.E, P = a.T * a.k;
    for (int e = tid; e < E; e += kCacheThreads) sel[e] = 0;
    if (tid == 0) s_cp = 0;
    __syncthreads();
    for (int p = tid; p < P; p += kCacheThreads) {
        const int e = a.idx[p];
        if ((unsigned)e < (unsigned)E) sel[e] = 1;
    }
    __syncthreads();
    if (tid < 64) {
        const int EPL = (E + 63) >> 6, e0 = lane * EPL;
        int c = 0;
        for (int j = 0; j < EPL; j++) c += (e0 + j < E) ? sel[e0 + j] : 0;
        int off = wave_incl_scan(c) - c;
        for (int j = 0; j < EPL; j++)
            if (e0 + j < E && sel[e0 + j]) list[off++] = e0 + j;
        if (lane == 63) s_nd = off;
    }
    __syncthreads();
    const int nd = s_nd;
    const int64_t kbase = (int64_t)a.layer * E;
    for (int e = tid; e < E; e += kCacheThreads)
        if (!sel[e]) a.table[e] = nullptr;
    for (int u = tid; u < nd; u += kCacheThreads) {
        const int e = list[u];
        const int s = a.where[kbase + e];
        uint8_t *dst = a.staging + (size_t)u * a.slot_bytes;
        a.table[e] = dst;
        a.jobs[u] = CacheJob{dst, s >= 0 ? a.pool + (size_t)s * a.slot_bytes : (const uint8_t *)a.src[kbase + e]};
        if (s >= 0) atomicAdd(&s_cp, 1);
    }
    __syncthreads();
    if (tid == 0) {
        *a.njobs = nd;
        a.stats[9] += s_cp;        // large_copies
        a.stats[10] += nd - s_cp;  // large_uploads
    }
}

__global__ void k_fill_zero(uint4 *p, size_t n16)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace
}  // namespace moe

// Scratch of moe_layer_forward_noalloc, for callers that cannot allocate:
// one array per GPU, held from the library's first use on that GPU until
// the process ends.  Host code never uses its name as an address; it takes
// the device address from hipGetSymbolAddress once per device.
static constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// host side

std::atomic<unsigned> g_spin{kSpinLimit};
std::atomic<int> g_withhold{0};
unsigned spin_limit() { return g_spin.load(std::memory_order_relaxed); }

#define HIP_OK(expr)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (expr);                                                          \
        if (e_ != hipSuccess) {                                                          \
            set_error("%s failed: %s", #expr, hipGetErrorString(e_));                    \
            return MOE_ERR_HIP;                                                          \
        }                                                                                \
    } while (0)

#define LAUNCH_OK(what)                                                                  \
    do {                                                                                 \
        hipError_t e_ = hipGetLastError();                                               \
        if (e_ != hipSuccess) {                                                          \
            set_error("launch of %s failed: %s", what, hipGetErrorString(e_));           \
            return MOE_ERR_HIP;                                                          \
        }                                                                                \
    } while (0)

struct Ws {
    WsLayout L;
    uint8_t *b;
    template <class T> T *at(size_t off) const { return (T *)(b + off); }
    Enc x() const { return Enc{at<uint8_t>(L.xenc)}; }
    Enc h() const { return Enc{at<uint8_t>(L.henc)}; }
    // items: the VALU FFN kernels' work items (kItemTok pairs at most),
    // else one entry per distinct expert (MFMA kernels)
    GroupOut group(bool items) const
    {
        GroupOut g{};
        g.nuniq = at<int>(L.nuniq);
        g.wt = at<WorkEntry>(L.wt);
        g.Umax = items ? L.UI : L.U;
        g.chunk = items ? kItemTok : 0;
        g.ptok = at<int>(L.ptok);
        g.inv = at<int>(L.inv);
        g.pw = at<float>(L.pw);
        return g;
    }
};

moe_status check_desc(const moe_expert_desc *d, ExpertGeom *g)
{
    if (!d) { set_error("null expert desc"); return MOE_ERR_ARG; }
    if (!qtype_ok(d->gate) || !qtype_ok(d->up) || !qtype_ok(d->down)) {
        set_error("unknown qtype (gate %d, up %d, down %d)", d->gate, d->up, d->down);
        return MOE_ERR_QTYPE;
    }
    if (d->gate != d->up) { set_error("gate and up must share one qtype"); return MOE_ERR_QTYPE; }
    if (!geom(*d, g) || enc_bytes(g->kd) > (size_t)kDnLds) {
        set_error("bad shape H=%d I=%d: H must be a multiple of 256 up to %d, I a multiple of 64 up to %d",
                  d->H, d->I, kMaxH, kDnLds / 4);
        return MOE_ERR_SHAPE;
    }
    return MOE_OK;
}

moe_status check_tke(int T, int k, int E, int ns, int tmax = kMaxT)
{
    if (T < 1 || T > tmax) { set_error("T=%d outside [1, %d]", T, tmax); return MOE_ERR_BATCH; }
    if (E < 1 || E > kMaxE) { set_error("E=%d outside [1, %d]", E, kMaxE); return MOE_ERR_ARG; }
    if (k < 1 || k > E || k > kMaxK) { set_error("k=%d outside [1, min(E=%d, %d)]", k, E, kMaxK); return MOE_ERR_ARG; }
    if (ns < 0 || ns > kMaxShared) { set_error("n_shared=%d outside [0, %d]", ns, kMaxShared); return MOE_ERR_ARG; }
    return MOE_OK;
}

moe_status check_ws(const moe_expert_desc &d, void *ws, size_t ws_bytes, int T, int k, int E, int ns, Ws *out)
{
    if (!ws) { set_error("null workspace"); return MOE_ERR_ARG; }
    out->L = ws_layout(d, T, k, E, ns);
    out->b = (uint8_t *)ws;
    if (ws_bytes < out->L.total) {
        set_error("workspace too small: %zu < %zu bytes", ws_bytes, out->L.total);
        return MOE_ERR_ARG;
    }
    return MOE_OK;
}

// The MFMA path takes batches of more than kMfmaMinT tokens whose expert
// matrices are all Q4_K (and H a multiple of 128).
constexpr int kMfmaMinT = 8;
bool use_mfma(const moe_expert_desc &d, int T)
{
    return T > kMfmaMinT && d.gate == MOE_Q4_K && d.up == MOE_Q4_K && d.down == MOE_Q4_K && d.H % 128 == 0;
}

// The integer-MFMA path takes batches of 2 .. kI8Tok tokens on all-Q4_K
// experts (one work entry per distinct expert, at most kI8Tok pairs each).
bool use_i8(const moe_expert_desc &d, int T)
{
    return T >= 2 && T <= kI8Tok && d.gate == MOE_Q4_K && d.up == MOE_Q4_K && d.down == MOE_Q4_K && d.I % 64 == 0 &&
           down_k(d) <= kDnI8MaxKd && d.H <= kI8MaxH;
}

// Work items of at most kItemTok pairs for the dot-product kernels; one
// entry per distinct expert for the MFMA kernels.
bool dot_items(const moe_expert_desc &d, int T) { return !use_mfma(d, T) && !use_i8(d, T); }

moe_status launch_ffn_i8(const moe_expert_desc &d, const ExpertGeom &g, const Ws &ws, int T, int E,
                         const void *const *eptr, const void *const *sptr, float *y, float *act_out, hipStream_t s,
                         bool defer)
{
    const WsLayout &L = ws.L;
    GateUpI8Args ga;
    ga.eptr = eptr; ga.sptr = sptr; ga.E = E;
    ga.wt = ws.at<WorkEntry>(L.wt); ga.nuniq = ws.at<int>(L.nuniq);
    ga.x = ws.x();
    ga.H = d.H; ga.I = d.I; ga.kd = g.kd; ga.up_off = g.up_off;
    ga.hf = ws.at<float>(L.hf); ga.act_out = act_out;
    ga.nrb = d.I / 64;
    ga.idx_in = defer ? ws.at<int>(L.idx) : nullptr;
    ga.w_in = ws.at<float>(L.w);
    ga.keys_in = defer && E <= kWaveTopE ? ws.at<uint32_t>(L.dlog) : nullptr;
    ga.status = ws.at<uint32_t>(L.status);
    ga.T = T; ga.k = L.k; ga.ns = L.ns; ga.Umax = L.U;
    ga.wt_out = ws.at<WorkEntry>(L.wt); ga.nuniq_out = ws.at<int>(L.nuniq);
    ga.ptok_out = ws.at<int>(L.ptok); ga.inv_out = ws.at<int>(L.inv); ga.pw_out = ws.at<float>(L.pw);
    if (defer) {
        const size_t lds = std::max(i8_gu_lds(d.H), i8_group_lds(E));
        k_gate_up_i8<true><<<L.U * ga.nrb, kGUI8Threads, lds, s>>>(ga);
    } else {
        k_gate_up_i8<false><<<L.U * ga.nrb, kGUI8Threads, i8_gu_lds(d.H), s>>>(ga);
    }
    LAUNCH_OK("k_gate_up_i8");
    DownI8Args da;
    da.eptr = eptr; da.sptr = sptr; da.E = E;
    da.nuniq = ga.nuniq; da.wt = ga.wt; da.hf = ga.hf;
    da.H = d.H; da.I = d.I; da.kd = g.kd; da.down_off = g.down_off;
    da.nrt = d.H / 64;
    da.ptok = ws.at<int>(L.ptok); da.pw = ws.at<float>(L.pw); da.y = y;
    da.pairlist = defer;
    k_down_i8<<<L.U * da.nrt, kDnI8Threads, (size_t)kI8Tok * i8_dn_rec(g.kd), s>>>(da);
    LAUNCH_OK("k_down_i8");
    return MOE_OK;
}

// The FFN launches add into y (moe_expert_ffn clears it first when not
// accumulating); the routing is the grouping in the workspace.
moe_status launch_ffn_mfma(const moe_expert_desc &d, const ExpertGeom &g, const Ws &ws, int T, int E,
                           const void *const *eptr, const void *const *sptr, float *y, float *act_out, hipStream_t s)
{
    const WsLayout &L = ws.L;
    // entries: one per distinct expert up to kMaxT tokens; chunks of
    // kMfmaCols pairs for larger batches (k_group_large)
    const int nent = T > kMaxT ? L.UI : L.U;
    const size_t lds = 2 * kStageBytes;
    static std::atomic<uint64_t> attr_set{0};  // one bit per device
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    const uint64_t bit = 1ull << (dev & 63);
    if (!(attr_set.load() & bit)) {
        HIP_OK(hipFuncSetAttribute((const void *)k_gate_up_mfma, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
        HIP_OK(hipFuncSetAttribute((const void *)k_down_mfma, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
        attr_set.fetch_or(bit);
    }
    GateUpMfmaArgs ga;
    ga.eptr = eptr; ga.sptr = sptr; ga.E = E;
    ga.wt = ws.at<WorkEntry>(L.wt); ga.ptok = ws.at<int>(L.ptok);
    ga.x16 = ws.at<uint8_t>(L.x16); ga.H = d.H; ga.I = d.I; ga.kd = g.kd; ga.up_off = g.up_off;
    ga.hf = ws.at<float>(L.hf); ga.act_out = act_out;
    ga.nrb = d.I / 64;
    ga.nuniq = ws.at<int>(L.nuniq);
    k_gate_up_mfma<<<nent * ga.nrb, kGUMfmaThreads, lds, s>>>(ga);
    LAUNCH_OK("k_gate_up_mfma");
    DownMfmaArgs da;
    da.eptr = eptr; da.sptr = sptr; da.E = E;
    da.nuniq = ws.at<int>(L.nuniq); da.wt = ga.wt; da.hf = ga.hf;
    da.H = d.H; da.I = d.I; da.kd = g.kd; da.down_off = g.down_off;
    da.nrt = d.H / 128;
    da.ptok = ws.at<int>(L.ptok); da.pw = ws.at<float>(L.pw); da.y = y;
    k_down_mfma<<<nent * da.nrt, kDnMfmaThreads, lds, s>>>(da);
    LAUNCH_OK("k_down_mfma");
    return MOE_OK;
}

// A single token's routing moves from the route launch's tail into the
// gate/up workgroups when the experts are few enough for their rank count
// (E <= 128) and the token's record fits the prefetch words.  The layer
// calls use it: moe_layer_route then only writes the logit keys (and runs
// its tail only when the caller asks for the routing), moe_layer_ffn routes.
bool defer_routing(const moe_expert_desc &d, int T, int E)
{
    return T == 1 && E <= 128 && enc_bytes(d.H) <= (size_t)kGUPre * kGUThreads * 16 && !use_mfma(d, T);
}

}  // namespace

bool route_defers(const moe_expert_desc &d, int T, int E) { return defer_routing(d, T, E); }

namespace {

// For 2 .. 8 tokens on the integer-MFMA kernels the grouping moves from the
// route launch's tail (which keeps the top-k and softmax) into the gate/up
// workgroups, when the pair indices fit a byte.
bool defer_grouping(const moe_expert_desc &d, int T, int k, int ns)
{
    return use_i8(d, T) && T * k <= kGUI8Threads && T * (k + ns) <= 256;
}

// With E <= kWaveTopE the top-k and softmax move there as well: the route
// launch leaves the logit keys and runs its tail only when the caller asks
// for the routing.
bool defer_topk(const moe_expert_desc &d, int T, int k, int ns, int E)
{
    static_assert(kI8Tok <= kDlogTok, "key region");
    return defer_grouping(d, T, k, ns) && E <= kWaveTopE;
}

// The down kernel's block for a single token, and whether the pair's record
// fits its registers (the one-pair-per-item kernel)
int down_block(const ExpertGeom &g)
{
    const int S = g.kd / 256;
    return 64 * (S < 8 ? S : 8);
}
bool down_one(const ExpertGeom &g, int T) { return T == 1 && enc_bytes(g.kd) <= (size_t)kDnPre * down_block(g) * 16; }

// workgroups of a single-token gate/up launch that copy a cached step's misses
// (16 keep the bus busy; with 64, each one's release per job cost more than
// the overlap gained)
constexpr int kFfnCopyWGs = 16;

moe_status launch_ffn_kernels(const moe_expert_desc &d, const ExpertGeom &g, const Ws &ws, int T, int E,
                              const void *const *eptr, const void *const *sptr, float *y,
                              float *act_out, hipStream_t s, bool defer = false, const Chain *ch = nullptr,
                              const CacheCopy *cc = nullptr)
{
    if (use_mfma(d, T)) return launch_ffn_mfma(d, g, ws, T, E, eptr, sptr, y, act_out, s);
    if (use_i8(d, T)) return launch_ffn_i8(d, g, ws, T, E, eptr, sptr, y, act_out, s, defer && T > 1);
    const WsLayout &L = ws.L;
    GateUpArgs ga{};
    ga.eptr = eptr; ga.sptr = sptr; ga.E = E;
    ga.wt = ws.at<WorkEntry>(L.wt); ga.ptok = ws.at<int>(L.ptok);
    ga.x = ws.x();
    ga.H = d.H; ga.I = d.I; ga.kd = g.kd; ga.up_off = g.up_off;
    ga.h = ws.h();
    ga.act_out = act_out;
    ga.ntile = d.I / 32;
    ga.tpass = (int)(kGULds / enc_bytes(d.H));
    if (ga.tpass > kTokPass) ga.tpass = kTokPass;
    ga.T = T;
    const size_t glds = (size_t)ga.tpass * enc_bytes(d.H);
    if (cc) {  // a cached single token: the first workgroups copy its misses
        ga.ncopy = kFfnCopyWGs;
        ga.jobs = cc->jobs; ga.njobs = cc->njobs; ga.jwait = cc->jwait; ga.done = cc->done;
        ga.slot_bytes = cc->slot_bytes;
        ga.status = ws.at<uint32_t>(L.status);
        ga.spin = spin_limit();
    }
    dim3 ggrid(L.UI * ga.ntile + ga.ncopy);
    // every token's record staged up front when they all fit the first pass
    const bool all = T <= 2 && T <= ga.tpass && (size_t)T * enc_bytes(d.H) <= (size_t)kGUPre * kGUThreads * 16;
    // a single token routed by the gate/up workgroups themselves (the layer's
    // route launch left its logit keys in the workspace)
    ga.dlog = defer ? ws.at<uint32_t>(L.dlog) : nullptr;
    ga.k = L.k; ga.ns = L.ns; ga.Umax = L.UI;
    ga.wt_out = ws.at<WorkEntry>(L.wt); ga.ptok_out = ws.at<int>(L.ptok); ga.inv = ws.at<int>(L.inv);
    ga.nuniq = ws.at<int>(L.nuniq); ga.pw = ws.at<float>(L.pw);
    if (ch) {
        ga.rp_in = ch->rp_in; ga.hs = y; ga.bias = ch->bias; ga.eps = ch->eps;
        ga.wn = ch->wn; ga.En = ch->En; ga.rp_out = ch->rp_out; ga.P = L.P;
        ga.dlog_keys = ch->dlog_keys ? 1 : 0;
    }
#define GATE_UP(Q)                                                                        \
    (ch && cc ? k_gate_up<Q, 1, true, true, true><<<ggrid, kGUThreads, glds, s>>>(ga)     \
     : ch ? k_gate_up<Q, 1, true, true><<<ggrid, kGUThreads, glds, s>>>(ga)              \
     : cc ? k_gate_up<Q, 1, true, false, true><<<ggrid, kGUThreads, glds, s>>>(ga)       \
     : defer ? k_gate_up<Q, 1, true><<<ggrid, kGUThreads, glds, s>>>(ga)                 \
     : all ? (T == 1 ? k_gate_up<Q, 1, false><<<ggrid, kGUThreads, glds, s>>>(ga)        \
                     : k_gate_up<Q, 2, false><<<ggrid, kGUThreads, glds, s>>>(ga))       \
           : k_gate_up<Q, kTokPass, false><<<ggrid, kGUThreads, glds, s>>>(ga))
    switch (d.gate) {
    case MOE_Q4_K: GATE_UP(MOE_Q4_K); break;
    case MOE_Q6_K: GATE_UP(MOE_Q6_K); break;
    case MOE_Q8_0: GATE_UP(MOE_Q8_0); break;
    }
#undef GATE_UP
    LAUNCH_OK("k_gate_up");

    DownArgs da{};
    da.eptr = eptr; da.sptr = sptr; da.E = E;
    da.nuniq = ws.at<int>(L.nuniq); da.wt = ga.wt;
    da.h = ga.h;
    da.H = d.H; da.kd = g.kd; da.down_off = g.down_off;
    da.nrt = d.H / 64;
    da.ptok = ws.at<int>(L.ptok); da.pw = ws.at<float>(L.pw); da.y = y;
    da.P = L.P;
    da.tpass = (int)(kDnLds / enc_bytes(g.kd));
    if (da.tpass > kItemTok) da.tpass = kItemTok;  // a work item has at most kItemTok pairs
    const size_t dlds = (size_t)da.tpass * enc_bytes(g.kd);
    dim3 dgrid(L.UI * da.nrt), dblock(down_block(g));
    // one token: item u is pair u, whose record is loaded up front when it fits
    const bool one = down_one(g, T);
    const bool dch = ch && ch->rp_out;
    if (dch) { da.wn = ch->wn; da.En = ch->En; da.rp_out = ch->rp_out; }
#define DOWN(Q)                                                                                   \
    (dch ? k_down<Q, true, true><<<dgrid, dblock, dlds, s>>>(da)                                  \
     : one ? k_down<Q, true><<<dgrid, dblock, dlds, s>>>(da) : k_down<Q, false><<<dgrid, dblock, dlds, s>>>(da))
    switch (d.down) {
    case MOE_Q4_K: DOWN(MOE_Q4_K); break;
    case MOE_Q6_K: DOWN(MOE_Q6_K); break;
    case MOE_Q8_0: DOWN(MOE_Q8_0); break;
    }
#undef DOWN
    LAUNCH_OK("k_down");
    return MOE_OK;
}

}  // namespace

moe_status launch_cache_device(const CacheDevArgs &a, hipStream_t s, hipStream_t cs, hipEvent_t fork, hipEvent_t done)
{
    const size_t lds = (size_t)a.n_slots * 8;
    static std::atomic<uint64_t> attr_set{0};  // one bit per device
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    const uint64_t bit = 1ull << (dev & 63);
    if (!(attr_set.load() & bit)) {
        HIP_OK(hipFuncSetAttribute((const void *)k_cache_lookup, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)((size_t)kCacheMaxSlots * 8)));
        attr_set.fetch_or(bit);
    }
    k_cache_lookup<<<1, kCacheThreads, lds, s>>>(a);
    LAUNCH_OK("k_cache_lookup");
    if (a.jwait) return MOE_OK;  // the FFN launch copies the misses
    if (fork) {
        HIP_OK(hipEventRecord(fork, s));
        HIP_OK(hipStreamWaitEvent(cs, fork, 0));
        s = cs;
    }
    k_cache_copy<<<128, kCacheCopyThreads, 0, s>>>(a.jobs, a.njobs, a.slot_bytes);
    LAUNCH_OK("k_cache_copy");
    if (done) HIP_OK(hipEventRecord(done, s));
    return MOE_OK;
}

moe_status launch_ffn_copy(const moe_expert_desc *d, float *h, int E, int k, const void *const *eptr,
                           const void *const *sptr, int n_shared, void *ws, size_t ws_bytes, hipStream_t s,
                           const CacheCopy *cc, const Chain *ch)
{
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(1, k, E, n_shared)) != MOE_OK) return st;
    if (!h || !eptr || (n_shared > 0 && !sptr)) { set_error("moe_cache_ffn_device: null pointer"); return MOE_ERR_ARG; }
    Ws W;
    if ((st = check_ws(*d, ws, ws_bytes, 1, k, E, n_shared, &W)) != MOE_OK) return st;
    if (!defer_routing(*d, 1, E)) {
        set_error("moe_cache_ffn_device: the single-token kernels are needed (E <= 128, H <= 4096)");
        return MOE_ERR_ARG;
    }
    return launch_ffn_kernels(*d, g, W, 1, E, eptr, sptr, h, nullptr, s, true, ch, cc);
}

moe_status launch_stage_device(const StageDevArgs &a, hipStream_t s)
{
    k_cache_stage<<<1, kCacheThreads, 0, s>>>(a);
    LAUNCH_OK("k_cache_stage");
    k_cache_copy<<<128, kCacheCopyThreads, 0, s>>>(a.jobs, a.njobs, a.slot_bytes);
    LAUNCH_OK("k_cache_copy");
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_rmsnorm(const float *h, int32_t T, int32_t H, float eps, float *xhat, hipStream_t s)
{
    if (!h || !xhat || T < 1 || H < 1) { set_error("moe_rmsnorm: bad argument"); return MOE_ERR_ARG; }
    k_rmsnorm<<<T, 256, 0, s>>>(h, H, eps, xhat);
    LAUNCH_OK("k_rmsnorm");
    return MOE_OK;
}

moe_status moe_route_topk(const float *x, int32_t T, int32_t H, const float *w_router, const float *bias, int32_t E,
                          int32_t k, int32_t *idx, float *w, float *logits, hipStream_t s)
{
    moe_status st = check_tke(T, k, E, 0, kMaxTLarge);
    if (st != MOE_OK) return st;
    if (!x || !w_router || !idx || !w) { set_error("moe_route_topk: null pointer"); return MOE_ERR_ARG; }
    if (H < 256 || H % 256 || H > kMaxH) { set_error("moe_route_topk: H=%d must be a multiple of 256 up to %d", H, kMaxH); return MOE_ERR_SHAPE; }
    k_route_token<<<T, kRouteTokThreads, 0, s>>>(x, H, w_router, bias, E, k, idx, w, logits);
    LAUNCH_OK("k_route_token");
    return MOE_OK;
}

moe_status moe_group_tokens(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *count, int32_t *offset,
                            int32_t *pairs, hipStream_t s)
{
    moe_status st = check_tke(T, k, E, 0);
    if (st != MOE_OK) return st;
    if (!idx || !count || !offset || !pairs) { set_error("moe_group_tokens: null pointer"); return MOE_ERR_ARG; }
    k_group<<<1, kRouteThreads, 0, s>>>(idx, T, k, E, count, offset, pairs);
    LAUNCH_OK("k_group");
    return MOE_OK;
}

size_t moe_workspace_bytes(const moe_expert_desc *d, int32_t T, int32_t k, int32_t E, int32_t n_shared)
{
    ExpertGeom g;
    if (!d || !geom(*d, &g) || check_tke(T, k, E, n_shared, kMaxTLarge) != MOE_OK) return 0;
    return ws_layout(*d, T, k, E, n_shared).total;
}


moe_status moe_expert_ffn(const moe_expert_desc *d, const float *x, int32_t T, int32_t k, int32_t E,
                          const int32_t *idx, const float *w, const void *const *expert_ptrs,
                          const void *const *shared_ptrs, int32_t n_shared, float *y, int32_t accumulate,
                          float *act_out, void *ws, size_t ws_bytes, hipStream_t s)
{
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(T, k, E, n_shared, kMaxTLarge)) != MOE_OK) return st;
    if (!x || !idx || !w || !expert_ptrs || !y || (n_shared > 0 && !shared_ptrs)) {
        set_error("moe_expert_ffn: null pointer");
        return MOE_ERR_ARG;
    }
    Ws W;
    if ((st = check_ws(*d, ws, ws_bytes, T, k, E, n_shared, &W)) != MOE_OK) return st;
    PrepArgs pa{};
    pa.x = x; pa.T = T; pa.H = d->H; pa.k = k; pa.E = E; pa.ns = n_shared; pa.idx = idx; pa.w = w;
    pa.yzero = accumulate ? nullptr : y;
    pa.xe = W.x(); pa.go = W.group(dot_items(*d, T)); pa.hpad = W.h(); pa.P = W.L.P; pa.I = d->I; pa.kd = g.kd;
    pa.x16 = use_mfma(*d, T) ? W.at<uint8_t>(W.L.x16) : nullptr;
    pa.sb_scale = use_i8(*d, T);
    pa.go.eptr = expert_ptrs; pa.go.sptr = shared_ptrs;
    k_prep<<<T, kRouteThreads, 0, s>>>(pa);
    LAUNCH_OK("k_prep");
    if (T > kMaxT) {
        // prompt-sized batch: work entries of at most kItemTok (dot-product
        // kernels) or kMfmaCols (MFMA) pairs, from per-expert token bitmaps
        GroupLargeArgs ga{};
        ga.idx = idx; ga.w = w; ga.T = T; ga.k = k; ga.E = E; ga.ns = n_shared;
        ga.chunk = use_mfma(*d, T) ? kMfmaCols : kItemTok;
        ga.go = pa.go;
        ga.go.Umax = W.L.UI;
        k_group_large<<<1, kGroupLargeThreads, 0, s>>>(ga);
        LAUNCH_OK("k_group_large");
    }
    return launch_ffn_kernels(*d, g, W, T, E, expert_ptrs, shared_ptrs, y, act_out, s);
}

moe_status moe_layer_route(const moe_expert_desc *d, const float *h, int32_t T, const float *w_router,
                           const float *bias, int32_t E, int32_t k, const void *const *expert_ptrs,
                           const void *const *shared_ptrs, int32_t n_shared, float eps, int32_t *idx_out,
                           float *w_out, void *ws, size_t ws_bytes, hipStream_t s)
{
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(T, k, E, n_shared)) != MOE_OK) return st;
    if (!h || !w_router) { set_error("moe_layer_route: null pointer"); return MOE_ERR_ARG; }
    if (expert_ptrs && n_shared > 0 && !shared_ptrs) { set_error("moe_layer_route: shared_ptrs missing"); return MOE_ERR_ARG; }
    Ws W;
    if ((st = check_ws(*d, ws, ws_bytes, T, k, E, n_shared, &W)) != MOE_OK) return st;
    RouteArgs a{};
    a.h = h; a.T = T; a.H = d->H; a.wr = w_router; a.bias = bias; a.E = E; a.k = k; a.eps = eps; a.normalize = 1;
    a.keys = W.at<unsigned>(W.L.keys); a.idx = W.at<int>(W.L.idx); a.w = W.at<float>(W.L.w);
    a.idx2 = idx_out; a.w2 = w_out; a.logits2 = nullptr;
    a.x = W.x();
    a.x16 = use_mfma(*d, T) ? W.at<uint8_t>(W.L.x16) : nullptr;
    a.sb_scale = use_i8(*d, T);
    // for 2 .. 8 tokens on the integer-MFMA kernels the tail stops after the
    // top-k and softmax: moe_layer_ffn's gate/up workgroups group the pairs
    a.group = !defer_grouping(*d, T, k, n_shared); a.ns = n_shared; a.go = W.group(dot_items(*d, T));
    a.go.eptr = expert_ptrs; a.go.sptr = shared_ptrs;
    a.hpad = W.h(); a.P = W.L.P; a.I = d->I; a.kd = g.kd;
    // router workgroups: row pairs x token groups of kRouteTok
    a.n_expert_blocks = (E + kRouteRows - 1) / kRouteRows * ((T + kRouteTok - 1) / kRouteTok);
    // above kTopkBlocksMinT tokens (the tail would rank them in several rounds
    // of its 8 waves), a top-k workgroup per token
    a.topk_blocks = T > kTopkBlocksMinT && E <= kWaveTopE ? T : 0;
    a.tk = W.at<unsigned long long>(W.L.tk);
    // a single token (and 2 .. 8 tokens on the integer-MFMA kernels) is
    // routed by moe_layer_ffn's gate/up workgroups from the logit keys; the
    // tail runs only when the caller wants the routing now
    const bool defer = defer_routing(*d, T, E) || defer_topk(*d, T, k, n_shared, E);
    a.dlog = defer ? W.at<uint32_t>(W.L.dlog) : nullptr;
    a.tail = !defer || idx_out || w_out;
    if (!a.tail) a.topk_blocks = 0;
    a.status = W.at<uint32_t>(W.L.status);
    a.spin = spin_limit();
    a.withhold = g_withhold.load(std::memory_order_relaxed);
    k_route<<<a.n_expert_blocks + T * ((d->H + kEncPos - 1) / kEncPos) + a.topk_blocks + (a.tail ? 1 : 0), kRouteWG, 0,
              s>>>(a);
    LAUNCH_OK("k_route");
    return MOE_OK;
}

moe_status moe_layer_ffn(const moe_expert_desc *d, float *h, int32_t T, int32_t E, int32_t k,
                         const void *const *expert_ptrs, const void *const *shared_ptrs, int32_t n_shared, void *ws,
                         size_t ws_bytes, hipStream_t s)
{
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(T, k, E, n_shared)) != MOE_OK) return st;
    if (!h || !expert_ptrs || (n_shared > 0 && !shared_ptrs)) { set_error("moe_layer_ffn: null pointer"); return MOE_ERR_ARG; }
    Ws W;
    if ((st = check_ws(*d, ws, ws_bytes, T, k, E, n_shared, &W)) != MOE_OK) return st;
    return launch_ffn_kernels(*d, g, W, T, E, expert_ptrs, shared_ptrs, h, nullptr, s,
                              defer_routing(*d, T, E) || defer_grouping(*d, T, k, n_shared));
}

moe_status moe_layer_forward(const moe_expert_desc *d, float *h, int32_t T, const float *w_router, const float *bias,
                             int32_t E, int32_t k, const void *const *expert_ptrs, const void *const *shared_ptrs,
                             int32_t n_shared, float eps, int32_t *idx_out, float *w_out, void *ws, size_t ws_bytes,
                             hipStream_t s)
{
    if (!expert_ptrs || (n_shared > 0 && !shared_ptrs)) { set_error("moe_layer_forward: null pointer"); return MOE_ERR_ARG; }
    moe_status st = moe_layer_route(d, h, T, w_router, bias, E, k, expert_ptrs, shared_ptrs, n_shared, eps, idx_out,
                                    w_out, ws, ws_bytes, s);
    if (st != MOE_OK) return st;
    return moe_layer_ffn(d, h, T, E, k, expert_ptrs, shared_ptrs, n_shared, ws, ws_bytes, s);
}

moe_status moe_layer_forward_chain(const moe_expert_desc *d, float *h, int32_t T, const float *w_router,
                                   const float *bias, int32_t E, int32_t k, const void *const *expert_ptrs,
                                   const void *const *shared_ptrs, int32_t n_shared, float eps, int32_t chain_in,
                                   const float *next_router, int32_t next_E, int32_t parity, void *ws,
                                   size_t ws_bytes, hipStream_t s)
{
    if (!chain_in && !next_router)
        return moe_layer_forward(d, h, T, w_router, bias, E, k, expert_ptrs, shared_ptrs, n_shared, eps, nullptr,
                                 nullptr, ws, ws_bytes, s);
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(T, k, E, n_shared)) != MOE_OK) return st;
    if (!h || !expert_ptrs || (n_shared > 0 && !shared_ptrs) || (!chain_in && !w_router)) {
        set_error("moe_layer_forward_chain: null pointer");
        return MOE_ERR_ARG;
    }
    if (!moe_layer_chain_supported(d, T, E)) {
        set_error("moe_layer_forward_chain: chaining takes one token, E <= %d, H <= %d and the single-token kernels "
                  "(T=%d E=%d H=%d I=%d)", kChainE, kChainMaxH, T, E, d->H, d->I);
        return MOE_ERR_ARG;
    }
    if (next_router && (next_E < 1 || next_E > kChainE)) {
        set_error("moe_layer_forward_chain: next_E=%d outside [1, %d]", next_E, kChainE);
        return MOE_ERR_ARG;
    }
    if (parity != 0 && parity != 1) {
        set_error("moe_layer_forward_chain: parity=%d (0 or 1)", parity);
        return MOE_ERR_ARG;
    }
    Ws W;
    if ((st = check_ws(*d, ws, ws_bytes, T, k, E, n_shared, &W)) != MOE_OK) return st;
    if (!chain_in) {
        st = moe_layer_route(d, h, T, w_router, bias, E, k, expert_ptrs, shared_ptrs, n_shared, eps, nullptr, nullptr,
                             ws, ws_bytes, s);
        if (st != MOE_OK) return st;
    }
    Chain c{};
    c.rp_in = chain_in ? chain_buf(ws, parity) : nullptr;
    c.rp_out = next_router ? chain_buf(ws, parity ^ 1) : nullptr;
    c.wn = next_router;
    c.En = next_E;
    c.bias = bias;
    c.eps = eps;
    return launch_ffn_kernels(*d, g, W, T, E, expert_ptrs, shared_ptrs, h, nullptr, s, true, &c);
}

int32_t moe_layer_chain_supported(const moe_expert_desc *d, int32_t T, int32_t E)
{
    ExpertGeom g;
    if (!d || !qtype_ok(d->gate) || !qtype_ok(d->up) || !qtype_ok(d->down) || !geom(*d, &g)) return 0;
    return defer_routing(*d, T, E) && down_one(g, T) && d->H <= kChainMaxH && E >= 1 && E <= kChainE;
}


}  // extern "C"

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

moe_status fill_zero(void *ws, size_t bytes, hipStream_t s)
{
    const size_t n16 = bytes / 16;
    int blocks = (int)((n16 + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    k_fill_zero<<<blocks, 256, 0, s>>>((uint4 *)ws, n16);
    LAUNCH_OK("k_fill_zero");
    return MOE_OK;
}

// The device address of this GPU's scratch array: taken once per device
// (with that device current) and kept; the first call also clears the
// whole array on s, since the routing hand-over words must start at zero
// (the kernels leave them at zero when they finish).  With setup == false
// no address is taken: *out is null if no call has taken it yet.
moe_status static_scratch(hipStream_t s, void **out, bool setup = true)
{
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d outside the %d devices the static scratch tracks", dev, kMaxDevices);
        return MOE_ERR_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev] && setup) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error("hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
            return MOE_ERR_HIP;
        }
        moe_status st = fill_zero(p, kStaticScratchBytes, s);
        if (st != MOE_OK) return st;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_expert_desc *d, float *h, int32_t T, const float *w_router,
                                     const float *bias, int32_t E, int32_t k, const void *const *expert_ptrs,
                                     const void *const *shared_ptrs, int32_t n_shared, float eps, int32_t *idx_out,
                                     float *w_out, hipStream_t s)
{
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(T, k, E, n_shared)) != MOE_OK) return st;
    if (!h || !w_router || !expert_ptrs || (n_shared > 0 && !shared_ptrs)) {
        set_error("moe_layer_forward_noalloc: null pointer");
        return MOE_ERR_ARG;
    }
    const size_t need = ws_layout(*d, T, k, E, n_shared).total;
    if (need > kStaticScratchBytes) {
        set_error("moe_layer_forward_noalloc: this layer needs %zu bytes of scratch, the static array holds %zu "
                  "(use moe_layer_forward with a workspace)", need, kStaticScratchBytes);
        return MOE_ERR_CAPACITY;
    }
    void *ws = nullptr;
    if ((st = static_scratch(s, &ws)) != MOE_OK) return st;
    return moe_layer_forward(d, h, T, w_router, bias, E, k, expert_ptrs, shared_ptrs, n_shared, eps, idx_out, w_out,
                             ws, kStaticScratchBytes, s);
}

moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t s)
{
    if (!ws) {
        // the static scratch of the current device
        void *p = nullptr;
        moe_status st = static_scratch(s, &p, false);
        if (st != MOE_OK) return st;
        if (!p) return static_scratch(s, &p);  // taken now, and cleared
        return fill_zero(p, kStaticScratchBytes, s);
    }
    if (ws_bytes & 15) { set_error("moe_workspace_init: size not a multiple of 16"); return MOE_ERR_ARG; }
    return fill_zero(ws, ws_bytes, s);
}

moe_status moe_workspace_status(const void *ws, size_t ws_bytes, uint32_t *status, hipStream_t s)
{
    if (!status) { set_error("moe_workspace_status: null status"); return MOE_ERR_ARG; }
    *status = 0;
    if (!ws) {
        void *p = nullptr;
        moe_status st = static_scratch(s, &p, false);
        if (st != MOE_OK) return st;
        if (!p) return MOE_OK;  // never used on this device
        ws = p;
        ws_bytes = kStaticScratchBytes;
    }
    if (ws_bytes < kStatus + 4) {
        set_error("moe_workspace_status: %zu bytes cannot hold the status word at offset %zu", ws_bytes, kStatus);
        return MOE_ERR_ARG;
    }
    HIP_OK(hipMemcpyAsync(status, (const uint8_t *)ws + kStatus, 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipStreamSynchronize(s));
    return MOE_OK;
}

void moe_set_spin_limit(uint32_t rounds, int32_t withhold_keys)
{
    g_spin.store(rounds ? rounds : kSpinLimit, std::memory_order_relaxed);
    g_withhold.store(withhold_keys ? 1 : 0, std::memory_order_relaxed);
}

}  // extern "C"
