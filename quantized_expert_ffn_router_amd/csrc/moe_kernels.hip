// moe_kernels.hip -- gfx950 kernels and compute entry points of libmoe.
//
// Decode path of one MoE layer (T <= 32 tokens), three launches:
//
//   k_route    router GEMV (+ RMSNorm and bias) by 8 expert rows per
//              workgroup; the last of those workgroups does softmax top-k and
//              the grouping of (token, expert) pairs into a work table;
//              T more workgroups encode each token's normalised state.
//   k_gate_up  one workgroup per (distinct expert, 32-row tile): the gate
//              and up rows of the expert against all of its tokens,
//              SiLU(g)*u, and the encoding of those 32 values.
//   k_down     one workgroup per (distinct expert, 64-row tile): down rows
//              against SiLU(g)*u; the last expert to finish a row tile adds
//              the weighted outputs of every token (and the residual).
//
// Gating follows the MoE offload blog (mhpn.cn, section 3.1: router logits,
// softmax, top-k; section 5.2: the batched form); matvecs that keep the
// weights in their quantized blocks follow the GPU-offload research notes
// (kwkr.cn, section 1.2); the gate/up/down expert tensors and the 32-token
// batch limit follow the T4 MoE-cache report (kongchang.com, section "What
// the MoE cache caches").
//
// Activation encoding.  Each block of 32 consecutive activation values v is
// stored as three int8 pieces with one fp32 scale s = max|v|/127:
//     v ~= s * (x0 + x1/254 + x2/254^2),   |xi| <= 127,
// an error below s * 7.8e-6 = max|v| * 6.1e-8, i.e. fp32 class.  Quantized
// weights are small integers times per-block scales, so the product of a
// weight block with an activation block is three exact integer dot products
// (v_dot4 on 4 int8 lanes) and a few fp32 operations per block.  This keeps
// the matvec near 1.3 VALU operations per weight, well under the ~2.7 that
// 8 TB/s of Q4_K leaves on 256 CUs, while the result stays within fp32
// rounding of the exact product.  The pieces live in global memory and every
// lane of a wavefront reads the same words (a lane owns a weight row), so
// the compiler loads them with scalar loads into SGPRs and feeds them
// straight to v_dot4.
//
// Cross-workgroup hand-off (route -> top-k, down -> combine) uses relaxed
// agent-scope atomic stores/loads for the handed-over data (coherent across
// the XCDs' L2 caches without whole-cache write-back or invalidation), a
// wait for their completion, and a relaxed arrival counter.
#include <hip/hip_runtime.h>
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
constexpr int kRouteRows = kRouteThreads / 64;  // router rows per workgroup
constexpr int kEncThreads = 256;                // positions encoded per workgroup
constexpr int kMaxK = 64;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

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

__device__ __forceinline__ uint32_t comp(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float half_lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }

__device__ __forceinline__ int dot4(uint32_t a, int b, int c) { return __builtin_amdgcn_sdot4((int)a, b, c, false); }

__device__ __forceinline__ void st_coh(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_coh(const float *p) { return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Arrival of a workgroup whose hand-over stores (st_coh) are issued: waits
// for their completion, then counts the workgroup.  Returns true in every
// thread of the last of `target` arriving workgroups, which also resets the
// counter for the next launch.
__device__ bool arrive(unsigned *cnt, unsigned target, int *flag)
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = old == target - 1;
        if (*flag) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return *flag != 0;
}

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
// Activation encoding of one 32-value block held by 32 consecutive lanes
// (lane r of the group holds position pos0 + r of a vector of K positions).
struct Enc {
    int8_t *q;     // [n][3][K]
    float *bs;     // [n][K/32]
    float *bsum;   // [n][K/32]
    int *ps;       // [n][3][K/16]
};

__device__ __forceinline__ void encode32(float v, int r, const Enc &e, int vec, int K, int pos0)
{
    const float a = group_max<32>(fabsf(v));
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
    const size_t qb = (size_t)vec * kPieces * K + pos0 + r;
    if ((r & 3) == 0) {
        *(int *)(e.q + qb) = w0;
        *(int *)(e.q + qb + K) = w1;
        *(int *)(e.q + qb + 2 * (size_t)K) = w2;
    }
    if ((r & 15) == 0) {
        const size_t pb = (size_t)vec * kPieces * (K / 16) + (pos0 + r) / 16;
        e.ps[pb] = s0;
        e.ps[pb + K / 16] = s1;
        e.ps[pb + 2 * (K / 16)] = s2;
    }
    if (r == 0) {
        e.bs[(size_t)vec * (K / 32) + pos0 / 32] = a / 127.0f;
        e.bsum[(size_t)vec * (K / 32) + pos0 / 32] = sm;
    }
}

// Zero blocks [b0, b1) of vector `vec` (padding columns of the down rows).
__device__ void zero_blocks(const Enc &e, int vec, int K, int b0, int b1, int tid, int nthr)
{
    for (int b = b0 + tid; b < b1; b += nthr) {
        for (int p = 0; p < kPieces; p++) {
            int *q = (int *)(e.q + (size_t)vec * kPieces * K + (size_t)p * K + 32 * b);
            for (int i = 0; i < 8; i++) q[i] = 0;
            e.ps[(size_t)vec * kPieces * (K / 16) + (size_t)p * (K / 16) + 2 * b] = 0;
            e.ps[(size_t)vec * kPieces * (K / 16) + (size_t)p * (K / 16) + 2 * b + 1] = 0;
        }
        e.bs[(size_t)vec * (K / 32) + b] = 0.f;
        e.bsum[(size_t)vec * (K / 32) + b] = 0.f;
    }
}

// ---------------------------------------------------------------------------
// Grouping (stable counting sort) of the T*k routed pairs plus T*ns shared
// pairs, run by one workgroup.  Routed pairs of expert e come first in
// ascending e, each expert's pairs by ascending token; shared expert s is
// pseudo-expert E+s with one pair per token.  Ids outside [0, E) are dropped.
struct WorkEntry {
    int e, p0, p1, pad;   // expert (E+s for shared s), grouped pairs [p0, p1)
    const void *ptr;      // expert's slot address, or null: read it from the pointer table
    const void *pad2;
};

struct GroupOut {
    int *nuniq;           // distinct experts (workspace)
    WorkEntry *wt;        // [Umax]; entries past nuniq are empty (p0 == p1)
    int Umax;
    int *ptok;            // [P] token of each grouped pair
    int *inv;             // [T][k+ns] grouped position of (t, j), -1 if dropped
    const void *const *eptr, *const *sptr;  // pointer tables to resolve, or null
    int *count, *offset, *pairs;  // moe_group_tokens outputs (may be null)
};

// Branch-free counting formulation over the P = T*k routed pairs q (in
// (token, slot) order; ids are distinct within a token, so that is also
// (token) order per expert):
//   count(e)  = #{q : e_q == e},   below(e) = #{q : e_q < e},
//   rank(p)   = #{q < p : e_q == e_p}       (stable position inside e_p)
//   pos(p)    = below(e_p) + rank(p)
//   u(p)      = #{q : e_q < e_p and rank(q) == 0}   (distinct-expert index)
// Shared expert s follows as pseudo-expert E+s with pair T*k + s*T + t.
__device__ void group_block(const int *sidx, int T, int k, int E, int ns, GroupOut g, int *lrank /* LDS [T*k] */)
{
    const int P = T * k;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int ep = sidx[p];
        int rank = 0;
        for (int q = 0; q < p; q++) rank += sidx[q] == ep;
        lrank[p] = (unsigned)ep < (unsigned)E ? rank : -1;
    }
    __syncthreads();
    int nu_local = 0;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int ep = sidx[p];
        const int t = p / k, j = p - t * k;
        if ((unsigned)ep >= (unsigned)E) {
            if (g.inv) g.inv[t * (k + ns) + j] = -1;
            continue;
        }
        int below = 0, cnt = 0, ubelow = 0;
        for (int q = 0; q < P; q++) {
            const int eq = sidx[q];
            const bool valid = (unsigned)eq < (unsigned)E;
            below += valid && eq < ep;
            cnt += eq == ep;
            ubelow += valid && eq < ep && lrank[q] == 0;
        }
        const int pos = below + lrank[p];
        if (g.pairs) g.pairs[pos] = p;
        if (g.ptok) {
            g.ptok[pos] = t;
            g.inv[t * (k + ns) + j] = pos;
        }
        if (lrank[p] == 0) {
            nu_local++;
            if (g.count) g.count[ep] = cnt;
            if (g.wt) {
                WorkEntry we;
                we.e = ep; we.p0 = below; we.p1 = below + cnt; we.pad = 0; we.pad2 = nullptr;
                we.ptr = g.eptr ? g.eptr[ep] : nullptr;
                g.wt[ubelow] = we;
            }
        }
    }
    // number of distinct routed experts, and the API's per-expert arrays
    __shared__ int s_nu, s_valid;
    if (threadIdx.x == 0) { s_nu = 0; s_valid = 0; }
    __syncthreads();
    if (nu_local) atomicAdd(&s_nu, nu_local);
    for (int p = threadIdx.x; p < P; p += blockDim.x)
        if (lrank[p] >= 0) atomicAdd(&s_valid, 1);
    __syncthreads();
    const int nu = s_nu, nvalid = s_valid;
    if (g.count || g.offset) {
        for (int e = threadIdx.x; e < E; e += blockDim.x) {
            int below = 0, cnt = 0;
            for (int q = 0; q < P; q++) {
                const int eq = sidx[q];
                below += (unsigned)eq < (unsigned)e;
                cnt += eq == e;
            }
            if (g.count && cnt == 0) g.count[e] = 0;
            if (g.offset) g.offset[e] = below;
        }
        if (g.offset && threadIdx.x == 0) g.offset[E] = nvalid;
    }
    if (g.wt) {
        for (int s2 = threadIdx.x; s2 < ns; s2 += blockDim.x) {
            WorkEntry we;
            we.e = E + s2; we.p0 = nvalid + s2 * T; we.p1 = nvalid + (s2 + 1) * T; we.pad = 0; we.pad2 = nullptr;
            we.ptr = g.eptr ? g.sptr[s2] : nullptr;
            g.wt[nu + s2] = we;
        }
        for (int u = nu + ns + threadIdx.x; u < g.Umax; u += blockDim.x) g.wt[u] = WorkEntry{0, 0, 0, 0, nullptr, nullptr};
        if (threadIdx.x == 0) *g.nuniq = nu + ns;
    }
    if (g.ptok) {
        for (int i = threadIdx.x; i < ns * T; i += blockDim.x) {
            const int s2 = i / T, t = i - s2 * T;
            const int pos = nvalid + s2 * T + t;
            g.ptok[pos] = t;
            g.inv[t * (k + ns) + k + s2] = pos;
        }
    }
}

// Top-k of one token by one wave.  Each candidate is a 64-bit key: the
// logit's bits mapped to an unsigned order (high word) and the inverted
// expert id (low word), so the unsigned maximum is the largest logit and,
// among equal logits, the lowest id.  Lane j receives the j-th selection.
__device__ __forceinline__ uint32_t ord_bits(float v)
{
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_bits(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
template <int S> __device__ __forceinline__ uint64_t max_step(uint64_t b)
{
    const uint32_t hi = xchg<S>((int)(uint32_t)(b >> 32));
    const uint32_t lo = xchg<S>((int)(uint32_t)b);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > b ? o : b;
}

template <int NVL>
__device__ __forceinline__ void topk_wave(const float *lg, int E, int k, float *mine, int *myid, float *top)
{
    const int lane = lane_id();
    uint64_t key[NVL];
#pragma unroll
    for (int i = 0; i < NVL; i++) {
        const int e = lane + 64 * i;
        key[i] = e < E ? ((uint64_t)ord_bits(ld_coh(lg + e)) << 32) | (uint32_t)~e : 0ull;
    }
    for (int j = 0; j < k; j++) {
        uint64_t b = key[0];
#pragma unroll
        for (int i = 1; i < NVL; i++) b = key[i] > b ? key[i] : b;
        b = max_step<1>(b); b = max_step<2>(b); b = max_step<4>(b);
        b = max_step<8>(b); b = max_step<16>(b); b = max_step<32>(b);
#pragma unroll
        for (int i = 0; i < NVL; i++) key[i] = key[i] == b ? 0ull : key[i];
        const float v = unord_bits((uint32_t)(b >> 32));
        if (j == 0) *top = v;
        if (lane == j) { *mine = v; *myid = (int)~(uint32_t)b; }
    }
}

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
    float *logits;          // [T][E] hand-over buffer
    int *idx;               // [T][k]
    float *w;               // [T][k]
    int *idx2;              // optional copies
    float *w2;
    float *logits2;
    Enc x;                  // [T] vectors of H
    int group;
    int ns;
    GroupOut go;
    Enc hpad;               // [P] vectors of kd: padding blocks zeroed here
    int P, I, kd;
    unsigned *counter;
    int n_expert_blocks;    // router workgroups; the rest encode (T * H/256)
};

// Router workgroup: 4 router rows, one per wave, against all T tokens.
// Encoding workgroup (t, c): RMS of token t, then positions [256c, 256c+256).
// The last router workgroup to finish does top-k and grouping.
__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a)
{
    __shared__ float red[8];
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ float sw[kMaxT * kMaxK];
    __shared__ int lstart[kMaxT * kMaxK];
    __shared__ int flag;

    const int H = a.H, T = a.T, E = a.E;
    const int blk = blockIdx.x;
    const int lane = lane_id();
    const int nv = H >> 8;  // float4 per lane per row
    if (blk >= a.n_expert_blocks) {
        const int g = blk - a.n_expert_blocks;
        const int t = g / nv, c = g - t * nv;
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
        for (int i = 0; i < kRouteThreads / 64; i++) ss += red[i];
        const float r = a.normalize ? 1.0f / sqrtf(ss / (float)H + a.eps) : 1.0f;
        const int pos = c * 256 + threadIdx.x;
        encode32(a.h[(size_t)t * H + pos] * r, threadIdx.x & 31, a.x, t, H, pos & ~31);
        if (a.kd > a.I) {
            const int nenc = T * nv;
            for (int p = g; p < a.P; p += nenc) zero_blocks(a.hpad, p, a.kd, a.I / 32, a.kd / 32, threadIdx.x, blockDim.x);
        }
        return;
    }

    const int e = blk * kRouteRows + wave_id();
    if (e < E) {
        const float4 *wrow = (const float4 *)(a.wr + (size_t)e * H);
        const float b = a.bias ? a.bias[e] : 0.f;
        for (int t0 = 0; t0 < T; t0 += 4) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f}, ss[4] = {0.f, 0.f, 0.f, 0.f};
            for (int i0 = 0; i0 < nv; i0 += 8) {
                // issue the router row chunk and 4 tokens' state chunks together
                float4 wv[8], hv[4][8];
#pragma unroll
                for (int i = 0; i < 8; i++)
                    if (i0 + i < nv) wv[i] = wrow[(i0 + i) * 64 + lane];
#pragma unroll
                for (int tt = 0; tt < 4; tt++)
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        if (t0 + tt < T && i0 + i < nv)
                            hv[tt][i] = ((const float4 *)(a.h + (size_t)(t0 + tt) * H))[(i0 + i) * 64 + lane];
#pragma unroll
                for (int tt = 0; tt < 4; tt++)
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        if (t0 + tt < T && i0 + i < nv) {
                            const float4 x = hv[tt][i];
                            acc[tt] += wv[i].x * x.x + wv[i].y * x.y + wv[i].z * x.z + wv[i].w * x.w;
                            ss[tt] += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
                        }
            }
#pragma unroll
            for (int tt = 0; tt < 4; tt++) {
                if (t0 + tt < T) {
                    const float d = wave_sum(acc[tt]);
                    const float q = wave_sum(ss[tt]);
                    if (lane == 0) {
                        const float rr = a.normalize ? 1.0f / sqrtf(q / (float)H + a.eps) : 1.0f;
                        const float lg = d * rr + b;
                        st_coh(a.logits + (size_t)(t0 + tt) * E + e, lg);
                        if (a.logits2) a.logits2[(size_t)(t0 + tt) * E + e] = lg;
                    }
                }
            }
        }
    }
    if (!arrive(a.counter, (unsigned)a.n_expert_blocks, &flag)) return;

    // last router workgroup: softmax top-k of every token (one wave per token)
    const int k = a.k;
    for (int t = wave_id(); t < T; t += kRouteThreads / 64) {
        float top = 0.f, mine = 0.f;
        int myid = 0;
        const float *lg = a.logits + (size_t)t * E;
        if (E <= 64) topk_wave<1>(lg, E, k, &mine, &myid, &top);
        else if (E <= 128) topk_wave<2>(lg, E, k, &mine, &myid, &top);
        else if (E <= 256) topk_wave<4>(lg, E, k, &mine, &myid, &top);
        else if (E <= 512) topk_wave<8>(lg, E, k, &mine, &myid, &top);
        else topk_wave<16>(lg, E, k, &mine, &myid, &top);
        // softmax over the k selected logits, lane j holding selection j
        const float ex = lane < k ? expf(mine - top) : 0.f;
        const float s = wave_sum(ex);
        if (lane < k) {
            const float wj = ex / s;
            sidx[t * k + lane] = myid;
            sw[t * k + lane] = wj;
            a.idx[t * k + lane] = myid;
            a.w[t * k + lane] = wj;
            if (a.idx2) a.idx2[t * k + lane] = myid;
            if (a.w2) a.w2[t * k + lane] = wj;
        }
    }
    __syncthreads();
    if (a.group) group_block(sidx, T, k, E, a.ns, a.go, lstart);
}

// ---------------------------------------------------------------------------
// k_prep: encode given token states (no normalisation), and group given
// routing (workgroup 0).
struct PrepArgs {
    const float *x;
    int T, H, k, E, ns;
    const int *idx;
    Enc xe;
    GroupOut go;
    Enc hpad;
    int P, I, kd;
};

__global__ __launch_bounds__(kRouteThreads) void k_prep(PrepArgs a)
{
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ int lstart[kMaxT * kMaxK];
    const int t = blockIdx.x;
    for (int pos = threadIdx.x; pos < a.H; pos += blockDim.x)
        encode32(a.x[(size_t)t * a.H + pos], threadIdx.x & 31, a.xe, t, a.H, pos & ~31);
    if (a.kd > a.I)
        for (int p = t; p < a.P; p += a.T) zero_blocks(a.hpad, p, a.kd, a.I / 32, a.kd / 32, threadIdx.x, blockDim.x);
    if (t != 0) return;
    for (int p = threadIdx.x; p < a.T * a.k; p += blockDim.x) sidx[p] = a.idx[p];
    __syncthreads();
    group_block(sidx, a.T, a.k, a.E, a.ns, a.go, lstart);
}

// k_group: moe_group_tokens (one workgroup).
__global__ __launch_bounds__(kRouteThreads) void k_group(const int *idx, int T, int k, int E, GroupOut go)
{
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ int lstart[kMaxT * kMaxK];
    for (int p = threadIdx.x; p < T * k; p += blockDim.x) sidx[p] = idx[p];
    __syncthreads();
    group_block(sidx, T, k, E, 0, go, lstart);
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
// Per-lane K-group dot products.  A lane owns one row of a 64-row tile and
// one 256-column K-group.  X points at the token's encoding of that K-group:
// w0..w2 its three pieces (64 int32 words each), bs / bsum its 8 block
// scales and sums, p0..p2 the per-16 sums of each piece (16 each).

struct XGroup {
    const int *__restrict__ w0, *__restrict__ w1, *__restrict__ w2;
    const float *__restrict__ bs, *__restrict__ bsum;
    const int *__restrict__ p0, *__restrict__ p1, *__restrict__ p2;
};

struct Q4KRegs { uint4 meta; uint4 q[8]; };
struct Q6KRegs { uint4 ql[8]; uint4 qh[4]; uint4 sc; uint32_t d; };
struct Q80Regs { uint4 q[16]; uint4 d; };

__device__ __forceinline__ void load_regs(Q4KRegs &r, const uint8_t *tile, int lt)
{
    r.meta = *(const uint4 *)(tile + lt * 16);
#pragma unroll
    for (int j = 0; j < 8; j++) r.q[j] = *(const uint4 *)(tile + 1024 + j * 1024 + lt * 16);
}

__device__ __forceinline__ void load_regs(Q6KRegs &r, const uint8_t *tile, int lt)
{
#pragma unroll
    for (int j = 0; j < 8; j++) r.ql[j] = *(const uint4 *)(tile + j * 1024 + lt * 16);
#pragma unroll
    for (int j = 0; j < 4; j++) r.qh[j] = *(const uint4 *)(tile + 8192 + j * 1024 + lt * 16);
    r.sc = *(const uint4 *)(tile + 12288 + lt * 16);
    r.d = *(const unsigned short *)(tile + 13312 + lt * 2);
}

__device__ __forceinline__ void load_regs(Q80Regs &r, const uint8_t *tile, int lt)
{
#pragma unroll
    for (int j = 0; j < 16; j++) r.q[j] = *(const uint4 *)(tile + j * 1024 + lt * 16);
    r.d = *(const uint4 *)(tile + 16384 + lt * 16);
}

__device__ __forceinline__ float fpieces(int a0, int a1, int a2)
{
    return (float)a0 + (float)a1 * kC1 + (float)a2 * kC2;
}

// Q4_K: sum_b bs_b*(d*sc_b*D_b) - dmin*m_b*bsum_b, D_b = piece dots of sub-block b.
__device__ __forceinline__ float kgroup_dot(const Q4KRegs &r, const XGroup &X)
{
    const uint32_t W0 = r.meta.y, W1 = r.meta.z, W2 = r.meta.w;
    const uint32_t sclo = W0 & 0x3F3F3F3Fu, mlo = W1 & 0x3F3F3F3Fu;
    const uint32_t schi = (W2 & 0x0F0F0F0Fu) | ((W0 >> 2) & 0x30303030u);
    const uint32_t mhi = ((W2 >> 4) & 0x0F0F0F0Fu) | ((W1 >> 2) & 0x30303030u);
    float acc = 0.f, accm = 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const uint32_t scw = c < 2 ? sclo : schi;
        const uint32_t mw = c < 2 ? mlo : mhi;
        const int sh0 = 8 * ((2 * c) & 3), sh1 = 8 * ((2 * c + 1) & 3);
        const int sc0 = (scw >> sh0) & 0xff, sc1 = (scw >> sh1) & 0xff;
        const int m0 = (mw >> sh0) & 0xff, m1 = (mw >> sh1) & 0xff;
        int a0 = 0, a1 = 0, a2 = 0, b0 = 0, b1 = 0, b2 = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t qd = comp(r.q[2 * c + (i >> 2)], i & 3);
            const uint32_t lo = qd & 0x0F0F0F0Fu;
            const uint32_t hi = (qd >> 4) & 0x0F0F0F0Fu;
            a0 = dot4(lo, X.w0[16 * c + i], a0);
            a1 = dot4(lo, X.w1[16 * c + i], a1);
            a2 = dot4(lo, X.w2[16 * c + i], a2);
            b0 = dot4(hi, X.w0[16 * c + 8 + i], b0);
            b1 = dot4(hi, X.w1[16 * c + 8 + i], b1);
            b2 = dot4(hi, X.w2[16 * c + 8 + i], b2);
        }
        acc += (float)sc0 * (X.bs[2 * c] * fpieces(a0, a1, a2)) + (float)sc1 * (X.bs[2 * c + 1] * fpieces(b0, b1, b2));
        accm += (float)m0 * X.bsum[2 * c] + (float)m1 * X.bsum[2 * c + 1];
    }
    return half_lo(r.meta.x) * acc - half_hi(r.meta.x) * accm;
}

// Q6_K: d * sum_b bs_b * sum_{j in b} sc_j * (Q_j - 32*S_j), Q_j, S_j piece dots / sums of sub-block j.
__device__ __forceinline__ float kgroup_dot(const Q6KRegs &r, const XGroup &X)
{
    float acc = 0.f;
#pragma unroll
    for (int n = 0; n < 2; n++) {
        int A[4][2][3];
#pragma unroll
        for (int ih = 0; ih < 2; ih++) {
            uint32_t qv[4][4];
#pragma unroll
            for (int i4 = 0; i4 < 4; i4++) {
                const int i = 4 * ih + i4;
                const uint32_t qlA = comp(r.ql[4 * n + (i >> 2)], i & 3);
                const uint32_t qlB = comp(r.ql[4 * n + 2 + (i >> 2)], i & 3);
                const uint32_t qhw = comp(r.qh[2 * n + (i >> 2)], i & 3);
                qv[0][i4] = (qlA & 0x0F0F0F0Fu) | ((qhw << 4) & 0x30303030u);
                qv[1][i4] = (qlB & 0x0F0F0F0Fu) | ((qhw << 2) & 0x30303030u);
                qv[2][i4] = ((qlA >> 4) & 0x0F0F0F0Fu) | (qhw & 0x30303030u);
                qv[3][i4] = ((qlB >> 4) & 0x0F0F0F0Fu) | ((qhw >> 2) & 0x30303030u);
            }
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const int wb = 32 * n + 8 * m + 4 * ih;
                int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
                for (int i4 = 0; i4 < 4; i4++) {
                    a0 = dot4(qv[m][i4], X.w0[wb + i4], a0);
                    a1 = dot4(qv[m][i4], X.w1[wb + i4], a1);
                    a2 = dot4(qv[m][i4], X.w2[wb + i4], a2);
                }
                A[m][ih][0] = a0; A[m][ih][1] = a1; A[m][ih][2] = a2;
            }
        }
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const int b = 4 * n + m;  // 32-position activation block = sub-blocks 2b, 2b+1
            int I0 = 0, I1 = 0, I2 = 0;
#pragma unroll
            for (int ih = 0; ih < 2; ih++) {
                const int j = 2 * b + ih;
                const int sc = (int)(int8_t)((comp(r.sc, j >> 2) >> (8 * (j & 3))) & 0xff);
                I0 += __mul24(sc, A[m][ih][0] - 32 * X.p0[j]);
                I1 += __mul24(sc, A[m][ih][1] - 32 * X.p1[j]);
                I2 += __mul24(sc, A[m][ih][2] - 32 * X.p2[j]);
            }
            acc += X.bs[b] * fpieces(I0, I1, I2);
        }
    }
    return half_lo(r.d) * acc;
}

// Q8_0: sum_b d_b * bs_b * D_b over the 8 blocks of 32.
__device__ __forceinline__ float kgroup_dot(const Q80Regs &r, const XGroup &X)
{
    float acc = 0.f;
#pragma unroll
    for (int b = 0; b < 8; b++) {
        int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int D = 8 * b + i;
            const uint32_t qd = comp(r.q[D >> 2], D & 3);
            a0 = dot4(qd, X.w0[D], a0);
            a1 = dot4(qd, X.w1[D], a1);
            a2 = dot4(qd, X.w2[D], a2);
        }
        const uint32_t dw = comp(r.d, b >> 1);
        const float db = (b & 1) ? half_hi(dw) : half_lo(dw);
        acc += db * (X.bs[b] * fpieces(a0, a1, a2));
    }
    return acc;
}

template <int QT> struct RegsOf;
template <> struct RegsOf<MOE_Q4_K> { using T = Q4KRegs; };
template <> struct RegsOf<MOE_Q6_K> { using T = Q6KRegs; };
template <> struct RegsOf<MOE_Q8_0> { using T = Q80Regs; };

template <int QT> constexpr int kTileBytes = QT == MOE_Q4_K ? 9216 : QT == MOE_Q6_K ? 13440 : 17408;

// Encoding of vector `vec` (K positions), K-group s.
__device__ __forceinline__ XGroup xgroup(const Enc &e, int vec, int K, int s)
{
    XGroup X;
    const int *q = (const int *)(e.q + (size_t)vec * kPieces * K) + s * 64;
    X.w0 = q;
    X.w1 = q + K / 4;
    X.w2 = q + K / 2;
    X.bs = e.bs + (size_t)vec * (K / 32) + s * 8;
    X.bsum = e.bsum + (size_t)vec * (K / 32) + s * 8;
    const int *ps = e.ps + (size_t)vec * kPieces * (K / 16) + s * 16;
    X.p0 = ps;
    X.p1 = ps + K / 16;
    X.p2 = ps + K / 8;
    return X;
}

// ---------------------------------------------------------------------------
// k_gate_up: workgroup (u, rt) = distinct expert u, rows [32rt, 32rt+32) of
// gate (lanes 0-31) and up (lanes 32-63); wave w takes K-groups w, w+8, ...

struct GateUpArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const WorkEntry *wt;
    const int *ptok;
    Enc x;            // token encodings, K = H
    int H, I, kd;
    unsigned long long up_off;
    Enc h;            // pair encodings, K = kd
    float *act_out;   // [P][kd] or null
    int ntile;        // I/32
};

constexpr int kGUThreads = 512;

template <int QT>
__global__ __launch_bounds__(kGUThreads) void k_gate_up(GateUpArgs a)
{
    __shared__ float part[8][kChunk][64];
    __shared__ float redv[kChunk][64];

    const int u = blockIdx.x / a.ntile;
    const int rt = blockIdx.x - u * a.ntile;
    const WorkEntry we = a.wt[u];
    const int e = we.e, p0 = we.p0, p1 = we.p1;
    if (p0 >= p1) return;
    const uint8_t *base = (const uint8_t *)(we.ptr ? we.ptr : e < a.E ? a.eptr[e] : a.sptr[e - a.E]);
    const int H = a.H, S = H >> 8;
    const int wv = wave_id(), lane = lane_id();
    const int row = rt * 32 + (lane & 31);
    const int tile64 = row >> 6, lt = row & 63;
    const uint8_t *mbase = base + ((lane >> 5) ? a.up_off : 0ull);
    const int nwv = S < 8 ? S : 8;

    for (int c0 = p0; c0 < p1; c0 += kChunk) {
        const int nt = p1 - c0 < kChunk ? p1 - c0 : kChunk;
        if (wv < nwv) {
            for (int s = wv; s < S; s += 8) {
                typename RegsOf<QT>::T r;
                load_regs(r, mbase + ((size_t)tile64 * S + s) * kTileBytes<QT>, lt);
                for (int tt = 0; tt < nt; tt++) {
                    const XGroup X = xgroup(a.x, a.ptok[c0 + tt], H, s);
                    const float v = kgroup_dot(r, X);
                    if (s == wv) part[wv][tt][lane] = v;
                    else part[wv][tt][lane] += v;
                }
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nt * 64; i += blockDim.x) {
            const int tt = i >> 6, ln = i & 63;
            float s = 0.f;
            for (int w = 0; w < nwv; w++) s += part[w][tt][ln];
            redv[tt][ln] = s;
        }
        __syncthreads();
        // SiLU(g)*u of rows [32rt, 32rt+32) and their encoding as block rt
        for (int i = threadIdx.x; i < nt * 32; i += blockDim.x) {
            const int tt = i >> 5, r = i & 31;
            const float g = redv[tt][r], up = redv[tt][32 + r];
            const float hv = g / (1.0f + expf(-g)) * up;
            encode32(hv, r, a.h, c0 + tt, a.kd, rt * 32);
            if (a.act_out) a.act_out[(size_t)(c0 + tt) * a.kd + rt * 32 + r] = hv;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// k_down: workgroup (u, rt) = distinct expert u, down rows [64rt, 64rt+64);
// wave w takes K-groups w, w+nw, ...  The last expert to finish row tile rt
// writes y for every token.

struct DownArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const int *nuniq;
    const WorkEntry *wt;
    Enc h;           // pair encodings, K = kd
    int H, kd;
    unsigned long long down_off;
    float *osc;      // [P][H] hand-over buffer
    unsigned *cnt;   // [H/64]
    int nrt;
    int T, k, ns;
    const int *inv;  // [T][k+ns]
    const float *w;  // [T][k]
    float *y;        // [T][H]
    int accumulate;
};

template <int QT>
__global__ __launch_bounds__(512) void k_down(DownArgs a)
{
    __shared__ float part[8][kChunk][64];
    __shared__ int sinv[kMaxT * (kMaxK + kMaxShared)];
    __shared__ float swt[kMaxT * kMaxK];
    __shared__ int flag;

    const int u = blockIdx.x / a.nrt;
    const int rt = blockIdx.x - u * a.nrt;
    const WorkEntry we = a.wt[u];
    const int e = we.e, p0 = we.p0, p1 = we.p1;
    if (p0 >= p1) return;
    const int nu = *a.nuniq;
    const uint8_t *base =
        (const uint8_t *)(we.ptr ? we.ptr : e < a.E ? a.eptr[e] : a.sptr[e - a.E]) + a.down_off;
    const int kd = a.kd, S = kd >> 8;
    const int nwv = (int)(blockDim.x >> 6);
    const int wv = wave_id(), lane = lane_id();

    for (int c0 = p0; c0 < p1; c0 += kChunk) {
        const int nt = p1 - c0 < kChunk ? p1 - c0 : kChunk;
        for (int s = wv; s < S; s += nwv) {
            typename RegsOf<QT>::T r;
            load_regs(r, base + ((size_t)rt * S + s) * kTileBytes<QT>, lane);
            for (int tt = 0; tt < nt; tt++) {
                const XGroup X = xgroup(a.h, c0 + tt, kd, s);
                const float v = kgroup_dot(r, X);
                if (s == wv) part[wv][tt][lane] = v;
                else part[wv][tt][lane] += v;
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nt * 64; i += blockDim.x) {
            const int tt = i >> 6, ln = i & 63;
            float s = 0.f;
            for (int w = 0; w < nwv && w < S; w++) s += part[w][tt][ln];
            st_coh(a.osc + (size_t)(c0 + tt) * a.H + rt * 64 + ln, s);
        }
        __syncthreads();
    }

    // routing of every token, staged before the arrival so that the last
    // workgroup only waits for the hand-over loads
    const int kk = a.k + a.ns;
    for (int i = threadIdx.x; i < a.T * kk; i += blockDim.x) sinv[i] = a.inv[i];
    for (int i = threadIdx.x; i < a.T * a.k; i += blockDim.x) swt[i] = a.w[i];
    if (!arrive(&a.cnt[rt], (unsigned)nu, &flag)) return;
    for (int i = threadIdx.x; i < a.T * 64; i += blockDim.x) {
        const int t = i >> 6, ln = i & 63;
        const size_t row = (size_t)rt * 64 + ln;
        float acc = a.accumulate ? a.y[(size_t)t * a.H + row] : 0.f;
        for (int j = 0; j < a.k; j++) {
            const int pj = sinv[t * kk + j];
            if (pj >= 0) acc += swt[t * a.k + j] * ld_coh(a.osc + (size_t)pj * a.H + row);
        }
        for (int s = 0; s < a.ns; s++) acc += ld_coh(a.osc + (size_t)sinv[t * kk + a.k + s] * a.H + row);
        a.y[(size_t)t * a.H + row] = acc;
    }
}

__global__ void k_fill_zero(uint4 *p, size_t n16)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// host side

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
    Enc x() const { return Enc{at<int8_t>(L.xq), at<float>(L.xbs), at<float>(L.xbsum), at<int>(L.xps)}; }
    Enc h() const { return Enc{at<int8_t>(L.hq), at<float>(L.hbs), at<float>(L.hbsum), at<int>(L.hps)}; }
    GroupOut group() const
    {
        GroupOut g{};
        g.nuniq = at<int>(L.nuniq);
        g.wt = at<WorkEntry>(L.wt);
        g.Umax = L.U;
        g.ptok = at<int>(L.ptok);
        g.inv = at<int>(L.inv);
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
    if (!geom(*d, g)) {
        set_error("bad shape H=%d I=%d: H must be a multiple of 256 and I of 64, both <= %d", d->H, d->I, kMaxH);
        return MOE_ERR_SHAPE;
    }
    return MOE_OK;
}

moe_status check_tke(int T, int k, int E, int ns)
{
    if (T < 1 || T > kMaxT) { set_error("T=%d outside [1, %d]", T, kMaxT); return MOE_ERR_BATCH; }
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

moe_status launch_ffn_kernels(const moe_expert_desc &d, const ExpertGeom &g, const Ws &ws, int T, int k, int E,
                              int ns, const void *const *eptr, const void *const *sptr, const float *wts, float *y,
                              int accumulate, float *act_out, hipStream_t s)
{
    const WsLayout &L = ws.L;
    GateUpArgs ga;
    ga.eptr = eptr; ga.sptr = sptr; ga.E = E;
    ga.wt = ws.at<WorkEntry>(L.wt); ga.ptok = ws.at<int>(L.ptok);
    ga.x = ws.x();
    ga.H = d.H; ga.I = d.I; ga.kd = g.kd; ga.up_off = g.up_off;
    ga.h = ws.h();
    ga.act_out = act_out;
    ga.ntile = d.I / 32;
    dim3 ggrid(L.U * ga.ntile);
    switch (d.gate) {
    case MOE_Q4_K: k_gate_up<MOE_Q4_K><<<ggrid, kGUThreads, 0, s>>>(ga); break;
    case MOE_Q6_K: k_gate_up<MOE_Q6_K><<<ggrid, kGUThreads, 0, s>>>(ga); break;
    case MOE_Q8_0: k_gate_up<MOE_Q8_0><<<ggrid, kGUThreads, 0, s>>>(ga); break;
    }
    LAUNCH_OK("k_gate_up");

    DownArgs da;
    da.eptr = eptr; da.sptr = sptr; da.E = E;
    da.nuniq = ws.at<int>(L.nuniq); da.wt = ga.wt;
    da.h = ga.h;
    da.H = d.H; da.kd = g.kd; da.down_off = g.down_off;
    da.osc = ws.at<float>(L.osc); da.cnt = ws.at<unsigned>(L.cnt_dn);
    da.nrt = d.H / 64;
    da.T = T; da.k = k; da.ns = ns; da.inv = ws.at<int>(L.inv); da.w = wts; da.y = y; da.accumulate = accumulate;
    const int S = g.kd / 256;
    dim3 dgrid(L.U * da.nrt), dblock(64 * (S < 8 ? S : 8));
    switch (d.down) {
    case MOE_Q4_K: k_down<MOE_Q4_K><<<dgrid, dblock, 0, s>>>(da); break;
    case MOE_Q6_K: k_down<MOE_Q6_K><<<dgrid, dblock, 0, s>>>(da); break;
    case MOE_Q8_0: k_down<MOE_Q8_0><<<dgrid, dblock, 0, s>>>(da); break;
    }
    LAUNCH_OK("k_down");
    return MOE_OK;
}

}  // namespace
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
    moe_status st = check_tke(T, k, E, 0);
    if (st != MOE_OK) return st;
    if (!x || !w_router || !idx || !w) { set_error("moe_route_topk: null pointer"); return MOE_ERR_ARG; }
    if (H < 256 || H % 256 || H > kMaxH) { set_error("moe_route_topk: H=%d must be a multiple of 256 up to %d", H, kMaxH); return MOE_ERR_SHAPE; }
    // small private scratch per thread and device: logits and the arrival counter
    static thread_local struct { void *p = nullptr; int dev = -1; } scr;
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    const size_t cap = (size_t)kMaxT * kMaxE * 4 + 256;
    if (!scr.p || scr.dev != dev) {
        scr.p = nullptr;
        HIP_OK(hipMalloc(&scr.p, cap));
        HIP_OK(hipMemset(scr.p, 0, cap));
        scr.dev = dev;
    }
    RouteArgs a{};
    a.h = x; a.T = T; a.H = H; a.wr = w_router; a.bias = bias; a.E = E; a.k = k; a.eps = 0.f; a.normalize = 0;
    a.logits = (float *)scr.p; a.idx = idx; a.w = w; a.logits2 = logits;
    a.counter = (unsigned *)((uint8_t *)scr.p + (size_t)kMaxT * kMaxE * 4);
    a.n_expert_blocks = (E + kRouteRows - 1) / kRouteRows;
    k_route<<<a.n_expert_blocks, kRouteThreads, 0, s>>>(a);
    LAUNCH_OK("k_route");
    return MOE_OK;
}

moe_status moe_group_tokens(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *count, int32_t *offset,
                            int32_t *pairs, hipStream_t s)
{
    moe_status st = check_tke(T, k, E, 0);
    if (st != MOE_OK) return st;
    if (!idx || !count || !offset || !pairs) { set_error("moe_group_tokens: null pointer"); return MOE_ERR_ARG; }
    GroupOut go{};
    go.count = count; go.offset = offset; go.pairs = pairs;
    k_group<<<1, kRouteThreads, 0, s>>>(idx, T, k, E, go);
    LAUNCH_OK("k_group");
    return MOE_OK;
}

size_t moe_workspace_bytes(const moe_expert_desc *d, int32_t T, int32_t k, int32_t E, int32_t n_shared)
{
    ExpertGeom g;
    if (!d || !geom(*d, &g) || check_tke(T, k, E, n_shared) != MOE_OK) return 0;
    return ws_layout(*d, T, k, E, n_shared).total;
}

moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t s)
{
    if (!ws || (ws_bytes & 15)) { set_error("moe_workspace_init: null or size not a multiple of 16"); return MOE_ERR_ARG; }
    const size_t n16 = ws_bytes / 16;
    int blocks = (int)((n16 + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    k_fill_zero<<<blocks, 256, 0, s>>>((uint4 *)ws, n16);
    LAUNCH_OK("k_fill_zero");
    return MOE_OK;
}

moe_status moe_expert_ffn(const moe_expert_desc *d, const float *x, int32_t T, int32_t k, int32_t E,
                          const int32_t *idx, const float *w, const void *const *expert_ptrs,
                          const void *const *shared_ptrs, int32_t n_shared, float *y, int32_t accumulate,
                          float *act_out, void *ws, size_t ws_bytes, hipStream_t s)
{
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(T, k, E, n_shared)) != MOE_OK) return st;
    if (!x || !idx || !w || !expert_ptrs || !y || (n_shared > 0 && !shared_ptrs)) {
        set_error("moe_expert_ffn: null pointer");
        return MOE_ERR_ARG;
    }
    Ws W;
    if ((st = check_ws(*d, ws, ws_bytes, T, k, E, n_shared, &W)) != MOE_OK) return st;
    PrepArgs pa{};
    pa.x = x; pa.T = T; pa.H = d->H; pa.k = k; pa.E = E; pa.ns = n_shared; pa.idx = idx;
    pa.xe = W.x(); pa.go = W.group(); pa.hpad = W.h(); pa.P = W.L.P; pa.I = d->I; pa.kd = g.kd;
    pa.go.eptr = expert_ptrs; pa.go.sptr = shared_ptrs;
    k_prep<<<T, kRouteThreads, 0, s>>>(pa);
    LAUNCH_OK("k_prep");
    return launch_ffn_kernels(*d, g, W, T, k, E, n_shared, expert_ptrs, shared_ptrs, w, y, accumulate, act_out, s);
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
    a.logits = W.at<float>(W.L.logits); a.idx = W.at<int>(W.L.idx); a.w = W.at<float>(W.L.w);
    a.idx2 = idx_out; a.w2 = w_out; a.logits2 = nullptr;
    a.x = W.x();
    a.group = 1; a.ns = n_shared; a.go = W.group();
    a.go.eptr = expert_ptrs; a.go.sptr = shared_ptrs;
    a.hpad = W.h(); a.P = W.L.P; a.I = d->I; a.kd = g.kd;
    a.counter = W.at<unsigned>(W.L.cnt_route);
    a.n_expert_blocks = (E + kRouteRows - 1) / kRouteRows;
    k_route<<<a.n_expert_blocks + T * (d->H / kEncThreads), kRouteThreads, 0, s>>>(a);
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
    return launch_ffn_kernels(*d, g, W, T, k, E, n_shared, expert_ptrs, shared_ptrs, W.at<float>(W.L.w), h, 1,
                              nullptr, s);
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

}  // extern "C"
