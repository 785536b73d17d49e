// moe_kernels.hip -- gfx950 kernels and compute entry points of libmoe.
//
// Decode path of one MoE layer (T <= 32 tokens), three launches:
//
//   k_route    router GEMV (+ optional RMSNorm and bias), then the last
//              workgroup to finish does softmax top-k and the grouping of
//              (token, expert) pairs; extra workgroups encode each token's
//              normalised state for the expert matvecs.
//   k_gate_up  one workgroup per (distinct expert, 32-row tile): gate and up
//              rows of the expert against the expert's tokens, SiLU(g)*u;
//              the last tile of an expert encodes its SiLU(g)*u vectors.
//   k_down     one workgroup per (distinct expert, 64-row tile): down rows
//              against SiLU(g)*u; the last expert to finish a row tile adds
//              the weighted outputs of every token (and the residual).
//
// Gating follows the MoE offload blog (mhpn.cn, section 3.1: router logits,
// softmax, top-k); matvecs that keep the weights in their quantized blocks
// follow the GPU-offload research notes (kwkr.cn, section 1.2); expert
// tensors gate/up/down, the slot-pool layout and the 32-token limit follow
// the T4 MoE-cache report (kongchang.com, section "What the MoE cache
// caches").
//
// Activation encoding.  A vector v is stored as three int8 pieces with one
// fp32 scale s = max|v|/127:  v ~= s*(x0 + x1/254 + x2/254^2), |xi| <= 127.
// The representation error is below max|v| * 6.2e-8, i.e. fp32 class.
// Quantized weights are integers times per-block scales, so each block's
// dot product is three exact integer dot products (v_dot4_i32_i8 on 4 int8
// lanes) and the block scales are applied once per block in fp32.  This
// keeps the matvec at about 1.2-2 VALU operations per weight, below the
// ~2.7 that 8 TB/s of Q4_K leaves on 256 CUs, while the result stays within
// fp32 rounding of the exact product.  The pieces live in global memory and
// every lane of a wavefront reads the same words, so the compiler loads them
// with scalar loads into SGPRs and feeds them straight to v_dot4.
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

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint32_t comp(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float half_lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }

__device__ __forceinline__ int dot4(uint32_t a, int b, int c) { return __builtin_amdgcn_sdot4((int)a, b, c, false); }

// Block-wide reductions through a small LDS scratch (>= 16 floats).
__device__ float block_sum(float v, float *red)
{
    v = wave_sum(v);
    int nw = blockDim.x >> 6;
    __syncthreads();
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < nw; i++) s += red[i];
    __syncthreads();
    return s;
}

__device__ float block_max(float v, float *red)
{
    v = wave_max(v);
    int nw = blockDim.x >> 6;
    __syncthreads();
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < nw; i++) s = fmaxf(s, red[i]);
    __syncthreads();
    return s;
}

// ---------------------------------------------------------------------------
// Activation encoding: v[0..n) (zeros up to K, K % 16 == 0) -> pieces
// q[3][K] (int8), scale, and per-16 sums of each piece sums[3][K/16].
// All threads of the block call it.
__device__ void encode_vector(const float *v, int n, int K, int8_t *q, float *scale, int *sums, float *red)
{
    float m = 0.f;
    for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, fabsf(v[i]));
    float amax = block_max(m, red);
    float inv = amax > 0.f ? 127.0f / amax : 0.f;
    if (threadIdx.x == 0) *scale = amax > 0.f ? amax / 127.0f : 1.0f;
    int ngroups = K >> 4;
    for (int g = threadIdx.x; g < ngroups; g += blockDim.x) {
        uint32_t w0[4], w1[4], w2[4];
        int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
        for (int i4 = 0; i4 < 4; i4++) {
            uint32_t p0 = 0, p1 = 0, p2 = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                int i = g * 16 + i4 * 4 + b;
                float x = i < n ? v[i] : 0.f;
                float r0 = x * inv;
                float x0 = rintf(r0);
                float r1 = (r0 - x0) * 254.0f;
                float x1 = rintf(r1);
                float r2 = (r1 - x1) * 254.0f;
                float x2 = rintf(r2);
                int i0 = (int)x0, i1 = (int)x1, i2 = (int)x2;
                s0 += i0; s1 += i1; s2 += i2;
                p0 |= ((uint32_t)(i0 & 0xff)) << (8 * b);
                p1 |= ((uint32_t)(i1 & 0xff)) << (8 * b);
                p2 |= ((uint32_t)(i2 & 0xff)) << (8 * b);
            }
            w0[i4] = p0; w1[i4] = p1; w2[i4] = p2;
        }
        *(uint4 *)(q + 0 * (size_t)K + g * 16) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        *(uint4 *)(q + 1 * (size_t)K + g * 16) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        *(uint4 *)(q + 2 * (size_t)K + g * 16) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
        sums[0 * ngroups + g] = s0;
        sums[1 * ngroups + g] = s1;
        sums[2 * ngroups + g] = s2;
    }
}

// ---------------------------------------------------------------------------
// Grouping (stable counting sort) of the T*k routed pairs plus T*ns shared
// pairs, run by one workgroup.  Routed pairs of expert e come first in
// ascending e, each expert's pairs by ascending token; shared expert s is
// pseudo-expert E+s with one pair per token.
struct GroupOut {
    int *nuniq, *uniq, *uoff, *ptok, *inv;  // workspace (may be null)
    float *pw;                              // workspace (may be null)
    int *count, *offset, *pairs;            // moe_group_tokens outputs (may be null)
};

__device__ void group_block(const int *sidx, const float *sw, int T, int k, int E, int ns, GroupOut g,
                            int *lstart /* LDS [E+ns+1] */)
{
    int ne = E + ns;
    for (int e = threadIdx.x; e < ne; e += blockDim.x) lstart[e] = e < E ? 0 : T;
    __syncthreads();
    for (int p = threadIdx.x; p < T * k; p += blockDim.x)
        if ((unsigned)sidx[p] < (unsigned)E) atomicAdd(&lstart[sidx[p]], 1);  // ids outside [0, E) are dropped
    __syncthreads();
    // exclusive scan of counts and compaction of non-empty experts (wave 0)
    if (threadIdx.x < 64) {
        int lane = lane_id();
        int run = 0, nu = 0;
        for (int base = 0; base < ne; base += 64) {
            int e = base + lane;
            int c = e < ne ? lstart[e] : 0;
            int x = c, f = c > 0 ? 1 : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                int y = __shfl_up(x, o, 64);
                int z = __shfl_up(f, o, 64);
                if (lane >= o) { x += y; f += z; }
            }
            int excl = run + x - c;
            int uidx = nu + f - (c > 0 ? 1 : 0);
            if (e < ne) {
                if (g.count && e < E) g.count[e] = c;
                if (g.offset && e < E) g.offset[e] = excl;
                if (c > 0 && g.uniq) { g.uniq[uidx] = e; g.uoff[uidx] = excl; }
            }
            run += __shfl(x, 63, 64);
            nu += __shfl(f, 63, 64);
            if (e < ne) lstart[e] = excl;
        }
        if (lane == 0) {
            if (g.offset) g.offset[E] = T * k;
            if (g.uniq) { g.uoff[nu] = run; *g.nuniq = nu; }
        }
    }
    __syncthreads();
    int kk = k + ns;
    for (int p = threadIdx.x; p < T * kk; p += blockDim.x) {
        int t = p / kk, j = p - t * kk;
        int pos;
        float wt;
        if (j < k) {
            int e = sidx[t * k + j];
            if ((unsigned)e >= (unsigned)E) {
                if (g.inv) g.inv[p] = -1;
                continue;
            }
            int rank = 0;
            for (int t2 = 0; t2 < t; t2++)
                for (int j2 = 0; j2 < k; j2++) rank += sidx[t2 * k + j2] == e;
            pos = lstart[e] + rank;
            wt = sw ? sw[t * k + j] : 0.f;
            if (g.pairs) g.pairs[pos] = t * k + j;
        } else {
            pos = lstart[E + (j - k)] + t;
            wt = 1.0f;
        }
        if (g.ptok) { g.ptok[pos] = t; g.pw[pos] = wt; g.inv[p] = pos; }
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
    int normalize;          // scale logits by 1/rms(h[t])
    float *logits;          // [T][E] workspace/user
    int *idx;               // [T][k]
    float *w;               // [T][k]
    int *idx2;              // optional second copy
    float *w2;
    float *logits2;
    int encode;             // encode normalised h for the matvecs
    int8_t *xq; float *xs; int *xsum;
    int group;
    int ns;
    GroupOut go;
    unsigned *counter;
    int n_expert_blocks;
};

constexpr int kRouteThreads = 256;
constexpr int kMaxK = 64;

__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a)
{
    __shared__ float red[16];
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ float sw[kMaxT * kMaxK];
    __shared__ int lstart[kMaxE + 8];
    __shared__ int is_last;
    extern __shared__ float xbuf[];  // [H] for the encoding workgroups

    const int H = a.H, T = a.T, E = a.E;
    const int blk = blockIdx.x;
    if (blk < a.n_expert_blocks) {
        const int e = blk * 4 + wave_id();
        const int lane = lane_id();
        if (e < E) {
            const float4 *wrow = (const float4 *)(a.wr + (size_t)e * H);
            const int nv = H >> 8;  // float4 per lane
            for (int t0 = 0; t0 < T; t0 += kChunk) {
                float acc[kChunk], ss[kChunk];
#pragma unroll
                for (int tt = 0; tt < kChunk; tt++) { acc[tt] = 0.f; ss[tt] = 0.f; }
                for (int i = 0; i < nv; i++) {
                    float4 wv = wrow[i * 64 + lane];
#pragma unroll
                    for (int tt = 0; tt < kChunk; tt++) {
                        if (t0 + tt < T) {
                            float4 hv = ((const float4 *)(a.h + (size_t)(t0 + tt) * H))[i * 64 + lane];
                            acc[tt] += wv.x * hv.x + wv.y * hv.y + wv.z * hv.z + wv.w * hv.w;
                            ss[tt] += hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w;
                        }
                    }
                }
#pragma unroll
                for (int tt = 0; tt < kChunk; tt++) {
                    if (t0 + tt < T) {
                        float d = wave_sum(acc[tt]);
                        float q = wave_sum(ss[tt]);
                        if (lane == 0) {
                            float r = a.normalize ? 1.0f / sqrtf(q / (float)H + a.eps) : 1.0f;
                            float lg = d * r + (a.bias ? a.bias[e] : 0.f);
                            a.logits[(size_t)(t0 + tt) * E + e] = lg;
                            if (a.logits2) a.logits2[(size_t)(t0 + tt) * E + e] = lg;
                        }
                    }
                }
            }
        }
    } else {
        // encode token t = blk - n_expert_blocks
        const int t = blk - a.n_expert_blocks;
        const float *ht = a.h + (size_t)t * H;
        float ss = 0.f;
        for (int i = threadIdx.x; i < H; i += blockDim.x) ss += ht[i] * ht[i];
        ss = block_sum(ss, red);
        float r = a.normalize ? 1.0f / sqrtf(ss / (float)H + a.eps) : 1.0f;
        for (int i = threadIdx.x; i < H; i += blockDim.x) xbuf[i] = ht[i] * r;
        __syncthreads();
        encode_vector(xbuf, H, H, a.xq + (size_t)t * kPieces * H, a.xs + t, a.xsum + (size_t)t * kPieces * (H / 16), red);
    }

    // completion count; the last workgroup does top-k (and grouping)
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(a.counter, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!is_last) return;
    __threadfence();

    const int k = a.k;
    const int lane = lane_id();
    for (int t = wave_id(); t < T; t += kRouteThreads / 64) {
        // each lane holds logits e = lane + 64*i
        float v[kMaxE / 64];
        uint32_t taken = 0;
#pragma unroll
        for (int i = 0; i < kMaxE / 64; i++) {
            int e = lane + 64 * i;
            v[i] = e < E ? __builtin_nontemporal_load(a.logits + (size_t)t * E + e) : -INFINITY;
        }
        float top = 0.f;
        for (int j = 0; j < k; j++) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < kMaxE / 64; i++) {
                int e = lane + 64 * i;
                if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                float ov = __shfl_xor(bv, o, 64);
                int oi = __shfl_xor(bi, o, 64);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
            if (j == 0) top = bv;
            if (lane == 0) { sidx[t * k + j] = bi; sw[t * k + j] = bv; }
        }
        // softmax over the k selected logits
        float s = 0.f;
        for (int j = lane; j < k; j += 64) s += expf(sw[t * k + j] - top);
        s = wave_sum(s);
        for (int j = lane; j < k; j += 64) {
            float wj = expf(sw[t * k + j] - top) / s;
            int id = sidx[t * k + j];
            sw[t * k + j] = wj;
            a.idx[t * k + j] = id;
            a.w[t * k + j] = wj;
            if (a.idx2) a.idx2[t * k + j] = id;
            if (a.w2) a.w2[t * k + j] = wj;
        }
    }
    __syncthreads();
    if (a.group) group_block(sidx, sw, T, k, E, a.ns, a.go, lstart);
    if (threadIdx.x == 0) *a.counter = 0u;
}

// ---------------------------------------------------------------------------
// k_prep: encode given token states (no normalisation) and group given
// routing.  Workgroup t encodes token t; the last one groups.
struct PrepArgs {
    const float *x;
    int T, H, k, E, ns;
    const int *idx;
    const float *w;
    int8_t *xq; float *xs; int *xsum;
    GroupOut go;
    unsigned *counter;
};

__global__ __launch_bounds__(kRouteThreads) void k_prep(PrepArgs a)
{
    __shared__ float red[16];
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ float sw[kMaxT * kMaxK];
    __shared__ int lstart[kMaxE + 8];
    __shared__ int is_last;
    const int t = blockIdx.x;
    encode_vector(a.x + (size_t)t * a.H, a.H, a.H, a.xq + (size_t)t * kPieces * a.H, a.xs + t,
                  a.xsum + (size_t)t * kPieces * (a.H / 16), red);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(a.counter, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    for (int p = threadIdx.x; p < a.T * a.k; p += blockDim.x) {
        sidx[p] = a.idx[p];
        sw[p] = a.w[p];
    }
    __syncthreads();
    group_block(sidx, sw, a.T, a.k, a.E, a.ns, a.go, lstart);
    if (threadIdx.x == 0) *a.counter = 0u;
}

// k_group: moe_group_tokens (one workgroup).
__global__ __launch_bounds__(kRouteThreads) void k_group(const int *idx, int T, int k, int E, GroupOut go)
{
    __shared__ int sidx[kMaxT * kMaxK];
    __shared__ int lstart[kMaxE + 8];
    for (int p = threadIdx.x; p < T * k; p += blockDim.x) sidx[p] = idx[p];
    __syncthreads();
    group_block(sidx, nullptr, T, k, E, 0, go, lstart);
}

// k_rmsnorm: one workgroup per token.
__global__ __launch_bounds__(kRouteThreads) void k_rmsnorm(const float *h, int H, float eps, float *out)
{
    __shared__ float red[16];
    const float *ht = h + (size_t)blockIdx.x * H;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += blockDim.x) ss += ht[i] * ht[i];
    ss = block_sum(ss, red);
    float r = 1.0f / sqrtf(ss / (float)H + eps);
    for (int i = threadIdx.x; i < H; i += blockDim.x) out[(size_t)blockIdx.x * H + i] = ht[i] * r;
}

// ---------------------------------------------------------------------------
// Per-lane K-group dot products.  A lane owns one row of a 64-row tile and
// one 256-column K-group; xw0..2 point at the token's three pieces for the
// K-group (64 int32 words each), xsm0..2 at their per-16 sums (16 each).

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

__device__ __forceinline__ float kgroup_dot(const Q4KRegs &r, const int *__restrict__ xw0, const int *__restrict__ xw1,
                                            const int *__restrict__ xw2, const int *__restrict__ xs0,
                                            const int *__restrict__ xs1, const int *__restrict__ xs2)
{
    const uint32_t W0 = r.meta.y, W1 = r.meta.z, W2 = r.meta.w;
    const uint32_t sclo = W0 & 0x3F3F3F3Fu, mlo = W1 & 0x3F3F3F3Fu;
    const uint32_t schi = (W2 & 0x0F0F0F0Fu) | ((W0 >> 2) & 0x30303030u);
    const uint32_t mhi = ((W2 >> 4) & 0x0F0F0F0Fu) | ((W1 >> 2) & 0x30303030u);
    int I0 = 0, I1 = 0, I2 = 0, J0 = 0, J1 = 0, J2 = 0;
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
            a0 = dot4(lo, xw0[16 * c + i], a0);
            a1 = dot4(lo, xw1[16 * c + i], a1);
            a2 = dot4(lo, xw2[16 * c + i], a2);
            b0 = dot4(hi, xw0[16 * c + 8 + i], b0);
            b1 = dot4(hi, xw1[16 * c + 8 + i], b1);
            b2 = dot4(hi, xw2[16 * c + 8 + i], b2);
        }
        I0 += __mul24(sc0, a0) + __mul24(sc1, b0);
        I1 += __mul24(sc0, a1) + __mul24(sc1, b1);
        I2 += __mul24(sc0, a2) + __mul24(sc1, b2);
        J0 += m0 * (xs0[4 * c] + xs0[4 * c + 1]) + m1 * (xs0[4 * c + 2] + xs0[4 * c + 3]);
        J1 += m0 * (xs1[4 * c] + xs1[4 * c + 1]) + m1 * (xs1[4 * c + 2] + xs1[4 * c + 3]);
        J2 += m0 * (xs2[4 * c] + xs2[4 * c + 1]) + m1 * (xs2[4 * c + 2] + xs2[4 * c + 3]);
    }
    const float d = half_lo(r.meta.x), dmin = half_hi(r.meta.x);
    const float fi = (float)I0 + (float)I1 * kC1 + (float)I2 * kC2;
    const float fj = (float)J0 + (float)J1 * kC1 + (float)J2 * kC2;
    return d * fi - dmin * fj;
}

__device__ __forceinline__ float kgroup_dot(const Q6KRegs &r, const int *__restrict__ xw0, const int *__restrict__ xw1,
                                            const int *__restrict__ xw2, const int *__restrict__ xs0,
                                            const int *__restrict__ xs1, const int *__restrict__ xs2)
{
    int I0 = 0, I1 = 0, I2 = 0;
#pragma unroll
    for (int n = 0; n < 2; n++) {
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
                const int j = 8 * n + 2 * m + ih;  // 16-weight sub-block
                const int wb = 32 * n + 8 * m + 4 * ih;
                int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
                for (int i4 = 0; i4 < 4; i4++) {
                    a0 = dot4(qv[m][i4], xw0[wb + i4], a0);
                    a1 = dot4(qv[m][i4], xw1[wb + i4], a1);
                    a2 = dot4(qv[m][i4], xw2[wb + i4], a2);
                }
                const int sc = (int)(int8_t)((comp(r.sc, j >> 2) >> (8 * (j & 3))) & 0xff);
                I0 += __mul24(sc, a0 - 32 * xs0[j]);
                I1 += __mul24(sc, a1 - 32 * xs1[j]);
                I2 += __mul24(sc, a2 - 32 * xs2[j]);
            }
        }
    }
    const float d = half_lo(r.d);
    return d * ((float)I0 + (float)I1 * kC1 + (float)I2 * kC2);
}

__device__ __forceinline__ float kgroup_dot(const Q80Regs &r, const int *__restrict__ xw0, const int *__restrict__ xw1,
                                            const int *__restrict__ xw2, const int *, const int *, const int *)
{
    float acc = 0.f;
#pragma unroll
    for (int b = 0; b < 8; b++) {
        int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int D = 8 * b + i;
            const uint32_t qd = comp(r.q[D >> 2], D & 3);
            a0 = dot4(qd, xw0[D], a0);
            a1 = dot4(qd, xw1[D], a1);
            a2 = dot4(qd, xw2[D], a2);
        }
        const uint32_t dw = comp(r.d, b >> 1);
        const float db = (b & 1) ? half_hi(dw) : half_lo(dw);
        acc += db * ((float)a0 + (float)a1 * kC1 + (float)a2 * kC2);
    }
    return acc;
}

template <int QT> struct RegsOf;
template <> struct RegsOf<MOE_Q4_K> { using T = Q4KRegs; };
template <> struct RegsOf<MOE_Q6_K> { using T = Q6KRegs; };
template <> struct RegsOf<MOE_Q8_0> { using T = Q80Regs; };

template <int QT> constexpr int kTileBytes = QT == MOE_Q4_K ? 9216 : QT == MOE_Q6_K ? 13440 : 17408;

// ---------------------------------------------------------------------------
// k_gate_up: workgroup (u, rt) = distinct expert u, rows [32rt, 32rt+32) of
// gate (lanes 0-31) and up (lanes 32-63); wave w takes K-groups w, w+8, ...

struct GateUpArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const int *nuniq, *uniq, *uoff, *ptok;
    const int8_t *xq; const float *xs; const int *xsum;  // [T][3][H], [T], [T][3][H/16]
    int H, I, kd;
    unsigned long long up_off;
    float *hact;                                           // [P][kd]
    int8_t *hq; float *hs; int *hsum;                      // [P][3][kd], [P], [P][3][kd/16]
    unsigned *cnt;                                         // [U]
    int ntile;                                             // I/32
};

constexpr int kGUThreads = 512;

template <int QT>
__global__ __launch_bounds__(kGUThreads) void k_gate_up(GateUpArgs a)
{
    __shared__ float part[8][kChunk][64];
    __shared__ float redv[kChunk][64];
    __shared__ float red[16];
    __shared__ int is_last;

    const int u = blockIdx.x / a.ntile;
    const int rt = blockIdx.x - u * a.ntile;
    if (u >= *a.nuniq) return;
    const int e = a.uniq[u];
    const uint8_t *base = (const uint8_t *)(e < a.E ? a.eptr[e] : a.sptr[e - a.E]);
    const int p0 = a.uoff[u], p1 = a.uoff[u + 1];
    const int H = a.H, S = H >> 8;
    const int wv = wave_id(), lane = lane_id();
    const int mat = lane >> 5;
    const int row = rt * 32 + (lane & 31);
    const int tile64 = row >> 6, lt = row & 63;
    const uint8_t *mbase = base + (mat ? a.up_off : 0ull);
    const int nwv = S < 8 ? S : 8;

    for (int c0 = p0; c0 < p1; c0 += kChunk) {
        const int nt = p1 - c0 < kChunk ? p1 - c0 : kChunk;
        if (wv < nwv) {
            for (int s = wv; s < S; s += 8) {
                typename RegsOf<QT>::T r;
                load_regs(r, mbase + ((size_t)tile64 * S + s) * kTileBytes<QT>, lt);
                for (int tt = 0; tt < nt; tt++) {
                    const int t = a.ptok[c0 + tt];
                    const int *xw = (const int *)(a.xq + (size_t)t * kPieces * H) + s * 64;
                    const int *xsm = a.xsum + (size_t)t * kPieces * (H / 16) + s * 16;
                    float v = kgroup_dot(r, xw, xw + H / 4, xw + H / 2, xsm, xsm + H / 16, xsm + H / 8) * a.xs[t];
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
        for (int i = threadIdx.x; i < nt * 32; i += blockDim.x) {
            const int tt = i >> 5, r = i & 31;
            const float g = redv[tt][r], up = redv[tt][32 + r];
            const float hv = g / (1.0f + expf(-g)) * up;
            a.hact[(size_t)(c0 + tt) * a.kd + rt * 32 + r] = hv;
        }
        __syncthreads();
    }

    // the last row tile of this expert encodes SiLU(g)*u of its pairs
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(&a.cnt[u], 1u) == (unsigned)(a.ntile - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    for (int p = p0; p < p1; p++)
        encode_vector(a.hact + (size_t)p * a.kd, a.I, a.kd, a.hq + (size_t)p * kPieces * a.kd, a.hs + p,
                      a.hsum + (size_t)p * kPieces * (a.kd / 16), red);
    if (threadIdx.x == 0) a.cnt[u] = 0u;
}

// ---------------------------------------------------------------------------
// k_down: workgroup (u, rt) = distinct expert u, down rows [64rt, 64rt+64);
// wave w takes K-groups w, w+nw, ...  The last expert to finish row tile rt
// writes y for every token.

struct DownArgs {
    const void *const *eptr;
    const void *const *sptr;
    int E;
    const int *nuniq, *uniq, *uoff;
    const int8_t *hq; const float *hs; const int *hsum;
    int H, kd;
    unsigned long long down_off;
    float *osc;   // [P][H]
    unsigned *cnt;  // [H/64]
    int nrt;
    int T, k, ns;
    const int *inv;   // [T][k+ns]
    const float *w;   // [T][k]
    float *y;         // [T][H]
    int accumulate;
};

template <int QT>
__global__ __launch_bounds__(512) void k_down(DownArgs a)
{
    __shared__ float part[8][kChunk][64];
    __shared__ int is_last;

    const int u = blockIdx.x / a.nrt;
    const int rt = blockIdx.x - u * a.nrt;
    const int nu = *a.nuniq;
    if (u >= nu) return;
    const int e = a.uniq[u];
    const uint8_t *base = (const uint8_t *)(e < a.E ? a.eptr[e] : a.sptr[e - a.E]) + a.down_off;
    const int p0 = a.uoff[u], p1 = a.uoff[u + 1];
    const int kd = a.kd, S = kd >> 8;
    const int nwv = (int)(blockDim.x >> 6);
    const int wv = wave_id(), lane = lane_id();

    for (int c0 = p0; c0 < p1; c0 += kChunk) {
        const int nt = p1 - c0 < kChunk ? p1 - c0 : kChunk;
        for (int s = wv; s < S; s += nwv) {
            typename RegsOf<QT>::T r;
            load_regs(r, base + ((size_t)rt * S + s) * kTileBytes<QT>, lane);
            for (int tt = 0; tt < nt; tt++) {
                const int p = c0 + tt;
                const int *xw = (const int *)(a.hq + (size_t)p * kPieces * kd) + s * 64;
                const int *xsm = a.hsum + (size_t)p * kPieces * (kd / 16) + s * 16;
                float v = kgroup_dot(r, xw, xw + kd / 4, xw + kd / 2, xsm, xsm + kd / 16, xsm + kd / 8) * a.hs[p];
                if (s == wv) part[wv][tt][lane] = v;
                else part[wv][tt][lane] += v;
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nt * 64; i += blockDim.x) {
            const int tt = i >> 6, ln = i & 63;
            float s = 0.f;
            for (int w = 0; w < nwv && w < S; w++) s += part[w][tt][ln];
            a.osc[(size_t)(c0 + tt) * a.H + rt * 64 + ln] = s;
        }
        __syncthreads();
    }

    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(&a.cnt[rt], 1u) == (unsigned)(nu - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    const int kk = a.k + a.ns;
    for (int i = threadIdx.x; i < a.T * 64; i += blockDim.x) {
        const int t = i >> 6, ln = i & 63;
        const size_t row = (size_t)rt * 64 + ln;
        float acc = a.accumulate ? a.y[(size_t)t * a.H + row] : 0.f;
        for (int j = 0; j < a.k; j++) {
            const int pj = a.inv[t * kk + j];
            if (pj >= 0) acc += a.w[t * a.k + j] * __builtin_nontemporal_load(a.osc + (size_t)pj * a.H + row);
        }
        for (int s = 0; s < a.ns; s++)
            acc += __builtin_nontemporal_load(a.osc + (size_t)a.inv[t * kk + a.k + s] * a.H + row);
        a.y[(size_t)t * a.H + row] = acc;
    }
    if (threadIdx.x == 0) a.cnt[rt] = 0u;
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
};

moe_status check_desc(const moe_expert_desc *d, ExpertGeom *g)
{
    if (!d) { set_error("null expert desc"); return MOE_ERR_ARG; }
    if (!qtype_ok(d->gate) || !qtype_ok(d->up) || !qtype_ok(d->down)) {
        set_error("unknown qtype (gate %d, up %d, down %d)", d->gate, d->up, d->down);
        return MOE_ERR_QTYPE;
    }
    if (!geom(*d, g)) {
        set_error("bad shape H=%d I=%d: H must be a positive multiple of 256, I of 64", d->H, d->I);
        return MOE_ERR_SHAPE;
    }
    return MOE_OK;
}

moe_status check_tke(int T, int k, int E, int ns)
{
    if (T < 1 || T > kMaxT) { set_error("T=%d outside [1, %d]", T, kMaxT); return MOE_ERR_BATCH; }
    if (E < 1 || E > kMaxE) { set_error("E=%d outside [1, %d]", E, kMaxE); return MOE_ERR_ARG; }
    if (k < 1 || k > E || k > kMaxK) { set_error("k=%d outside [1, min(E=%d, %d)]", k, E, kMaxK); return MOE_ERR_ARG; }
    if (ns < 0 || ns > 8) { set_error("n_shared=%d outside [0, 8]", ns); return MOE_ERR_ARG; }
    return MOE_OK;
}

moe_status launch_ffn_kernels(const moe_expert_desc &d, const ExpertGeom &g, const Ws &ws, int T, int k,
                              int E, int ns, const void *const *eptr, const void *const *sptr,
                              const float *wts, float *y, int accumulate, float *act_out, hipStream_t s)
{
    const WsLayout &L = ws.L;
    const int U = (E < T * k ? E : T * k) + ns;
    float *hact = act_out ? act_out : ws.at<float>(L.hact);
    GateUpArgs ga;
    ga.eptr = eptr; ga.sptr = sptr; ga.E = E;
    ga.nuniq = ws.at<int>(L.nuniq); ga.uniq = ws.at<int>(L.uniq); ga.uoff = ws.at<int>(L.uoff); ga.ptok = ws.at<int>(L.ptok);
    ga.xq = ws.at<int8_t>(L.xq); ga.xs = ws.at<float>(L.xs); ga.xsum = ws.at<int>(L.xsum);
    ga.H = d.H; ga.I = d.I; ga.kd = g.kd; ga.up_off = g.up_off;
    ga.hact = hact; ga.hq = ws.at<int8_t>(L.hq); ga.hs = ws.at<float>(L.hs); ga.hsum = ws.at<int>(L.hsum);
    ga.cnt = ws.at<unsigned>(L.cnt_gu);
    ga.ntile = d.I / 32;
    if (d.gate != d.up) { set_error("gate and up must share one qtype"); return MOE_ERR_QTYPE; }
    dim3 ggrid(U * ga.ntile);
    switch (d.gate) {
    case MOE_Q4_K: k_gate_up<MOE_Q4_K><<<ggrid, kGUThreads, 0, s>>>(ga); break;
    case MOE_Q6_K: k_gate_up<MOE_Q6_K><<<ggrid, kGUThreads, 0, s>>>(ga); break;
    case MOE_Q8_0: k_gate_up<MOE_Q8_0><<<ggrid, kGUThreads, 0, s>>>(ga); break;
    }
    LAUNCH_OK("k_gate_up");

    DownArgs da;
    da.eptr = eptr; da.sptr = sptr; da.E = E;
    da.nuniq = ga.nuniq; da.uniq = ga.uniq; da.uoff = ga.uoff;
    da.hq = ga.hq; da.hs = ga.hs; da.hsum = ga.hsum;
    da.H = d.H; da.kd = g.kd; da.down_off = g.down_off;
    da.osc = ws.at<float>(L.osc); da.cnt = ws.at<unsigned>(L.cnt_dn);
    da.nrt = d.H / 64;
    da.T = T; da.k = k; da.ns = ns; da.inv = ws.at<int>(L.inv); da.w = wts; da.y = y; da.accumulate = accumulate;
    const int S = g.kd / 256;
    dim3 dgrid(U * da.nrt), dblock(64 * (S < 8 ? S : 8));
    switch (d.down) {
    case MOE_Q4_K: k_down<MOE_Q4_K><<<dgrid, dblock, 0, s>>>(da); break;
    case MOE_Q6_K: k_down<MOE_Q6_K><<<dgrid, dblock, 0, s>>>(da); break;
    case MOE_Q8_0: k_down<MOE_Q8_0><<<dgrid, dblock, 0, s>>>(da); break;
    }
    LAUNCH_OK("k_down");
    return MOE_OK;
}

GroupOut ws_group_out(const Ws &ws)
{
    const WsLayout &L = ws.L;
    GroupOut go{};
    go.nuniq = ws.at<int>(L.nuniq); go.uniq = ws.at<int>(L.uniq); go.uoff = ws.at<int>(L.uoff);
    go.ptok = ws.at<int>(L.ptok); go.pw = ws.at<float>(L.pw); go.inv = ws.at<int>(L.inv);
    return go;
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

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_rmsnorm(const float *h, int32_t T, int32_t H, float eps, float *xhat, hipStream_t s)
{
    if (!h || !xhat || T < 1 || H < 1) { set_error("moe_rmsnorm: bad argument"); return MOE_ERR_ARG; }
    k_rmsnorm<<<T, kRouteThreads, 0, s>>>(h, H, eps, xhat);
    LAUNCH_OK("k_rmsnorm");
    return MOE_OK;
}

moe_status moe_route_topk(const float *x, int32_t T, int32_t H, const float *w_router, const float *bias,
                          int32_t E, int32_t k, int32_t *idx, float *w, float *logits, hipStream_t s)
{
    moe_status st = check_tke(T, k, E, 0);
    if (st != MOE_OK) return st;
    if (!x || !w_router || !idx || !w) { set_error("moe_route_topk: null pointer"); return MOE_ERR_ARG; }
    if (H < 256 || H % 256) { set_error("moe_route_topk: H=%d must be a multiple of 256", H); return MOE_ERR_SHAPE; }
    // small private scratch: logits and the completion counter
    static thread_local struct { void *p = nullptr; size_t n = 0; int dev = -1; } scr;
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    size_t need = align256((size_t)T * E * 4) + 256;
    if (scr.n < need || scr.dev != dev) {
        if (scr.p) (void)hipFree(scr.p);
        scr.p = nullptr; scr.n = 0;
        HIP_OK(hipMalloc(&scr.p, kMaxT * kMaxE * 4 + 256));
        HIP_OK(hipMemset(scr.p, 0, kMaxT * kMaxE * 4 + 256));
        scr.n = kMaxT * kMaxE * 4 + 256; scr.dev = dev;
    }
    RouteArgs a{};
    a.h = x; a.T = T; a.H = H; a.wr = w_router; a.bias = bias; a.E = E; a.k = k; a.eps = 0.f; a.normalize = 0;
    a.logits = (float *)scr.p; a.idx = idx; a.w = w; a.logits2 = logits;
    a.counter = (unsigned *)((uint8_t *)scr.p + kMaxT * kMaxE * 4);
    a.n_expert_blocks = (E + 3) / 4;
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
    size_t n16 = ws_bytes / 16;
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
    pa.x = x; pa.T = T; pa.H = d->H; pa.k = k; pa.E = E; pa.ns = n_shared; pa.idx = idx; pa.w = w;
    pa.xq = W.at<int8_t>(W.L.xq); pa.xs = W.at<float>(W.L.xs); pa.xsum = W.at<int>(W.L.xsum);
    pa.go = ws_group_out(W);
    pa.counter = W.at<unsigned>(W.L.cnt_route);
    k_prep<<<T, kRouteThreads, 0, s>>>(pa);
    LAUNCH_OK("k_prep");
    return launch_ffn_kernels(*d, g, W, T, k, E, n_shared, expert_ptrs, shared_ptrs, w, y, accumulate, act_out, s);
}

moe_status moe_layer_route(const moe_expert_desc *d, const float *h, int32_t T, const float *w_router,
                           const float *bias, int32_t E, int32_t k, int32_t n_shared, float eps, int32_t *idx_out,
                           float *w_out, void *ws, size_t ws_bytes, hipStream_t s)
{
    ExpertGeom g;
    moe_status st = check_desc(d, &g);
    if (st != MOE_OK) return st;
    if ((st = check_tke(T, k, E, n_shared)) != MOE_OK) return st;
    if (!h || !w_router) { set_error("moe_layer_route: null pointer"); return MOE_ERR_ARG; }
    Ws W;
    if ((st = check_ws(*d, ws, ws_bytes, T, k, E, n_shared, &W)) != MOE_OK) return st;
    RouteArgs a{};
    a.h = h; a.T = T; a.H = d->H; a.wr = w_router; a.bias = bias; a.E = E; a.k = k; a.eps = eps; a.normalize = 1;
    a.logits = W.at<float>(W.L.logits); a.idx = W.at<int>(W.L.idx); a.w = W.at<float>(W.L.w);
    a.idx2 = idx_out; a.w2 = w_out; a.logits2 = nullptr;
    a.encode = 1; a.xq = W.at<int8_t>(W.L.xq); a.xs = W.at<float>(W.L.xs); a.xsum = W.at<int>(W.L.xsum);
    a.group = 1; a.ns = n_shared; a.go = ws_group_out(W);
    a.counter = W.at<unsigned>(W.L.cnt_route);
    a.n_expert_blocks = (E + 3) / 4;
    k_route<<<a.n_expert_blocks + T, kRouteThreads, (size_t)d->H * 4, s>>>(a);
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
    moe_status st = moe_layer_route(d, h, T, w_router, bias, E, k, n_shared, eps, idx_out, w_out, ws, ws_bytes, s);
    if (st != MOE_OK) return st;
    return moe_layer_ffn(d, h, T, E, k, expert_ptrs, shared_ptrs, n_shared, ws, ws_bytes, s);
}

}  // extern "C"
