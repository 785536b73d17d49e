/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle for the decode-time MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and
 * bench.py's cpu_baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the only thing both sides
 * share is the seeded input generator (workloads/), which holds none of the
 * method's arithmetic.
 *
 * What it computes, and where each step comes from:
 *
 *  - Quantized block formats: Q8_0 (34-byte block of 32 weights: fp16 scale d
 *    then 32 int8 quants; the 34-byte size is stated in the GPU-offload
 *    research notes, kwkr.cn, section 1.2), Q4_K and Q6_K super-blocks of 256
 *    weights.  The bit packing is not on the pages; the public GGUF layout is
 *    taken as the definition.  Values are the closed forms
 *        Q8_0: v = d*q
 *        Q4_K: v = d*sc_b*q - dmin*m_b      (b = 32-weight sub-block)
 *        Q6_K: v = d*sc_j*(q - 32)          (j = 16-weight sub-block)
 *    All are dyadic rationals, exact in fp64.
 *  - Router: logits = <x, W_e> + b_e, softmax, top-k (gating as in the MoE
 *    offload blog, mhpn.cn, sections 3.1 and 5.2), with the k selected
 *    probabilities renormalised to sum to one.
 *  - Expert FFN: down( SiLU(gate x) * (up x) ), weighted sum over the k
 *    selected experts plus always-active shared experts of weight one
 *    (shared experts: laptop 16B MoE post, lpnh.cn, section 2.1; the T4
 *    MoE-cache report, kongchang.com, section "What the MoE cache caches",
 *    names the gate/up/down expert tensors).
 *  - Grouping of (token, slot) pairs by expert: a stable counting sort.
 *  - Slot planner and LRU over (layer, expert) keys in one pool per
 *    (type, shape) group: T4 MoE-cache report, sections "What the MoE cache
 *    caches" and "Size your experts before configuring".
 *
 * Readings of points the pages leave open are listed where they are used.
 * Everything accumulates in fp64; sums run in plain index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q8_0 1
#define ORC_Q4_K 2
#define ORC_Q6_K 3

/* ------------------------------------------------------------------ */
/* IEEE-754 binary16 -> double, exact.                                  */
double orc_half(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* zero / subnormal */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);    /* 1.man * 2^(ex-15) */
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int orc_block_weights(int qtype)
{
    return qtype == ORC_Q8_0 ? 32 : (qtype == ORC_Q4_K || qtype == ORC_Q6_K) ? 256 : 0;
}

int orc_block_bytes(int qtype)
{
    return qtype == ORC_Q8_0 ? 34 : qtype == ORC_Q4_K ? 144 : qtype == ORC_Q6_K ? 210 : 0;
}

/* Q8_0 block: bytes 0-1 fp16 d, bytes 2..33 int8 q[0..31]. */
static void deq_q8_0(const uint8_t *b, double *out)
{
    double d = orc_half(rd16(b));
    for (int i = 0; i < 32; i++)
        out[i] = d * (double)(int8_t)b[2 + i];
}

/* Q4_K scale / min of sub-block j (0..7) from the 12 packed scale bytes.
 * Sub-blocks 0-3 keep their 6-bit scale and min in the low 6 bits of bytes j
 * and j+4.  Sub-blocks 4-7 keep the low 4 bits in the two nibbles of byte
 * j+4 (scale low, min high) and the top 2 bits in the top 2 bits of bytes
 * j-4 (scale) and j (min). */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Q4_K super-block: fp16 d, fp16 dmin, 12 scale bytes, 128 quant bytes.
 * Quant byte 32c+i holds weight 64c+i in its low nibble and weight 64c+32+i
 * in its high nibble (c = 0..3, i = 0..31). */
static void deq_q4_k(const uint8_t *b, double *out)
{
    double d = orc_half(rd16(b));
    double dmin = orc_half(rd16(b + 2));
    const uint8_t *s = b + 4;
    const uint8_t *qs = b + 16;
    for (int c = 0; c < 4; c++) {
        int sc0, m0, sc1, m1;
        q4k_scale_min(s, 2 * c, &sc0, &m0);
        q4k_scale_min(s, 2 * c + 1, &sc1, &m1);
        for (int i = 0; i < 32; i++) {
            int lo = qs[32 * c + i] & 15;
            int hi = qs[32 * c + i] >> 4;
            out[64 * c + i] = d * sc0 * lo - dmin * m0;
            out[64 * c + 32 + i] = d * sc1 * hi - dmin * m1;
        }
    }
}

/* Q6_K super-block: 128 bytes of low 4 bits (ql), 64 bytes of high 2 bits
 * (qh), 16 int8 sub-scales, fp16 d.  Each half n (128 weights) uses
 * ql[64n..64n+63] and qh[32n..32n+31]; for l = 0..31 the byte pair
 * (ql[64n+l], ql[64n+32+l]) and qh[32n+l] carry the weights 128n+l,
 * 128n+32+l, 128n+64+l, 128n+96+l: low nibbles first, then high nibbles,
 * with qh bit pairs 0-1, 2-3, 4-5, 6-7 in that order.  The sub-scale of a
 * weight is sc[weight/16]. */
static void deq_q6_k(const uint8_t *b, double *out)
{
    const uint8_t *ql = b;
    const uint8_t *qh = b + 128;
    const int8_t *sc = (const int8_t *)(b + 192);
    double d = orc_half(rd16(b + 208));
    int q[256];
    for (int n = 0; n < 2; n++) {
        for (int l = 0; l < 32; l++) {
            int a = ql[64 * n + l], c = ql[64 * n + 32 + l], h = qh[32 * n + l];
            q[128 * n + l] = (a & 15) | ((h & 3) << 4);
            q[128 * n + 32 + l] = (c & 15) | (((h >> 2) & 3) << 4);
            q[128 * n + 64 + l] = (a >> 4) | (((h >> 4) & 3) << 4);
            q[128 * n + 96 + l] = (c >> 4) | (((h >> 6) & 3) << 4);
        }
    }
    for (int p = 0; p < 256; p++)
        out[p] = d * (double)sc[p / 16] * (double)(q[p] - 32);
}

/* Dequantize one row of k weights (k a multiple of the block size). */
int orc_dequant_row(int qtype, const uint8_t *row, int k, double *out)
{
    int bw = orc_block_weights(qtype), bb = orc_block_bytes(qtype);
    if (bw == 0 || k % bw)
        return -1;
    for (int b = 0; b < k / bw; b++) {
        const uint8_t *blk = row + (size_t)b * bb;
        if (qtype == ORC_Q8_0)
            deq_q8_0(blk, out + (size_t)b * bw);
        else if (qtype == ORC_Q4_K)
            deq_q4_k(blk, out + (size_t)b * bw);
        else
            deq_q6_k(blk, out + (size_t)b * bw);
    }
    return 0;
}

/* y[r] = sum_c W[r][c] * x[c] for an [n, k] quantized matrix (row-major rows
 * of whole blocks).  Each row is dequantized to fp64 and dotted with x. */
int orc_qmatvec(int qtype, const uint8_t *w, int n, int k, const double *x, double *y)
{
    int bw = orc_block_weights(qtype), bb = orc_block_bytes(qtype);
    if (bw == 0 || k % bw)
        return -1;
    size_t row_bytes = (size_t)(k / bw) * bb;
    int bad = 0;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (size_t)k);
        if (!buf) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int r = 0; r < n; r++) {
                orc_dequant_row(qtype, w + row_bytes * (size_t)r, k, buf);
                double acc = 0.0;
                for (int c = 0; c < k; c++)
                    acc += buf[c] * x[c];
                y[r] = acc;
            }
            free(buf);
        }
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------ */
/* Layer-stack normalisation.  The pages give no composition for a stack of
 * MoE layers; the reading used here is a pre-norm residual block with a
 * weightless RMSNorm:  xhat = h / sqrt(mean(h^2) + eps). */
void orc_rmsnorm(const double *h, int n, double eps, double *out)
{
    double ss = 0.0;
    for (int i = 0; i < n; i++)
        ss += h[i] * h[i];
    double r = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; i++)
        out[i] = h[i] * r;
}

/* Router for one token: logits, top-k ids ordered by (logit desc, id asc),
 * renormalised softmax weights over the selected k, and the gap between the
 * k-th and (k+1)-th largest logit (+inf when k == E).
 * Softmax is monotone, so choosing by logit is choosing by probability, and
 * the full softmax restricted to the k winners and renormalised equals a
 * softmax over the k winning logits. */
int orc_route(const double *x, const float *wr, const float *bias, int E, int H, int k,
              int32_t *idx, double *w, double *logits, double *gap)
{
    if (k < 1 || k > E)
        return -1;
    for (int e = 0; e < E; e++) {
        double acc = 0.0;
        for (int i = 0; i < H; i++)
            acc += x[i] * (double)wr[(size_t)e * H + i];
        logits[e] = acc + (bias ? (double)bias[e] : 0.0);
    }
    unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
    if (!taken)
        return -2;
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++)
            if (!taken[e] && (best < 0 || logits[e] > logits[best]))
                best = e;                /* strict '>' keeps the lower id on ties */
        taken[best] = 1;
        idx[j] = best;
    }
    double next = -INFINITY;
    for (int e = 0; e < E; e++)
        if (!taken[e] && logits[e] > next)
            next = logits[e];
    *gap = (k == E) ? INFINITY : logits[idx[k - 1]] - next;
    free(taken);
    double mx = logits[idx[0]], s = 0.0;
    for (int j = 0; j < k; j++) {
        w[j] = exp(logits[idx[j]] - mx);
        s += w[j];
    }
    for (int j = 0; j < k; j++)
        w[j] /= s;
    return 0;
}

double orc_silu(double g) { return g / (1.0 + exp(-g)); }

/* One expert on one token: g = Wg x, u = Wu x, a = SiLU(g)*u (zero-padded to
 * the down matrix's padded row length kd), o = Wd a.  Any output pointer may
 * be NULL except o. */
int orc_expert_ffn(int qg, int qu, int qd, int H, int I, int kd,
                   const uint8_t *gate, const uint8_t *up, const uint8_t *down,
                   const double *x, double *g_out, double *u_out, double *a_out, double *o)
{
    double *g = (double *)malloc(sizeof(double) * (size_t)I);
    double *u = (double *)malloc(sizeof(double) * (size_t)I);
    double *a = (double *)calloc((size_t)kd, sizeof(double));
    int rc = 0;
    if (!g || !u || !a) {
        rc = -2;
        goto done;
    }
    if ((rc = orc_qmatvec(qg, gate, I, H, x, g)) != 0)
        goto done;
    if ((rc = orc_qmatvec(qu, up, I, H, x, u)) != 0)
        goto done;
    for (int i = 0; i < I; i++)
        a[i] = orc_silu(g[i]) * u[i];
    if ((rc = orc_qmatvec(qd, down, H, kd, a, o)) != 0)
        goto done;
    if (g_out)
        memcpy(g_out, g, sizeof(double) * (size_t)I);
    if (u_out)
        memcpy(u_out, u, sizeof(double) * (size_t)I);
    if (a_out)
        memcpy(a_out, a, sizeof(double) * (size_t)kd);
done:
    free(g);
    free(u);
    free(a);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Grouping: count[e] = number of (t, j) with idx[t][j] == e; offset is the
 * exclusive prefix sum (E+1 entries); pairs lists t*k+j ordered by expert,
 * then token, then slot. */
int orc_group(const int32_t *idx, int T, int k, int E, int32_t *count, int32_t *offset, int32_t *pairs)
{
    for (int e = 0; e < E; e++)
        count[e] = 0;
    for (int p = 0; p < T * k; p++) {
        if (idx[p] < 0 || idx[p] >= E)
            return -1;
        count[idx[p]]++;
    }
    offset[0] = 0;
    for (int e = 0; e < E; e++)
        offset[e + 1] = offset[e] + count[e];
    int n = 0;
    for (int e = 0; e < E; e++)
        for (int t = 0; t < T; t++)
            for (int j = 0; j < k; j++)
                if (idx[t * k + j] == e)
                    pairs[n++] = t * k + j;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Slot planner.  Each group g (one per expert type+shape) with per-expert
 * bytes s_g shared by L_g layers gets the same fraction of its experts:
 *     slots_g = floor(B * L_g / sum_h L_h * s_h) - 1,
 * and a group whose count falls below top_k is disabled (0 slots).  Returns
 * 0, or -1 when every group is disabled.  The "- 1" and the top_k floor are
 * the reading that reproduces all three printed facts of the T4 MoE-cache
 * report (section "Size your experts before configuring"): 1,834 slots per
 * group at 10,000 MiB, 50 MiB accepted, 49 MiB rejected. */
int orc_cache_plan(int n_groups, const int64_t *expert_bytes, const int32_t *layers,
                   uint64_t budget, int top_k, int32_t *slots)
{
    unsigned __int128 denom = 0;
    for (int g = 0; g < n_groups; g++)
        denom += (unsigned __int128)expert_bytes[g] * (uint64_t)layers[g];
    int any = 0;
    for (int g = 0; g < n_groups; g++) {
        unsigned __int128 q = denom ? ((unsigned __int128)budget * (uint64_t)layers[g]) / denom : 0;
        long long s = (long long)q - 1;
        if (s < top_k)
            s = 0;
        slots[g] = (int32_t)s;
        if (s > 0)
            any = 1;
    }
    return any ? 0 : -1;
}

/* Exact LRU over (layer, expert) keys, one pool per group.
 *
 * lookups: n_lookups (layer, expert) pairs in the order the decode visits
 * them (step by step, layer by layer, and within a layer-step each distinct
 * expert once in ascending id).  layer_group[l] maps a layer to its pool.
 * The pool starts empty.  A hit makes the key most recent.  A miss takes the
 * lowest free slot, or else evicts the pool's least recently used key and
 * takes its slot.  Outputs per lookup: hit (0/1), the victim's layer and
 * expert (-1 when none) and the slot used.  Recency is kept as a last-use
 * stamp per slot; the victim is the resident key with the oldest stamp. */
int orc_lru(int n_groups, const int32_t *slots, const int32_t *layer_group, int n_layers,
            int n_lookups, const int32_t *lk_layer, const int32_t *lk_expert,
            uint8_t *hit, int32_t *victim_layer, int32_t *victim_expert, int32_t *slot_out)
{
    int32_t **kl = (int32_t **)calloc((size_t)n_groups, sizeof(int32_t *));
    int32_t **ke = (int32_t **)calloc((size_t)n_groups, sizeof(int32_t *));
    int64_t **st = (int64_t **)calloc((size_t)n_groups, sizeof(int64_t *));
    int rc = 0;
    if (!kl || !ke || !st) {
        rc = -2;
        goto done;
    }
    for (int g = 0; g < n_groups; g++) {
        kl[g] = (int32_t *)malloc(sizeof(int32_t) * (size_t)(slots[g] > 0 ? slots[g] : 1));
        ke[g] = (int32_t *)malloc(sizeof(int32_t) * (size_t)(slots[g] > 0 ? slots[g] : 1));
        st[g] = (int64_t *)malloc(sizeof(int64_t) * (size_t)(slots[g] > 0 ? slots[g] : 1));
        if (!kl[g] || !ke[g] || !st[g]) {
            rc = -2;
            goto done;
        }
        for (int s = 0; s < slots[g]; s++) {
            kl[g][s] = -1;
            ke[g][s] = -1;
            st[g][s] = -1;
        }
    }
    for (int i = 0; i < n_lookups; i++) {
        int l = lk_layer[i], e = lk_expert[i];
        if (l < 0 || l >= n_layers) {
            rc = -1;
            goto done;
        }
        int g = layer_group[l], ns = slots[g];
        if (ns <= 0) {
            rc = -1;
            goto done;
        }
        int found = -1, freeslot = -1, oldest = -1;
        for (int s = 0; s < ns; s++) {
            if (kl[g][s] == l && ke[g][s] == e)
                found = s;
            if (kl[g][s] < 0 && freeslot < 0)
                freeslot = s;
            if (kl[g][s] >= 0 && (oldest < 0 || st[g][s] < st[g][oldest]))
                oldest = s;
        }
        victim_layer[i] = -1;
        victim_expert[i] = -1;
        if (found >= 0) {
            hit[i] = 1;
            slot_out[i] = found;
        } else {
            hit[i] = 0;
            int s = freeslot;
            if (s < 0) {
                s = oldest;
                victim_layer[i] = kl[g][s];
                victim_expert[i] = ke[g][s];
            }
            kl[g][s] = l;
            ke[g][s] = e;
            slot_out[i] = s;
            found = s;
        }
        st[g][found] = i;
    }
done:
    for (int g = 0; g < n_groups && kl && ke && st; g++) {
        free(kl[g]);
        free(ke[g]);
        free(st[g]);
    }
    free(kl);
    free(ke);
    free(st);
    return rc;
}
