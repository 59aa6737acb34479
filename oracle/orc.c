/*
 * orc.c -- plain, slow, CPU oracle for one decode step of one sequence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the bench's
 * cpu_baseline leg do.  It shares no source, header, table or helper with
 * the HIP library: it has its own bf16 codec, its own selection code and its
 * own attention arithmetic, and it is built by gcc, not hipcc.
 *
 * Source: "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
 * Decoding" (ByteCross), GitHub README page.  Sections cited per function.
 *
 * Arithmetic conventions
 *   - bf16 values travel as uint16_t bit patterns.
 *   - GEMV, RMSNorm, RoPE, SwiGLU and attention accumulate in double and round
 *     to bf16 (round to nearest even) only where the decode step stores bf16.
 *   - Block scores are computed in float in one documented order, because they
 *     decide an integer result (which history blocks are kept).
 *   - Threads (OpenMP) only split independent outputs; results never depend
 *     on the thread count.
 *   - Build with -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* bf16 codec written from the format's definition: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits; value = (-1)^s * 1.f * 2^(e-127) for
 * 0 < e < 255, (-1)^s * 0.f * 2^-126 for e == 0.                            */

double orc_bf16_to_double(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 0xFF, f = b & 0x7F;
    double v;
    if (e == 0xFF)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -133);              /* f * 2^-7 * 2^-126 */
    else
        v = ldexp((double)(f | 0x80), e - 134);  /* (128+f) * 2^(e-127-7) */
    return s ? -v : v;
}

/* Round a double to the nearest bf16, ties to even. */
uint16_t orc_bf16_from_double(double v)
{
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e2;
    frexp(a, &e2);                 /* a = m * 2^e2, m in [0.5, 1) */
    int ue = e2 - 1;               /* unbiased exponent of a      */
    if (ue < -126) {
        /* subnormal range: the grid spacing is 2^-133 */
        double r = nearbyint(ldexp(a, 133));   /* 0..128; 128 is the smallest normal */
        return sign | (uint16_t)r;
    }
    double r = nearbyint(ldexp(a, 7 - ue));   /* significand in units of 2^(ue-7): [128, 256] */
    if (r == 256.0) { r = 128.0; ue += 1; }
    if (ue > 127) return sign | 0x7F80;
    return sign | (uint16_t)(((ue + 127) << 7) | ((int)r - 128));
}

void orc_bf16_to_double_array(const uint16_t* in, double* out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = orc_bf16_to_double(in[i]);
}

void orc_bf16_from_double_array(const double* in, uint16_t* out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = orc_bf16_from_double(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Channel selection (README "What it does in one picture" and "Timing and
 * quality on a GPU": a token's own activations decide which projection
 * weights are read; TEAL on all seven projections).  Read here as the
 * exact per-step top-k of |x|: the key of channel i is its bf16 magnitude
 * bits, larger key first, equal keys by lower index; k channels are kept and
 * reported in ascending channel order.                                       */

typedef struct { uint32_t key; int32_t pos; } orc_keyed;

static int orc_cmp_desc_key_asc_pos(const void* a, const void* b)
{
    const orc_keyed* x = (const orc_keyed*)a;
    const orc_keyed* y = (const orc_keyed*)b;
    if (x->key != y->key) return x->key > y->key ? -1 : 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int orc_cmp_int32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Sort all n keys (largest first, ties by lower position), keep the first k
 * positions, return them ascending.  Brute force by construction. */
static void orc_topk_positions(const uint32_t* keys, int n, int k, int32_t* out)
{
    orc_keyed* a = (orc_keyed*)malloc(sizeof(orc_keyed) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) { a[i].key = keys[i]; a[i].pos = i; }
    qsort(a, (size_t)n, sizeof(orc_keyed), orc_cmp_desc_key_asc_pos);
    for (int i = 0; i < k; ++i) out[i] = a[i].pos;
    qsort(out, (size_t)k, sizeof(int32_t), orc_cmp_int32);
    free(a);
}

/* Number of channels kept: k = floor(r_p * d_in + 1/2), clamped to [1, d_in];
 * r_p >= 1 keeps every channel. */
int orc_channel_keep(double r_p, int d_in)
{
    if (r_p >= 1.0) return d_in;
    long k = (long)floor(r_p * (double)d_in + 0.5);
    if (k < 1) k = 1;
    if (k > d_in) k = d_in;
    return (int)k;
}

void orc_select_channels(const uint16_t* x, int d_in, int k, int32_t* idx_out)
{
    uint32_t* keys = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(d_in > 0 ? d_in : 1));
    for (int i = 0; i < d_in; ++i) keys[i] = (uint32_t)(x[i] & 0x7FFF);   /* |x|: drop the sign bit */
    orc_topk_positions(keys, d_in, k, idx_out);
    free(keys);
}

/* ------------------------------------------------------------------------ */
/* Sparse projection GEMV (README "Timing and quality on a GPU"; "What it
 * does": only the weight columns of selected input channels are read).
 * wt is W transposed: wt[i*d_out + o] = W[o][i].  With idx == NULL every
 * channel 0..k-1 is used (the dense GEMV).  Sum in double over the selected
 * channels in list order; y64 (optional) gets the unrounded sums.            */
void orc_sparse_gemv(const uint16_t* wt, int d_in, int d_out, const uint16_t* x,
                     const int32_t* idx, int k, double* y64, uint16_t* y_bf16)
{
    (void)d_in;
    double* acc = (double*)calloc((size_t)d_out, sizeof(double));
    double* xv = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    for (int j = 0; j < k; ++j) xv[j] = orc_bf16_to_double(x[idx ? idx[j] : j]);
#pragma omp parallel for schedule(static)
    for (int o0 = 0; o0 < d_out; o0 += 256) {
        int o1 = o0 + 256 < d_out ? o0 + 256 : d_out;
        for (int j = 0; j < k; ++j) {
            const uint16_t* row = wt + (size_t)(idx ? idx[j] : j) * (size_t)d_out;
            for (int o = o0; o < o1; ++o) acc[o] += orc_bf16_to_double(row[o]) * xv[j];
        }
    }
    for (int o = 0; o < d_out; ++o) {
        if (y64) y64[o] = acc[o];
        if (y_bf16) y_bf16[o] = orc_bf16_from_double(acc[o]);
    }
    free(xv);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Layer glue (not on the pages; the plain Llama reading of "Llama-3.1-8B").
 * RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, in double, rounded to bf16.   */
void orc_rmsnorm(const uint16_t* x, const uint16_t* g, int d, double eps, uint16_t* out)
{
    double ss = 0.0;
    for (int i = 0; i < d; ++i) { double v = orc_bf16_to_double(x[i]); ss += v * v; }
    double inv = 1.0 / sqrt(ss / (double)d + eps);
    for (int i = 0; i < d; ++i)
        out[i] = orc_bf16_from_double(orc_bf16_to_double(x[i]) * inv * orc_bf16_to_double(g[i]));
}

/* Rotary embedding, rotate-half form: within each head of width D the pair
 * (i, i + D/2) turns by angle pos * theta^(-2i/D).  In-place on double data. */
void orc_rope(double* v, int n_heads, int D, int pos, double theta)
{
    int h2 = D / 2;
    for (int hh = 0; hh < n_heads; ++hh) {
        double* r = v + (size_t)hh * D;
        for (int i = 0; i < h2; ++i) {
            double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)D);
            double c = cos(ang), s = sin(ang);
            double a = r[i], b = r[i + h2];
            r[i] = a * c - b * s;
            r[i + h2] = b * c + a * s;
        }
    }
}

/* SwiGLU: out_i = silu(gate_i) * up_i, silu(z) = z / (1 + e^-z), in double. */
void orc_swiglu(const double* gate, const double* up, int n, uint16_t* out)
{
    for (int i = 0; i < n; ++i) {
        double z = gate[i];
        out[i] = orc_bf16_from_double(z / (1.0 + exp(-z)) * up[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* Per-block key summaries (read of the KV branch as query-aware block
 * scoring, in the Quest form the pages list among the paper's ancestors).
 * k is one KV head's keys [n_cap][D]; blocks of 16 tokens aligned at 0.
 * For every block holding at least one of the first n tokens, store per dim
 * (min, max) over the block's tokens below n: out[(b*D + d)*2 + 0] = min,
 * out[(b*D + d)*2 + 1] = max.  Exact (a min/max of bf16 values is bf16).     */
void orc_kv_summary(const uint16_t* k, int n, int D, uint16_t* out)
{
    int nb = (n + 15) / 16;
    for (int b = 0; b < nb; ++b) {
        int t1 = (b + 1) * 16 < n ? (b + 1) * 16 : n;
        for (int d = 0; d < D; ++d) {
            double mn = INFINITY, mx = -INFINITY;
            uint16_t bmn = 0, bmx = 0;
            for (int t = b * 16; t < t1; ++t) {
                uint16_t u = k[(size_t)t * D + d];
                double v = orc_bf16_to_double(u);
                if (v < mn) { mn = v; bmn = u; }
                if (v > mx) { mx = v; bmx = u; }
            }
            out[((size_t)b * D + d) * 2 + 0] = bmn;
            out[((size_t)b * D + d) * 2 + 1] = bmx;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* KV budget (README "What it does in one picture": the kept entries are the
 * first tokens, a share of the older history and the newest tokens; block
 * size 16).  T = min(n, floor(r_kv*n + 1/2)); sinks
 * S' = min(sinks, T); window W' = min(window, T - S'); whole 16-token blocks
 * fill the rest: k_blk = floor((T - S' - W') / 16), capped by the number of
 * candidate blocks, which are the aligned blocks lying wholly in [S', n - W').
 * r_kv >= 1 means the dense list 0..n-1.
 * out[0]=T_sel out[1]=k_blk out[2]=n_cand out[3]=b_lo out[4]=S' out[5]=W'.  */
void orc_kv_budget(int n, double r_kv, int sinks, int window, int* out)
{
    if (r_kv >= 1.0) {
        out[0] = n; out[1] = 0; out[2] = 0; out[3] = 0; out[4] = 0; out[5] = 0;
        return;
    }
    long T = (long)floor(r_kv * (double)n + 0.5);
    if (T > n) T = n;
    if (T < 0) T = 0;
    int sp = sinks < T ? sinks : (int)T;
    int wp = window < (int)T - sp ? window : (int)T - sp;
    int kb = ((int)T - sp - wp) / 16;
    int b_lo = (sp + 15) / 16;
    int b_hi = (n - wp) / 16;
    int nc = b_hi > b_lo ? b_hi - b_lo : 0;
    if (kb > nc) kb = nc;
    out[0] = sp + wp + 16 * kb;
    out[1] = kb;
    out[2] = nc;
    out[3] = b_lo;
    out[4] = sp;
    out[5] = wp;
}

/* Adjacent-pair tree sum in float: v[i] <- v[2i] + v[2i+1] until one value
 * is left.  len must be a power of two.  Destroys v. */
static float orc_pair_tree(float* v, int len)
{
    while (len > 1) {
        for (int i = 0; i < len / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
        len /= 2;
    }
    return v[0];
}

/* Score of one candidate block for one KV head: an upper bound of q_j . k_t
 * over the block's tokens, summed over the G query heads of the group.  Per
 * dim d the group's positive and negative query parts are summed first,
 *   P_d = adjacent-pair tree over j of (q_{j,d} > 0 ? q_{j,d} : 0)
 *   N_d = adjacent-pair tree over j of (q_{j,d} > 0 ? 0 : q_{j,d}),
 * since sum_j max(q kmax, q kmin) = kmax P + kmin N when kmax >= kmin; then
 *   t_d = fmaf(kmax_d, P_d, kmin_d * N_d)
 *   a_p = (t_{4p} + t_{4p+1}) + (t_{4p+2} + t_{4p+3})
 *   s   = adjacent-pair tree over p = 0 .. D/4-1 of a_p
 * all in float, in exactly this order.  q is [G][D] bf16, summ is [D][2]. */
float orc_block_score(const uint16_t* q, const uint16_t* summ, int G, int D)
{
    int P = D / 4;
    float* a = (float*)malloc(sizeof(float) * (size_t)P);
    float* pos = (float*)malloc(sizeof(float) * (size_t)G);
    float* neg = (float*)malloc(sizeof(float) * (size_t)G);
    for (int p = 0; p < P; ++p) {
        float t[4];
        for (int u = 0; u < 4; ++u) {
            int d = 4 * p + u;
            for (int j = 0; j < G; ++j) {
                float qv = (float)orc_bf16_to_double(q[(size_t)j * D + d]);
                pos[j] = qv > 0.0f ? qv : 0.0f;
                neg[j] = qv > 0.0f ? 0.0f : qv;
            }
            float pd = orc_pair_tree(pos, G);
            float nd = orc_pair_tree(neg, G);
            float mn = (float)orc_bf16_to_double(summ[(size_t)d * 2 + 0]);
            float mx = (float)orc_bf16_to_double(summ[(size_t)d * 2 + 1]);
            float lo = mn * nd;
            t[u] = fmaf(mx, pd, lo);
        }
        a[p] = (t[0] + t[1]) + (t[2] + t[3]);
    }
    float s = orc_pair_tree(a, P);
    free(neg);
    free(pos);
    free(a);
    return s;
}

/* Map a float to an unsigned key with the same order (larger float, larger
 * key); -0 and +0 get different keys, -0 below +0. */
static uint32_t orc_float_order_key(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

/* Attention-scored KV selection for every KV head.
 *   q     [H][D] bf16, post-rotary query of the current token
 *   summ  [Hkv][nb_cap][D][2] bf16 (layout of orc_kv_summary per head)
 * For KV head g the query heads g*G .. g*G+G-1 (G = H/Hkv) score each
 * candidate block; the k_blk highest scores are kept (equal scores: lower
 * block first); the list is sinks, kept blocks' tokens and the window, in
 * ascending token order: idx_out [Hkv][T_sel].  scores_out (optional) gets
 * [Hkv][n_cand] in candidate order.  r_kv >= 1 gives 0..n-1 for every head. */
void orc_kv_select(const uint16_t* q, const uint16_t* summ, int nb_cap, int n,
                   int H, int Hkv, int D, double r_kv, int sinks, int window,
                   int32_t* idx_out, float* scores_out)
{
    int bud[6];
    orc_kv_budget(n, r_kv, sinks, window, bud);
    int T_sel = bud[0], kb = bud[1], nc = bud[2], b_lo = bud[3], sp = bud[4], wp = bud[5];
    int G = H / Hkv;
    if (r_kv >= 1.0) {
        for (int g = 0; g < Hkv; ++g)
            for (int t = 0; t < n; ++t) idx_out[(size_t)g * n + t] = t;
        return;
    }
#pragma omp parallel for schedule(static)
    for (int g = 0; g < Hkv; ++g) {
        uint32_t* keys = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(nc > 0 ? nc : 1));
        int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)(kb > 0 ? kb : 1));
        for (int c = 0; c < nc; ++c) {
            int b = b_lo + c;
            float s = orc_block_score(q + (size_t)g * G * D,
                                      summ + ((size_t)g * nb_cap + b) * D * 2, G, D);
            if (scores_out) scores_out[(size_t)g * nc + c] = s;
            keys[c] = orc_float_order_key(s);
        }
        orc_topk_positions(keys, nc, kb, chosen);
        int32_t* out = idx_out + (size_t)g * T_sel;
        int w = 0;
        for (int t = 0; t < sp; ++t) out[w++] = t;
        for (int i = 0; i < kb; ++i)
            for (int u = 0; u < 16; ++u) out[w++] = 16 * (b_lo + chosen[i]) + u;
        for (int t = n - wp; t < n; ++t) out[w++] = t;
        free(chosen);
        free(keys);
    }
}

/* ------------------------------------------------------------------------ */
/* Select-once KV policy in the SnapKV form (README FAQ "How is this different
 * from TEAL and SnapKV?": the KV branch follows SnapKV, selecting once after
 * prefill; README "Timing and quality on a GPU" and "API at a glance": the
 * selection is gathered into one buffer by select_and_compact).  SnapKV
 * scores every cached token by the attention an observation window of the
 * last queries pays it, pooled over neighbouring tokens, and keeps the
 * highest-scored ones.
 *
 * Votes.  The observation queries are q_obs[i][j][:], i = 0..w-1 at
 * position p_i = n - w + i, j = 0..H-1 (post-rotary, bf16).  For KV head g and
 * its query heads j = g*G .. g*G+G-1:
 *   z_{i,j,t} = scale * (q_{i,j} . k_t)              for t <= p_i
 *   A_{i,j,t} = exp(z_{i,j,t} - max_t z) / sum_t exp(z_{i,j,t} - max_t z)
 *   votes[g][t] = sum_i sum_j A_{i,j,t}   (A = 0 for t > p_i),  t = 0..n-1.
 * Everything in double; rows are summed i outer, j inner.                   */
void orc_snapkv_votes(const uint16_t* q_obs, const uint16_t* K, int n_cap, int n, int w, int H, int Hkv,
                      int D, double scale, double* votes)
{
    int G = H / Hkv;
    int rows = w * G;
    /* the keys and queries in double, once */
    double* kd = (double*)malloc(sizeof(double) * (size_t)Hkv * n * D);
    double* qd = (double*)malloc(sizeof(double) * (size_t)w * H * D);
#pragma omp parallel for schedule(static)
    for (long r = 0; r < (long)Hkv * n; ++r) {
        long g = r / n, t = r % n;
        for (int d = 0; d < D; ++d) kd[(size_t)r * D + d] = orc_bf16_to_double(K[((size_t)g * n_cap + t) * D + d]);
    }
    for (long e = 0; e < (long)w * H * D; ++e) qd[e] = orc_bf16_to_double(q_obs[e]);
    double* mrow = (double*)malloc(sizeof(double) * (size_t)Hkv * rows);
    double* lrow = (double*)malloc(sizeof(double) * (size_t)Hkv * rows);
    /* pass 1: per row, the max and the sum over its causal range */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int g = 0; g < Hkv; ++g) {
        for (int r = 0; r < rows; ++r) {
            int i = r / G, j = g * G + r % G;
            long p = (long)n - w + i;
            const double* q = qd + ((size_t)i * H + j) * D;
            double* z = (double*)malloc(sizeof(double) * (size_t)(p + 1));
            double mx = -INFINITY;
            for (long t = 0; t <= p; ++t) {
                const double* k = kd + ((size_t)g * n + t) * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += q[d] * k[d];
                z[t] = acc * scale;
                if (z[t] > mx) mx = z[t];
            }
            double sum = 0.0;
            for (long t = 0; t <= p; ++t) sum += exp(z[t] - mx);
            mrow[(size_t)g * rows + r] = mx;
            lrow[(size_t)g * rows + r] = sum;
            free(z);
        }
    }
    /* pass 2: per token, the normalised weights summed over the rows */
#pragma omp parallel for collapse(2) schedule(static)
    for (int g = 0; g < Hkv; ++g) {
        for (long t = 0; t < n; ++t) {
            const double* k = kd + ((size_t)g * n + t) * D;
            double v = 0.0;
            for (int r = 0; r < rows; ++r) {
                int i = r / G, j = g * G + r % G;
                if (t > (long)n - w + i) continue;
                const double* q = qd + ((size_t)i * H + j) * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += q[d] * k[d];
                v += exp(acc * scale - mrow[(size_t)g * rows + r]) / lrow[(size_t)g * rows + r];
            }
            votes[(size_t)g * n + t] = v;
        }
    }
    free(lrow);
    free(mrow);
    free(qd);
    free(kd);
}

/* Average pooling of one vote vector over neighbouring tokens (SnapKV's
 * clustering step): out_t = (1/ks) * sum_{u = t-ks/2}^{t+ks/2} v_u, with
 * v_u = 0 outside [0, n); ks odd.  Summed in u order, in double.           */
void orc_avg_pool(const double* v, int n, int ks, double* out)
{
    int r = ks / 2;
    for (int t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int u = t - r; u <= t + r; ++u)
            if (u >= 0 && u < n) acc += v[u];
        out[t] = acc / (double)ks;
    }
}

/* Token budget of the select-once policy: T = min(n, floor(r_kv*n + 1/2));
 * sinks S' = min(sinks, T); window W' = min(window, T - S'); the history
 * candidates are tokens [S', n - W'), of which k = T - S' - W' are kept, so
 * T_sel = T.  r_kv >= 1 keeps all n.  out[0]=T_sel out[1]=k out[2]=S'
 * out[3]=W'.                                                                 */
void orc_token_budget(int n, double r_kv, int sinks, int window, int* out)
{
    if (r_kv >= 1.0) { out[0] = n; out[1] = 0; out[2] = 0; out[3] = 0; return; }
    long T = (long)floor(r_kv * (double)n + 0.5);
    if (T > n) T = n;
    if (T < 0) T = 0;
    int sp = sinks < T ? sinks : (int)T;
    int wp = window < (int)T - sp ? window : (int)T - sp;
    out[0] = (int)T;
    out[1] = (int)T - sp - wp;
    out[2] = sp;
    out[3] = wp;
}

static uint32_t orc_float_order_key(float f);

/* Token selection from given float scores [Hkv][n] (one list per KV head):
 * the k highest-scored candidates of [S', n - W') (equal scores: lower token
 * first), with the sinks and the window, ascending: idx_out [Hkv][T_sel].
 * The decision is taken on the float values as given.                      */
void orc_token_select(const float* scores, int n, int Hkv, double r_kv, int sinks, int window, int32_t* idx_out)
{
    int bud[4];
    orc_token_budget(n, r_kv, sinks, window, bud);
    int T_sel = bud[0], k = bud[1], sp = bud[2], wp = bud[3];
    int nc = n - wp - sp;
    for (int g = 0; g < Hkv; ++g) {
        int32_t* out = idx_out + (size_t)g * T_sel;
        if (r_kv >= 1.0) {
            for (int t = 0; t < n; ++t) out[t] = t;
            continue;
        }
        uint32_t* keys = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(nc > 0 ? nc : 1));
        int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
        for (int c = 0; c < nc; ++c) keys[c] = orc_float_order_key(scores[(size_t)g * n + sp + c]);
        orc_topk_positions(keys, nc, k, chosen);
        int w = 0;
        for (int t = 0; t < sp; ++t) out[w++] = t;
        for (int c = 0; c < k; ++c) out[w++] = sp + chosen[c];
        for (int t = n - wp; t < n; ++t) out[w++] = t;
        free(chosen);
        free(keys);
    }
}

/* ------------------------------------------------------------------------ */
/* Split-K decode attention, partial pass (README "Overview": one split-K
 * attention kernel reads the cache in every mode).  For query head j (KV
 * head g = j / G) and split s covering list positions [s*c, min(n_sel,
 * (s+1)*c)), c = ceil(n_sel / S):
 *   z_t = scale * (q_j . k_t),  m = max z,  l = sum e^(z - m),
 *   o = sum e^(z - m) v_t   (unnormalised; m in natural-log units).
 * An empty split gives (-inf, 0, 0).  idx == NULL reads tokens 0..n_sel-1.
 * K and V are [Hkv][n_cap][D]; idx is [Hkv][n_sel]; m, l are [H][S]; o is
 * [H][S][D].  Everything in double.                                         */
void orc_attn_partial(const uint16_t* q, const uint16_t* K, const uint16_t* V, int n_cap,
                      const int32_t* idx, int n_sel, int H, int Hkv, int D, int S,
                      double scale, double* m, double* l, double* o)
{
    int G = H / Hkv;
    long c = S > 0 ? ((long)n_sel + S - 1) / S : 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int j = 0; j < H; ++j) {
        for (int s = 0; s < S; ++s) {
            int g = j / G;
            double qd[512];
            for (int d = 0; d < D; ++d) qd[d] = orc_bf16_to_double(q[(size_t)j * D + d]);
            long lo = (long)s * c, hi = lo + c < n_sel ? lo + c : n_sel;
            double* oo = o + ((size_t)j * S + s) * D;
            for (int d = 0; d < D; ++d) oo[d] = 0.0;
            if (lo >= hi) {
                m[(size_t)j * S + s] = -INFINITY;
                l[(size_t)j * S + s] = 0.0;
                continue;
            }
            double* z = (double*)malloc(sizeof(double) * (size_t)(hi - lo));
            double mx = -INFINITY;
            for (long p = lo; p < hi; ++p) {
                long t = idx ? idx[(size_t)g * n_sel + p] : p;
                const uint16_t* kr = K + ((size_t)g * n_cap + t) * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += qd[d] * orc_bf16_to_double(kr[d]);
                z[p - lo] = acc * scale;
                if (z[p - lo] > mx) mx = z[p - lo];
            }
            double sum = 0.0;
            for (long p = lo; p < hi; ++p) {
                long t = idx ? idx[(size_t)g * n_sel + p] : p;
                const uint16_t* vr = V + ((size_t)g * n_cap + t) * D;
                double e = exp(z[p - lo] - mx);
                sum += e;
                for (int d = 0; d < D; ++d) oo[d] += e * orc_bf16_to_double(vr[d]);
            }
            m[(size_t)j * S + s] = mx;
            l[(size_t)j * S + s] = sum;
            free(z);
        }
    }
}

/* Merge of the split partials: M = max_s m_s; out = sum_s o_s e^(m_s - M) /
 * sum_s l_s e^(m_s - M).  All splits empty gives 0.  out64 optional. */
void orc_attn_reduce(const double* m, const double* l, const double* o, int H, int S, int D,
                     double* out64, uint16_t* out)
{
    for (int j = 0; j < H; ++j) {
        double M = -INFINITY;
        for (int s = 0; s < S; ++s) if (m[(size_t)j * S + s] > M) M = m[(size_t)j * S + s];
        double den = 0.0;
        double num[512];
        for (int d = 0; d < D; ++d) num[d] = 0.0;
        if (M != -INFINITY) {
            for (int s = 0; s < S; ++s) {
                double ms = m[(size_t)j * S + s];
                if (ms == -INFINITY) continue;
                double w = exp(ms - M);
                den += w * l[(size_t)j * S + s];
                for (int d = 0; d < D; ++d) num[d] += w * o[((size_t)j * S + s) * D + d];
            }
        }
        for (int d = 0; d < D; ++d) {
            double v = den > 0.0 ? num[d] / den : 0.0;
            if (out64) out64[(size_t)j * D + d] = v;
            if (out) out[(size_t)j * D + d] = orc_bf16_from_double(v);
        }
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
