/*
 * CPU oracle for the sigmoid-routed mixture-of-experts feed-forward layer (GLM-5 / GLM-4.7-Flash).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
 * may load or call this library. The product path (the HIP kernels behind include/moe.h) never does, and
 * the two share no code: this file has its own bf16 decode, its own loops and libm's exp.
 *
 * What it computes is the plain definition, written out per token, with every sum in double precision in
 * a fixed ascending order and one rounding to fp32 per stored value:
 *
 *   z = x W_r                          router logits       (open-model-atlas, GLM-5 "MoE transformer block",
 *   s = sigmoid(z)                     scores               "All 43 steps", the mixture-of-experts equations;
 *   sel = top_k(s + b)                 biased choice        nnterp encyclopedia glm_moe_dsa / glm4_moe_lite,
 *   G_i = scale s_i / sum_sel s_j      gates                "The mixture: sigmoid scores, a selection bias,
 *   E_i = (silu(x W1_i) * (x W3_i)) W2_i   SwiGLU expert    renormalized weights")
 *   y_routed = sum_sel G_i E_i
 *   y_shared = (silu(x Ws1) * (x Ws3)) Ws2
 *   out = y_routed + y_shared
 *
 * and the steps on either side of the mixture in a GLM-5 block, plus the dense MLP of the dense-first
 * blocks (same pages: "All 43 steps" x_ffn = RMSNorm(x'_n) and x_{n+1} = x'_n + delta_ffn; the nnterp
 * module trees' post_attention_layernorm with eps 1e-5 and the dense gate/up/down MLP):
 *
 *   x_ffn = RMSNorm(x') = gamma * x' / sqrt(mean(x'^2) + eps)   rounded once to bf16
 *   x_next = x' + out(x_ffn)
 *   y_dense = (silu(x W1) * (x W3)) W2
 *
 * Weights are stored [out, in] like nn.Linear, so "x W1" is sum_h x[h] W1[n, h]. W1 is the gate (it gets
 * the sigmoid-weighted linear unit), W3 the up projection, W2 the down projection.
 *
 * Readings where the pages are silent (each one is listed with its reason in the design notes):
 *  - top-k ties go to the lower expert index; the k slots are ordered by descending s + b, then index;
 *  - z, s and c = s + b are fp32 values; z is the fp32 rounding of the exact (double) dot product;
 *  - b is fp32;
 *  - a zero gate denominator (never reached by these workloads) gives zero gates;
 *  - no intermediate of the expert MLPs is rounded; the output is fp32;
 *  - RMSNorm is the textbook definition (the pages name the module and its eps, not its formula), in
 *    double with the product taken as (x * rstd) * gamma, and its output is rounded once to bf16, the
 *    dtype the mixture takes.
 *
 * Parity status: every function here is pinned by a CPU test (brute-force top-k, crafted ties, the
 * sigmoid's closed forms, gate sums, the bias-only-moves-the-choice property, k = E dense mixture,
 * E = 1 dense SwiGLU MLP, linearity, token independence, the stable-sort permutation, the skewed
 * workload's closed forms and the pages' GLM-5 parameter count; the bf16 rounding against fp32 rounding
 * and crafted ties, RMSNorm's scale invariance and one-hot / constant rows, the block's residual wiring,
 * and the dense MLP against numpy matrix products).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 storage -> double: bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t v) {
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* s = sigma(z) = 1 / (1 + e^-z), evaluated in double and rounded once to fp32. */
float oracle_sigmoid(float z) { return (float)(1.0 / (1.0 + exp(-(double)z))); }

/* double -> bf16 storage, round to nearest, ties to even, straight from the double (no detour through
 * fp32, which could round twice). |v| = m 2^e with m in [0.5, 1); a normal bf16 keeps 8 significant bits,
 * so q = m 2^8 is split into its integer part (the kept bits) and the exact remainder. Below 2^-126 the
 * quantum is the subnormal step 2^-133. */
uint16_t oracle_round_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) return 0x7FC0u;
    if (isinf(a)) return sign | 0x7F80u;
    if (a == 0.0) return sign;
    int e;
    double m = frexp(a, &e); /* a = m 2^e */
    int biased = e - 1 + 127;
    double q = biased >= 1 ? ldexp(m, 8) : ldexp(a, 133);
    double whole = floor(q);
    double rem = q - whole;
    uint32_t n = (uint32_t)whole;
    if (rem > 0.5 || (rem == 0.5 && (n & 1u))) n++;
    if (biased < 1) return sign | (uint16_t)n; /* n == 128 is the smallest normal, which the same bits encode */
    if (n == 256u) {
        n = 128u;
        biased++;
    }
    if (biased >= 255) return sign | 0x7F80u;
    return sign | (uint16_t)((uint32_t)biased << 7) | (uint16_t)(n - 128u);
}

/* RMSNorm of one row: rstd = 1 / sqrt(sum_h x[h]^2 / H + eps) in double (h ascending), then
 * out[h] = bf16((x[h] * rstd) * gamma[h]). */
static void rmsnorm_row(int H, double eps, const uint16_t* xrow, const uint16_t* gamma, uint16_t* out) {
    double ss = 0.0;
    for (int h = 0; h < H; ++h) {
        double xv = oracle_bf16_to_double(xrow[h]);
        ss += xv * xv;
    }
    double rstd = 1.0 / sqrt(ss / (double)H + eps);
    for (int h = 0; h < H; ++h)
        out[h] = oracle_round_bf16(oracle_bf16_to_double(xrow[h]) * rstd * oracle_bf16_to_double(gamma[h]));
}

/* One token's router logits: z[e] = fp32(sum_h x[h] W_r[e, h]), h ascending. */
static void token_logits(int H, int E, const uint16_t* xrow, const uint16_t* wr, float* z) {
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        const uint16_t* w = wr + (size_t)e * (size_t)H;
        for (int h = 0; h < H; ++h) acc += oracle_bf16_to_double(xrow[h]) * oracle_bf16_to_double(w[h]);
        z[e] = (float)acc;
    }
}

/*
 * One token's routing. Fills ids[k] (slot order: descending c, then ascending index), the double gates
 * gd[k], and returns the gap between the k-th and (k+1)-th biased scores (+inf when k == E).
 * `s` and `c` are caller scratch of E floats; `taken` E chars.
 */
static double token_route(int E, int k, float scale, const float* z, const float* b, float* s, float* c,
                          char* taken, int32_t* ids, double* gd) {
    for (int e = 0; e < E; ++e) {
        s[e] = oracle_sigmoid(z[e]);
        c[e] = s[e] + b[e]; /* fp32 add, round to nearest even */
        taken[e] = 0;
    }
    /* Selection: k passes, each takes the largest c among the untaken experts; a strict comparison while
     * scanning upward keeps the lower index among equal scores. */
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || c[e] > c[best])) best = e;
        taken[best] = 1;
        ids[j] = best;
    }
    double gap = INFINITY;
    if (k < E) {
        int next = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (next < 0 || c[e] > c[next])) next = e;
        gap = (double)c[ids[k - 1]] - (double)c[next];
    }
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += (double)s[ids[j]];
    for (int j = 0; j < k; ++j) gd[j] = den > 0.0 ? (double)scale * (double)s[ids[j]] / den : 0.0;
    return gap;
}

/* SwiGLU MLP of one token, all in double: g = x W1, u = x W3, h = g sigma(g) u, y = h W2.
 * W1, W3: [Iw, H]; W2: [H, Iw]; y: [H]; hbuf: [Iw] scratch. */
static void swiglu_mlp(int H, int Iw, const uint16_t* xrow, const uint16_t* W1, const uint16_t* W3,
                       const uint16_t* W2, double* y, double* hbuf) {
    for (int n = 0; n < Iw; ++n) {
        const uint16_t* r1 = W1 + (size_t)n * (size_t)H;
        const uint16_t* r3 = W3 + (size_t)n * (size_t)H;
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            double xv = oracle_bf16_to_double(xrow[h]);
            g += xv * oracle_bf16_to_double(r1[h]);
            u += xv * oracle_bf16_to_double(r3[h]);
        }
        double a = g / (1.0 + exp(-g));
        hbuf[n] = a * u;
    }
    for (int m = 0; m < H; ++m) {
        const uint16_t* r2 = W2 + (size_t)m * (size_t)Iw;
        double acc = 0.0;
        for (int n = 0; n < Iw; ++n) acc += hbuf[n] * oracle_bf16_to_double(r2[n]);
        y[m] = acc;
    }
}

/*
 * Routing of the tokens listed in rows[0..nrows) (rows == NULL: tokens 0..nrows-1) of x [*, H].
 * Outputs are indexed by list position: ids/gates [nrows, k], logits [nrows, E] (nullable),
 * gap [nrows] (nullable). Returns 0, or -1 on bad arguments or allocation failure.
 */
int oracle_route(int H, int E, int k, float scale, const uint16_t* x, const uint16_t* wr, const float* b,
                 const int32_t* rows, int nrows, int32_t* ids, float* gates, float* logits, double* gap) {
    if (H <= 0 || E <= 0 || k < 1 || k > E || nrows < 0) return -1;
    float* z = (float*)malloc(sizeof(float) * (size_t)E * 3);
    char* taken = (char*)malloc((size_t)E);
    double* gd = (double*)malloc(sizeof(double) * (size_t)k);
    if (!z || !taken || !gd) { free(z); free(taken); free(gd); return -1; }
    float* s = z + E;
    float* c = z + 2 * E;
    for (int r = 0; r < nrows; ++r) {
        size_t t = rows ? (size_t)rows[r] : (size_t)r;
        token_logits(H, E, x + t * (size_t)H, wr, z);
        double g = token_route(E, k, scale, z, b, s, c, taken, ids + (size_t)r * k, gd);
        for (int j = 0; j < k; ++j) gates[(size_t)r * k + j] = (float)gd[j];
        if (logits) memcpy(logits + (size_t)r * E, z, sizeof(float) * (size_t)E);
        if (gap) gap[r] = g;
    }
    free(z); free(taken); free(gd);
    return 0;
}

/*
 * The whole layer for the tokens listed in rows[0..nrows) (rows == NULL: tokens 0..nrows-1).
 * x [*, H]; wr [E, H]; b [E]; w1, w3 [E, I, H]; w2 [E, H, I]; ws1, ws3 [Is, H]; ws2 [H, Is] (Is == 0:
 * no shared expert, ws* unused). Outputs by list position: out [nrows, H] = fp32(routed + shared);
 * optional ids/gates [nrows, k], gap [nrows], routed/shared [nrows, H] (each rounded to fp32 on its own).
 * Returns 0, or -1 on bad arguments or allocation failure.
 */
/* Per-call scratch of the mixture on one token. */
typedef struct {
    float *z, *s, *c;
    char* taken;
    double *gd, *y, *routed, *shared, *hbuf;
    int32_t* sel;
} MixScratch;

static void mix_free(MixScratch* m) {
    free(m->z); free(m->taken); free(m->gd); free(m->sel); free(m->y); free(m->routed); free(m->shared);
    free(m->hbuf);
}

static int mix_alloc(MixScratch* m, int H, int E, int k, int wmax) {
    m->z = (float*)malloc(sizeof(float) * (size_t)E * 3);
    m->taken = (char*)malloc((size_t)E);
    m->gd = (double*)malloc(sizeof(double) * (size_t)k);
    m->sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    m->y = (double*)malloc(sizeof(double) * (size_t)H);
    m->routed = (double*)malloc(sizeof(double) * (size_t)H);
    m->shared = (double*)malloc(sizeof(double) * (size_t)H);
    m->hbuf = (double*)malloc(sizeof(double) * (size_t)wmax);
    if (!m->z || !m->taken || !m->gd || !m->sel || !m->y || !m->routed || !m->shared || !m->hbuf) {
        mix_free(m);
        return -1;
    }
    m->s = m->z + E;
    m->c = m->z + 2 * E;
    return 0;
}

/* The mixture on one token x (a bf16 row): routing into m->sel / m->gd, the gated routed sum into
 * m->routed and the shared expert into m->shared (both double, unrounded). Returns the selection gap. */
static double token_mixture(int H, int E, int k, int I, int Is, float scale, const uint16_t* xrow,
                            const uint16_t* wr, const float* b, const uint16_t* w1, const uint16_t* w3,
                            const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2,
                            MixScratch* m) {
    const size_t expert_in = (size_t)I * (size_t)H;
    token_logits(H, E, xrow, wr, m->z);
    double g = token_route(E, k, scale, m->z, b, m->s, m->c, m->taken, m->sel, m->gd);
    for (int i = 0; i < H; ++i) m->routed[i] = 0.0;
    for (int j = 0; j < k; ++j) {
        size_t e = (size_t)m->sel[j];
        swiglu_mlp(H, I, xrow, w1 + e * expert_in, w3 + e * expert_in, w2 + e * expert_in, m->y, m->hbuf);
        for (int i = 0; i < H; ++i) m->routed[i] += m->gd[j] * m->y[i];
    }
    if (Is > 0) swiglu_mlp(H, Is, xrow, ws1, ws3, ws2, m->shared, m->hbuf);
    else for (int i = 0; i < H; ++i) m->shared[i] = 0.0;
    return g;
}

static void store_routing(const MixScratch* m, int k, int r, double g, int32_t* ids, float* gates, double* gap) {
    if (ids) memcpy(ids + (size_t)r * k, m->sel, sizeof(int32_t) * (size_t)k);
    if (gates) for (int j = 0; j < k; ++j) gates[(size_t)r * k + j] = (float)m->gd[j];
    if (gap) gap[r] = g;
}

int oracle_forward(int H, int E, int k, int I, int Is, float scale, const uint16_t* x, const uint16_t* wr,
                   const float* b, const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                   const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2, const int32_t* rows, int nrows,
                   float* out, int32_t* ids, float* gates, double* gap, float* routed_out, float* shared_out) {
    if (H <= 0 || E <= 0 || k < 1 || k > E || I <= 0 || Is < 0 || nrows < 0) return -1;
    MixScratch m;
    if (mix_alloc(&m, H, E, k, I > Is ? I : Is) != 0) return -1;
    for (int r = 0; r < nrows; ++r) {
        size_t t = rows ? (size_t)rows[r] : (size_t)r;
        double g = token_mixture(H, E, k, I, Is, scale, x + t * (size_t)H, wr, b, w1, w3, w2, ws1, ws3, ws2, &m);
        for (int i = 0; i < H; ++i) out[(size_t)r * H + i] = (float)(m.routed[i] + m.shared[i]);
        if (routed_out) for (int i = 0; i < H; ++i) routed_out[(size_t)r * H + i] = (float)m.routed[i];
        if (shared_out) for (int i = 0; i < H; ++i) shared_out[(size_t)r * H + i] = (float)m.shared[i];
        store_routing(&m, k, r, g, ids, gates, gap);
    }
    mix_free(&m);
    return 0;
}

/*
 * RMSNorm of the listed rows of x [*, H] with weight gamma [H]: out [nrows, H] bf16 by list position.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_rmsnorm(int H, double eps, const uint16_t* x, const uint16_t* gamma, const int32_t* rows, int nrows,
                   uint16_t* out) {
    if (H <= 0 || nrows < 0 || !(eps >= 0.0)) return -1;
    for (int r = 0; r < nrows; ++r) {
        size_t t = rows ? (size_t)rows[r] : (size_t)r;
        rmsnorm_row(H, eps, x + t * (size_t)H, gamma, out + (size_t)r * H);
    }
    return 0;
}

/*
 * The mixture half of a GLM-5 block on the residual stream x' [*, H]: x_ffn = RMSNorm(x') (bf16), the
 * mixture on x_ffn, and the residual add out = fp32(x' + routed + shared). Outputs by list position:
 * out [nrows, H]; optional x_norm [nrows, H] bf16, ids/gates [nrows, k], gap [nrows].
 */
int oracle_block_forward(int H, int E, int k, int I, int Is, float scale, double eps, const uint16_t* resid,
                         const uint16_t* gamma, const uint16_t* wr, const float* b, const uint16_t* w1,
                         const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3,
                         const uint16_t* ws2, const int32_t* rows, int nrows, float* out, uint16_t* x_norm,
                         int32_t* ids, float* gates, double* gap) {
    if (H <= 0 || E <= 0 || k < 1 || k > E || I <= 0 || Is < 0 || nrows < 0 || !(eps >= 0.0)) return -1;
    MixScratch m;
    if (mix_alloc(&m, H, E, k, I > Is ? I : Is) != 0) return -1;
    uint16_t* xn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
    if (!xn) {
        mix_free(&m);
        return -1;
    }
    for (int r = 0; r < nrows; ++r) {
        size_t t = rows ? (size_t)rows[r] : (size_t)r;
        const uint16_t* xr = resid + t * (size_t)H;
        rmsnorm_row(H, eps, xr, gamma, xn);
        double g = token_mixture(H, E, k, I, Is, scale, xn, wr, b, w1, w3, w2, ws1, ws3, ws2, &m);
        for (int i = 0; i < H; ++i)
            out[(size_t)r * H + i] = (float)(oracle_bf16_to_double(xr[i]) + m.routed[i] + m.shared[i]);
        if (x_norm) memcpy(x_norm + (size_t)r * H, xn, sizeof(uint16_t) * (size_t)H);
        store_routing(&m, k, r, g, ids, gates, gap);
    }
    free(xn);
    mix_free(&m);
    return 0;
}

/*
 * Dense SwiGLU MLP of the listed rows of x [*, H]: out [nrows, H] = fp32((silu(x W1) * (x W3)) W2), with
 * W1, W3 [Id, H] and W2 [H, Id]. Returns 0, or -1 on bad arguments or allocation failure.
 */
int oracle_dense_mlp(int H, int Id, const uint16_t* x, const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                     const int32_t* rows, int nrows, float* out) {
    if (H <= 0 || Id <= 0 || nrows < 0) return -1;
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* hbuf = (double*)malloc(sizeof(double) * (size_t)Id);
    if (!y || !hbuf) {
        free(y);
        free(hbuf);
        return -1;
    }
    for (int r = 0; r < nrows; ++r) {
        size_t t = rows ? (size_t)rows[r] : (size_t)r;
        swiglu_mlp(H, Id, x + t * (size_t)H, w1, w3, w2, y, hbuf);
        for (int i = 0; i < H; ++i) out[(size_t)r * H + i] = (float)y[i];
    }
    free(y);
    free(hbuf);
    return 0;
}

/*
 * The layer with the routing given instead of computed: slot j of token t goes to expert ids[t, j] with
 * gate gates[t, j], exactly as written (no renormalisation). This is the pages' ablation: zeroing the
 * gate of every slot that chose an expert leaves the other slots' gates as they were (nnterp
 * encyclopedia glm_moe_dsa, "The mixture", the ablation example). Gates are widened to double.
 * ids and gates are [*, k] indexed by token (not by list position); out is [nrows, H] by list position.
 */
int oracle_forward_routed(int H, int E, int k, int I, int Is, const uint16_t* x, const int32_t* ids,
                          const float* gates, const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                          const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2, const int32_t* rows,
                          int nrows, float* out) {
    if (H <= 0 || E <= 0 || k < 1 || I <= 0 || Is < 0 || nrows < 0) return -1;
    int wmax = I > Is ? I : Is;
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    double* shared = (double*)malloc(sizeof(double) * (size_t)H);
    double* hbuf = (double*)malloc(sizeof(double) * (size_t)wmax);
    if (!y || !acc || !shared || !hbuf) { free(y); free(acc); free(shared); free(hbuf); return -1; }
    const size_t expert_in = (size_t)I * (size_t)H;
    for (int r = 0; r < nrows; ++r) {
        size_t t = rows ? (size_t)rows[r] : (size_t)r;
        const uint16_t* xrow = x + t * (size_t)H;
        for (int m = 0; m < H; ++m) acc[m] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[t * (size_t)k + j];
            if (e < 0 || e >= E) { free(y); free(acc); free(shared); free(hbuf); return -1; }
            swiglu_mlp(H, I, xrow, w1 + (size_t)e * expert_in, w3 + (size_t)e * expert_in,
                       w2 + (size_t)e * expert_in, y, hbuf);
            double gj = (double)gates[t * (size_t)k + j];
            for (int m = 0; m < H; ++m) acc[m] += gj * y[m];
        }
        if (Is > 0) swiglu_mlp(H, Is, xrow, ws1, ws3, ws2, shared, hbuf);
        else for (int m = 0; m < H; ++m) shared[m] = 0.0;
        for (int m = 0; m < H; ++m) out[(size_t)r * H + m] = (float)(acc[m] + shared[m]);
    }
    free(y); free(acc); free(shared); free(hbuf);
    return 0;
}

/*
 * Permutation of the T*k routing slots into expert-contiguous rows: a stable counting sort by expert.
 * counts[e] = number of slots routed to e; offsets = exclusive prefix sum (offsets[E] = T*k); rows of
 * expert e are offsets[e] .. offsets[e+1]-1 in ascending token order. row_token[r] = the token of row r;
 * slot_row[t*k + j] = the row that slot j of token t went to. Returns 0, or -1 on an id out of range.
 */
int oracle_permute(int T, int E, int k, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* row_token, int32_t* slot_row) {
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (size_t i = 0; i < (size_t)T * (size_t)k; ++i) {
        if (ids[i] < 0 || ids[i] >= E) return -1;
        counts[ids[i]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return -1;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            int32_t r = offsets[e] + fill[e]++;
            row_token[r] = t;
            slot_row[(size_t)t * k + j] = r;
        }
    free(fill);
    return 0;
}

/* Element count of one MoE block's parameters as this layer takes them: routed W1, W3, W2 (E of each,
 * I x H), shared Ws1, Ws3, Ws2 (Is x H), router W_r (E x H) and the selection bias (E). */
uint64_t oracle_param_count(uint64_t H, uint64_t E, uint64_t I, uint64_t Is) {
    return 3 * E * I * H + 3 * Is * H + E * H + E;
}
