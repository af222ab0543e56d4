/*
 * moe_oracle.c — plain CPU oracle of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this code; the product path never does.  It shares
 * no code, header, table or constant generator with the GPU library: it is
 * written from the pages and the slot-format / routing-contract text alone.
 *
 * What it computes (sources cited by page title and section):
 *  - Routing: softmax over the E router logits and top-k ("RFC: stream MoE
 *    experts from disk in from_pretrained", Motivation: a token uses 10 of 512
 *    experts; only its top-k experts are read), with weights renormalised over
 *    the chosen k.  The decision is taken in fp32, the precision the GPU kernel
 *    takes it in, with the routing contract's own exp (Cody-Waite reduction and
 *    a Taylor polynomial) and summation order, so ids and weights are comparable
 *    bit for bit.
 *  - Cache-aware substitution (BigMoeOnEdge commit message adding it, after
 *    Skliar et al.): each cached expert's score gains L x (max - min of the
 *    token's scores) and the k winners are picked again from the adjusted
 *    scores; k experts still run.
 *  - Sort by expert and passes of at most 64 hit experts ("POC: Experts
 *    offload", commit messages: the sorted prefill handles the hit experts in
 *    batches of 64; RFC, How the prototype works, Prefill).
 *  - Router logits for the lookahead guesses ("RFC ...", How the prototype
 *    works, Reads: the two following layers' routers are applied to the present
 *    hidden state to predict their experts): logits[m][t][e] = sum_i x[t][i] *
 *    Wr_m[e][i] in fp64 over the bf16 values, a plain linear map per layer.
 *  - The layer ("RFC ...", How the prototype works: experts are gated,
 *    concatenated, untransposed and without bias, run on the slot pool through a
 *    map from expert id to slot for each layer; quantized experts in a
 *    group-wise affine format, each expert a single unbroken row):
 *        out[t] = sum_j w[t,j] * Wd_e (silu(Wg_e x_t) * (Wu_e x_t)),  e = ids[t,j]
 *    written out directly in fp64 with plain loops.  Dequantization s*q + z is
 *    exact in fp64.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC -lm.
 * -ffp-contract=off keeps every fp32 multiply and add of the routing separate
 * unless fmaf() is written.  OpenMP only splits independent tokens across
 * threads; each output value is computed by one thread in a fixed order.
 *
 * Return codes: 0 ok, 1 invalid argument, 2 routed expert not resident,
 * 3 slot out of range, 4 non-finite logit, 5 expert id out of range.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_INVALID 1
#define OR_NOT_RESIDENT 2
#define OR_BAD_SLOT 3
#define OR_NONFINITE 4
#define OR_BAD_ID 5

/* ------------------------------------------------------------------------- */
/* exp for the routing contract: e^x = 2^n * e^r, x = n*ln2 + r, |r| <= ln2/2  */
/* (Cody & Waite argument reduction, ln2 split in a high and a low part), e^r  */
/* by its Taylor series to degree 7 evaluated with Horner's rule.              */
/* ------------------------------------------------------------------------- */
static float bits_to_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float oracle_exp_c(float x)
{
    if (x < -86.0f) return 0.0f;
    const float log2e = 1.44269502f;
    const float ln2_hi = bits_to_float(0x3f317218u);
    const float ln2_lo = bits_to_float(0xb102e308u);
    float n = rintf(x * log2e);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    /* Taylor coefficients 1/k!, k = 7 .. 0, as fp32 */
    const float c7 = (float)(1.0 / 5040.0);
    const float c6 = (float)(1.0 / 720.0);
    const float c5 = (float)(1.0 / 120.0);
    const float c4 = (float)(1.0 / 24.0);
    const float c3 = (float)(1.0 / 6.0);
    float p = c7;
    p = fmaf(p, r, c6);
    p = fmaf(p, r, c5);
    p = fmaf(p, r, c4);
    p = fmaf(p, r, c3);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int ni = (int)n; /* in [-125, 0] for x in [-86, 0] */
    float two_n = bits_to_float((uint32_t)(ni + 127) << 23);
    return p * two_n;
}

/* Softmax probabilities of one token (fp32, the contract's summation order). */
static int softmax_row(const float* l, int E, float* p)
{
    float m = l[0];
    for (int i = 0; i < E; i++) {
        if (!isfinite(l[i])) return OR_NONFINITE;
        if (l[i] > m) m = l[i];
    }
    for (int i = 0; i < E; i++) p[i] = oracle_exp_c(l[i] - m);
    float S[64];
    for (int lane = 0; lane < 64; lane++) {
        float s = 0.0f;
        for (int i = lane; i < E; i += 64) s = s + p[i];
        S[lane] = s;
    }
    for (int off = 32; off >= 1; off /= 2)
        for (int lane = 0; lane < off; lane++) S[lane] = S[lane] + S[lane + off];
    float Z = S[0];
    for (int i = 0; i < E; i++) p[i] = p[i] / Z;
    return OR_OK;
}

int oracle_softmax(const float* logits, int T, int E, float* p)
{
    if (T < 0 || E < 1 || E > 1024) return OR_INVALID;
    for (int t = 0; t < T; t++) {
        int rc = softmax_row(logits + (size_t)t * E, E, p + (size_t)t * E);
        if (rc) return rc;
    }
    return OR_OK;
}

/*
 * Route T tokens.  mode 0: plain softmax top-k.  mode 1: cache-aware
 * substitution with strength L, resident = slot_table[e] >= 0.
 * ids/w: [T, k]; p_out (may be NULL): [T, E] probabilities.
 */
int oracle_route(const float* logits, int T, int E, int k, int mode, float L,
                 const int32_t* slot_table, int32_t* ids, float* w, float* p_out)
{
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 32) return OR_INVALID;
    if (mode != 0 && mode != 1) return OR_INVALID;
    if (mode == 1 && !slot_table) return OR_INVALID;
    float* p = (float*)malloc(sizeof(float) * (size_t)E);
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    int rc = OR_OK;
    for (int t = 0; t < T && rc == OR_OK; t++) {
        rc = softmax_row(logits + (size_t)t * E, E, p);
        if (rc) break;
        if (p_out) memcpy(p_out + (size_t)t * E, p, sizeof(float) * (size_t)E);
        /* selection key */
        if (mode == 0) {
            for (int i = 0; i < E; i++) key[i] = p[i];
        } else {
            float pmax = p[0], pmin = p[0];
            for (int i = 1; i < E; i++) {
                if (p[i] > pmax) pmax = p[i];
                if (p[i] < pmin) pmin = p[i];
            }
            float range = pmax - pmin;
            float c = L * range;
            for (int i = 0; i < E; i++) key[i] = (slot_table[i] >= 0) ? p[i] + c : p[i];
        }
        /* top-k by repeated argmax: larger key first, ties to the smaller id */
        memset(taken, 0, (size_t)E);
        int32_t* id_row = ids + (size_t)t * k;
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int i = 0; i < E; i++) {
                if (taken[i]) continue;
                if (best < 0 || key[i] > key[best]) best = i;
            }
            taken[best] = 1;
            id_row[j] = best;
        }
        /* renormalised weights from the unbiased probabilities */
        float s = 0.0f;
        for (int j = 0; j < k; j++) s = s + p[id_row[j]];
        for (int j = 0; j < k; j++) w[(size_t)t * k + j] = p[id_row[j]] / s;
    }
    free(p);
    free(key);
    free(taken);
    return rc;
}

/*
 * Stable counting sort of pair ids p = t*k + j by expert, and the pass table
 * (hit experts ascending, in passes of at most P).
 * pass_table: [0] n_hit, [1] n_passes, [2..2+E) hit ids then -1,
 *             [2+E .. 2+E+ceil(E/P)+1) pass starts (unused = n_hit).
 */
int oracle_sort(const int32_t* ids, int T, int k, int E, int P,
                int32_t* offsets, int32_t* sorted_pairs, int32_t* pass_table)
{
    if (T < 0 || k < 1 || E < 1 || P < 1) return OR_INVALID;
    int64_t n = (int64_t)T * k;
    for (int64_t q = 0; q < n; q++)
        if (ids[q] < 0 || ids[q] >= E) return OR_BAD_ID;
    /* counts, exclusive prefix sums */
    for (int e = 0; e <= E; e++) offsets[e] = 0;
    for (int64_t q = 0; q < n; q++) offsets[ids[q] + 1]++;
    for (int e = 0; e < E; e++) offsets[e + 1] += offsets[e];
    /* stable placement: visit pairs in ascending id */
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; e++) cursor[e] = offsets[e];
    for (int64_t q = 0; q < n; q++) sorted_pairs[cursor[ids[q]]++] = (int32_t)q;
    free(cursor);
    /* pass table */
    int n_pass_max = (E + P - 1) / P;
    int n_hit = 0;
    for (int e = 0; e < E; e++) pass_table[2 + e] = -1;
    for (int e = 0; e < E; e++)
        if (offsets[e + 1] > offsets[e]) pass_table[2 + n_hit++] = e;
    int n_pass = (n_hit + P - 1) / P;
    pass_table[0] = n_hit;
    pass_table[1] = n_pass;
    for (int q = 0; q <= n_pass_max; q++) {
        int start = q * P;
        pass_table[2 + E + q] = start < n_hit ? start : n_hit;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Slot format                                                                */
/* ------------------------------------------------------------------------- */
static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

/* offs[0..4] = gate_up codes, gate_up scale/bias, down codes, down scale/bias,
 * slot bytes.  Blocks start at multiples of 256 bytes.  Width 16 means
 * unquantized bf16 weights ("RFC ...", How the prototype works, Cache: BF16
 * experts run from the same pool): the values themselves in row order, and an
 * empty scale/bias block. */
static int width_ok(int b) { return b == 3 || b == 4 || b == 6 || b == 8 || b == 16; }

int oracle_layout(int H, int I, int bits_gu, int bits_d, int64_t* offs)
{
    if (H <= 0 || I <= 0 || H % 64 || I % 64) return OR_INVALID;
    if (!width_ok(bits_gu) || !width_ok(bits_d)) return OR_INVALID;
    int64_t gu_codes = (int64_t)2 * I * H * bits_gu / 8;
    int64_t gu_sb = bits_gu == 16 ? 0 : (int64_t)2 * I * (H / 64) * 4;
    int64_t d_codes = (int64_t)H * I * bits_d / 8;
    int64_t d_sb = bits_d == 16 ? 0 : (int64_t)H * (I / 64) * 4;
    offs[0] = 0;
    offs[1] = round_up(offs[0] + gu_codes, 256);
    offs[2] = round_up(offs[1] + gu_sb, 256);
    offs[3] = round_up(offs[2] + d_codes, 256);
    offs[4] = round_up(offs[3] + d_sb, 256);
    return OR_OK;
}

/* Code of column c in a code row of `bits`-bit values: the bits [bits*i,
 * bits*i + bits) of pack unit c/32 read as a little-endian bit string. */
uint32_t oracle_code(const uint8_t* row, int bits, int c)
{
    const uint8_t* unit = row + (size_t)(c / 32) * 4 * (size_t)bits;
    int first = bits * (c % 32);
    uint32_t q = 0;
    for (int b = 0; b < bits; b++) {
        int bit = first + b;
        q |= (uint32_t)((unit[bit / 8] >> (bit % 8)) & 1u) << b;
    }
    return q;
}

static double half_to_double(uint16_t h)
{
    int sign = h >> 15, ex = (h >> 10) & 0x1f, man = h & 0x3ff;
    double v;
    if (ex == 0) v = ldexp((double)man, -24);
    else if (ex == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(man | 0x400), ex - 25);
    return sign ? -v : v;
}

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Dequantized weight [n][c] of an R x C matrix given its code block and
 * scale/bias block: s*q + z, exact in double; width 16: the bf16 value. */
static double weight_at(const uint8_t* codes, const uint8_t* sb, int C, int bits, int n, int c)
{
    const uint8_t* row = codes + (size_t)n * (size_t)C * bits / 8;
    uint32_t q = oracle_code(row, bits, c);
    if (bits == 16) return bf16_to_double((uint16_t)q);
    const uint8_t* g = sb + ((size_t)n * (C / 64) + c / 64) * 4;
    uint16_t s16 = (uint16_t)(g[0] | (g[1] << 8));
    uint16_t z16 = (uint16_t)(g[2] | (g[3] << 8));
    return half_to_double(s16) * (double)q + half_to_double(z16);
}

/* Whole dequantized matrix of one expert row: which = 0 gate_up [2I x H],
 * 1 down [H x I]; out row-major doubles. */
int oracle_dequant(const uint8_t* slot_row, int H, int I, int bits_gu, int bits_d, int which,
                   double* out)
{
    int64_t offs[5];
    if (oracle_layout(H, I, bits_gu, bits_d, offs)) return OR_INVALID;
    const uint8_t* codes = slot_row + offs[which == 0 ? 0 : 2];
    const uint8_t* sb = slot_row + offs[which == 0 ? 1 : 3];
    int R = which == 0 ? 2 * I : H, C = which == 0 ? H : I, b = which == 0 ? bits_gu : bits_d;
    for (int n = 0; n < R; n++)
        for (int c = 0; c < C; c++) out[(size_t)n * C + c] = weight_at(codes, sb, C, b, n, c);
    return OR_OK;
}

/*
 * The layer for a subset of tokens (tokens == NULL: all T).  out[n_out, H] in
 * double, row r for token tokens[r].  Pool rows are slot_row = pool +
 * slot*slot_bytes with slot = slot_table[e] in [0, n_slots).
 */
int oracle_layer(const uint16_t* x, int T, int H, int I, int bits_gu, int bits_d,
                 const int32_t* ids, const float* w, int k, int E,
                 const int32_t* slot_table, const uint8_t* pool, int64_t n_slots,
                 const int32_t* tokens, int n_out, double* out, int nthreads)
{
    int64_t offs[5];
    if (oracle_layout(H, I, bits_gu, bits_d, offs)) return OR_INVALID;
    if (T < 0 || k < 1 || E < 1) return OR_INVALID;
    if (!tokens) n_out = T;
    /* validate every routed expert first */
    for (int r = 0; r < n_out; r++) {
        int t = tokens ? tokens[r] : r;
        if (t < 0 || t >= T) return OR_INVALID;
        for (int j = 0; j < k; j++) {
            int e = ids[(size_t)t * k + j];
            if (e < 0 || e >= E) return OR_BAD_ID;
            if (slot_table[e] < 0) return OR_NOT_RESIDENT;
            if (slot_table[e] >= n_slots) return OR_BAD_SLOT;
        }
    }
    const int64_t sbytes = offs[4];
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int r = 0; r < n_out; r++) {
        int t = tokens ? tokens[r] : r;
        double* xt = (double*)malloc(sizeof(double) * (size_t)H);
        double* h = (double*)malloc(sizeof(double) * (size_t)I);
        double* o = out + (size_t)r * H;
        for (int i = 0; i < H; i++) xt[i] = bf16_to_double(x[(size_t)t * H + i]);
        for (int n = 0; n < H; n++) o[n] = 0.0;
        for (int j = 0; j < k; j++) {
            int e = ids[(size_t)t * k + j];
            const uint8_t* row = pool + (size_t)slot_table[e] * (size_t)sbytes;
            const uint8_t* gu_c = row + offs[0];
            const uint8_t* gu_s = row + offs[1];
            const uint8_t* d_c = row + offs[2];
            const uint8_t* d_s = row + offs[3];
            /* gate/up and SwiGLU */
            for (int n = 0; n < I; n++) {
                double g = 0.0, u = 0.0;
                for (int c = 0; c < H; c++) {
                    g += weight_at(gu_c, gu_s, H, bits_gu, n, c) * xt[c];
                    u += weight_at(gu_c, gu_s, H, bits_gu, I + n, c) * xt[c];
                }
                h[n] = g / (1.0 + exp(-g)) * u;
            }
            /* down, weighted combine */
            double wj = (double)w[(size_t)t * k + j];
            for (int n = 0; n < H; n++) {
                double y = 0.0;
                for (int c = 0; c < I; c++) y += weight_at(d_c, d_s, I, bits_d, n, c) * h[c];
                o[n] += wj * y;
            }
        }
        free(xt);
        free(h);
    }
    return OR_OK;
}

/*
 * Router logits of n_mats consecutive layers on the same hidden states:
 * logits[m][t][e] = sum_i x[t][i] * w[m][e][i], x bf16 [T][H], w bf16
 * [n_mats][E][H], accumulated in fp64 with i ascending.
 */
int oracle_router_logits(const uint16_t* x, int T, int H, const uint16_t* w, int n_mats, int E,
                         double* logits)
{
    if (!x || !w || !logits || T < 0 || H < 1 || n_mats < 1 || E < 1) return OR_INVALID;
    for (int m = 0; m < n_mats; m++)
        for (int t = 0; t < T; t++)
            for (int e = 0; e < E; e++) {
                const uint16_t* wr = w + ((size_t)m * E + e) * (size_t)H;
                const uint16_t* xr = x + (size_t)t * H;
                double acc = 0.0;
                for (int i = 0; i < H; i++) acc += bf16_to_double(xr[i]) * bf16_to_double(wr[i]);
                logits[((size_t)m * T + t) * E + e] = acc;
            }
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* One-time conversion of expert weights into slot rows                       */
/* ------------------------------------------------------------------------- */
/*
 * Source: "RFC: stream MoE experts from disk in from_pretrained", How the
 * prototype works, Quantized experts bullet: an optional offline pass converts
 * the experts to the affine quantized format and writes each expert as one
 * contiguous row.  The pages print no rule for choosing scale and bias; the
 * reading taken here is plain min/max affine quantization per group of 64
 * inputs: scale = (max - min) / (2^b - 1) and bias = min, each rounded to the
 * nearest fp16 (ties to even mantissa), code = (w - bias) / scale rounded to
 * the nearest integer (ties to even) and clamped to [0, 2^b - 1], computed in
 * double from the fp16 scale and bias; a group whose fp16 scale is 0 gets code 0.
 * A minimum of zero is stored as +0.  Width 16 stores the weights rounded to the
 * nearest bf16 (ties to even).  Weights must be finite.
 */

/* Nearest value of a 16-bit float format to x, ties to the even bit pattern:
 * a binary search over the format's non-negative finite patterns, which are
 * ordered like their values, then the closer neighbour.  dec() decodes a
 * pattern, top is the largest finite pattern; beyond the largest finite value
 * plus half its spacing the result is infinity (pattern top + 1). */
static uint16_t nearest16(double x, double (*dec)(uint16_t), uint16_t top)
{
    const uint16_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x8000u : 0u;
    const double a = fabs(x);
    uint16_t lo = 0, hi = top;  /* dec(lo) <= a is kept true where possible */
    if (a >= dec(top)) {
        const double spacing = dec(top) - dec((uint16_t)(top - 1));
        if (a > dec(top) + spacing / 2 || (a == dec(top) + spacing / 2 && (top & 1)))
            return (uint16_t)(sign | (top + 1));
        return (uint16_t)(sign | top);
    }
    while (hi - lo > 1) {  /* dec(lo) <= a < dec(hi) */
        uint16_t mid = (uint16_t)((lo + hi) / 2);
        if (dec(mid) <= a) lo = mid;
        else hi = mid;
    }
    const double dl = a - dec(lo), dh = dec(hi) - a;
    uint16_t r;
    if (dl < dh) r = lo;
    else if (dh < dl) r = hi;
    else r = (lo & 1) ? hi : lo;
    return (uint16_t)(sign | r);
}

uint16_t oracle_round_half(double x) { return nearest16(x, half_to_double, 0x7BFF); }
uint16_t oracle_round_bf16(double x) { return nearest16(x, bf16_to_double, 0x7F7F); }

/* Group-wise affine quantization of an R x C fp32 matrix (C a multiple of 64):
 * codes[r][c] (one byte each), scale16 / bias16 [r][c / 64] fp16 patterns. */
int oracle_quantize(const float* w, int R, int C, int bits, uint8_t* codes, uint16_t* scale16,
                    uint16_t* bias16)
{
    if (!w || !codes || !scale16 || !bias16 || R < 0 || C <= 0 || C % 64) return OR_INVALID;
    if (!(bits == 3 || bits == 4 || bits == 6 || bits == 8)) return OR_INVALID;
    const double qmax = (double)((1 << bits) - 1);
    for (int r = 0; r < R; r++)
        for (int g = 0; g < C / 64; g++) {
            const float* v = w + (size_t)r * C + (size_t)g * 64;
            double mn = v[0], mx = v[0];
            for (int i = 1; i < 64; i++) {
                if (v[i] < mn) mn = v[i];
                if (v[i] > mx) mx = v[i];
            }
            const uint16_t s16 = oracle_round_half((mx - mn) / qmax);
            const uint16_t z16 = oracle_round_half(mn + 0.0);  /* -0 + 0 = +0: one pattern for zero */
            const double s = half_to_double(s16), z = half_to_double(z16);
            scale16[(size_t)r * (C / 64) + g] = s16;
            bias16[(size_t)r * (C / 64) + g] = z16;
            for (int i = 0; i < 64; i++) {
                double q = 0.0;
                if (s != 0.0) {
                    q = nearbyint(((double)v[i] - z) / s);  /* default mode: ties to even */
                    if (q < 0) q = 0;
                    if (q > qmax) q = qmax;
                }
                codes[(size_t)r * C + (size_t)g * 64 + i] = (uint8_t)q;
            }
        }
    return OR_OK;
}

/* Write code q of column c into a code row: bit b of q becomes bit bits*(c%32)+b
 * of pack unit c/32 read as a little-endian bit string (the inverse of
 * oracle_code). */
static void put_code(uint8_t* row, int bits, int c, uint32_t q)
{
    uint8_t* unit = row + (size_t)(c / 32) * 4 * (size_t)bits;
    int first = bits * (c % 32);
    for (int b = 0; b < bits; b++) {
        int bit = first + b;
        if ((q >> b) & 1u) unit[bit / 8] |= (uint8_t)(1u << (bit % 8));
        else unit[bit / 8] &= (uint8_t)~(1u << (bit % 8));
    }
}

/* One matrix into its code block and scale/bias block (scale low half, bias
 * high half of each little-endian 32-bit word). */
static int convert_matrix(const float* w, int R, int C, int bits, uint8_t* code_blk, uint8_t* sb_blk)
{
    const size_t row_bytes = (size_t)C * bits / 8;
    if (bits == 16) {
        for (int r = 0; r < R; r++)
            for (int c = 0; c < C; c++)
                put_code(code_blk + (size_t)r * row_bytes, 16, c, oracle_round_bf16(w[(size_t)r * C + c]));
        return OR_OK;
    }
    uint8_t* q = (uint8_t*)malloc((size_t)R * C);
    uint16_t* s = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)R * (C / 64));
    uint16_t* z = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)R * (C / 64));
    int rc = (q && s && z) ? oracle_quantize(w, R, C, bits, q, s, z) : OR_INVALID;
    if (rc == OR_OK) {
        for (int r = 0; r < R; r++)
            for (int c = 0; c < C; c++) put_code(code_blk + (size_t)r * row_bytes, bits, c, q[(size_t)r * C + c]);
        for (size_t i = 0; i < (size_t)R * (C / 64); i++) {
            sb_blk[4 * i + 0] = (uint8_t)(s[i] & 0xFF);
            sb_blk[4 * i + 1] = (uint8_t)(s[i] >> 8);
            sb_blk[4 * i + 2] = (uint8_t)(z[i] & 0xFF);
            sb_blk[4 * i + 3] = (uint8_t)(z[i] >> 8);
        }
    }
    free(q);
    free(s);
    free(z);
    return rc;
}

/* One expert's slot row from fp32 gate_up [2I][H] (gate rows, then up rows) and
 * down [H][I]; padding between blocks is zero. */
int oracle_convert_expert(const float* w_gu, const float* w_d, int H, int I, int bits_gu, int bits_d,
                          uint8_t* row)
{
    int64_t offs[5];
    if (!w_gu || !w_d || !row || oracle_layout(H, I, bits_gu, bits_d, offs)) return OR_INVALID;
    memset(row, 0, (size_t)offs[4]);
    int rc = convert_matrix(w_gu, 2 * I, H, bits_gu, row + offs[0], row + offs[1]);
    if (rc == OR_OK) rc = convert_matrix(w_d, H, I, bits_d, row + offs[2], row + offs[3]);
    return rc;
}
