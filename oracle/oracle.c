/*
 * oracle.c -- plain, slow CPU reference of the mixed-precision AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant
 * generator with the HIP library: every function below is written from the
 * pages it cites, in the order and notation those pages use.
 *
 * Pages cited (by title and section):
 *   [LLMC]  "04 · 多 GPU 与混合精度" -- the llm.c multi-GPU and mixed-precision
 *           chapter: §2.1 precision roles, §2.2 the AdamW kernel, §2.3
 *           stochastic rounding, §3.2 ZeRO-1 sharding rule, §4 the training
 *           step (grad norm and clip), §5.2 bit-perfect resume.
 *   [LEC13] "第 13 讲：扩大 LLM——优化与并行训练" -- §1.4 Adam, §1.7 bias
 *           correction and AdamW, §2.1 number formats, §2.3 fp32 master
 *           weights, §5.2 ZeRO-1, §7.3 exercises 1 and 5.
 *   [DIST]  "LLM 分布式训练实战：CUDA/ROCm 多卡并行优化详解" -- §3.1 the
 *           ZeRO stage-1 sharded update (offset rank * total / world).
 *   Philox4x32-10: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 *           "Parallel random numbers: as easy as 1, 2, 3", SC'11 (the pages
 *           name a counter-based noise hash for the rounding draws but print
 *           neither its code nor its constants; this published generator is
 *           used in its place).
 *
 * Floating point: every float operation here is one IEEE-754 binary32
 * operation with round-to-nearest-even.  Build with -ffp-contract=off and
 * without -ffast-math so that no multiply-add is fused except the explicit
 * fmaf() calls, division and sqrtf are correctly rounded and subnormals are
 * kept.  Sums of squares are formed in binary64.
 */
#define _DEFAULT_SOURCE
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOTDIVISIBLE (-2)
#define ORACLE_ERANGE (-3)
#define ORACLE_ETABLE (-5)

#define ORACLE_ROUND_SR 0
#define ORACLE_ROUND_RNE 1

/* One entry of the flat parameter buffer: tensor k occupies global elements
 * [offset, offset + numel); bit 0 of flags says the tensor takes weight decay. */
typedef struct {
    uint64_t offset;
    uint64_t numel;
    uint32_t flags;
    uint32_t pad;
} oracle_tensor;

typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int32_t bias_correction;
} oracle_hparams;

/* ------------------------------------------------------------------ */
/* bf16 <-> f32 bit patterns                                           */
/* ------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* [LEC13] §2.1: bf16 keeps fp32's sign and 8 exponent bits and the top 7
 * mantissa bits, i.e. it is the upper half of a binary32 pattern.  Widening
 * is therefore exact: the pattern goes to the upper 16 bits. */
float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* Value of a bf16 pattern as a double, for the distance comparisons below.
 * The pattern one past the largest finite value (exponent field all ones,
 * mantissa zero) stands for 2^128 here: it is the neighbour that IEEE
 * round-to-nearest compares against when deciding overflow. */
static double bf16_value_for_rounding(uint16_t h) {
    if ((h & 0x7FFF) == 0x7F80) return (h & 0x8000) ? -ldexp(1.0, 128) : ldexp(1.0, 128);
    return (double)oracle_bf16_to_f32(h);
}

/* Round-to-nearest, ties to even ([LLMC] §2.3 "ordinary rounding to the
 * nearest bf16"; [LEC13] §7.3 exercise 5: 1 + 2^-8 lies exactly half way and
 * goes to the even neighbour 1, 257 goes to 256).  Written as the
 * definition: of the two bf16 values that bracket x, return the nearer one
 * and, on a tie, the one whose last mantissa bit is 0.  NaN stays a quiet
 * NaN with its sign. */
uint16_t oracle_round_nearest_even(float x) {
    uint32_t bits = f32_bits(x);
    if (isnan(x)) return (uint16_t)((bits >> 16) | 0x0040);
    uint16_t toward_zero = (uint16_t)(bits >> 16);    /* |value| <= |x| */
    if ((bits & 0xFFFFu) == 0) return toward_zero;      /* x is a bf16 value */
    uint16_t away = (uint16_t)(toward_zero + 1);         /* next bf16 away from 0 */
    double ax = fabs((double)x);
    double below = fabs(bf16_value_for_rounding(toward_zero));
    double above = fabs(bf16_value_for_rounding(away));
    double d_below = ax - below, d_above = above - ax;    /* both exact in binary64 */
    if (d_below < d_above) return toward_zero;
    if (d_above < d_below) return away;
    return (toward_zero & 1) ? away : toward_zero;
}

/* Stochastic rounding ([LLMC] §2.3): the 16 bits that bf16 drops, lo16, are
 * the fraction of one bf16 step by which x exceeds its truncation; round to
 * the far neighbour when lo16 > r, else keep the truncation.  With r uniform
 * on [0, 65536) the far neighbour is taken with probability lo16 / 65536, so
 * the expected result is x.  "Up" means away from zero for both signs (for a
 * negative x the dropped bits measure the distance below the truncation), the
 * only reading under which the expectation equals x.  NaN stays a quiet NaN. */
uint16_t oracle_round_stochastic(float x, uint16_t r) {
    uint32_t bits = f32_bits(x);
    if (isnan(x)) return (uint16_t)((bits >> 16) | 0x0040);
    uint16_t truncated = (uint16_t)(bits >> 16);
    uint32_t lo16 = bits & 0xFFFFu;
    if (lo16 > (uint32_t)r) return (uint16_t)(truncated + 1);  /* next bf16 away from zero */
    return truncated;
}

/* ------------------------------------------------------------------ */
/* Counter-based draws: Philox4x32-10 (Salmon et al., SC'11)            */
/* ------------------------------------------------------------------ */

/* Round multipliers and key increments as published for Philox4x32. */
static const uint32_t PHILOX_M4x32_0 = 0xD2511F53u;
static const uint32_t PHILOX_M4x32_1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W32_0 = 0x9E3779B9u;
static const uint32_t PHILOX_W32_1 = 0xBB67AE85u;

/* One Philox S-box round: two 32x32->64 products of counter words 0 and 2,
 * whose high halves are mixed with the other two words and the round key,
 * and whose low halves are passed through; the words are permuted so that
 * the products feed the other pair in the next round. */
static void philox4x32_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M4x32_0 * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)PHILOX_M4x32_1 * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t out0 = hi1 ^ c[1] ^ k[0];
    uint32_t out1 = lo1;
    uint32_t out2 = hi0 ^ c[3] ^ k[1];
    uint32_t out3 = lo0;
    c[0] = out0; c[1] = out1; c[2] = out2; c[3] = out3;
}

/* Philox4x32 with 10 rounds: the key is bumped by the Weyl constants
 * between rounds. */
void oracle_philox4x32_10(const uint32_t counter[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {counter[0], counter[1], counter[2], counter[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k[0] += PHILOX_W32_0; k[1] += PHILOX_W32_1; }
        philox4x32_round(c, k);
    }
    memcpy(out, c, sizeof c);
}

/* The 16-bit rounding draw of global element i under a 64-bit seed.  The
 * pages key each parameter's draw on a reproducible (position, seed) pair
 * ([LLMC] §2.3, §5.2); here the position is the element's global index in
 * the flat buffer, so the draw does not depend on launch shape or on the
 * number of shards.  One Philox block serves the aligned group of 8
 * elements i>>3: counter = (lo32(i>>3), hi32(i>>3), 0, 0),
 * key = (lo32(seed), hi32(seed)); element i takes output word (i>>1)&3,
 * low half when i is even, high half when i is odd. */
uint16_t oracle_rng16(uint64_t i, uint64_t seed) {
    uint64_t group = i >> 3;
    uint32_t counter[4] = {(uint32_t)group, (uint32_t)(group >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(counter, key, out);
    uint32_t word = out[(i >> 1) & 3];
    return (uint16_t)((i & 1) ? (word >> 16) : (word & 0xFFFFu));
}

void oracle_rng16_fill(uint64_t first, uint64_t count, uint64_t seed, uint16_t *out) {
    for (uint64_t k = 0; k < count; ++k) out[k] = oracle_rng16(first + k, seed);
}

void oracle_round_stochastic_array(const float *x, const uint16_t *r, uint64_t count, uint16_t *out) {
    for (uint64_t k = 0; k < count; ++k) out[k] = oracle_round_stochastic(x[k], r[k]);
}

void oracle_round_nearest_even_array(const float *x, uint64_t count, uint16_t *out) {
    for (uint64_t k = 0; k < count; ++k) out[k] = oracle_round_nearest_even(x[k]);
}

/* ------------------------------------------------------------------ */
/* ZeRO-1 shard and tensor table                                        */
/* ------------------------------------------------------------------ */

/* [LLMC] §3.2: each rank owns "parameter count / process count" elements,
 * and the count must divide exactly, otherwise it is an error.  [DIST] §3.1:
 * rank r's slice starts at r * (total / world).  Errors: world = 0 is
 * invalid, rank >= world is out of range, n mod world != 0 is not divisible. */
int oracle_shard_range(uint64_t n, uint32_t world, uint32_t rank, uint64_t *begin, uint64_t *end) {
    if (world == 0) return ORACLE_EINVAL;
    if (rank >= world) return ORACLE_ERANGE;
    if (n % world != 0) return ORACLE_ENOTDIVISIBLE;
    uint64_t per_rank = n / world;
    *begin = (uint64_t)rank * per_rank;
    *end = *begin + per_rank;
    return ORACLE_OK;
}

/* The table must list the tensors in buffer order, each starting where the
 * previous one ends, from 0; only flag bit 0 is defined.  On success *total
 * is the buffer length n. */
int oracle_table_check(const oracle_tensor *t, uint32_t count, uint64_t *total) {
    uint64_t expect = 0;
    for (uint32_t k = 0; k < count; ++k) {
        if (t[k].offset != expect) return ORACLE_ETABLE;
        if (t[k].flags & ~1u) return ORACLE_ETABLE;
        if (t[k].numel > UINT64_MAX - expect) return ORACLE_ETABLE;
        expect += t[k].numel;
    }
    *total = expect;
    return ORACLE_OK;
}

/* [LLMC] §2.2: weight decay applies to 2-D tensors (embeddings and
 * matrices) and not to LayerNorm weights or biases; the table's flag bit
 * records that choice per tensor.  Writes 1 for each element of
 * [begin, begin + count) whose tensor decays, else 0. */
int oracle_decay_mask(const oracle_tensor *t, uint32_t ntensors, uint64_t begin, uint64_t count, uint8_t *out) {
    uint64_t n;
    int rc = oracle_table_check(t, ntensors, &n);
    if (rc != ORACLE_OK) return rc;
    if (begin > n || count > n - begin) return ORACLE_ERANGE;
    for (uint64_t j = 0; j < count; ++j) {
        uint64_t i = begin + j;
        out[j] = 0;
        for (uint32_t k = 0; k < ntensors; ++k)
            if (i >= t[k].offset && i - t[k].offset < t[k].numel) { out[j] = (uint8_t)(t[k].flags & 1u); break; }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Global gradient norm and clip scale                                  */
/* ------------------------------------------------------------------ */

/* [LLMC] §4: grad_norm is the L2 norm of all gradients (under ZeRO-1 the
 * local shard's sum of squares, combined across ranks), and the update uses
 * grad_scale = min(1, 1/grad_norm), i.e. clipping to norm 1.0.  Here: the
 * sum of squares of the widened bf16 values in binary64, added in ascending
 * index order (every bf16 square is exact in binary64); norm is its square
 * root rounded to binary32; scale is max_norm / norm when norm exceeds
 * max_norm, else 1 (for max_norm = 1 this is min(1, 1/norm)).
 * oracle_norm_from_sumsq is that last part alone, for a sum of squares
 * added up elsewhere (e.g. the shards' parts, added before the root). */
void oracle_norm_from_sumsq(double sumsq, float max_norm, float *norm, float *scale) {
    float nrm = (float)sqrt(sumsq);
    *norm = nrm;
    *scale = (nrm > max_norm) ? max_norm / nrm : 1.0f;
}

void oracle_grad_norm(const uint16_t *g, uint64_t count, float max_norm,
                      double *sumsq, float *norm, float *scale) {
    double s = 0.0;
    for (uint64_t j = 0; j < count; ++j) {
        double x = (double)oracle_bf16_to_f32(g[j]);
        s += x * x;
    }
    *sumsq = s;
    oracle_norm_from_sumsq(s, max_norm, norm, scale);
}

/* ------------------------------------------------------------------ */
/* AdamW step                                                           */
/* ------------------------------------------------------------------ */

/* [LEC13] §1.7: m and v start at 0, so without correction the step is scaled
 * by (1 - beta1^t) / sqrt(1 - beta2^t); dividing m by 1 - beta1^t and v by
 * 1 - beta2^t removes it.  beta^t is formed as pow() in binary64 and
 * 1 - beta^t is rounded once to binary32.  t is the 1-based step number
 * ([LLMC] §4 passes step + 1). */
void oracle_bias_corrections(float beta1, float beta2, uint64_t t, int bias_correction,
                             float *bc1, float *bc2) {
    if (!bias_correction) { *bc1 = 1.0f; *bc2 = 1.0f; return; }
    *bc1 = (float)(1.0 - pow((double)beta1, (double)t));
    *bc2 = (float)(1.0 - pow((double)beta2, (double)t));
}

/* [LLMC] §2.2, with the lerp of the same section computed by two fused
 * multiply-adds: lerp(start, end, w) = start + w * (end - start)
 *                                    = fma(w, end, fma(-w, start, start)). */
static float lerp2fma(float start, float end, float w) {
    return fmaf(w, end, fmaf(-w, start, start));
}

/* The AdamW step, per element ([LLMC] §2.2, with [LEC13] §1.7 for the bias
 * correction and the decoupled weight decay):
 *   grad = grad_scale * f32(G)
 *   m    = lerp(grad, m, beta1)           v = lerp(grad*grad, v, beta2)
 *   m_hat = m / bc1                       v_hat = v / bc2
 *   old  = master ? M : f32(P)
 *   p    = old - lr * (m_hat / (sqrt(v_hat) + eps) + wd * old)
 *   P    = SR(p, r16(i, seed))   or RNE(p)
 *   M    = p                     (master path only)
 * wd is the table's weight decay for 2-D tensors and 0 for the rest.
 * adamw_element does one element (global index i, decay w); each of its
 * lines is one binary32 operation, in the order above. */
static void adamw_element(uint64_t i, float w, uint16_t *P, const uint16_t *G, float *M, float *m, float *v,
                          const oracle_hparams *hp, float bc1, float bc2, float grad_scale,
                          uint64_t seed, int rounding) {
    float grad = grad_scale * oracle_bf16_to_f32(*G);
    float m1 = lerp2fma(grad, *m, hp->beta1);
    float gg = grad * grad;
    float v1 = lerp2fma(gg, *v, hp->beta2);
    float m_hat = m1 / bc1;
    float v_hat = v1 / bc2;
    float denom = sqrtf(v_hat) + hp->eps;
    float adam = m_hat / denom;
    float old = M ? *M : oracle_bf16_to_f32(*P);
    float decay = w * old;
    float sum = adam + decay;
    float step = hp->lr * sum;
    float p = old - step;

    *m = m1;
    *v = v1;
    if (M) *M = p;
    *P = (rounding == ORACLE_ROUND_SR) ? oracle_round_stochastic(p, oracle_rng16(i, seed))
                                       : oracle_round_nearest_even(p);
}

static int step_args_check(const oracle_tensor *table, uint32_t ntensors, uint64_t *n, uint64_t t, int rounding) {
    int rc = oracle_table_check(table, ntensors, n);
    if (rc != ORACLE_OK) return rc;
    if (t == 0) return ORACLE_EINVAL;
    if (rounding != ORACLE_ROUND_SR && rounding != ORACLE_ROUND_RNE) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* Index of the tensor holding global element i, searching forward from *k
 * (and from 0 again when i lies before tensor *k). */
static uint32_t tensor_of(const oracle_tensor *table, uint32_t ntensors, uint64_t i, uint32_t *k) {
    if (*k >= ntensors || i < table[*k].offset) *k = 0;
    while (*k < ntensors && i - table[*k].offset >= table[*k].numel) ++*k;
    return *k;
}

/* One step over global elements [begin, begin + count); element j of every
 * array holds global element begin + j. */
int oracle_adamw_step(const oracle_tensor *table, uint32_t ntensors,
                      uint64_t begin, uint64_t count,
                      uint16_t *P, const uint16_t *G, float *M, float *m, float *v,
                      const oracle_hparams *hp, float grad_scale,
                      uint64_t t, uint64_t seed, int rounding) {
    uint64_t n;
    int rc = step_args_check(table, ntensors, &n, t, rounding);
    if (rc != ORACLE_OK) return rc;
    if (begin > n || count > n - begin) return ORACLE_ERANGE;
    float bc1, bc2;
    oracle_bias_corrections(hp->beta1, hp->beta2, t, hp->bias_correction, &bc1, &bc2);
    uint32_t k = 0;
    for (uint64_t j = 0; j < count; ++j) {
        uint64_t i = begin + j;
        tensor_of(table, ntensors, i, &k);
        float w = (table[k].flags & 1u) ? hp->weight_decay : 0.0f;
        adamw_element(i, w, &P[j], &G[j], M ? &M[j] : NULL, &m[j], &v[j], hp, bc1, bc2, grad_scale, seed,
                      rounding);
    }
    return ORACLE_OK;
}

/* The same step for a shard given as a list of global indices: shard
 * element j is global element gidx[j]; P and G are the full n-element
 * buffers (indexed by global index), M, m and v are shard-local. */
int oracle_adamw_step_mapped(const oracle_tensor *table, uint32_t ntensors,
                             const uint64_t *gidx, uint64_t count,
                             uint16_t *P, const uint16_t *G, float *M, float *m, float *v,
                             const oracle_hparams *hp, float grad_scale,
                             uint64_t t, uint64_t seed, int rounding) {
    uint64_t n;
    int rc = step_args_check(table, ntensors, &n, t, rounding);
    if (rc != ORACLE_OK) return rc;
    for (uint64_t j = 0; j < count; ++j)
        if (gidx[j] >= n) return ORACLE_ERANGE;
    float bc1, bc2;
    oracle_bias_corrections(hp->beta1, hp->beta2, t, hp->bias_correction, &bc1, &bc2);
    uint32_t k = 0;
    for (uint64_t j = 0; j < count; ++j) {
        uint64_t i = gidx[j];
        tensor_of(table, ntensors, i, &k);
        float w = (table[k].flags & 1u) ? hp->weight_decay : 0.0f;
        adamw_element(i, w, &P[i], &G[i], M ? &M[j] : NULL, &m[j], &v[j], hp, bc1, bc2, grad_scale, seed,
                      rounding);
    }
    return ORACLE_OK;
}

/* [LLMC] §3.2 and §6: llm.c shards every tensor, so each tensor's size must
 * divide by the process count; rank r owns the r-th 1/N slice of each
 * tensor, and its shard is those slices in table order.  Writes the global
 * index of every shard position (count = n / world). */
int oracle_shard_map_per_tensor(const oracle_tensor *table, uint32_t ntensors, uint32_t world, uint32_t rank,
                                uint64_t *gidx, uint64_t capacity, uint64_t *count) {
    uint64_t n;
    int rc = oracle_table_check(table, ntensors, &n);
    if (rc != ORACLE_OK) return rc;
    if (world == 0) return ORACLE_EINVAL;
    if (rank >= world) return ORACLE_ERANGE;
    for (uint32_t k = 0; k < ntensors; ++k)
        if (table[k].numel % world != 0) return ORACLE_ENOTDIVISIBLE;
    uint64_t j = 0;
    for (uint32_t k = 0; k < ntensors; ++k) {
        uint64_t slice = table[k].numel / world;
        for (uint64_t e = 0; e < slice; ++e) {
            if (j >= capacity) return ORACLE_ERANGE;
            gidx[j++] = table[k].offset + (uint64_t)rank * slice + e;
        }
    }
    *count = j;
    return ORACLE_OK;
}

/* [LLMC] §5.2: on resume the bf16 weights are not read from the checkpoint
 * but rebuilt from the fp32 master with the same rounding draws as the
 * update that produced it, so they come back bit-identical.  P = SR(M,
 * r16(i, seed)) over global elements [begin, begin + count). */
void oracle_master_to_bf16_sr(const float *M, uint64_t begin, uint64_t count, uint64_t seed, uint16_t *P) {
    for (uint64_t j = 0; j < count; ++j)
        P[j] = oracle_round_stochastic(M[j], oracle_rng16(begin + j, seed));
}

/* The same for a shard given by global indices: P_full[gidx[j]] = SR(M[j]). */
void oracle_master_to_bf16_sr_mapped(const float *M, const uint64_t *gidx, uint64_t count, uint64_t seed,
                                     uint16_t *P_full) {
    for (uint64_t j = 0; j < count; ++j)
        P_full[gidx[j]] = oracle_round_stochastic(M[j], oracle_rng16(gidx[j], seed));
}

/* Array helper for the test harness: widen bf16 patterns to binary32. */
void oracle_bf16_to_f32_array(const uint16_t *h, uint64_t count, float *out) {
    for (uint64_t k = 0; k < count; ++k) out[k] = oracle_bf16_to_f32(h[k]);
}

/* ------------------------------------------------------------------ */
/* Step control: learning-rate schedules and the outlier z-score        */
/* ------------------------------------------------------------------ */

#define ORACLE_LR_CONSTANT 0
#define ORACLE_LR_LINEAR 1
#define ORACLE_LR_COSINE 2
#define ORACLE_LR_WSD 3

/* [LLMC] §4 names four schedules (cosine, linear, constant, wsd) without
 * formulas; the readings, for 0-based step s, peak lr_max, floor
 * lr_min = final_frac * lr_max, W warm-up steps and T total steps:
 *   warm-up (s < W): lr_max * (s + 1) / W, for every kind;
 *   afterwards, with progress p = (s - W) / (T - W) clamped to [0, 1]:
 *   constant: lr_max;
 *   linear:   lr_max - (lr_max - lr_min) * p;
 *   cosine:   lr_min + (lr_max - lr_min) * (1 + cos(pi * p)) / 2;
 *   wsd:      lr_max while s < T - D, then linear from lr_max to lr_min over
 *             the last D = decay_frac * T steps (warm-up, stable, decay).
 * Evaluated in binary64 and rounded once to binary32. */
float oracle_lr_at(int kind, uint64_t step, uint64_t warmup, uint64_t total, float lr_max,
                   float final_frac, float decay_frac) {
    double peak = (double)lr_max;
    double floor_lr = (double)final_frac * peak;
    if (step < warmup) return (float)(peak * (double)(step + 1) / (double)warmup);
    if (kind == ORACLE_LR_CONSTANT) return lr_max;
    if (kind == ORACLE_LR_WSD) {
        double decay_steps = (double)decay_frac * (double)total;
        double decay_start = (double)total - decay_steps;
        if ((double)step < decay_start || decay_steps <= 0.0) return lr_max;
        double q = ((double)step - decay_start) / decay_steps;
        if (q > 1.0) q = 1.0;
        return (float)(peak - (peak - floor_lr) * q);
    }
    double span = (double)total - (double)warmup;
    double p = span > 0.0 ? ((double)step - (double)warmup) / span : 1.0;
    if (p > 1.0) p = 1.0;
    if (kind == ORACLE_LR_LINEAR) return (float)(peak - (peak - floor_lr) * p);
    return (float)(floor_lr + (peak - floor_lr) * (1.0 + cos(M_PI * p)) / 2.0);
}

/* [LLMC] §4: a z-score of the grad norm (or loss) over a window of the 128
 * previous values; the update is skipped when it exceeds a threshold.
 * Reading: mean and variance (population, divide by the window length) of
 * the previous `window` finite values, summed in binary64 from oldest to
 * newest; z = (x - mean) / sqrt(variance), NaN until the window is full;
 * skip when x is not finite, or when threshold > 0 and z > threshold.  x
 * then joins the window (oldest value dropped) unless it is not finite. */
typedef struct {
    uint32_t window, count, head, pad;
    float values[4096];
} oracle_outlier;

int oracle_outlier_init(oracle_outlier *d, uint32_t window) {
    if (window == 0 || window > 4096) return ORACLE_EINVAL;
    memset(d, 0, sizeof *d);
    d->window = window;
    return ORACLE_OK;
}

void oracle_outlier_update(oracle_outlier *d, float x, float threshold, float *z_out, int32_t *skip_out) {
    double z = NAN;
    if (d->count == d->window) {
        double sum = 0.0;
        for (uint32_t k = 0; k < d->window; ++k) sum += (double)d->values[(d->head + k) % d->window];
        double mean = sum / (double)d->window;
        double sq = 0.0;
        for (uint32_t k = 0; k < d->window; ++k) {
            double dev = (double)d->values[(d->head + k) % d->window] - mean;
            sq += dev * dev;
        }
        z = ((double)x - mean) / sqrt(sq / (double)d->window);
    }
    int finite = isfinite(x);
    *z_out = (float)z;
    *skip_out = (!finite || (threshold > 0.0f && z > (double)threshold)) ? 1 : 0;
    if (finite) {
        d->values[d->head] = x;
        d->head = (d->head + 1) % d->window;
        if (d->count < d->window) ++d->count;
    }
}
