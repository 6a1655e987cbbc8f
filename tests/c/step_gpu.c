/* A plain C caller of the whole step on the GPU, with no Python and no torch:
 * device memory from the HIP runtime's C API, every step through the
 * library's C ABI (grad_global_norm, adamw_sr_step, master_to_bf16_sr), and
 * the result checked against the CPU oracle (oracle/liboracle.so) bit for bit.
 *
 * Workload: a 3-tensor flat buffer of n = 2 * 15,401 elements (2-D, 1-D,
 * 2-D), rank 1 of 2, so the shard starts mid-tensor and ends ragged; three
 * steps with grads large enough that the clip scale is active, the rebuild,
 * then three more steps replayed from a HIP graph recorded once through the
 * HIP C API (grad_global_norm, adamw_sr_step_scheduled, bfo_cursor_advance),
 * the grads refilled between replays.  Prints one line per check and exits
 * non-zero on the first mismatch. */
#include "bf16opt.h"

#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's C entry points (test infrastructure; see oracle/oracle.c). */
typedef struct {
    uint64_t offset, numel;
    uint32_t flags, pad;
} oracle_tensor;
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int32_t bias_correction;
} oracle_hparams;
void oracle_grad_norm(const uint16_t *g, uint64_t count, float max_norm, double *sumsq, float *norm, float *scale);
int oracle_adamw_step(const oracle_tensor *table, uint32_t ntensors, uint64_t begin, uint64_t count, uint16_t *P,
                      const uint16_t *G, float *M, float *m, float *v, const oracle_hparams *hp, float grad_scale,
                      uint64_t t, uint64_t seed, int rounding);
void oracle_master_to_bf16_sr(const float *M, uint64_t begin, uint64_t count, uint64_t seed, uint16_t *P);

#define HIP_OK(x)                                                             \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            printf("FAIL HIP error %d at line %d\n", (int)e_, __LINE__);     \
            return 1;                                                         \
        }                                                                     \
    } while (0)
#define BFO_OK_(x)                                                                       \
    do {                                                                                 \
        int rc_ = (x);                                                                   \
        if (rc_ != BFO_OK) {                                                             \
            printf("FAIL %s at line %d: %s\n", #x, __LINE__, bfo_status_string(rc_));   \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

/* splitmix64: input generator only. */
static uint64_t mix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

/* A bf16 pattern of a value in about +-scale, never NaN or Inf. */
static uint16_t bf16_from(uint64_t h, float scale) {
    const float u = (float)((double)(h >> 11) / 9007199254740992.0) * 2.0f - 1.0f;
    const float x = u * scale;
    uint32_t b;
    memcpy(&b, &x, 4);
    return (uint16_t)(b >> 16);
}

static float f32_of(uint16_t h) {
    const uint32_t b = (uint32_t)h << 16;
    float x;
    memcpy(&x, &b, 4);
    return x;
}

int main(void) {
    const uint64_t sizes[3] = {4096 * 3 + 37, 1201, 15401 * 2 - (4096 * 3 + 37) - 1201};
    const uint32_t flags[3] = {BFO_FLAG_DECAY, 0, BFO_FLAG_DECAY};
    bfo_tensor tab[3];
    oracle_tensor otab[3];
    uint64_t n = 0;
    for (int k = 0; k < 3; ++k) {
        memset(&tab[k], 0, sizeof tab[k]);
        memset(&otab[k], 0, sizeof otab[k]);
        tab[k].offset = otab[k].offset = n;
        tab[k].numel = otab[k].numel = sizes[k];
        tab[k].flags = otab[k].flags = flags[k];
        n += sizes[k];
    }
    const uint32_t world = 2, rank = 1;
    uint64_t b = 0, e = 0;
    BFO_OK_(shard_range(n, world, rank, &b, &e));
    const uint64_t S = e - b;
    printf("ok   n = %llu, shard [%llu, %llu)\n", (unsigned long long)n, (unsigned long long)b,
           (unsigned long long)e);

    uint16_t *hP = malloc(n * 2), *hG = malloc(S * 2), *oP = malloc(S * 2), *gP = malloc(n * 2);
    float *hM = malloc(S * 4), *oM = malloc(S * 4), *om = calloc(S, 4), *ov = calloc(S, 4);
    float *gM = malloc(S * 4), *gm = malloc(S * 4), *gv = malloc(S * 4);
    uint16_t *rebuilt = malloc(S * 2);
    if (!hP || !hG || !oP || !gP || !hM || !oM || !om || !ov || !gM || !gm || !gv || !rebuilt) return 1;
    for (uint64_t i = 0; i < n; ++i) hP[i] = bf16_from(mix64(i), 0.05f);
    for (uint64_t j = 0; j < S; ++j) {
        oP[j] = hP[b + j];
        hM[j] = oM[j] = f32_of(hP[b + j]);
    }

    uint16_t *dP, *dG;
    float *dM, *dm, *dv;
    bfo_norm_result *dres;
    HIP_OK(hipMalloc((void **)&dP, n * 2));
    HIP_OK(hipMalloc((void **)&dG, S * 2));
    HIP_OK(hipMalloc((void **)&dM, S * 4));
    HIP_OK(hipMalloc((void **)&dm, S * 4));
    HIP_OK(hipMalloc((void **)&dv, S * 4));
    HIP_OK(hipMalloc((void **)&dres, sizeof(bfo_norm_result)));
    HIP_OK(hipMemcpy(dP, hP, n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dM, hM, S * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(dm, 0, S * 4));
    HIP_OK(hipMemset(dv, 0, S * 4));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    bfo_table tb = NULL;
    BFO_OK_(bfo_table_create(tab, 3, world, rank, &tb));
    /* the eager steps bring their own norm workspace; the graph uses the table's */
    uint64_t wsBytes = 0;
    BFO_OK_(bfo_norm_workspace_bytes(tb, &wsBytes));
    void *dws = NULL;
    HIP_OK(hipMalloc(&dws, wsBytes ? wsBytes : 8));
    const bfo_adamw_hparams hp = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1};
    const oracle_hparams ohp = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1};
    int failures = 0;
    uint64_t seed = 0;
    for (uint64_t t = 1; t <= 3; ++t) {
        seed = (1337ull << 32) | t;
        for (uint64_t j = 0; j < S; ++j) hG[j] = bf16_from(mix64((t << 40) ^ (b + j)), 0.02f);
        HIP_OK(hipMemcpyAsync(dG, hG, S * 2, hipMemcpyHostToDevice, stream));
        BFO_OK_(grad_global_norm(tb, dG, 1.0f, dws, dres, stream));
        BFO_OK_(adamw_sr_step(tb, dP + b, dG, dM, dm, dv, &hp, &dres->scale, NULL, t, seed, BFO_ROUND_SR, stream));
        bfo_norm_result res;
        HIP_OK(hipMemcpyAsync(&res, dres, sizeof res, hipMemcpyDeviceToHost, stream));
        HIP_OK(hipStreamSynchronize(stream));

        double osum;
        float onorm, oscale;
        oracle_grad_norm(hG, S, 1.0f, &osum, &onorm, &oscale);
        const double rel = res.sumsq > osum ? (res.sumsq - osum) / osum : (osum - res.sumsq) / osum;
        const int norm_ok = rel <= 1e-12 && res.scale < 1.0f;
        printf("%s step %llu: sumsq %.17g vs oracle %.17g, scale %.9g\n", norm_ok ? "ok  " : "FAIL",
               (unsigned long long)t, res.sumsq, osum, (double)res.scale);
        failures += !norm_ok;
        if (oracle_adamw_step(otab, 3, b, S, oP, hG, oM, om, ov, &ohp, res.scale, t, seed, BFO_ROUND_SR) != 0) {
            printf("FAIL oracle_adamw_step\n");
            return 1;
        }
    }
    HIP_OK(hipMemcpy(gP, dP, n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gM, dM, S * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gm, dm, S * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gv, dv, S * 4, hipMemcpyDeviceToHost));
    const int p_ok = memcmp(gP + b, oP, S * 2) == 0;
    const int outside_ok = memcmp(gP, hP, b * 2) == 0 && memcmp(gP + e, hP + e, (n - e) * 2) == 0;
    const int state_ok = memcmp(gM, oM, S * 4) == 0 && memcmp(gm, om, S * 4) == 0 && memcmp(gv, ov, S * 4) == 0;
    printf("%s bf16 params equal the oracle's bit for bit after 3 steps\n", p_ok ? "ok  " : "FAIL");
    printf("%s params outside the shard untouched\n", outside_ok ? "ok  " : "FAIL");
    printf("%s master, m, v equal the oracle's bit for bit\n", state_ok ? "ok  " : "FAIL");
    failures += !p_ok + !outside_ok + !state_ok;

    /* resume-time rebuild: the master and the last seed give the same bf16 */
    HIP_OK(hipMemset(dP + b, 0, S * 2));
    BFO_OK_(master_to_bf16_sr(tb, dM, dP + b, seed, stream));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(rebuilt, dP + b, S * 2, hipMemcpyDeviceToHost));
    uint16_t *orebuilt = malloc(S * 2);
    if (!orebuilt) return 1;
    oracle_master_to_bf16_sr(oM, b, S, seed, orebuilt);
    const int rb_ok = memcmp(rebuilt, oP, S * 2) == 0 && memcmp(orebuilt, oP, S * 2) == 0;
    printf("%s master_to_bf16_sr rebuilds the last step's bf16 params (GPU and oracle)\n", rb_ok ? "ok  " : "FAIL");
    failures += !rb_ok;

    /* the allocation-free norm and the one-call step, on copies of the state:
     * the same bits as grad_global_norm and as the two calls */
    {
        bfo_norm_result *dres2, *dres3;
        uint16_t *dP2, *dP3;
        float *dS2, *dS3;   /* master, m, v of each copy, each on a 16-byte boundary */
        const uint64_t Sp = (S + 3) / 4 * 4;
        HIP_OK(hipMalloc((void **)&dres2, sizeof(bfo_norm_result)));
        HIP_OK(hipMalloc((void **)&dres3, sizeof(bfo_norm_result)));
        HIP_OK(hipMalloc((void **)&dP2, n * 2));
        HIP_OK(hipMalloc((void **)&dP3, n * 2));
        HIP_OK(hipMalloc((void **)&dS2, 3 * Sp * 4));
        HIP_OK(hipMalloc((void **)&dS3, 3 * Sp * 4));
        HIP_OK(hipMemcpy(dP2, dP, n * 2, hipMemcpyDeviceToDevice));
        HIP_OK(hipMemcpy(dP3, dP, n * 2, hipMemcpyDeviceToDevice));
        const float *src[3] = {dM, dm, dv};
        for (int a = 0; a < 3; ++a) {
            HIP_OK(hipMemcpy(dS2 + a * Sp, src[a], S * 4, hipMemcpyDeviceToDevice));
            HIP_OK(hipMemcpy(dS3 + a * Sp, src[a], S * 4, hipMemcpyDeviceToDevice));
        }
        BFO_OK_(grad_global_norm(tb, dG, 1.0f, dws, dres2, stream));
        BFO_OK_(grad_global_norm_noalloc(tb, dG, 1.0f, dres3, stream));
        bfo_norm_result r2, r3;
        HIP_OK(hipMemcpyAsync(&r2, dres2, sizeof r2, hipMemcpyDeviceToHost, stream));
        HIP_OK(hipMemcpyAsync(&r3, dres3, sizeof r3, hipMemcpyDeviceToHost, stream));
        HIP_OK(hipStreamSynchronize(stream));
        const int na_ok = memcmp(&r2, &r3, sizeof r2) == 0;
        printf("%s grad_global_norm_noalloc gives grad_global_norm's bits\n", na_ok ? "ok  " : "FAIL");
        failures += !na_ok;
        const uint64_t t7 = 7, seed7 = (1337ull << 32) | 7;
        BFO_OK_(adamw_sr_step(tb, dP2 + b, dG, dS2, dS2 + Sp, dS2 + 2 * Sp, &hp, &dres2->scale, NULL, t7, seed7,
                              BFO_ROUND_SR, stream));
        BFO_OK_(adamw_sr_step_with_norm(tb, dP3 + b, dG, dS3, dS3 + Sp, dS3 + 2 * Sp, &hp, 1.0f, dws, dres3, NULL,
                                        t7, seed7, BFO_ROUND_SR, stream));
        HIP_OK(hipStreamSynchronize(stream));
        uint16_t *c2 = malloc(n * 2), *c3 = malloc(n * 2);
        float *s2 = malloc(3 * Sp * 4), *s3 = malloc(3 * Sp * 4);
        if (!c2 || !c3 || !s2 || !s3) return 1;
        HIP_OK(hipMemcpy(c2, dP2, n * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(c3, dP3, n * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(s2, dS2, 3 * Sp * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(s3, dS3, 3 * Sp * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(&r3, dres3, sizeof r3, hipMemcpyDeviceToHost));
        int state_same = 1;
        for (int a = 0; a < 3; ++a) state_same &= memcmp(s2 + a * Sp, s3 + a * Sp, S * 4) == 0;
        const int oc_ok = memcmp(c2, c3, n * 2) == 0 && state_same &&
                          memcmp(&r2, &r3, sizeof r2) == 0 && memcmp(c2, gP, n * 2) != 0;
        printf("%s adamw_sr_step_with_norm gives the two calls' bits (norm, params, master, m, v)\n",
               oc_ok ? "ok  " : "FAIL");
        failures += !oc_ok;
        free(c2); free(c3); free(s2); free(s3);
        HIP_OK(hipFree(dres2));
        HIP_OK(hipFree(dres3));
        HIP_OK(hipFree(dP2));
        HIP_OK(hipFree(dP3));
        HIP_OK(hipFree(dS2));
        HIP_OK(hipFree(dS3));
    }

    /* steps 4..6 from a graph: per-step scalars in device memory, a cursor */
    bfo_step_scalars hsteps[3];
    for (int k = 0; k < 3; ++k) BFO_OK_(bfo_step_scalars_fill(&hp, 4 + k, hp.lr, (1337ull << 32) | (4 + k), &hsteps[k]));
    bfo_step_scalars *dsteps;
    uint64_t *dcursor;
    HIP_OK(hipMalloc((void **)&dsteps, sizeof hsteps));
    HIP_OK(hipMalloc((void **)&dcursor, sizeof(uint64_t)));
    HIP_OK(hipMemcpy(dsteps, hsteps, sizeof hsteps, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(dcursor, 0, sizeof(uint64_t)));
    hipGraph_t graph;
    hipGraphExec_t exec;
    HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
    BFO_OK_(grad_global_norm(tb, dG, 1.0f, NULL, dres, stream));
    BFO_OK_(adamw_sr_step_scheduled(tb, dP + b, dG, dM, dm, dv, &hp, dsteps, 3, dcursor, &dres->scale, NULL,
                                    BFO_ROUND_SR, stream));
    BFO_OK_(bfo_cursor_advance(dcursor, stream));
    HIP_OK(hipStreamEndCapture(stream, &graph));
    HIP_OK(hipGraphInstantiateWithFlags(&exec, graph, 0));
    for (uint64_t t = 4; t <= 6; ++t) {
        seed = (1337ull << 32) | t;
        for (uint64_t j = 0; j < S; ++j) hG[j] = bf16_from(mix64((t << 40) ^ (b + j)), 0.02f);
        HIP_OK(hipMemcpyAsync(dG, hG, S * 2, hipMemcpyHostToDevice, stream));
        HIP_OK(hipGraphLaunch(exec, stream));
        bfo_norm_result res;
        HIP_OK(hipMemcpyAsync(&res, dres, sizeof res, hipMemcpyDeviceToHost, stream));
        HIP_OK(hipStreamSynchronize(stream));
        double osum;
        float onorm, oscale;
        oracle_grad_norm(hG, S, 1.0f, &osum, &onorm, &oscale);
        const double rel = res.sumsq > osum ? (res.sumsq - osum) / osum : (osum - res.sumsq) / osum;
        const int norm_ok = rel <= 1e-12 && res.scale < 1.0f;
        printf("%s graph replay, step %llu: sumsq %.17g vs oracle %.17g\n", norm_ok ? "ok  " : "FAIL",
               (unsigned long long)t, res.sumsq, osum);
        failures += !norm_ok;
        if (oracle_adamw_step(otab, 3, b, S, oP, hG, oM, om, ov, &ohp, res.scale, t, seed, BFO_ROUND_SR) != 0) {
            printf("FAIL oracle_adamw_step\n");
            return 1;
        }
    }
    uint64_t cursor = 0;
    HIP_OK(hipMemcpy(&cursor, dcursor, sizeof cursor, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gP, dP, n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gM, dM, S * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gm, dm, S * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gv, dv, S * 4, hipMemcpyDeviceToHost));
    const int graph_ok = cursor == 3 && memcmp(gP + b, oP, S * 2) == 0 && memcmp(gM, oM, S * 4) == 0 &&
                         memcmp(gm, om, S * 4) == 0 && memcmp(gv, ov, S * 4) == 0 &&
                         memcmp(gP, hP, b * 2) == 0 && memcmp(gP + e, hP + e, (n - e) * 2) == 0;
    printf("%s after 3 graph replays: params, master, m, v equal the oracle's bit for bit, cursor %llu\n",
           graph_ok ? "ok  " : "FAIL", (unsigned long long)cursor);
    failures += !graph_ok;
    HIP_OK(hipGraphExecDestroy(exec));
    HIP_OK(hipGraphDestroy(graph));
    HIP_OK(hipFree(dsteps));
    HIP_OK(hipFree(dcursor));

    BFO_OK_(bfo_table_destroy(tb));
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(dP));
    HIP_OK(hipFree(dG));
    HIP_OK(hipFree(dM));
    HIP_OK(hipFree(dm));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(dres));
    HIP_OK(hipFree(dws));
    free(hP); free(hG); free(oP); free(gP); free(hM); free(oM); free(om); free(ov);
    free(gM); free(gm); free(gv); free(rebuilt); free(orebuilt);
    return failures ? 1 : 0;
}
