/*
 * A plain C99 program that uses the library through include/tree_attn.h only:
 * device memory from the HIP runtime's C API, descriptors filled by hand, no
 * Python and no torch. It checks results that have a closed form:
 *
 *  1. Constant keys: every logit of a row is equal, so the softmax weights are
 *     uniform and out is the mean of the V rows over the sequence's tokens, with
 *     lse = s + ln n ("Core Innovation 2" of "Tree Attention Guide:
 *     Topology-Aware LLM Decoding": the softmax over the row). A ragged batch
 *     with a GQA group of 4 and a chunk that does not divide n.
 *  2. A sequence of length 0: out = 0 and lse = -inf.
 *  3. ta_combine of one state is that state, and of two states with equal lse
 *     is their mean with lse + ln 2 (the merge operator of the same section).
 *  4. Validation: chunk 0 is refused with TA_ERR_ARG and a message, before any
 *     launch.
 *  5. ta_partial followed by ta_combine reproduces ta_decode bit for bit (the
 *     same states merged by the same tree), on the ragged batch of check 1 with
 *     random keys.
 *  6. ta_combine_k (arity 8) and ta_combine_chain give the mean of two states of
 *     equal lse, with lse + ln 2, like ta_combine.
 *  7. ta_stream_read refuses a NULL buffer and a size that is not a multiple of
 *     16 bytes, before any launch, and reads a valid buffer.
 *
 * Exit status 0 when every check holds; it prints what failed otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tree_attn.h"

static int failures = 0;

#define CHECK(cond, ...)                      \
    do {                                      \
        if (!(cond)) {                        \
            fprintf(stderr, "FAIL: ");        \
            fprintf(stderr, __VA_ARGS__);     \
            fprintf(stderr, "\n");            \
            ++failures;                       \
        }                                     \
    } while (0)

#define HIP(x)                                                                       \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

/* A descriptor of a contiguous tensor. */
static ta_tensor contiguous(void* data, ta_dtype dtype, int ndim, const int64_t* shape) {
    ta_tensor t;
    memset(&t, 0, sizeof t);
    t.data = data;
    t.dtype = dtype;
    t.ndim = ndim;
    int64_t acc = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        t.shape[i] = shape[i];
        t.stride[i] = acc;
        acc *= shape[i];
    }
    return t;
}

static void* device_alloc(size_t bytes) {
    void* dev = NULL;
    HIP(hipMalloc(&dev, bytes ? bytes : 16));
    return dev;
}

static void* upload(const void* host, size_t bytes) {
    void* dev = device_alloc(bytes);
    if (bytes) HIP(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
    return dev;
}

static float value_at(int b, int g, int j, int c) {  /* a V entry with no pattern the mean could hide */
    return (float)sin(0.37 * (b + 1) + 0.11 * (g + 1) * (j + 1) + 0.013 * c * (j % 7 + 1));
}

static void check_constant_keys(void) {
    enum { B = 3, HQ = 8, HKV = 2, N = 1000, D = 128, CHUNK = 64 };
    const int32_t lens[B] = {1000, 377, 0};
    const size_t nq = (size_t)B * HQ * D, nkv = (size_t)B * HKV * N * D;
    float* q = malloc(nq * sizeof(float));
    float* k = malloc(nkv * sizeof(float));
    float* v = malloc(nkv * sizeof(float));
    for (size_t i = 0; i < nq; ++i) q[i] = 0.5f;
    for (size_t i = 0; i < nkv; ++i) k[i] = 1.0f;
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < HKV; ++g)
            for (int j = 0; j < N; ++j)
                for (int c = 0; c < D; ++c) v[(((size_t)b * HKV + g) * N + j) * D + c] = value_at(b, g, j, c);

    void* dq = upload(q, nq * sizeof(float));
    void* dk = upload(k, nkv * sizeof(float));
    void* dv = upload(v, nkv * sizeof(float));
    void* dl = upload(lens, sizeof lens);
    void* dout = device_alloc((size_t)B * HQ * D * sizeof(float));
    void* dlse = device_alloc((size_t)B * HQ * sizeof(float));

    const int64_t sq[3] = {B, HQ, D}, skv[4] = {B, HKV, N, D}, so[3] = {B, HQ, D}, sl[2] = {B, HQ};
    ta_tensor tq = contiguous(dq, TA_F32, 3, sq), tk = contiguous(dk, TA_F32, 4, skv),
              tv = contiguous(dv, TA_F32, 4, skv), to = contiguous(dout, TA_F32, 3, so),
              tl = contiguous(dlse, TA_F32, 2, sl);
    int rc = ta_decode(&tq, &tk, &tv, (const int32_t*)dl, &to, &tl, CHUNK, NULL);
    CHECK(rc == TA_OK, "ta_decode returned %d: %s", rc, ta_last_error());
    HIP(hipDeviceSynchronize());

    float* out = malloc((size_t)B * HQ * D * sizeof(float));
    float lse[B * HQ];
    HIP(hipMemcpy(out, dout, (size_t)B * HQ * D * sizeof(float), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(lse, dlse, sizeof lse, hipMemcpyDeviceToHost));

    const double s = 0.5 * D / sqrt((double)D);  /* q . k / sqrt(d), the same for every token */
    double worst = 0.0, worst_lse = 0.0;
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < HQ; ++h) {
            const int g = h / (HQ / HKV), n = lens[b];
            const float* o = out + ((size_t)b * HQ + h) * D;
            if (n == 0) {
                CHECK(isinf(lse[b * HQ + h]) && lse[b * HQ + h] < 0, "empty sequence: lse %g", lse[b * HQ + h]);
                for (int c = 0; c < D; ++c) CHECK(o[c] == 0.0f, "empty sequence: out[%d] = %g", c, o[c]);
                continue;
            }
            for (int c = 0; c < D; ++c) {
                double mean = 0.0;
                for (int j = 0; j < n; ++j) mean += v[(((size_t)b * HKV + g) * N + j) * D + c];
                mean /= n;
                const double err = fabs(o[c] - mean);
                if (err > worst) worst = err;
            }
            const double want = s + log((double)n);
            const double lerr = fabs(lse[b * HQ + h] - want) / fabs(want);
            if (lerr > worst_lse) worst_lse = lerr;
        }
    }
    CHECK(worst <= 1e-5, "constant keys: max |out - mean of V| = %g", worst);
    CHECK(worst_lse <= 1e-4, "constant keys: max relative lse error = %g", worst_lse);
    printf("constant keys, GQA 8/2, lengths 1000/377/0, chunk 64: max |out - mean| %.2e, lse rel %.2e\n", worst,
           worst_lse);

    /* validation happens before any launch */
    rc = ta_decode(&tq, &tk, &tv, (const int32_t*)dl, &to, &tl, 0, NULL);
    CHECK(rc == TA_ERR_ARG && strlen(ta_last_error()) > 0, "chunk 0: rc %d, message '%s'", rc, ta_last_error());

    HIP(hipFree(dq)); HIP(hipFree(dk)); HIP(hipFree(dv)); HIP(hipFree(dl)); HIP(hipFree(dout)); HIP(hipFree(dlse));
    free(q); free(k); free(v); free(out);
}

static void check_partial_then_combine(void) {
    enum { B = 3, HQ = 8, HKV = 2, N = 1000, D = 128, CHUNK = 64, P = (N + CHUNK - 1) / CHUNK };
    const int32_t lens[B] = {1000, 377, 0};
    const size_t nq = (size_t)B * HQ * D, nkv = (size_t)B * HKV * N * D;
    float* q = malloc(nq * sizeof(float));
    float* k = malloc(nkv * sizeof(float));
    float* v = malloc(nkv * sizeof(float));
    for (size_t i = 0; i < nq; ++i) q[i] = (float)sin(0.7 * i + 0.1);
    for (size_t i = 0; i < nkv; ++i) k[i] = (float)cos(0.31 * i + 0.2);
    for (size_t i = 0; i < nkv; ++i) v[i] = (float)sin(0.17 * i + 0.3);
    void* dq = upload(q, nq * sizeof(float));
    void* dk = upload(k, nkv * sizeof(float));
    void* dv = upload(v, nkv * sizeof(float));
    void* dl = upload(lens, sizeof lens);
    void* dpo = device_alloc((size_t)B * HQ * P * D * sizeof(float));
    void* dpl = device_alloc((size_t)B * HQ * P * sizeof(float));
    void* dout1 = device_alloc(nq * sizeof(float));
    void* dlse1 = device_alloc((size_t)B * HQ * sizeof(float));
    void* dout2 = device_alloc(nq * sizeof(float));
    void* dlse2 = device_alloc((size_t)B * HQ * sizeof(float));
    const int64_t sq[3] = {B, HQ, D}, skv[4] = {B, HKV, N, D}, spo[4] = {B, HQ, P, D}, spl[3] = {B, HQ, P},
                  sl[2] = {B, HQ};
    ta_tensor tq = contiguous(dq, TA_F32, 3, sq), tk = contiguous(dk, TA_F32, 4, skv),
              tv = contiguous(dv, TA_F32, 4, skv), tpo = contiguous(dpo, TA_F32, 4, spo),
              tpl = contiguous(dpl, TA_F32, 3, spl), to1 = contiguous(dout1, TA_F32, 3, sq),
              tl1 = contiguous(dlse1, TA_F32, 2, sl), to2 = contiguous(dout2, TA_F32, 3, sq),
              tl2 = contiguous(dlse2, TA_F32, 2, sl);
    int rc = ta_partial(&tq, &tk, &tv, (const int32_t*)dl, &tpo, &tpl, CHUNK, NULL);
    CHECK(rc == TA_OK, "ta_partial returned %d: %s", rc, ta_last_error());
    rc = ta_combine(&tpo, &tpl, P, &to1, &tl1, NULL);
    CHECK(rc == TA_OK, "ta_combine returned %d: %s", rc, ta_last_error());
    rc = ta_decode(&tq, &tk, &tv, (const int32_t*)dl, &to2, &tl2, CHUNK, NULL);
    CHECK(rc == TA_OK, "ta_decode returned %d: %s", rc, ta_last_error());
    HIP(hipDeviceSynchronize());
    float* o1 = malloc(nq * sizeof(float));
    float* o2 = malloc(nq * sizeof(float));
    float l1[B * HQ], l2[B * HQ];
    HIP(hipMemcpy(o1, dout1, nq * sizeof(float), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(o2, dout2, nq * sizeof(float), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(l1, dlse1, sizeof l1, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(l2, dlse2, sizeof l2, hipMemcpyDeviceToHost));
    CHECK(memcmp(o1, o2, nq * sizeof(float)) == 0, "ta_combine(ta_partial) out differs from ta_decode");
    CHECK(memcmp(l1, l2, sizeof l1) == 0, "ta_combine(ta_partial) lse differs from ta_decode");
    printf("ta_partial + ta_combine reproduce ta_decode bit for bit (ragged batch, %d chunks)\n", P);
    HIP(hipFree(dq)); HIP(hipFree(dk)); HIP(hipFree(dv)); HIP(hipFree(dl)); HIP(hipFree(dpo)); HIP(hipFree(dpl));
    HIP(hipFree(dout1)); HIP(hipFree(dlse1)); HIP(hipFree(dout2)); HIP(hipFree(dlse2));
    free(q); free(k); free(v); free(o1); free(o2);
}

static void check_stream_read(void) {
    const size_t bytes = 1 << 20;
    void* buf = device_alloc(bytes);
    void* sink = device_alloc(sizeof(uint32_t));
    HIP(hipMemset(buf, 0, bytes));
    int rc = ta_stream_read(NULL, 16, (uint32_t*)sink, NULL);
    CHECK(rc == TA_ERR_NULL && strlen(ta_last_error()) > 0, "stream_read(NULL): rc %d", rc);
    rc = ta_stream_read(buf, 17, (uint32_t*)sink, NULL);
    CHECK(rc == TA_ERR_ARG && strlen(ta_last_error()) > 0, "stream_read(17 bytes): rc %d", rc);
    rc = ta_stream_read(buf, (int64_t)bytes, (uint32_t*)sink, NULL);
    CHECK(rc == TA_OK, "stream_read(1 MiB) returned %d: %s", rc, ta_last_error());
    HIP(hipDeviceSynchronize());
    printf("ta_stream_read: NULL and ragged sizes refused, 1 MiB read\n");
    HIP(hipFree(buf)); HIP(hipFree(sink));
}

static void check_combine(void) {
    enum { H = 3, P = 2, D = 64 };
    float o[H * P * D], l[H * P];
    for (int i = 0; i < H * P * D; ++i) o[i] = (float)cos(0.1 * i);
    for (int h = 0; h < H; ++h) l[h * P] = l[h * P + 1] = 2.5f + h;
    void* dpo = upload(o, sizeof o);
    void* dpl = upload(l, sizeof l);
    void* dout = device_alloc(H * D * sizeof(float));
    void* dlse = device_alloc(H * sizeof(float));
    const int64_t spo[4] = {1, H, P, D}, spl[3] = {1, H, P}, so[3] = {1, H, D}, sl[2] = {1, H};
    ta_tensor tpo = contiguous(dpo, TA_F32, 4, spo), tpl = contiguous(dpl, TA_F32, 3, spl),
              to = contiguous(dout, TA_F32, 3, so), tl = contiguous(dlse, TA_F32, 2, sl);
    float out[H * D], lse[H];

    int rc = ta_combine(&tpo, &tpl, 1, &to, &tl, NULL);  /* one state: the identity */
    CHECK(rc == TA_OK, "ta_combine(1) returned %d: %s", rc, ta_last_error());
    HIP(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(lse, dlse, sizeof lse, hipMemcpyDeviceToHost));
    for (int h = 0; h < H; ++h) {
        CHECK(lse[h] == l[h * P], "n_parts 1: lse %g != %g", lse[h], l[h * P]);
        for (int c = 0; c < D; ++c)
            CHECK(out[h * D + c] == o[(h * P) * D + c], "n_parts 1: out differs at head %d, channel %d", h, c);
    }

    rc = ta_combine(&tpo, &tpl, 2, &to, &tl, NULL);  /* equal lse: the mean, lse + ln 2 */
    CHECK(rc == TA_OK, "ta_combine(2) returned %d: %s", rc, ta_last_error());
    HIP(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(lse, dlse, sizeof lse, hipMemcpyDeviceToHost));
    double worst = 0.0;
    for (int h = 0; h < H; ++h) {
        CHECK(fabs(lse[h] - (l[h * P] + log(2.0))) <= 1e-6 * fabs(l[h * P] + log(2.0)), "n_parts 2: lse %g", lse[h]);
        for (int c = 0; c < D; ++c) {
            const double mean = 0.5 * ((double)o[(h * P) * D + c] + (double)o[(h * P + 1) * D + c]);
            const double err = fabs(out[h * D + c] - mean);
            if (err > worst) worst = err;
        }
    }
    CHECK(worst <= 1e-6, "n_parts 2: max |out - mean| = %g", worst);
    printf("ta_combine: one state is the identity, two equal-lse states give the mean (max err %.2e)\n", worst);

    for (int which = 0; which < 2; ++which) {  /* the arity-8 tree and the chain, the same two states */
        rc = which == 0 ? ta_combine_k(&tpo, &tpl, 2, 8, &to, &tl, NULL) : ta_combine_chain(&tpo, &tpl, 2, &to, &tl, NULL);
        const char* name = which == 0 ? "ta_combine_k(arity 8)" : "ta_combine_chain";
        CHECK(rc == TA_OK, "%s returned %d: %s", name, rc, ta_last_error());
        HIP(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(lse, dlse, sizeof lse, hipMemcpyDeviceToHost));
        double w = 0.0;
        for (int h = 0; h < H; ++h) {
            CHECK(fabs(lse[h] - (l[h * P] + log(2.0))) <= 1e-6 * fabs(l[h * P] + log(2.0)), "%s: lse %g", name, lse[h]);
            for (int c = 0; c < D; ++c) {
                const double mean = 0.5 * ((double)o[(h * P) * D + c] + (double)o[(h * P + 1) * D + c]);
                const double err = fabs(out[h * D + c] - mean);
                if (err > w) w = err;
            }
        }
        CHECK(w <= 1e-6, "%s: max |out - mean| = %g", name, w);
        printf("%s: two equal-lse states give the mean (max err %.2e)\n", name, w);
    }
    HIP(hipFree(dpo)); HIP(hipFree(dpl)); HIP(hipFree(dout)); HIP(hipFree(dlse));
}

int main(void) {
    printf("tree_attn ABI version %d\n", ta_version());
    check_constant_keys();
    check_partial_then_combine();
    check_combine();
    check_stream_read();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("all checks passed\n");
    return 0;
}
