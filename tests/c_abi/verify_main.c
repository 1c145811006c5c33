/* A caller of the C ABI with no Python and no framework: HIP runtime calls
 * for device memory and a stream, then sv_workspace_bytes, sv_verify and
 * sv_accept_histogram.  Checks the structure of the outputs (an accepted
 * prefix equal to the drafts, one token in range, -1 after it), that the
 * histogram counts n_accepted, and that a repeated call is bit-identical.
 * Exit status 0 on success.  Built by tests/test_c_abi.py. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "specverify.h"

#define CHECK(x)                                                              \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
            return 2;                                                         \
        }                                                                     \
    } while (0)

/* xorshift64*: a seeded stand-in for logits, uniform in [-4, 4) */
static float next_logit(uint64_t *s) {
    *s ^= *s >> 12;
    *s ^= *s << 25;
    *s ^= *s >> 27;
    const uint64_t r = *s * 2685821657736338717ull;
    return (float)((r >> 40) * (1.0 / 16777216.0)) * 8.0f - 4.0f;
}

int main(void) {
    const int32_t B = 64, G = 4, V = 5003;
    const size_t nt = (size_t)B * (G + 1) * V, nd = (size_t)B * G * V;
    float *ht = malloc(nt * sizeof(float)), *hd = malloc(nd * sizeof(float));
    int32_t *htok = malloc((size_t)B * G * sizeof(int32_t));
    uint64_t s = 0x9E3779B97F4A7C15ull;
    for (size_t i = 0; i < nt; ++i) ht[i] = next_logit(&s);
    for (size_t i = 0; i < nd; ++i) hd[i] = ht[(i / V / G) * (G + 1) * V + (i % ((size_t)G * V))] + 0.3f * next_logit(&s);
    for (int i = 0; i < B * G; ++i) htok[i] = (int32_t)((next_logit(&s) + 4.0f) / 8.0f * V) % V;

    float *dt, *dd;
    int32_t *dtok, *dout, *dn, *dhist;
    void *ws;
    const size_t wsb = sv_workspace_bytes(B, G, V, 0, SV_F32);
    if (wsb == 0) { fprintf(stderr, "workspace size 0\n"); return 1; }
    CHECK(hipMalloc((void **)&dt, nt * sizeof(float)));
    CHECK(hipMalloc((void **)&dd, nd * sizeof(float)));
    CHECK(hipMalloc((void **)&dtok, (size_t)B * G * sizeof(int32_t)));
    CHECK(hipMalloc((void **)&dout, (size_t)B * (G + 1) * sizeof(int32_t)));
    CHECK(hipMalloc((void **)&dn, (size_t)B * sizeof(int32_t)));
    CHECK(hipMalloc((void **)&dhist, (size_t)(G + 2) * sizeof(int32_t)));
    CHECK(hipMalloc(&ws, wsb));
    CHECK(hipMemcpy(dt, ht, nt * sizeof(float), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dd, hd, nd * sizeof(float), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dtok, htok, (size_t)B * G * sizeof(int32_t), hipMemcpyHostToDevice));
    hipStream_t st;
    CHECK(hipStreamCreate(&st));

    int32_t *out[2], *n[2], hist[66];
    for (int call = 0; call < 2; ++call) {
        sv_status r = sv_verify(dt, dd, dtok, B, G, V, SV_F32, 0.9f, 0, 1.0f, 1234u, 0u, dout, dn, ws, wsb, st);
        if (r != SV_OK) { fprintf(stderr, "sv_verify: %s\n", sv_status_string(r)); return 1; }
        r = sv_accept_histogram(dn, B, G, dhist, st);
        if (r != SV_OK) { fprintf(stderr, "sv_accept_histogram: %s\n", sv_status_string(r)); return 1; }
        CHECK(hipStreamSynchronize(st));
        out[call] = malloc((size_t)B * (G + 1) * sizeof(int32_t));
        n[call] = malloc((size_t)B * sizeof(int32_t));
        CHECK(hipMemcpy(out[call], dout, (size_t)B * (G + 1) * sizeof(int32_t), hipMemcpyDeviceToHost));
        CHECK(hipMemcpy(n[call], dn, (size_t)B * sizeof(int32_t), hipMemcpyDeviceToHost));
        CHECK(hipMemcpy(hist, dhist, (size_t)(G + 2) * sizeof(int32_t), hipMemcpyDeviceToHost));
    }
    int count[66] = {0};
    for (int b = 0; b < B; ++b) {
        const int k = n[0][b];
        if (k < 0 || k > G) { fprintf(stderr, "n[%d] = %d\n", b, k); return 1; }
        count[k + 1]++;
        for (int i = 0; i < k; ++i)
            if (out[0][b * (G + 1) + i] != htok[b * G + i]) { fprintf(stderr, "prefix of %d\n", b); return 1; }
        const int t = out[0][b * (G + 1) + k];
        if (t < 0 || t >= V) { fprintf(stderr, "token of %d: %d\n", b, t); return 1; }
        for (int i = k + 1; i <= G; ++i)
            if (out[0][b * (G + 1) + i] != -1) { fprintf(stderr, "padding of %d\n", b); return 1; }
    }
    for (int i = 0; i < G + 2; ++i)
        if (hist[i] != count[i]) { fprintf(stderr, "histogram bin %d: %d != %d\n", i, hist[i], count[i]); return 1; }
    if (memcmp(out[0], out[1], (size_t)B * (G + 1) * sizeof(int32_t)) || memcmp(n[0], n[1], (size_t)B * sizeof(int32_t))) {
        fprintf(stderr, "repeated call differs\n");
        return 1;
    }
    printf("c abi ok: %s; n histogram", sv_version());
    for (int i = 0; i < G + 2; ++i) printf(" %d", hist[i]);
    printf("\n");
    return 0;
}
