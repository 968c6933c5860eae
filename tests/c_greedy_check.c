/*
 * A plain C caller of libspecverify: device memory from the HIP runtime, one
 * greedy-chain verification on the null stream, and the result checked
 * against the greedy rule itself (keep drafts while each equals the argmax of
 * the row that scores it, lowest id on ties; then emit that row's argmax).
 * Exits 0 when every output matches.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify.h"

enum { B = 16, K = 5, V = 3001, R = K + 1 };

static uint32_t next(uint32_t *s) {
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

static float bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* an exactly representable bf16 value: k / 16 for an integer k in [-128, 128] */
static uint16_t bf16_bits(int k) {
    float f = (float)k / 16.0f;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

#define CHECK(call)                                                          \
    do {                                                                     \
        hipError_t e_ = (call);                                              \
        if (e_ != hipSuccess) {                                              \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));      \
            return 3;                                                        \
        }                                                                    \
    } while (0)

int main(void) {
    static uint16_t L[B * R * V];
    static int32_t amax[B * R], x[B * K], n_want[B], tok_want[B * R], n_got[B], tok_got[B * R], st_got[B];
    uint32_t s = 20261202u;
    for (size_t i = 0; i < sizeof L / sizeof L[0]; ++i) L[i] = bf16_bits((int)(next(&s) % 257) - 128);
    for (int r = 0; r < B * R; ++r) {  /* first maximum (ties are frequent on this grid) */
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (bf16_value(L[(size_t)r * V + v]) > bf16_value(L[(size_t)r * V + best])) best = v;
        amax[r] = best;
    }
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < K; ++i)
            x[b * K + i] = (next(&s) % 4 != 0) ? amax[b * R + i] : (int32_t)(next(&s) % V);
        int n = K;
        for (int i = 0; i < K; ++i)
            if (x[b * K + i] != amax[b * R + i]) { n = i; break; }
        n_want[b] = n;
        for (int i = 0; i < R; ++i) tok_want[b * R + i] = i < n ? x[b * K + i] : (i == n ? amax[b * R + n] : -1);
    }

    void *dL, *dx, *dn, *dtok, *dst, *ws;
    const size_t ws_bytes = sv_greedy_workspace_bytes(B, R, V, SV_BF16);
    CHECK(hipMalloc(&dL, sizeof L));
    CHECK(hipMalloc(&dx, sizeof x));
    CHECK(hipMalloc(&dn, sizeof n_got));
    CHECK(hipMalloc(&dtok, sizeof tok_got));
    CHECK(hipMalloc(&dst, sizeof st_got));
    CHECK(hipMalloc(&ws, ws_bytes)); /* hipMalloc returns 256-byte aligned memory */
    CHECK(hipMemcpy(dL, L, sizeof L, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dx, x, sizeof x, hipMemcpyHostToDevice));
    const sv_status st = spec_verify_greedy(dL, (const int32_t *)dx, B, K, V, SV_BF16, (int32_t *)dn,
                                            (int32_t *)dtok, (int32_t *)dst, ws, ws_bytes, NULL);
    if (st != SV_OK) {
        fprintf(stderr, "spec_verify_greedy: %s\n", sv_status_string(st));
        return 2;
    }
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(n_got, dn, sizeof n_got, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(tok_got, dtok, sizeof tok_got, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(st_got, dst, sizeof st_got, hipMemcpyDeviceToHost));
    int bad = 0, accepted = 0;
    for (int b = 0; b < B; ++b) {
        accepted += n_got[b];
        if (n_got[b] != n_want[b] || st_got[b] != 0) ++bad;
        for (int i = 0; i < R; ++i)
            if (tok_got[b * R + i] != tok_want[b * R + i]) { ++bad; break; }
    }
    printf("c caller: B=%d K=%d V=%d, %d drafts accepted, %d requests differ\n", B, K, V, accepted, bad);
    hipFree(dL);
    hipFree(dx);
    hipFree(dn);
    hipFree(dtok);
    hipFree(dst);
    hipFree(ws);
    return bad == 0 ? 0 : 1;
}
