/* Drives the oracle under AddressSanitizer/UndefinedBehaviorSanitizer on
 * ordinary, boundary and non-finite inputs of every function. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_decode_m_e4(uint16_t);
uint16_t oracle_encode_m_e4(float);
float oracle_decode_r_e4(uint16_t);
uint16_t oracle_encode_r_e4(float);
float oracle_decode_f16(uint16_t);
uint16_t oracle_encode_f16(float);
float oracle_decode_bf16(uint16_t);
uint16_t oracle_encode_bf16(float);
void oracle_scalars(double, double, double, double, double, long long, float[8]);
unsigned long long oracle_step_fp32(float*, const float*, float*, float*, size_t, const float[8]);
unsigned long long oracle_step_packed(int, float*, const float*, uint32_t*, size_t, const float[8]);
unsigned long long oracle_step_typed(int, int, int, void*, const void*, void*, void*, size_t, const float[8]);
unsigned long long oracle_step_blockwise(const float*, const float*, uint8_t*, float*, uint8_t*, float*,
                                         const float*, const float*, uint16_t*, size_t, const float[8]);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng ^= rng << 13; rng ^= rng >> 17; rng ^= rng << 5; return rng; }
static float bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

int main(void) {
    unsigned long long sink = 0;
    for (uint32_t c = 0; c < 65536; ++c) {
        sink += oracle_encode_m_e4(oracle_decode_m_e4((uint16_t)c));
        sink += oracle_encode_r_e4(oracle_decode_r_e4((uint16_t)c));
        sink += oracle_encode_f16(oracle_decode_f16((uint16_t)c));
        sink += oracle_encode_bf16(oracle_decode_bf16((uint16_t)c));
    }
    for (int i = 0; i < 200000; ++i) {
        float x = bits(next());
        sink += oracle_encode_m_e4(x) + oracle_encode_r_e4(x) + oracle_encode_f16(x) + oracle_encode_bf16(x);
    }
    enum { N = 3 * 2048 };
    float s[8];
    oracle_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 3, s);
    float* p = malloc(N * sizeof(float));
    float* g = malloc(N * sizeof(float));
    float* m = malloc(N * sizeof(float));
    float* v = malloc(N * sizeof(float));
    uint32_t* w = malloc(N * sizeof(uint32_t));
    uint16_t* h = malloc(N * sizeof(uint16_t));
    uint16_t* hg = malloc(N * sizeof(uint16_t));
    for (int i = 0; i < N; ++i) {
        p[i] = (float)((int)(next() % 2001) - 1000) * 1e-5f;
        g[i] = i % 97 == 0 ? NAN : i % 89 == 0 ? INFINITY : bits(next() & 0xBFFFFFFFu) * 1e-20f;
        m[i] = 0.0f;
        v[i] = 0.0f;
        w[i] = next();
        h[i] = oracle_encode_bf16(p[i]);
        hg[i] = oracle_encode_bf16(g[i]);
    }
    sink += oracle_step_fp32(p, g, m, v, N, s);
    sink += oracle_step_packed(1, p, g, w, N, s);
    sink += oracle_step_packed(2, p, g, w, N, s);
    sink += oracle_step_typed(1, 1, 1, h, hg, w, NULL, N, s);
    sink += oracle_step_typed(0, 2, 0, h, g, m, v, N, s);
    float qm[256], qv[256], am[3] = {0}, av[3] = {0};
    for (int j = 0; j < 256; ++j) {
        qm[j] = -1.0f + 2.0f * (float)j / 255.0f;
        qv[j] = (float)j / 255.0f;
    }
    uint8_t* mc = calloc(N, 1);
    uint8_t* vc = calloc(N, 1);
    sink += oracle_step_blockwise(p, g, mc, am, vc, av, qm, qv, h, N, s);
    sink += oracle_step_blockwise(p, g, mc, am, vc, av, qm, qv, h, N - 7, s);   /* rejected length */
    free(p); free(g); free(m); free(v); free(w); free(h); free(hg); free(mc); free(vc);
    printf("oracle driver ok %llu\n", sink & 0xFF);
    return 0;
}
