/*
 * Exhaustive pins of the oracle's two scalar encoders over every finite fp32
 * bit pattern, each against an independent formulation:
 *   - E2M1 encode vs the round-to-nearest-even threshold table of the 8
 *     magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} (ties at the midpoints 0.25,
 *     0.75, 1.25, 1.75, 2.5, 3.5, 5 go to the even code; past 6 saturates);
 *   - bf16 round-to-nearest-even vs the integer add-and-shift formulation.
 * It also prints an order-independent checksum of the oracle's codes over
 * the same patterns, sum of (code + 1) * mix(pattern) mod 2^64 with mix the
 * splitmix64 finaliser (Vigna), which the device encoders are checked
 * against without moving 2^32 codes.
 * Usage: exhaustive <lib.so> <first_pattern> <count>; prints mismatch counts
 * and the checksums.
 */
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static unsigned table_e2m1(float v)
{
    float m = fabsf(v);
    unsigned c;
    if (m <= 0.25f) c = 0;
    else if (m < 0.75f) c = 1;
    else if (m <= 1.25f) c = 2;
    else if (m < 1.75f) c = 3;
    else if (m <= 2.5f) c = 4;
    else if (m < 3.5f) c = 5;
    else if (m <= 5.0f) c = 6;
    else c = 7;
    return c | (signbit(v) ? 8u : 0u);
}

static uint64_t mix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint16_t trick_bf16(uint32_t u)
{
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

int main(int argc, char **argv)
{
    if (argc < 4) return 2;
    void *h = dlopen(argv[1], RTLD_NOW);
    if (!h) { fprintf(stderr, "%s\n", dlerror()); return 2; }
    unsigned (*enc)(float) = (unsigned (*)(float))dlsym(h, "orc_e2m1_encode");
    uint16_t (*bf)(float) = (uint16_t (*)(float))dlsym(h, "orc_bf16_from_f32");
    uint64_t first = strtoull(argv[2], 0, 0), count = strtoull(argv[3], 0, 0);
    uint64_t bad_e = 0, bad_b = 0, tested = 0, sum_e = 0, sum_b = 0;
    #pragma omp parallel for reduction(+:bad_e,bad_b,tested,sum_e,sum_b) schedule(static, 65536)
    for (uint64_t i = first; i < first + count; ++i) {
        uint32_t u = (uint32_t)i;
        float x;
        memcpy(&x, &u, 4);
        if (!isfinite(x)) continue;
        ++tested;
        const unsigned ce = enc(x);
        const uint16_t cb = bf(x);
        if (ce != table_e2m1(x)) ++bad_e;
        if (cb != trick_bf16(u)) ++bad_b;
        const uint64_t m = mix64(u);
        sum_e += (uint64_t)(ce + 1) * m;
        sum_b += (uint64_t)(cb + 1u) * m;
    }
    printf("tested=%llu e2m1_mismatch=%llu bf16_mismatch=%llu\n", (unsigned long long)tested,
           (unsigned long long)bad_e, (unsigned long long)bad_b);
    printf("e2m1_sum=0x%016llx bf16_sum=0x%016llx\n", (unsigned long long)sum_e, (unsigned long long)sum_b);
    return (bad_e || bad_b) ? 1 : 0;
}
