/*
 * Seeded synthetic int32 inputs for the top-k / reduction workloads.
 *
 * This module holds no arithmetic of the method under test: it only draws
 * numbers.  Both the CPU oracle and the GPU path consume its output; neither
 * links it.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-style: element i
 * is the (i+1)-th output of a SplitMix64 stream whose state starts at
 * mix64(seed).  Any element can therefore be produced independently of the
 * others, which lets a large array be filled in parallel chunks.
 *
 * Value mapping from the high 32 bits h of the 64-bit output:
 *   range == 0 : the full int32 range, value = (int32_t)h (bit reinterpretation)
 *   range  > 0 : lo + floor(h * range / 2^32), i.e. [lo, lo + range)
 *                (Lemire's multiply-shift; bias at most range / 2^32).
 */
#include <stdint.h>
#include <pthread.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

typedef struct {
    uint64_t base;     /* mix64(seed) */
    int64_t begin, end;
    int32_t lo;
    uint32_t range;
    int32_t *out;
} chunk_t;

static void fill_chunk(const chunk_t *c)
{
    for (int64_t i = c->begin; i < c->end; ++i) {
        uint64_t v = sm64_mix(c->base + (uint64_t)(i + 1) * SM64_GAMMA);
        uint32_t h = (uint32_t)(v >> 32);
        if (c->range == 0)
            c->out[i] = (int32_t)h;
        else
            c->out[i] = c->lo + (int32_t)(((uint64_t)h * c->range) >> 32);
    }
}

static void *fill_thread(void *arg)
{
    fill_chunk((const chunk_t *)arg);
    return 0;
}

/* Fill out[0..n) with the seeded stream.  threads <= 1 runs inline.
 * Returns 0 on success, -1 on bad arguments. */
int synth_fill_i32(uint64_t seed, int64_t n, int32_t lo, uint32_t range,
                   int32_t *out, int threads)
{
    if (n < 0 || (n > 0 && !out))
        return -1;
    if (threads < 1)
        threads = 1;
    if (threads > 64)
        threads = 64;
    if (n < (int64_t)1 << 20)
        threads = 1;
    uint64_t base = sm64_mix(seed);
    chunk_t chunks[64];
    pthread_t tids[64];
    for (int t = 0; t < threads; ++t) {
        chunks[t].base = base;
        chunks[t].begin = n * t / threads;
        chunks[t].end = n * (t + 1) / threads;
        chunks[t].lo = lo;
        chunks[t].range = range;
        chunks[t].out = out;
    }
    if (threads == 1) {
        fill_chunk(&chunks[0]);
        return 0;
    }
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        if (pthread_create(&tids[t], 0, fill_thread, &chunks[t]) != 0)
            break;
        ++started;
    }
    for (int t = started; t < threads; ++t)
        fill_chunk(&chunks[t]);
    for (int t = 0; t < started; ++t)
        pthread_join(tids[t], 0);
    return 0;
}

/* Raw 64-bit output for element i (lets tests check the stream itself). */
uint64_t synth_raw_u64(uint64_t seed, int64_t i)
{
    return sm64_mix(sm64_mix(seed) + (uint64_t)(i + 1) * SM64_GAMMA);
}
