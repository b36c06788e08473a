/*
 * Seeded synthetic inputs for the attention tests and the bench.
 *
 * This file holds no attention arithmetic. It only turns (seed, stream, index)
 * into numbers, so that the CPU oracle and the HIP path can be fed the very same
 * bytes. Both sides consume the buffers it fills; neither side links it.
 *
 * Generator definition (published methods, restated):
 *   - SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): state advances by the golden gamma
 *     0x9e3779b97f4a7c15 and each output is the state passed through the
 *     "mix64" finaliser (xor-shift 30, multiply, xor-shift 27, multiply,
 *     xor-shift 31).
 *   - Counter-based use: the key of a stream is the (stream+1)-th SplitMix64
 *     output of a generator whose state starts at `seed`; draw i of the stream
 *     is the (i+1)-th SplitMix64 output of a generator whose state starts at
 *     that key. Every draw is therefore addressable without generating the
 *     ones before it, which is what lets OpenMP fill huge buffers in parallel.
 *   - Uniforms in (0, 1]: ((x >> 11) + 1) * 2^-53.
 *   - Normals: Box & Muller (1958). Pair p uses draws 2p and 2p+1 as u1, u2;
 *     element 2p is r*cos(2*pi*u2) and element 2p+1 is r*sin(2*pi*u2) with
 *     r = sqrt(-2 ln u1), all in double precision.
 *   - Narrowing: the double is rounded to float, multiplied by sigma in float,
 *     then rounded to bfloat16 with round-to-nearest-even on the bit pattern.
 *   - Integers in [lo, hi]: lo + draw mod (hi - lo + 1) (bias below 2^-40).
 *   - Permutations: Fisher & Yates (Durstenfeld's form), i from n-1 down to 1,
 *     j = draw_i mod (i + 1), swap a[i] and a[j], starting from the identity.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* (index+1)-th output of SplitMix64 started at `state`. */
static inline uint64_t sm64_at(uint64_t state, uint64_t index) {
    return mix64(state + (index + 1) * GOLDEN_GAMMA);
}

uint64_t gen_stream_key(uint64_t seed, uint64_t stream) { return sm64_at(seed, stream); }

uint64_t gen_draw(uint64_t seed, uint64_t stream, uint64_t index) {
    return sm64_at(sm64_at(seed, stream), index);
}

static inline double unit_open0(uint64_t x) {
    return (double)((x >> 11) + 1) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Element `e` of the stream's normal sequence, as double. */
static inline double normal_at(uint64_t key, uint64_t e) {
    uint64_t p = e >> 1;
    double u1 = unit_open0(sm64_at(key, 2 * p));
    double u2 = unit_open0(sm64_at(key, 2 * p + 1));
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    return (e & 1) ? r * sin(t) : r * cos(t);
}

/* out[i] = bf16(sigma * float(N(0,1) element offset+i)), i in [0, n). */
void gen_normal_bf16(uint64_t seed, uint64_t stream, float sigma, uint64_t offset, uint64_t n,
                     uint16_t* out) {
    uint64_t key = gen_stream_key(seed, stream);
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < nn; ++i) {
        float f = (float)normal_at(key, offset + (uint64_t)i);
        out[i] = f32_to_bf16_rne(f * sigma);
    }
}

/* Same sequence, kept in float (before the bf16 narrowing); used by tests. */
void gen_normal_f32(uint64_t seed, uint64_t stream, float sigma, uint64_t offset, uint64_t n,
                    float* out) {
    uint64_t key = gen_stream_key(seed, stream);
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < nn; ++i) out[i] = (float)normal_at(key, offset + (uint64_t)i) * sigma;
}

/* out[i] = lo + draw(offset+i) mod (hi-lo+1); requires lo <= hi. */
void gen_uniform_int(uint64_t seed, uint64_t stream, int64_t lo, int64_t hi, uint64_t offset,
                     uint64_t n, int64_t* out) {
    uint64_t key = gen_stream_key(seed, stream);
    uint64_t span = (uint64_t)(hi - lo) + 1u;
    for (uint64_t i = 0; i < n; ++i) out[i] = lo + (int64_t)(sm64_at(key, offset + i) % span);
}

/* Durstenfeld shuffle of the identity on [0, n). */
void gen_permutation(uint64_t seed, uint64_t stream, uint64_t n, int64_t* out) {
    uint64_t key = gen_stream_key(seed, stream);
    for (uint64_t i = 0; i < n; ++i) out[i] = (int64_t)i;
    if (n < 2) return;
    for (uint64_t i = n - 1; i >= 1; --i) {
        uint64_t j = sm64_at(key, n - 1 - i) % (i + 1);
        int64_t t = out[i];
        out[i] = out[j];
        out[j] = t;
    }
}
