/*
 * synth.c -- seeded synthetic inputs, shared by the tests, the benchmark and
 * the oracle's test harness.  It holds none of the activation/quantisation
 * arithmetic: only random streams and the rounding of a sample to bf16.
 *
 * Every value is a pure function of (stream key, element index), so any row
 * of a large tensor can be regenerated on its own:
 *   u64(key, i)   = SplitMix64 output for counter state key + (i+1)*gamma
 *                   (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *                   generators", OOPSLA 2014; gamma = 0x9E3779B97F4A7C15).
 *   uniform(key,i)= (u64 >> 11) * 2^-53, in [0, 1).
 *   normal: Box-Muller on the pair p = i/2: u1 = 1 - uniform(key, 2p),
 *           u2 = uniform(key, 2p+1), rho = sqrt(-2 ln u1);
 *           even i -> rho cos(2 pi u2), odd i -> rho sin(2 pi u2).
 *   bf16:   sigma * normal in fp64, rounded to fp32 (nearest-even), then to
 *           bf16 (nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const uint64_t kGamma = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_u64(uint64_t key, int64_t i) { return mix64(key + (uint64_t)(i + 1) * kGamma); }

static inline double uniform(uint64_t key, int64_t i)
{
    return (double)(synth_u64(key, i) >> 11) * 0x1p-53;
}

/* FNV-1a over a name, then one SplitMix64 mix: the key of a named stream. */
uint64_t synth_key(const char* name)
{
    uint64_t h = 0xCBF29CE484222325ull;
    for (const unsigned char* p = (const unsigned char*)name; *p; ++p) {
        h ^= *p;
        h *= 0x100000001B3ull;
    }
    return mix64(h);
}

static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u); /* finite inputs only */
    return (uint16_t)(b >> 16);
}

void synth_uniform(uint64_t key, int64_t first, int64_t count, double* out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = uniform(key, first + i);
}

void synth_normal_bf16(uint64_t key, int64_t first, int64_t count, double sigma, uint16_t* out)
{
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t k = 0; k < count; ++k) {
        const int64_t i = first + k;
        const int64_t p = i >> 1;
        const double u1 = 1.0 - uniform(key, 2 * p);
        const double u2 = uniform(key, 2 * p + 1);
        const double rho = sqrt(-2.0 * log(u1));
        const double z = (i & 1) ? rho * sin(two_pi * u2) : rho * cos(two_pi * u2);
        out[k] = f32_to_bf16_rne((float)(sigma * z));
    }
}

/* Replace element i by +-value with probability p (independent per element):
 * the choice uses stream key_p, the sign uses the top bit of stream key_s. */
void synth_outliers_bf16(uint64_t key_p, uint64_t key_s, int64_t first, int64_t count, double p,
                         double value, uint16_t* inout)
{
    for (int64_t k = 0; k < count; ++k) {
        const int64_t i = first + k;
        if (uniform(key_p, i) < p) {
            const double v = (synth_u64(key_s, i) >> 63) ? -value : value;
            inout[k] = f32_to_bf16_rne((float)v);
        }
    }
}
