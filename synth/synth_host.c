/*
 * synth_host.c -- seeded synthetic inputs for the MXFP4 sparse-MoE decode layer (host side).
 *
 * This module only draws random numbers.  It holds none of the MoE method's arithmetic: both
 * the CPU oracle and the GPU library consume the bytes it writes, and neither links the other.
 *
 * Counter-based generator (every value is a pure function of its coordinates):
 *   fmix64(z)       the SplitMix64 output mix (Steele, Lea & Flood, OOPSLA 2014):
 *                   z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31
 *   sm(s, i)        fmix64(s + (i+1) * 0x9E3779B97F4A7C15)              (all arithmetic mod 2^64)
 *   key             sm(sm(sm(sm(seed, layer), tensor), expert), attempt)
 *   r_i             sm(key, i)
 *
 * Tensor ids: 0 router, 1 gate/up codes, 2 gate/up scales, 3 down codes, 4 down scales,
 *             5 activations x, 6 LM-head weights.
 *
 * Integer quantities (bit-identical to the device twin in synth_device.hip):
 *   E2M1 code byte i   = byte (i & 7) (little-endian) of r_(i >> 3)   -> two nibbles uniform over 16 codes
 *   E8M0 scale byte i  = 121 + (r_i mod 5)                            -> exponents uniform in [-6, -2]
 * Normals (host only): Box-Muller on the pair (r_2p, r_2p+1) with u = ((r >> 11) + 0.5) * 2^-53;
 *   element 2p takes the cosine branch, element 2p+1 the sine branch; the value is sigma * z,
 *   rounded to fp32, and for bf16 outputs then rounded to bf16 (nearest, ties to even).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static uint64_t fmix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static uint64_t sm(uint64_t s, uint64_t i) { return fmix64(s + (i + 1) * 0x9E3779B97F4A7C15ULL); }

uint64_t synth_key(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t expert, uint32_t attempt) {
    return sm(sm(sm(sm(seed, layer), tensor), expert), attempt);
}

uint64_t synth_hash(uint64_t key, uint64_t i) { return sm(key, i); }

/* E2M1 code bytes [i0, i0+n) of the tensor identified by key. */
void synth_codes(uint8_t* out, uint64_t i0, uint64_t n, uint64_t key) {
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t i = i0 + j;
        uint64_t r = sm(key, i >> 3);
        out[j] = (uint8_t)(r >> (8 * (i & 7)));
    }
}

/* E8M0 scale bytes [i0, i0+n). */
void synth_scales(uint8_t* out, uint64_t i0, uint64_t n, uint64_t key) {
    for (uint64_t j = 0; j < n; ++j) out[j] = (uint8_t)(121 + sm(key, i0 + j) % 5);
}

static double normal_at(uint64_t key, uint64_t i) {
    uint64_t p = i >> 1;
    uint64_t r0 = sm(key, 2 * p), r1 = sm(key, 2 * p + 1);
    double u1 = ((double)(r0 >> 11) + 0.5) * 0x1p-53;
    double u2 = ((double)(r1 >> 11) + 0.5) * 0x1p-53;
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

void synth_normal_f32(float* out, uint64_t i0, uint64_t n, uint64_t key, double sigma) {
    for (uint64_t j = 0; j < n; ++j) out[j] = (float)(sigma * normal_at(key, i0 + j));
}

/* fp32 -> bf16, nearest with ties to even (the generated values are finite). */
static uint16_t to_bf16(float f) {
    union { float f; uint32_t u; } v = { f };
    uint32_t u = v.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void synth_normal_bf16(uint16_t* out, uint64_t i0, uint64_t n, uint64_t key, double sigma) {
    for (uint64_t j = 0; j < n; ++j) out[j] = to_bf16((float)(sigma * normal_at(key, i0 + j)));
}
