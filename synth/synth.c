/*
 * Seeded synthetic inputs for the MoE expert-offload workloads: the bytes of
 * MXFP4 expert weight blobs.  This file holds no arithmetic of the method
 * itself (no dequantisation, routing, caching or FFN); it only produces the
 * random codes and scales that both the HIP library and the CPU oracle take
 * as input.  Integer-only, so it gives the same bytes on every machine.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast Splittable
 * Pseudorandom Number Generators", OOPSLA 2014), used counter-style: the
 * n-th 64-bit word of the stream with state k is mix64(k + (n+1)*GAMMA).
 * Stream keys are derived by chaining the same step over (seed, kind, a, b, c).
 *
 * Logical blob (the input format of one expert, 3*H*I*17/32 bytes):
 *   gate codes  [I][H/2]   gate scales [I][H/32]
 *   up   codes  [I][H/2]   up   scales [I][H/32]
 *   down codes  [H][I/2]   down scales [H][I/32]
 * A code byte holds element 2j in its low nibble and element 2j+1 in its high
 * nibble; a scale byte is the E8M0 exponent of 32 consecutive elements along
 * the row (the reduction dimension).  Codes are uniform on all 16 values (so
 * every code byte is uniform on 0..255); scale bytes are uniform on 123..127.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

enum {
    KIND_CODES = 1,     /* + matrix index 0..2 */
    KIND_SCALES = 11,   /* + matrix index 0..2 */
};

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t kind, uint64_t a, uint64_t b, uint64_t c) {
    uint64_t k = mix64(seed + GAMMA);
    k = mix64(k + GAMMA * (kind + 1));
    k = mix64(k + GAMMA * (a + 1));
    k = mix64(k + GAMMA * (b + 1));
    k = mix64(k + GAMMA * (c + 1));
    return k;
}

static inline uint64_t word(uint64_t key, uint64_t n) { return mix64(key + GAMMA * (n + 1)); }

/* n random bytes: byte j is byte (j % 8) (little-endian) of word j/8 */
void synth_bytes(uint64_t key, uint8_t* out, size_t n) {
    size_t nw = n / 8;
    for (size_t w = 0; w < nw; ++w) {
        uint64_t r = word(key, w);
        memcpy(out + 8 * w, &r, 8);  /* little-endian host */
    }
    if (n % 8) {
        uint64_t r = word(key, nw);
        for (size_t j = 0; j < n % 8; ++j) out[8 * nw + j] = (uint8_t)(r >> (8 * j));
    }
}

/* n E8M0 scale bytes uniform on lo..lo+span-1: lo + floor(hi32(word) * span / 2^32) */
void synth_scales(uint64_t key, uint8_t* out, size_t n, uint32_t lo, uint32_t span) {
    for (size_t j = 0; j < n; ++j) {
        uint64_t hi = word(key, j) >> 32;
        out[j] = (uint8_t)(lo + ((hi * span) >> 32));
    }
}

/* expert id used in the stream key of shared expert s (routed ids are < 2^20) */
#define SHARED_ID_BASE 1000000ULL

/* Fill one logical blob.  expert >= 0: routed expert; expert < 0: shared expert -1-expert. */
void synth_expert_blob(uint64_t seed, int32_t layer, int32_t expert, int32_t H, int32_t I,
                       uint8_t* out) {
    uint64_t eid = expert >= 0 ? (uint64_t)expert : SHARED_ID_BASE + (uint64_t)(-1 - expert);
    size_t hi = (size_t)H * (size_t)I;
    uint8_t* p = out;
    for (int m = 0; m < 3; ++m) {
        size_t ncode = hi / 2, nscale = hi / 32;
        synth_bytes(synth_key(seed, KIND_CODES + m, (uint64_t)layer, eid, 0), p, ncode);
        p += ncode;
        synth_scales(synth_key(seed, KIND_SCALES + m, (uint64_t)layer, eid, 0), p, nscale, 123, 5);
        p += nscale;
    }
}

/* Callback with the signature the library's pool filler takes:
 *   void fill(void* user, int32_t layer, int32_t expert, uint8_t* dst_logical_blob)
 * user points at a synth_fill_args.  Safe to call from several threads at once. */
typedef struct {
    uint64_t seed;
    int32_t hidden, inter;
} synth_fill_args;

void synth_fill_cb(void* user, int32_t layer, int32_t expert, uint8_t* dst) {
    const synth_fill_args* a = (const synth_fill_args*)user;
    synth_expert_blob(a->seed, layer, expert, a->hidden, a->inter, dst);
}
