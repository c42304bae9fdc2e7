/*
 * Reference bit packing with the x86 BMI2 instructions PEXT (parallel bit
 * extract) and PDEP (parallel bit deposit), used by the tests as a library
 * routine that pins the oracle's bit order: packing the non-invariant bits of
 * a tensor, LSB-first and in ascending position, is a chain of PEXT over its
 * 64-bit little-endian words with selector ~Mask; unpacking is PDEP.
 * Test infrastructure only; word-level code on purpose (the oracle works bit
 * by bit).
 */
#include <immintrin.h>
#include <stdint.h>
#include <string.h>

/* Appends _pext_u64(src[i], sel[i]) for i = 0..n-1 to a bit stream at dst
 * (dst_bytes bytes, cleared first).  Returns the stream length in bits. */
uint64_t pext_stream(const uint64_t *src, const uint64_t *sel, uint64_t n,
                     uint8_t *dst, uint64_t dst_bytes)
{
    unsigned __int128 acc = 0;
    unsigned fill = 0;
    uint64_t pos = 0, total = 0;
    memset(dst, 0, dst_bytes);
    for (uint64_t i = 0; i < n; i++) {
        uint64_t v = _pext_u64(src[i], sel[i]);
        unsigned k = (unsigned)__builtin_popcountll(sel[i]);
        acc |= (unsigned __int128)v << fill;
        fill += k;
        total += k;
        if (fill >= 64) {
            uint64_t w = (uint64_t)acc;
            memcpy(dst + pos, &w, 8);
            pos += 8;
            acc >>= 64;
            fill -= 64;
        }
    }
    if (fill) {
        uint64_t w = (uint64_t)acc;
        memcpy(dst + pos, &w, (fill + 7) / 8);
    }
    return total;
}

/* Inverse: dst[i] = _pdep_u64(next popcount(sel[i]) stream bits, sel[i]).
 * stream must be readable for 8 bytes past its last used byte. */
void pdep_stream(const uint8_t *stream, const uint64_t *sel, uint64_t n, uint64_t *dst)
{
    unsigned __int128 acc = 0;
    unsigned fill = 0;
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        unsigned k = (unsigned)__builtin_popcountll(sel[i]);
        if (fill < k) {
            uint64_t w;
            memcpy(&w, stream + pos, 8);
            pos += 8;
            acc |= (unsigned __int128)w << fill;
            fill += 64;
        }
        uint64_t bits = k == 64 ? (uint64_t)acc : (uint64_t)acc & ((1ull << k) - 1);
        dst[i] = _pdep_u64(bits, sel[i]);
        acc >>= k;
        fill -= k;
    }
}
