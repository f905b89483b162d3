// nvfp4_lut.hpp -- compile-time table for NVFP4 -> E4M3 dequantization on gfx950.
//
// The dequantized byte of an element is e4m3_rn_satfinite(e2m1(code) * e4m3(scale))
// (vLLM API page "gather_nvfp4_index_k", module description).  The magnitude
// of that byte depends only on the 3-bit code magnitude and the scale byte
// without its sign; the sign is the XOR of the code's and the scale's sign bits.
// So each of the 256 scale bytes gets one 64-bit table entry holding the eight
// magnitude bytes, entry byte c = |e2m1 code c| * |scale| rounded to E4M3.
// Kernels fetch the entry for a group's scale once and then map four codes per
// v_perm_b32 (the byte-select instruction indexes an 8-byte table).
//
// The rounding below works on integers in units of 2^-10: an E2M1 magnitude
// is a multiple of 0.5 and an E4M3 magnitude a multiple of 2^-9, so their
// product is an exact integer number of 2^-10 units (below 2^22).
#pragma once

#include <cstdint>

namespace pagescore {

// |E2M1| of the magnitude code 0..7, in units of 0.5: 0 .5 1 1.5 2 3 4 6.
constexpr uint32_t e2m1_mag_half_units(int c)
{
    constexpr uint32_t v[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    return v[c & 7];
}

// |E4M3| of the 7-bit magnitude field in units of 2^-9 (exponent bias 7,
// exponent 0 subnormal).  Only meaningful for fields other than 0x7F (NaN).
constexpr uint32_t e4m3_mag_units9(int f)
{
    const int e = (f >> 3) & 15, m = f & 7;
    return e == 0 ? uint32_t(m) : uint32_t(8 + m) << (e - 1);
}

constexpr int floor_log2(uint64_t x)
{
    int n = -1;
    while (x) {
        x >>= 1;
        ++n;
    }
    return n;
}

// Round p * 2^-10 (p >= 0) to an E4M3 magnitude byte: nearest, ties to even
// mantissa, saturating at 448 (= 448 * 1024 units).
constexpr uint8_t e4m3_round_units10(uint64_t p)
{
    if (p >= (uint64_t(448) << 10))
        return 0x7E;
    if (p == 0)
        return 0;
    const int lg = floor_log2(p);
    // Step between E4M3 values: 2^-9 (2 units) below 2^-5, else 1/8 of the binade.
    const int sh = lg < 4 ? 1 : lg - 3;
    uint64_t q = p >> sh;
    const uint64_t rem = p & ((uint64_t(1) << sh) - 1);
    const uint64_t half = uint64_t(1) << (sh - 1);
    if (rem > half || (rem == half && (q & 1)))
        ++q;
    const uint64_t r = q << sh;                 // rounded magnitude, units of 2^-10
    if (r < 16)                                  // below 2^-6: subnormal m * 2^-9
        return uint8_t(r >> 1);
    const int lr = floor_log2(r);                // r in [2^lr, 2^(lr+1))
    const int biased = lr - 10 + 7;
    return uint8_t((biased << 3) | ((r >> (lr - 3)) & 7));
}

constexpr uint64_t lut_entry(int scale_byte)
{
    const int f = scale_byte & 0x7F;
    if (f == 0x7F)                               // NaN scale: NaN for every code
        return 0x7F7F7F7F7F7F7F7Full;
    uint64_t e = 0;
    for (int c = 0; c < 8; ++c)
        e |= uint64_t(e4m3_round_units10(uint64_t(e2m1_mag_half_units(c)) * e4m3_mag_units9(f)))
             << (8 * c);
    return e;
}

struct Nvfp4Lut {
    uint64_t entry[256];
};

constexpr Nvfp4Lut make_nvfp4_lut()
{
    Nvfp4Lut t{};
    for (int s = 0; s < 256; ++s)
        t.entry[s] = lut_entry(s);
    return t;
}

}  // namespace pagescore
