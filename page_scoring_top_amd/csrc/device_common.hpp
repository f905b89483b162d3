// device_common.hpp -- small gfx950 device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "nvfp4_lut.hpp"

namespace pagescore {

constexpr int kWave = 64;
constexpr int kPageTokens = 128;
constexpr int kDepth = 128;
constexpr int kCodeBytes = 8192;
constexpr int kPageBytes = 9216;
constexpr int kSlots = 8;
constexpr int kDecodeHeads = 4;
constexpr int kDecodeRows = kSlots * kDecodeHeads;  // 32 score rows per request
constexpr int kTopk = 16;

// The dequantization table, baked into the code object at compile time.
__device__ constexpr Nvfp4Lut kNvfp4Lut = make_nvfp4_lut();

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two E4M3 bytes of a word (bytes 0,1 or bytes 2,3) as two f16, in one
// v_cvt_scalef32_pk_f16_fp8 with scale 1.0.  Every E4M3 value is exact in f16;
// the conversion was checked on all 256 bytes in both positions on gfx950.
template <bool kHighPair>
__device__ __forceinline__ uint32_t f16x2_of_e4m3(uint32_t bytes)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f,
                                                                                 kHighPair));
}

// v_perm_b32 on the 8-byte value {hi:lo}: result byte i is byte sel.byte[i]
// (0..7) of that value, byte 0 being the lowest byte of lo.
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Dequantize the 8 E2M1 codes of one 32-bit word (element 2i in the low
// nibble of byte i) against a table entry {hi:lo}.  Returns the E4M3 bytes of
// the even elements (0,2,4,6) in `even` and of the odd elements (1,3,5,7) in
// `odd`; the sign of each byte is the code's sign bit.  The caller folds the
// scale's sign into the codes beforehand (XOR of 0x88888888) when it is set.
__device__ __forceinline__ void dequant_word(uint32_t codes, uint32_t lut_hi, uint32_t lut_lo,
                                             uint32_t &even, uint32_t &odd)
{
    const uint32_t mag_e = byte_perm(lut_hi, lut_lo, codes & 0x07070707u);
    const uint32_t mag_o = byte_perm(lut_hi, lut_lo, (codes >> 4) & 0x07070707u);
    even = mag_e | ((codes << 4) & 0x80808080u);
    odd = mag_o | (codes & 0x80808080u);
}

// Code-sign flip mask for a scale byte: every nibble's sign bit when the
// scale is negative.
__device__ __forceinline__ uint32_t scale_sign_flip(uint32_t scale_byte)
{
    return (scale_byte & 0x80u) ? 0x88888888u : 0u;
}

__device__ __forceinline__ bool scale_is_nan(uint32_t scale_byte)
{
    return (scale_byte & 0x7Fu) == 0x7Fu;
}

// Orders LDS stores of some lanes of a wave before loads of other lanes of
// the same wave (and the reverse): a wave-scope release/acquire around the
// wave barrier.  At wavefront scope this emits no instruction; it only keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A raw buffer descriptor over `bytes` bytes at `base` (wave-uniform by
// construction).  Loads at or past `bytes` read zeros and stores there are
// dropped, without touching memory; a descriptor of 0 bytes makes every
// access free.  The fields go through v_readfirstlane so the descriptor sits
// in scalar registers (one the compiler cannot prove uniform costs a loop
// per access); the address halves are widened as unsigned values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uintptr_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0, (int)n, 0x00020000);
}

}  // namespace pagescore
