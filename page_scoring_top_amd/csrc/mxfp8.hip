// mxfp8.hip -- K5: MXFP8 E4M3 quantization of bf16 rows (vLLM pull request
// #65508, "How it works": output layout and arithmetic items).
//
// Every 32 consecutive elements of a row form one MX block with one E8M0
// scale byte.  The block's largest magnitude is taken on the bf16 bit
// patterns with the sign cleared, and the scale byte is
//     sb = clamp(exponent_field - 8 + (fraction > 0.75), 0, 254)
// (= ceil(log2(amax / 448)) + 127, as 448 = 1.75 * 2^8).  Each element is
// multiplied by 2^(127 - sb), which is exact, and converted to E4M3 with
// round to nearest even.  The block maximum scaled this way is at most 448,
// so no element saturates.  An element that is +-inf or NaN is written as
// the canonical NaN byte 0x7F.
//
// Mapping to gfx950.  A lane takes 8 consecutive elements (one 16-byte
// load), so each load instruction of a wave reads 1 KiB of one row
// contiguously; the four lanes of a quad hold one 32-element block and join
// their maxima with two DPP quad permutes.  Each lane then converts its 8
// elements, two per v_cvt_pk_fp8_f32 (the second conversion of a pair
// writes the upper half of the same dword), and stores 8 bytes; the quad's
// first lane stores the scale byte.  A wave walks 4 x 64 lanes of one row
// (2,048 elements), four loads in flight.  The kernel is bound by HBM at
// 3 + 1/32 bytes per element.
#include "device_common.hpp"
#include "launch.hpp"

namespace pagescore {

namespace {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMxWaves = 4;                        // rows per work-group
constexpr int kMxSteps = 4;                        // 64-lane steps per wave
constexpr int kMxUnitsPerWave = kMxSteps * kWave;  // 8-element units of a row per wave

__device__ __forceinline__ uint32_t quad_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    return v;
}

__global__ __launch_bounds__(kMxWaves * kWave) void mxfp8_quant_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int32_t rows, int32_t units_per_row,
    uint8_t *__restrict__ q, int64_t ldq, uint8_t *__restrict__ scales, int64_t lds)
{
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int u0 = blockIdx.x * kMxUnitsPerWave + lane;
    for (int64_t r = (int64_t)blockIdx.y * kMxWaves + wave; r < rows;
         r += (int64_t)gridDim.y * kMxWaves) {
        // Unit u holds elements [8u, 8u + 8) of row r; units past the row
        // (whole quads, as a row has a multiple of 4 units) load zeros and
        // store nothing.
        // Inputs are read once and codes written once: both streamed past the
        // caches (nontemporal), 20.0 -> 17.7-18.1 us at 16,384 x 2,048.
        u32x4 v[kMxSteps];
#pragma unroll
        for (int j = 0; j < kMxSteps; ++j) {
            const int u = u0 + j * kWave;
            v[j] = u < units_per_row
                       ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + r * ldx + 8 * u))
                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kMxSteps; ++j) {
            const int u = u0 + j * kWave;
            const uint32_t w[4] = {v[j][0], v[j][1], v[j][2], v[j][3]};
            u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
            for (int i = 1; i < 4; ++i)
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
            const uint32_t amax = quad_max(m.x > m.y ? m.x : m.y);
            int sb = (int)(amax >> 7) - 8 + ((amax & 0x7Fu) > 96u ? 1 : 0);   // fraction > 0.75
            sb = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
            const float mul = __uint_as_float((uint32_t)(254 - sb) << 23);    // 2^(127 - sb)
            uint32_t out[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t a = w[2 * k], c = w[2 * k + 1];
                int o = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(a << 16) * mul,
                                                        __uint_as_float(a & 0xFFFF0000u) * mul, 0, false);
                o = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(c << 16) * mul,
                                                    __uint_as_float(c & 0xFFFF0000u) * mul, o, true);
                out[k] = (uint32_t)o;
            }
            if (amax >= 0x7F80u) {
                // The block holds an infinity or a NaN: those elements become 0x7F.
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (((w[e / 2] >> (16 * (e % 2))) & 0x7F80u) == 0x7F80u)
                        out[e / 4] = (out[e / 4] & ~(0xFFu << (8 * (e % 4)))) | (0x7Fu << (8 * (e % 4)));
                }
            }
            if (u < units_per_row) {
                __builtin_nontemporal_store(u32x2{out[0], out[1]},
                                            reinterpret_cast<u32x2 *>(q + r * ldq + 8 * u));
                if ((lane & 3) == 0)
                    scales[r * lds + u / 4] = (uint8_t)sb;
            }
        }
    }
}

}  // namespace

hipError_t launch_mxfp8_quant(const uint16_t *x, int64_t ldx, int32_t rows, int32_t cols, uint8_t *q,
                              int64_t ldq, uint8_t *scales, int64_t lds, hipStream_t stream)
{
    const int32_t units_per_row = cols / 8;
    const int32_t chunks = (units_per_row + kMxUnitsPerWave - 1) / kMxUnitsPerWave;
    const int64_t row_groups = ((int64_t)rows + kMxWaves - 1) / kMxWaves;
    const uint32_t gy = (uint32_t)(row_groups < 65535 ? row_groups : 65535);
    hipLaunchKernelGGL(mxfp8_quant_kernel, dim3((uint32_t)chunks, gy), dim3(kMxWaves * kWave), 0, stream,
                       x, ldx, rows, units_per_row, q, ldq, scales, lds);
    return hipGetLastError();
}

}  // namespace pagescore
