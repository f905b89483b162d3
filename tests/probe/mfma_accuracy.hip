// mfma_accuracy.hip -- TEST PROBE, not part of the product library.
//
// Computes one 16 x 16 tile of depth-128 dot products of E4M3 vectors per
// work-group with three gfx950 matrix instructions, so a test can compare
// each with the exact dot products:
//   method 0: four chained v_mfma_f32_16x16x32_f16 on E4M3 values converted
//             to f16 (exact), the form the indexer kernels use;
//   method 1: four chained v_mfma_f32_16x16x32_fp8_fp8 on the E4M3 bytes;
//   method 2: one v_mfma_scale_f32_16x16x128_f8f6f4 on the E4M3 bytes with
//             unit block scales (E8M0 byte 127 on both operands).
// A dot product does not depend on how the depth index is spread over the
// lanes as long as both operands spread it the same way, which they do here.
//
//   a, b   [tiles][16][128] E4M3 bytes (rows of the M and N operands)
//   out    [tiles][3][16][16] f32: out[t][method][i][j] = a[t][i] . b[t][j]
// Returns 0, or the HIP error of the launch.
#include <hip/hip_runtime.h>
#include <cstdint>

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));

namespace {

__device__ __forceinline__ uint32_t f16_pair(uint32_t bytes, bool high)
{
    return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, true)
                                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, false));
}

__global__ __launch_bounds__(64) void probe_kernel(const uint8_t *__restrict__ a,
                                                   const uint8_t *__restrict__ b, float *__restrict__ out)
{
    const int t = blockIdx.x;
    const int l = threadIdx.x;
    const int r = l % 16, g = l / 16;
    const uint8_t *ar = a + ((size_t)t * 16 + r) * 128;
    const uint8_t *br = b + ((size_t)t * 16 + r) * 128;
    v4f acc[3] = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint2 av = *reinterpret_cast<const uint2 *>(ar + 32 * s + 8 * g);
        const uint2 bv = *reinterpret_cast<const uint2 *>(br + 32 * s + 8 * g);
        const uint32_t ah[4] = {f16_pair(av.x, false), f16_pair(av.x, true), f16_pair(av.y, false),
                                f16_pair(av.y, true)};
        const uint32_t bh[4] = {f16_pair(bv.x, false), f16_pair(bv.x, true), f16_pair(bv.y, false),
                                f16_pair(bv.y, true)};
        v8h A, B;
        __builtin_memcpy(&A, ah, 16);
        __builtin_memcpy(&B, bh, 16);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[0], 0, 0, 0);
        const long a8 = (long)(((uint64_t)av.y << 32) | av.x);
        const long b8 = (long)(((uint64_t)bv.y << 32) | bv.x);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8, b8, acc[1], 0, 0, 0);
    }
    v8i A32, B32;
    __builtin_memcpy(&A32, ar + 32 * g, 32);
    __builtin_memcpy(&B32, br + 32 * g, 32);
    acc[2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A32, B32, acc[2], 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[(((size_t)t * 3 + m) * 16 + 4 * g + i) * 16 + r] = acc[m][i];
}

}  // namespace

extern "C" int mfma_accuracy_probe(const uint8_t *a, const uint8_t *b, int tiles, float *out,
                                   void *stream)
{
    if (tiles <= 0)
        return 0;
    hipLaunchKernelGGL(probe_kernel, dim3((unsigned)tiles), dim3(64), 0, (hipStream_t)stream, a, b,
                       out);
    return (int)hipGetLastError();
}
