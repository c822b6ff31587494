// Moves cached keys to new positions under rotary position embedding, in
// place, for gfx950.
//
// What it computes (TurboRAG summary, implementation notes: with rotary
// position embedding the position IDs a chunk's cache was built with must
// agree with those it is used at; the pages give no formula, and this is the
// standard rotary embedding in the rotate-half arrangement): for every key
// row x of a segment moved by delta positions and every i < d/2,
//   y_i       = x_i cos(a_i) - x_{i+d/2} sin(a_i)
//   y_{i+d/2} = x_{i+d/2} cos(a_i) + x_i sin(a_i),   a_i = delta * base^(-2i/d).
// The host evaluates cos and sin of the angles in double per segment; the
// kernel rotates in float32 and rounds once to the stored type.
//
// Pure streaming, bound by HBM: a lane takes eight consecutive pairs of a row
// (16 + 16 bytes in bf16, 32 + 32 in float32), with its eight cos/sin pairs
// held in registers for the whole workgroup, which covers kRopeRowsPerItem
// rows of one segment.
#include "crkv_internal.h"
#include "device_util.h"

namespace crkv {

template <int D, bool BF16>
__global__ void __launch_bounds__(kRopeThreads) rope_shift_kernel(const RopeArgs a)
{
    constexpr int HALF = D / 2;
    constexpr int LPR = HALF / 8;                     // lanes per row
    constexpr int RPP = kRopeThreads / LPR;           // rows per pass of the workgroup
    constexpr int ES = BF16 ? 2 : 4;                  // element bytes
    const RopeItem it = a.items[blockIdx.x];
    const RopeSeg sg = a.segs[it.seg];
    const int g = threadIdx.x % LPR;                  // pairs 8g .. 8g+7
    float c[8], s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        c[e] = as_global(sg.cs)[8 * g + e];
        s[e] = as_global(sg.cs)[HALF + 8 * g + e];
    }
    const int row_end = min(sg.rows, it.row0 + kRopeRowsPerItem);
    for (int r = it.row0 + (int)threadIdx.x / LPR; r < row_end; r += RPP) {
        unsigned char *row = static_cast<unsigned char *>(sg.K) + (size_t)r * D * ES;
        float x1[8], x2[8];
        if (BF16) {
            const gptr<u32x4> p1 = as_global(reinterpret_cast<u32x4 *>(row + 8 * g * 2));
            const gptr<u32x4> p2 = as_global(reinterpret_cast<u32x4 *>(row + (HALF + 8 * g) * 2));
            const u32x4 v1 = *p1, v2 = *p2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x1[2 * q] = __uint_as_float(v1[q] << 16);
                x1[2 * q + 1] = __uint_as_float(v1[q] & 0xFFFF0000u);
                x2[2 * q] = __uint_as_float(v2[q] << 16);
                x2[2 * q + 1] = __uint_as_float(v2[q] & 0xFFFF0000u);
            }
            u32x4 o1, o2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e0 = 2 * q, e1 = 2 * q + 1;
                const __bf16 a0 = (__bf16)(x1[e0] * c[e0] - x2[e0] * s[e0]);
                const __bf16 a1 = (__bf16)(x1[e1] * c[e1] - x2[e1] * s[e1]);
                const __bf16 b0 = (__bf16)(x2[e0] * c[e0] + x1[e0] * s[e0]);
                const __bf16 b1 = (__bf16)(x2[e1] * c[e1] + x1[e1] * s[e1]);
                o1[q] = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
                o2[q] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            }
            *p1 = o1;
            *p2 = o2;
        } else {
            const gptr<u32x4> p1 = as_global(reinterpret_cast<u32x4 *>(row + 8 * g * 4));
            const gptr<u32x4> p2 = as_global(reinterpret_cast<u32x4 *>(row + (HALF + 8 * g) * 4));
            const u32x4 v1a = p1[0], v1b = p1[1], v2a = p2[0], v2b = p2[1];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x1[q] = __uint_as_float(v1a[q]);
                x1[4 + q] = __uint_as_float(v1b[q]);
                x2[q] = __uint_as_float(v2a[q]);
                x2[4 + q] = __uint_as_float(v2b[q]);
            }
            u32x4 o1a, o1b, o2a, o2b;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o1a[q] = __float_as_uint(x1[q] * c[q] - x2[q] * s[q]);
                o1b[q] = __float_as_uint(x1[4 + q] * c[4 + q] - x2[4 + q] * s[4 + q]);
                o2a[q] = __float_as_uint(x2[q] * c[q] + x1[q] * s[q]);
                o2b[q] = __float_as_uint(x2[4 + q] * c[4 + q] + x1[4 + q] * s[4 + q]);
            }
            p1[0] = o1a;
            p1[1] = o1b;
            p2[0] = o2a;
            p2[1] = o2b;
        }
    }
}

hipError_t launch_rope_shift(int d, bool bf16, const RopeArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    const dim3 grid(n_items), block(kRopeThreads);
    if (d == 128 && bf16)
        hipLaunchKernelGGL((rope_shift_kernel<128, true>), grid, block, 0, stream, args);
    else if (d == 128)
        hipLaunchKernelGGL((rope_shift_kernel<128, false>), grid, block, 0, stream, args);
    else if (bf16)
        hipLaunchKernelGGL((rope_shift_kernel<64, true>), grid, block, 0, stream, args);
    else
        hipLaunchKernelGGL((rope_shift_kernel<64, false>), grid, block, 0, stream, args);
    return hipGetLastError();
}

}  // namespace crkv
