// Small device helpers shared by the gfx950 attention kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "crkv_internal.h"

namespace crkv {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef short i16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Pointers into the global address space: loads and stores through them are
// global_* instructions, which count only against vmcnt. Generic (flat)
// accesses also count against lgkmcnt, so every wait for an LDS read would
// wait for outstanding HBM loads as well.
template <typename T>
using gptr = __attribute__((address_space(1))) T *;

template <typename T>
__device__ __forceinline__ gptr<T> as_global(T *p)
{
    return (gptr<T>)p;
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1); every lane of the
// row receives the total.
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_mov<0x128>(x);
    x += dpp_mov<0x124>(x);
    x += dpp_mov<0x122>(x);
    x += dpp_mov<0x121>(x);
    return x;
}

// Sums of eight per-lane values v[0..7] over the 16 lanes of a DPP row,
// transposed while they are summed: lane li of the row receives the totals
// of values 2 (li / 4) (s0) and 2 (li / 4) + 1 (s1). Each of the first two
// steps pairs lanes (li ^ 8, then the mirror image within each half of 8)
// so that each lane keeps half of the values it holds; the last two sum
// within quads. 22 vector instructions against 48 for eight row16_sum.
__device__ __forceinline__ void row16_sum8(const float (&v)[8], int li, float &s0, float &s1)
{
    const bool lo8 = li < 8;
    const bool lo4 = (li & 4) == 0;
    float r1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)   // r1[k]: value k + 4 (li >= 8), over lanes li and li ^ 8
        r1[k] = (lo8 ? v[k] : v[k + 4]) + dpp_mov<0x128>(lo8 ? v[k + 4] : v[k]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {   // value j + 2 ((li & 4) != 0) + 4 (li >= 8), over 4 lanes
        float r = (lo4 ? r1[j] : r1[j + 2]) + dpp_mov<0x141>(lo4 ? r1[j + 2] : r1[j]);
        r += dpp_mov<0x4E>(r);   // quad lanes ^ 2
        r += dpp_mov<0xB1>(r);   // quad lanes ^ 1
        (j == 0 ? s0 : s1) = r;
    }
}

// Combine two (max, sum) softmax states; maxima are raw scores, the sums are
// of exp2((s - max) * c).
__device__ __forceinline__ void merge_state(float &m, float &l, float m2, float l2, float c)
{
    const float mn = fmaxf(m, m2);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float a = (m == -INFINITY) ? 0.f : exp2_hw((m - mu) * c);
    const float b = (m2 == -INFINITY) ? 0.f : exp2_hw((m2 - mu) * c);
    l = l * a + l2 * b;
    m = mn;
}

// Segment of a position: the number of segments that end at or before it.
__device__ __forceinline__ int segment_of(const SegDesc *segs, int n_seg, int pos)
{
    int s = 0;
    for (int c = 0; c < n_seg - 1; ++c)
        s += (segs[c].start + segs[c].len <= pos) ? 1 : 0;
    return s;
}

}  // namespace crkv
