// Top-k selection over the impact vector for gfx950 (CacheBlend summary,
// selective-recompute listing: topk over the document slice of the impact,
// k = max(1, int(N_doc * r))).
//
// One workgroup per vector. The fp32 values are mapped to unsigned keys that
// order like the floats (-0 below +0). A four-pass, 8-bit radix select finds
// the k-th largest key T. Every key above T is taken, and of the keys equal
// to T the lowest indices are taken (an ordered scan over contiguous index
// ranges, one per thread). The k winners are then sorted by (key descending,
// index ascending) with a bitonic network in LDS, packed as 64-bit words
// (key << 32 | ~index) so one descending sort does both orders.
#include <hip/hip_runtime.h>

#include "crkv_internal.h"

namespace crkv {

__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 256;

__device__ void topk_body(const TopkDesc td)
{
    __shared__ uint32_t hist[256];
    __shared__ int scan[kTopkThreads];
    __shared__ uint32_t s_digit;
    __shared__ int s_above;
    __shared__ int s_gt;
    __shared__ unsigned long long sel[kTopkMaxK];

    const int tid = threadIdx.x;
    const int n = td.n, k = td.k;
    const float *v = td.value;

    uint32_t prefix = 0, mask = 0;
    int remaining = k;   // how many of the keys matching `prefix` still to take
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t key = order_key(v[i]);
            if ((key & mask) == prefix)
                atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            int cum = 0;
            uint32_t dsel = 0;
            for (int dg = 255; dg >= 0; --dg) {
                const int h = (int)hist[dg];
                if (cum + h >= remaining) {
                    dsel = (uint32_t)dg;
                    break;
                }
                cum += h;
            }
            s_digit = dsel;
            s_above = cum;
        }
        __syncthreads();
        prefix |= s_digit << shift;
        mask |= 255u << shift;
        remaining -= s_above;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int n_gt = k - remaining;   // keys strictly above T, all taken

    // Ordered selection of the ties: thread t scans indices [t*chunk, ...).
    const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
    const int b = min(n, tid * chunk), e = min(n, b + chunk);
    int eq = 0;
    for (int i = b; i < e; ++i)
        eq += order_key(v[i]) == T ? 1 : 0;
    scan[tid] = eq;
    if (tid == 0)
        s_gt = 0;
    __syncthreads();
    for (int off = 1; off < kTopkThreads; off <<= 1) {   // inclusive Hillis-Steele scan
        const int add = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
    }
    int rank = scan[tid] - eq;   // ties before this thread's range
    for (int i = b; i < e; ++i) {
        const uint32_t key = order_key(v[i]);
        const unsigned long long packed =
            ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
        if (key > T) {
            sel[atomicAdd(&s_gt, 1)] = packed;
        } else if (key == T) {
            if (rank < remaining)
                sel[n_gt + rank] = packed;
            ++rank;
        }
    }
    int P = 1;
    while (P < k)
        P <<= 1;
    for (int i = k + tid; i < P; i += kTopkThreads)
        sel[i] = 0ull;   // below every real entry
    __syncthreads();

    // Bitonic sort, descending.
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < P / 2; t += kTopkThreads) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long x = sel[lo], y = sel[hi];
                if ((x < y) == desc) {
                    sel[lo] = y;
                    sel[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < k; i += kTopkThreads)
        td.idx[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(sel[i] & 0xFFFFFFFFull));
}

__global__ void __launch_bounds__(kTopkThreads) topk_one_kernel(const TopkDesc td) { topk_body(td); }

__global__ void __launch_bounds__(kTopkThreads) topk_batched_kernel(const TopkDesc *descs)
{
    topk_body(descs[blockIdx.x]);
}

hipError_t launch_topk_one(const TopkDesc &td, hipStream_t stream)
{
    hipLaunchKernelGGL(topk_one_kernel, dim3(1), dim3(kTopkThreads), 0, stream, td);
    return hipGetLastError();
}

hipError_t launch_topk_batched(const TopkDesc *descs, int n, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(topk_batched_kernel, dim3(n), dim3(kTopkThreads), 0, stream, descs);
    return hipGetLastError();
}

}  // namespace crkv
