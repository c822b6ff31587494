// Top-k selection over the impact vector for gfx950 (CacheBlend summary,
// selective-recompute listing: topk over the document slice of the impact,
// k = max(1, int(N_doc * r))).
//
// One workgroup of 1024 threads per vector. The fp32 values are mapped to
// unsigned keys that order like the floats (-0 below +0). Radix select then
// finds the k-th largest key T, eight bits at a time, starting below the bits
// every key shares (the common prefix of the minimum and maximum keys), so the
// first histogram is spread over many bins even when all values have the same
// sign and a narrow exponent range. Histograms are private per wave to keep
// LDS atomic contention low. Every key above T is taken; of the keys equal to
// T the lowest indices are taken (an ordered scan over contiguous index
// ranges, one per thread). The k winners are sorted by (key descending, index
// ascending) with a bitonic network in LDS, packed as 64-bit words
// (key << 32 | ~index) so that one descending sort gives both orders.
#include <hip/hip_runtime.h>

#include "crkv_internal.h"

namespace crkv {

__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkLdsKeys = 16384;   // vectors up to this length are held in LDS

// Inclusive prefix sum over the workgroup (every thread calls it).
__device__ __forceinline__ int block_inclusive_scan(int x, int *wave_tot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        wave_tot[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w)
        before += wave_tot[w];
    __syncthreads();
    return x + before;
}

__device__ void topk_body(const TopkDesc td)
{
    __shared__ uint32_t keys[kTopkLdsKeys];
    __shared__ uint32_t whist[kTopkWaves][256];
    __shared__ unsigned long long sel[kTopkMaxK];
    __shared__ int wave_tot[kTopkWaves];
    __shared__ uint32_t red_min[kTopkWaves], red_max[kTopkWaves];
    __shared__ uint32_t s_digit;
    __shared__ int s_above, s_gt;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = td.n, k = td.k;
    const bool in_lds = n <= kTopkLdsKeys;
    auto key_at = [&](int i) -> uint32_t { return in_lds ? keys[i] : order_key(td.value[i]); };

    // keys, and the common prefix of all of them
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t kk = order_key(td.value[i]);
        if (in_lds)
            keys[i] = kk;
        mn = min(mn, kk);
        mx = max(mx, kk);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    }
    if (lane == 0) {
        red_min[wave] = mn;
        red_max[wave] = mx;
    }
    __syncthreads();
    mn = red_min[0];
    mx = red_max[0];
    for (int w = 1; w < kTopkWaves; ++w) {
        mn = min(mn, red_min[w]);
        mx = max(mx, red_max[w]);
    }
    int shift = (mn == mx) ? 0 : 32 - __clz((int)(mn ^ mx));   // bits below the common prefix
    uint32_t pmask = shift >= 32 ? 0u : ~((1u << shift) - 1u);
    uint32_t prefix = mn & pmask;
    int remaining = k;   // keys still to take among those matching `prefix`

    while (shift > 0) {
        const int bits = shift >= 8 ? 8 : shift;
        shift -= bits;
        const uint32_t dmask = (1u << bits) - 1u;
        for (int b = lane; b < 256; b += 64)
            whist[wave][b] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t kk = key_at(i);
            if ((kk & pmask) == prefix)
                atomicAdd(&whist[wave][(kk >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l owns digits 255-4l .. 252-4l (scanning from the top)
            int c[4], tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dg = 255 - 4 * lane - q;
                int h = 0;
                for (int w = 0; w < kTopkWaves; ++w)
                    h += (int)whist[w][dg];
                c[q] = h;
                tot += h;
            }
            int incl = tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (lane >= off)
                    incl += y;
            }
            int cum = incl - tot;   // keys in higher digits than this lane's first
            const unsigned long long hit = __ballot(incl >= remaining);
            const int first = __ffsll((long long)hit) - 1;   // lowest lane reaching `remaining`
            if (lane == first) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (cum + c[q] >= remaining) {
                        s_digit = (uint32_t)(255 - 4 * lane - q);
                        s_above = cum;
                        break;
                    }
                    cum += c[q];
                }
            }
        }
        __syncthreads();
        prefix |= s_digit << shift;
        pmask |= dmask << shift;
        remaining -= s_above;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int n_gt = k - remaining;   // keys strictly above T: all taken

    // ordered selection of the ties: thread t scans indices [t*chunk, ...)
    const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
    const int b = min(n, tid * chunk), e = min(n, b + chunk);
    int eq = 0;
    for (int i = b; i < e; ++i)
        eq += key_at(i) == T ? 1 : 0;
    if (tid == 0)
        s_gt = 0;
    int rank = block_inclusive_scan(eq, wave_tot) - eq;
    for (int i = b; i < e; ++i) {
        const uint32_t kk = key_at(i);
        const unsigned long long packed =
            ((unsigned long long)kk << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
        if (kk > T) {
            sel[atomicAdd(&s_gt, 1)] = packed;   // any order: the sort orders them
        } else if (kk == T) {
            if (rank < remaining)
                sel[n_gt + rank] = packed;
            ++rank;
        }
    }
    int P = 128;   // at least one 128-entry block (see the sort)
    while (P < k)
        P <<= 1;
    for (int i = k + tid; i < P; i += kTopkThreads)
        sel[i] = 0ull;   // below every real entry
    __syncthreads();

    // Bitonic sort, descending, of P = 2^j >= 128 entries. Stages whose
    // stride is at least 128 compare entries of different 128-entry blocks
    // and go through LDS with a barrier each. The others stay inside a block:
    // wave w holds block w (and w + 16, ...) in registers, lane l entries l
    // and l + 64, and such a run of stages is done with lane shuffles and no
    // LDS traffic.
    auto reg_run = [&](int size_lo, int size_hi, int stride_first) {
        for (int blk = wave; blk < P / 128; blk += kTopkWaves) {
            const int base = blk * 128;
            unsigned long long x0 = sel[base + lane], x1 = sel[base + lane + 64];
            const int i0 = base + lane, i1 = i0 + 64;
            for (int size = size_lo; size <= size_hi; size <<= 1) {
                for (int stride = (size == size_lo ? stride_first : size >> 1); stride > 0; stride >>= 1) {
                    if (stride == 64) {   // pair (i0, i1) of this lane
                        const bool desc = (i0 & size) == 0;
                        if ((x0 < x1) == desc) {
                            const unsigned long long t = x0;
                            x0 = x1;
                            x1 = t;
                        }
                    } else {
                        const unsigned long long y0 = __shfl_xor(x0, stride), y1 = __shfl_xor(x1, stride);
                        const bool lo = (lane & stride) == 0;
                        // the lower position of a pair keeps the larger entry in a descending block
                        const bool max0 = lo == ((i0 & size) == 0), max1 = lo == ((i1 & size) == 0);
                        x0 = max0 ? (x0 > y0 ? x0 : y0) : (x0 < y0 ? x0 : y0);
                        x1 = max1 ? (x1 > y1 ? x1 : y1) : (x1 < y1 ? x1 : y1);
                    }
                }
            }
            sel[base + lane] = x0;
            sel[base + lane + 64] = x1;
        }
        __syncthreads();
    };
    reg_run(2, 128, 1);   // every stage of the sizes up to 128
    for (int size = 256; size <= P; size <<= 1) {
        int stride = size >> 1;
        for (; stride >= 128; stride >>= 1) {
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
        reg_run(size, size, 64);
    }
    __syncthreads();
    for (int i = tid; i < k; i += kTopkThreads)
        td.idx[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(sel[i] & 0xFFFFFFFFull));
}

__global__ void __launch_bounds__(kTopkThreads) topk_one_kernel(const TopkDesc td) { topk_body(td); }

__global__ void __launch_bounds__(kTopkThreads) topk_batched_kernel(const TopkDesc *descs)
{
    topk_body(descs[blockIdx.x]);
}

__global__ void __launch_bounds__(kTopkThreads) topk_inline_kernel(const TopkInline t)
{
    topk_body(t.d[blockIdx.x]);
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

hipError_t launch_topk_inline(const TopkDesc *descs, int n, hipStream_t stream)
{
    if (n <= 0 || n > kTopkInline)
        return hipErrorInvalidValue;
    TopkInline t{};
    for (int i = 0; i < n; ++i)
        t.d[i] = descs[i];
    hipLaunchKernelGGL(topk_inline_kernel, dim3(n), dim3(kTopkThreads), 0, stream, t);
    return hipGetLastError();
}

}  // namespace crkv
